// Single-token recurrent decode step on gfx950 (the recurrence of the
// Mamba-3-Lite README applied once, real Mamba-2 form):
//   h[b,h,p,:] <- exp(A_h delta) h[b,h,p,:] + delta x[b,h,p] B[b,g,:]
//   y[b,h,p]    = h[b,h,p,:] . C[b,g,:] + D_h x[b,h,p]
// One workgroup per (b, h).  A row of N state values is spread over N/4
// consecutive lanes, one float4 each, so every load and store is a 16-byte
// coalesced access; the workgroup walks its P rows with 8 rows in flight per
// thread.  The dot product with C is reduced across the row's lanes with
// cross-lane shuffles.  The state is read once and written once: the kernel
// is bound by HBM bandwidth.  Its loads and stores are nontemporal (each state
// byte is touched once per step; nothing else is displaced from the caches).

#include "ssd_chunk_common.h"

namespace ssd {

typedef float f4v __attribute__((ext_vector_type(4)));

template <int N>
__global__ __launch_bounds__(kThreads) void ssd_decode_kernel(
    float* __restrict__ h, const float* __restrict__ x, const float* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ C,
    const float* __restrict__ D, const float* __restrict__ dt_bias, float lo, float hi,
    float* __restrict__ y, int H, int P, int G) {
  constexpr int LPR = N / 4;            // lanes per state row
  constexpr int RPP = kThreads / LPR;   // rows covered by one pass of the block
  constexpr int UNR = 8;                // rows in flight per thread
  const int bh = blockIdx.x;
  const int b = bh / H, hh = bh % H, g = hh / (H / G);
  const int col = threadIdx.x % LPR, rsub = threadIdx.x / LPR;

  const float delta = step_size(dt[bh], dt_bias ? dt_bias[hh] : 0.0f, lo, hi);
  const float a = __expf(A[hh] * delta);
  const float Dh = D ? D[hh] : 0.0f;
  const float4 bv = *reinterpret_cast<const float4*>(B + (static_cast<size_t>(b) * G + g) * N + col * 4);
  const float4 cv = *reinterpret_cast<const float4*>(C + (static_cast<size_t>(b) * G + g) * N + col * 4);
  float* hrow = h + static_cast<size_t>(bh) * P * N + col * 4;
  const float* xr = x + static_cast<size_t>(bh) * P;
  float* yr = y + static_cast<size_t>(bh) * P;

  for (int r0 = rsub; r0 < P; r0 += UNR * RPP) {
    float4 v[UNR];
    float xv[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int r = r0 + k * RPP;
      if (r < P) {
        const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(hrow + static_cast<size_t>(r) * N));
        v[k] = make_float4(t.x, t.y, t.z, t.w);
        xv[k] = xr[r];
      }
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int r = r0 + k * RPP;
      float part = 0.0f;
      if (r < P) {
        const float u = delta * xv[k];
        float4 n;
        n.x = a * v[k].x + u * bv.x;
        n.y = a * v[k].y + u * bv.y;
        n.z = a * v[k].z + u * bv.z;
        n.w = a * v[k].w + u * bv.w;
        __builtin_nontemporal_store(f4v{n.x, n.y, n.z, n.w},
                                    reinterpret_cast<f4v*>(hrow + static_cast<size_t>(r) * N));
        part = n.x * cv.x + n.y * cv.y + n.z * cv.z + n.w * cv.w;
      }
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, kWave);
      if (r < P && col == 0) yr[r] = part + Dh * xv[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Complex form (the complex promotion of the recurrence in the Mamba-3-Lite
// README), one token:
//   h[b,h,p,n] <- e^{(alpha_h + i beta_h) delta} h[b,h,p,n] + B[b,g,n] x[b,h,p]
//   y[b,h,p]    = Re(sum_n C[b,g,n] h[b,h,p,n])
// with no step factor on the input and no D (the readings of the complex
// forward).  The state is complex64, (re, im) pairs, so a row of N values is
// 8N bytes: N/2 lanes, one float4 (two complex values) each; the layout,
// schedule and nontemporal state traffic are those of the real kernel.
// ---------------------------------------------------------------------------
template <int N>
__global__ __launch_bounds__(kThreads) void ssd_complex_decode_kernel(
    float* __restrict__ h, const float* __restrict__ x, const float* __restrict__ dt,
    const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ C,
    const float* __restrict__ dt_bias, float lo, float hi, float* __restrict__ y, int H, int P,
    int G) {
  constexpr int LPR = N / 2;            // lanes per state row
  constexpr int RPP = kThreads / LPR;   // rows covered by one pass of the block
  constexpr int UNR = 8;                // rows in flight per thread
  const int bh = blockIdx.x;
  const int b = bh / H, hh = bh % H, g = hh / (H / G);
  const int col = threadIdx.x % LPR, rsub = threadIdx.x / LPR;

  // a = e^{alpha delta} (cos beta delta, sin beta delta)
  const float delta = step_size(dt[bh], dt_bias ? dt_bias[hh] : 0.0f, lo, hi);
  const float mag = __expf(A[2 * hh] * delta);
  float ca, sa;
  rot_cs(static_cast<double>(A[2 * hh + 1]) * static_cast<double>(delta), ca, sa);
  const float ar = mag * ca, ai = mag * sa;
  // this lane's two complex values of B and C: (re, im, re, im)
  const float4 bv = *reinterpret_cast<const float4*>(B + (static_cast<size_t>(b) * G + g) * N * 2 + col * 4);
  const float4 cv = *reinterpret_cast<const float4*>(C + (static_cast<size_t>(b) * G + g) * N * 2 + col * 4);
  float* hrow = h + static_cast<size_t>(bh) * P * N * 2 + col * 4;
  const float* xr = x + static_cast<size_t>(bh) * P;
  float* yr = y + static_cast<size_t>(bh) * P;

  for (int r0 = rsub; r0 < P; r0 += UNR * RPP) {
    float4 v[UNR];
    float xv[UNR];
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int r = r0 + k * RPP;
      if (r < P) {
        const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(hrow + static_cast<size_t>(r) * N * 2));
        v[k] = make_float4(t.x, t.y, t.z, t.w);
        xv[k] = xr[r];
      }
    }
#pragma unroll
    for (int k = 0; k < UNR; ++k) {
      const int r = r0 + k * RPP;
      float part = 0.0f;
      if (r < P) {
        const float u = xv[k];
        float4 n;
        n.x = ar * v[k].x - ai * v[k].y + u * bv.x;
        n.y = ar * v[k].y + ai * v[k].x + u * bv.y;
        n.z = ar * v[k].z - ai * v[k].w + u * bv.z;
        n.w = ar * v[k].w + ai * v[k].z + u * bv.w;
        __builtin_nontemporal_store(f4v{n.x, n.y, n.z, n.w},
                                    reinterpret_cast<f4v*>(hrow + static_cast<size_t>(r) * N * 2));
        part = (cv.x * n.x - cv.y * n.y) + (cv.z * n.z - cv.w * n.w);  // Re(c h), two values
      }
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, kWave);
      if (r < P && col == 0) yr[r] = part;
    }
  }
}

hipError_t run_complex_decode(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.Bsz * a.H);
#define SSD_CDECODE_CASE(NN)                                                                       \
  case NN:                                                                                        \
    launch_k(true, ssd_complex_decode_kernel<NN>, grid, dim3(kThreads), st, a.events, a.h, a.x,     \
             a.dt, a.A, a.B, a.C, a.dt_bias, a.dt_min, a.dt_max, a.y, a.H, a.P, a.G);               \
    break;
  switch (a.N) {
    SSD_CDECODE_CASE(16)
    SSD_CDECODE_CASE(32)
    SSD_CDECODE_CASE(64)
    SSD_CDECODE_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef SSD_CDECODE_CASE
  return hipGetLastError();
}

hipError_t run_decode(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.Bsz * a.H);
#define SSD_DECODE_CASE(NN)                                                                  \
  case NN:                                                                                   \
    launch_k(true, ssd_decode_kernel<NN>, grid, dim3(kThreads), st, a.events, a.h, a.x, a.dt,  \
             a.A, a.B, a.C, a.D, a.dt_bias, a.dt_min, a.dt_max, a.y, a.H, a.P, a.G);         \
    break;
  switch (a.N) {
    SSD_DECODE_CASE(16)
    SSD_DECODE_CASE(32)
    SSD_DECODE_CASE(64)
    SSD_DECODE_CASE(128)
    SSD_DECODE_CASE(256)
    default:
      return hipErrorInvalidValue;
  }
#undef SSD_DECODE_CASE
  return hipGetLastError();
}

}  // namespace ssd
