// Depthwise causal convolution (kernel size 4) of the Mamba-2 layer over its
// x|B|C channels, with the split into the scan's three inputs.
//
// What is computed (Mamba-3-Lite block page, section 5.1 "Zero causal
// convolution": Mamba-1/2 mix each channel's positions t-3 .. t with learned
// weights before the scan):
//   v[b,t,c]   = bias[c] + sum_j w[c,j] in[b, t-3+j, c]      (j = 0..3)
//   out[b,t,c] = SiLU(v) = v / (1 + e^-v)  when act = 1, else v
// with in[b,p,c] for p < 0 taken from the carried state (the 3 raw inputs
// that preceded the segment).  Channel c < HP goes to x, the next GN to B,
// the last GN to C, each written contiguous, (Bsz,T,HP) and (Bsz,T,GN).
//
// The operation streams: 4 FLOPs per input element against 4 (bf16) or 8
// (fp32) bytes moved, so HBM bandwidth bounds it.  A thread owns one 16-byte
// vector of channels (8 bf16 or 4 fp32) over a run of TT tokens: it issues all
// TT + 3 row loads at once (3 halo rows before the run) and keeps the
// 3-position window in registers, so each input row is read once from HBM
// (the halo rows of a run are the last rows of the neighbouring wave's run,
// served by the cache).  A wave covers 64 consecutive vectors of one row, so
// every load and store instruction touches 1 KiB (bf16) contiguous bytes.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_chunk_common.h"
#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {

namespace {

constexpr int kConvK = 4;     // taps
constexpr int kConvTT = 8;    // tokens per thread (measured: 8 beats 4, 12, 16 and 32)
constexpr int kRunsPerBlock = 4;  // one run per wave

template <typename TIn>
struct ConvVec;
template <>
struct ConvVec<float> {
  static constexpr int V = 4;  // channels per 16-byte vector
  __device__ static void widen(uint4 r, float* f) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
  __device__ static uint4 narrow(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <>
struct ConvVec<uint16_t> {
  static constexpr int V = 8;
  __device__ static void widen(uint4 r, float* f) {
    const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(u[i] << 16);
      f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
  __device__ static uint4 narrow(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

// SiLU(v) = v / (1 + e^-v) from the hardware base-2 exponential and
// reciprocal (about 1 ulp each; v_exp_f32 gives +inf for v << 0, whose
// reciprocal 0 gives the limit -0, and 0 for v >> 0, giving v).  The
// correctly rounded division and libm exp cost ~20 VALU instructions per
// element, which made the kernel VALU-bound.
template <bool SILU>
__device__ __forceinline__ float conv_act(float v) {
  if (SILU) {
    const float e = __builtin_amdgcn_exp2f(v * -1.4426950408889634f);
    return v * __builtin_amdgcn_rcpf(1.0f + e);
  }
  return v;
}

// Grid: x = channel blocks of 64 vectors, y = blocks of 4 token runs, z = batch.
// Straight-line code: every load and store is a buffer access whose offset is
// pushed out of range where it must not happen (loads there return zero,
// stores are dropped), so no access sits in a branch and the waits on the
// token rows count down one row at a time, overlapping each row's arithmetic
// with the loads still in flight.
template <typename TIn, bool SILU>
__global__ __launch_bounds__(256) void ssd_conv1d_kernel(
    const TIn* __restrict__ xbc, int ld, const float* __restrict__ w,
    const float* __restrict__ bias, const float* __restrict__ state_in, TIn* __restrict__ xo,
    TIn* __restrict__ bo, TIn* __restrict__ co, float* __restrict__ state_out, int T, int HP,
    int GN, const int* __restrict__ cu) {
  using CV = ConvVec<TIn>;
  constexpr int V = CV::V;
  constexpr int ES = sizeof(TIn);
  constexpr uint32_t kOOB = 0xFFFFFFF0u;
  const int Ch = HP + 2 * GN;
  const int vec = blockIdx.x * kWave + (threadIdx.x & (kWave - 1));
  const bool active = vec * V < Ch;
  const int c0 = active ? vec * V : 0;
  const int b = blockIdx.z;
  // the sequence's rows: b of Bsz sequences of T tokens, or (variable
  // lengths) the rows cu[b] .. cu[b+1]-1 of the packed batch
  size_t row0 = static_cast<size_t>(b) * T;
  if (cu) {
    row0 = static_cast<size_t>(cu[b]);
    T = cu[b + 1] - cu[b];
  }
  const int run = blockIdx.y * kRunsPerBlock + wave_id();
  const int t0 = run * kConvTT;
  const int nruns = T > 0 ? (T + kConvTT - 1) / kConvTT : 1;
  if (run >= nruns) return;  // wave-uniform; no LDS, no barriers

  // taps and bias first, so that the waits below count down over the rows
  const buf_t wb = make_buf(w, static_cast<uint32_t>(Ch) * kConvK * 4);
  const buf_t bb = make_buf(bias, bias ? static_cast<uint32_t>(Ch) * 4 : 0u);
  uint4 wq[V], bq[V / 4];
#pragma unroll
  for (int v = 0; v < V; ++v)
    wq[v] = buf_load16(wb, active ? static_cast<uint32_t>(c0 + v) * kConvK * 4 : kOOB);
#pragma unroll
  for (int v = 0; v < V / 4; ++v)
    bq[v] = buf_load16(bb, active ? static_cast<uint32_t>(c0 + 4 * v) * 4 : kOOB);

  // the 3 positions before the run: positions >= 0 from the rows, < 0 from
  // the carried state (a NULL state is an empty range: zeros)
  const buf_t xb = make_buf(xbc + row0 * ld,
                            static_cast<uint32_t>(static_cast<size_t>(T) * ld * ES));
  const buf_t sb = make_buf(state_in + static_cast<size_t>(b) * (kConvK - 1) * Ch,
                            state_in ? static_cast<uint32_t>(kConvK - 1) * Ch * 4 : 0u);
  auto row_off = [&](int p) -> uint32_t {
    return (p >= 0 && active) ? static_cast<uint32_t>((static_cast<size_t>(p) * ld + c0) * ES)
                              : kOOB;
  };
  auto state_off = [&](int p, int v) -> uint32_t {
    return (p < 0 && active)
               ? static_cast<uint32_t>(((kConvK - 1 + p) * static_cast<size_t>(Ch) + c0 + v) * 4)
               : kOOB;
  };
  uint4 sq[kConvK - 1][V / 4], hr[kConvK - 1], rr[kConvTT];
#pragma unroll
  for (int j = 0; j < kConvK - 1; ++j) {
    const int p = t0 - (kConvK - 1) + j;
#pragma unroll
    for (int v = 0; v < V / 4; ++v) sq[j][v] = buf_load16(sb, state_off(p, 4 * v));
    hr[j] = buf_load16(xb, row_off(p));
  }
#pragma unroll
  for (int i = 0; i < kConvTT; ++i) rr[i] = buf_load16(xb, row_off(t0 + i));

  float wt[V][kConvK], bs[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    wt[v][0] = __uint_as_float(wq[v].x);
    wt[v][1] = __uint_as_float(wq[v].y);
    wt[v][2] = __uint_as_float(wq[v].z);
    wt[v][3] = __uint_as_float(wq[v].w);
  }
#pragma unroll
  for (int v = 0; v < V / 4; ++v) {
    bs[4 * v] = __uint_as_float(bq[v].x);
    bs[4 * v + 1] = __uint_as_float(bq[v].y);
    bs[4 * v + 2] = __uint_as_float(bq[v].z);
    bs[4 * v + 3] = __uint_as_float(bq[v].w);
  }
  // window of the 3 positions before the current token (one of the two loads
  // of each position is zero)
  float win[kConvK - 1][V];
#pragma unroll
  for (int j = 0; j < kConvK - 1; ++j) {
    CV::widen(hr[j], win[j]);
#pragma unroll
    for (int v = 0; v < V / 4; ++v) {
      win[j][4 * v] += __uint_as_float(sq[j][v].x);
      win[j][4 * v + 1] += __uint_as_float(sq[j][v].y);
      win[j][4 * v + 2] += __uint_as_float(sq[j][v].z);
      win[j][4 * v + 3] += __uint_as_float(sq[j][v].w);
    }
  }

  // outputs of this batch entry; rows at or past T are out of range
  const buf_t xob = make_buf(xo + row0 * HP,
                             static_cast<uint32_t>(static_cast<size_t>(T) * HP * ES));
  const buf_t bob = make_buf(bo + row0 * GN,
                             static_cast<uint32_t>(static_cast<size_t>(T) * GN * ES));
  const buf_t cob = make_buf(co + row0 * GN,
                             static_cast<uint32_t>(static_cast<size_t>(T) * GN * ES));
  // a block whose vectors all lie in x issues one store per token; the block
  // holding the x|B|C boundary issues three, each lane's offset in range for
  // one of them
  const bool all_x = static_cast<int>(blockIdx.x + 1) * kWave * V <= HP;
  const bool in_x = active && c0 < HP;
  const bool in_b = active && c0 >= HP && c0 < HP + GN;
  const bool in_c = active && c0 >= HP + GN;

#pragma unroll
  for (int i = 0; i < kConvTT; ++i) {
    float cur[V], o[V];
    CV::widen(rr[i], cur);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float a = bs[v];
      a = fmaf(wt[v][0], win[0][v], a);
      a = fmaf(wt[v][1], win[1][v], a);
      a = fmaf(wt[v][2], win[2][v], a);
      a = fmaf(wt[v][3], cur[v], a);
      o[v] = conv_act<SILU>(a);
    }
    const uint4 ov = CV::narrow(o);
    const uint32_t t = static_cast<uint32_t>(t0 + i);
    if (all_x) {
      buf_store16(xob, (t * HP + c0) * ES, ov);
    } else {
      buf_store16(xob, in_x ? (t * HP + c0) * ES : kOOB, ov);
      buf_store16(bob, in_b ? (t * GN + (c0 - HP)) * ES : kOOB, ov);
      buf_store16(cob, in_c ? (t * GN + (c0 - HP - GN)) * ES : kOOB, ov);
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      win[0][v] = win[1][v];
      win[1][v] = win[2][v];
      win[2][v] = cur[v];
    }
  }

  // the wave of the last run writes the raw inputs at positions T-3 .. T-1
  if (state_out && run == nruns - 1) {
    const buf_t ob = make_buf(state_out + static_cast<size_t>(b) * (kConvK - 1) * Ch,
                              static_cast<uint32_t>(kConvK - 1) * Ch * 4);
#pragma unroll
    for (int j = 0; j < kConvK - 1; ++j) {
      const int p = T - (kConvK - 1) + j;
      float f[V];
      CV::widen(buf_load16(xb, row_off(p)), f);
#pragma unroll
      for (int v = 0; v < V / 4; ++v) {
        const uint4 q = buf_load16(sb, state_off(p, 4 * v));
        const uint32_t off =
            active ? static_cast<uint32_t>((j * static_cast<size_t>(Ch) + c0 + 4 * v) * 4) : kOOB;
        buf_store16(ob, off,
                    make_uint4(__float_as_uint(f[4 * v] + __uint_as_float(q.x)),
                               __float_as_uint(f[4 * v + 1] + __uint_as_float(q.y)),
                               __float_as_uint(f[4 * v + 2] + __uint_as_float(q.z)),
                               __float_as_uint(f[4 * v + 3] + __uint_as_float(q.w))));
      }
    }
  }
}

// One token per sequence, in place on the fp32 state (Bsz, 3, Ch): a thread
// owns 4 channels of kStepRows consecutive sequences.  One sequence per thread
// measured faster than four (more waves in flight for a 36 MB step at the
// BitMamba decode batch; the taps come from the cache either way).
// Grid: x = channel blocks of 256 vectors, y = groups of kStepRows sequences.
constexpr int kStepRows = 1;

template <bool SILU>
__global__ __launch_bounds__(256) void ssd_conv1d_step_kernel(
    float* __restrict__ state, const float* __restrict__ xt, int ld, const float* __restrict__ w,
    const float* __restrict__ bias, float* __restrict__ xo, float* __restrict__ bo,
    float* __restrict__ co, int Bsz, int HP, int GN) {
  const int Ch = HP + 2 * GN;
  const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (c0 >= Ch) return;
  const int b0 = blockIdx.y * kStepRows;
  float4 q[kConvK];
#pragma unroll
  for (int v = 0; v < 4; ++v)
    q[v] = *reinterpret_cast<const float4*>(w + static_cast<size_t>(c0 + v) * kConvK);
  float4 bq = make_float4(0.f, 0.f, 0.f, 0.f);
  if (bias) bq = *reinterpret_cast<const float4*>(bias + c0);
  float4 s0[kStepRows], s1[kStepRows], s2[kStepRows], x[kStepRows];
#pragma unroll
  for (int r = 0; r < kStepRows; ++r) {
    const int b = min(b0 + r, Bsz - 1);  // rows past Bsz recompute the last one, not stored
    const float* s = state + static_cast<size_t>(b) * (kConvK - 1) * Ch + c0;
    s0[r] = *reinterpret_cast<const float4*>(s);
    s1[r] = *reinterpret_cast<const float4*>(s + Ch);
    s2[r] = *reinterpret_cast<const float4*>(s + 2 * Ch);
    x[r] = *reinterpret_cast<const float4*>(xt + static_cast<size_t>(b) * ld + c0);
  }
  const float bv[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
  for (int r = 0; r < kStepRows; ++r) {
    const int b = b0 + r;
    if (b >= Bsz) break;
    const float in[kConvK][4] = {{s0[r].x, s0[r].y, s0[r].z, s0[r].w},
                                 {s1[r].x, s1[r].y, s1[r].z, s1[r].w},
                                 {s2[r].x, s2[r].y, s2[r].z, s2[r].w},
                                 {x[r].x, x[r].y, x[r].z, x[r].w}};
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float a = bv[v];
      a = fmaf(q[v].x, in[0][v], a);
      a = fmaf(q[v].y, in[1][v], a);
      a = fmaf(q[v].z, in[2][v], a);
      a = fmaf(q[v].w, in[3][v], a);
      o[v] = conv_act<SILU>(a);
    }
    float* d = c0 < HP ? xo + static_cast<size_t>(b) * HP + c0
             : c0 < HP + GN ? bo + static_cast<size_t>(b) * GN + (c0 - HP)
                            : co + static_cast<size_t>(b) * GN + (c0 - HP - GN);
    *reinterpret_cast<float4*>(d) = make_float4(o[0], o[1], o[2], o[3]);
    float* s = state + static_cast<size_t>(b) * (kConvK - 1) * Ch + c0;
    *reinterpret_cast<float4*>(s) = s1[r];
    *reinterpret_cast<float4*>(s + Ch) = s2[r];
    *reinterpret_cast<float4*>(s + 2 * Ch) = x[r];
  }
}

// cu: the device copy of the sequence offsets (variable lengths; a.Bsz
// sequences, a.T the longest), or NULL
template <typename TIn>
void launch_conv(const ConvArgs& a, hipStream_t st, const int* cu) {
  constexpr int V = ConvVec<TIn>::V;
  const int Ch = a.HP + 2 * a.GN;
  const int nvec = Ch / V;
  const int nruns = a.T > 0 ? (a.T + kConvTT - 1) / kConvTT : 1;
  const dim3 grid((nvec + kWave - 1) / kWave, (nruns + kRunsPerBlock - 1) / kRunsPerBlock, a.Bsz);
  const TIn* x = static_cast<const TIn*>(a.xbc);
  TIn* xo = static_cast<TIn*>(a.x);
  TIn* bo = static_cast<TIn*>(a.B);
  TIn* co = static_cast<TIn*>(a.C);
  if (a.act)
    launch_k(true, ssd_conv1d_kernel<TIn, true>, grid, dim3(kThreads), st, a.events, x, a.ld, a.w,
             a.bias, a.state_in, xo, bo, co, a.state_out, a.T, a.HP, a.GN, cu);
  else
    launch_k(true, ssd_conv1d_kernel<TIn, false>, grid, dim3(kThreads), st, a.events, x, a.ld,
             a.w, a.bias, a.state_in, xo, bo, co, a.state_out, a.T, a.HP, a.GN, cu);
}

}  // namespace

int conv_tokens_per_thread() { return kConvTT; }

hipError_t run_conv1d(const ConvArgs& a, hipStream_t st) {
  if (a.dtype == 1)
    launch_conv<uint16_t>(a, st, nullptr);
  else
    launch_conv<float>(a, st, nullptr);
  return hipGetLastError();
}

hipError_t run_conv1d_varlen(const ConvArgs& a, const int* cu, void* workspace, hipStream_t st) {
  // the offsets go to the workspace (the call returns once the copy has the
  // host data); a.Bsz = nseq, a.T = the longest sequence
  hipError_t e = hipMemcpyAsync(workspace, cu, (static_cast<size_t>(a.Bsz) + 1) * sizeof(int),
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  const int* cud = static_cast<const int*>(workspace);
  if (a.dtype == 1)
    launch_conv<uint16_t>(a, st, cud);
  else
    launch_conv<float>(a, st, cud);
  return hipGetLastError();
}

hipError_t run_conv1d_step(const ConvArgs& a, hipStream_t st) {
  const int Ch = a.HP + 2 * a.GN;
  const dim3 grid((Ch / 4 + kThreads - 1) / kThreads, (a.Bsz + kStepRows - 1) / kStepRows);
  float* state = a.state_out;  // in place
  const float* xt = static_cast<const float*>(a.xbc);
  float* xo = static_cast<float*>(a.x);
  float* bo = static_cast<float*>(a.B);
  float* co = static_cast<float*>(a.C);
  if (a.act)
    launch_k(true, ssd_conv1d_step_kernel<true>, grid, dim3(kThreads), st, a.events, state, xt,
             a.ld, a.w, a.bias, xo, bo, co, a.Bsz, a.HP, a.GN);
  else
    launch_k(true, ssd_conv1d_step_kernel<false>, grid, dim3(kThreads), st, a.events, state, xt,
             a.ld, a.w, a.bias, xo, bo, co, a.Bsz, a.HP, a.GN);
  return hipGetLastError();
}

}  // namespace ssd
