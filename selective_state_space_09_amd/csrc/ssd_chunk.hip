// Chunked SSD forward on gfx950: three kernels per call.
//
//   ssd_state_kernel  one workgroup per (chunk c, head h, batch b): the state a
//                     chunk leaves behind when it starts from zero,
//                     S_c = sum_s w_s x_s (x) B_s  (MFMA, contraction over s),
//                     plus the chunk's total decay factor.
//   ssd_pass_kernel   the inter-chunk recurrence h_in(c+1) = decay_c h_in(c)
//                     + S_c, sequential over chunks and parallel over the
//                     (b, h, p, n) state elements; h_in(c) overwrites S_c.
//   ssd_scan_kernel   one workgroup per (c, h, b): the output of the chunk,
//                     y = ((C B^T) o L) (delta x) + e^{cs} C h_in(c) + D x,
//                     with both products on MFMA and y written once.
//
// The chunkwise algebra is the one of "Numerical Stability in Mamba-3-Lite",
// section 4: L[l,s] = exp(cs_l - cs_s) 1[l >= s] inside a chunk, and chunk
// ends carried across chunks by their total log-decay.  The pages carry all
// earlier chunks at once through a strictly lower-triangular chunk-decay
// matrix; here the carry is the equivalent linear scan, one state per chunk.
//
// The step-size gate and the per-chunk cumulative sums are a prologue of the
// state and scan kernels (each workgroup recomputes them for its own chunk from
// dt): the cumulative sums run in double, so decay exponents spread over
// hundreds of units keep fp32 accuracy in their differences.
//
// Complex form (Mamba-3-Lite): with u_l the cumulative step inside the chunk
// and theta_l = beta u_l, exp(A (u_l - u_s)) = e^{alpha (u_l - u_s)}
// e^{i theta_l} e^{-i theta_s}.  Rotating C'_l = C_l e^{i theta_l} and
// B'_s = B_s e^{-i theta_s} turns the real part of the complex decay-weighted
// product into one real product with K = 2N:
//   Re(C'_l . B'_s) = [C'_re | C'_im] . [B'_re | -B'_im],
// so the complex path is the real kernel with K = 2N and no delta factor.

#include <type_traits>

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {

constexpr int kST = 64;  // tokens per LDS stage of the s (source) dimension

template <typename E>
struct Pad;
template <>
struct Pad<uint16_t> {
  static constexpr int row = 8;  // bf16 elements of padding per LDS row
};
template <>
struct Pad<float> {
  static constexpr int row = 4;
};

// ---------------------------------------------------------------------------
// Per-chunk prologue: step sizes and cumulative decay exponents.
//
// Thread l < Q handles token l of the chunk (l >= Lc is padding: step 0).
// Writes dl[l] (step size), cs_hi/cs_lo[l] (double-float of the inclusive
// cumulative exponent: A*sum(delta) real, alpha*sum(delta) complex) and, for
// the complex form, the cosine/sine of theta_l = beta * sum(delta).
// Returns the cumulative sum of this thread (double) and, through tot, the
// chunk total (u or A*u at the last token).
// ---------------------------------------------------------------------------
template <bool CPLX>
__device__ __forceinline__ double chunk_prologue(
    const float* __restrict__ dt, size_t dt_base, int H, int Lc, float a_re,
    float a_im, float bias, float lo, float hi, float* dl, float* cs_hi,
    float* cs_lo, float* cth, float* sth, double* wsum, double* tot, int Q) {
  const int l = threadIdx.x;
  float d = 0.0f;
  if (l < Lc) d = step_size(dt[dt_base + static_cast<size_t>(l) * H], bias, lo, hi);
  const double v = CPLX ? static_cast<double>(d)
                        : static_cast<double>(a_re) * static_cast<double>(d);
  const double cum = block_inclusive_scan(v, wsum);  // u (complex) or A*u (real)
  if (l < Q) {
    dl[l] = d;
    const double e = CPLX ? static_cast<double>(a_re) * cum : cum;
    const float ehi = static_cast<float>(e);
    cs_hi[l] = ehi;
    cs_lo[l] = static_cast<float>(e - static_cast<double>(ehi));
    if (CPLX) {
      float c, s;
      rot_cs(static_cast<double>(a_im) * cum, c, s);
      cth[l] = c;
      sth[l] = s;
    }
    if (l == Q - 1) *tot = cum;
  }
  __syncthreads();
  return cum;
}

// exp(cs_l - cs_s) from double-float exponents (both <= ~1e3 in magnitude).
__device__ __forceinline__ float decay_between(float hl, float ll, float hs, float ls) {
  return __expf((hl - hs) + (ll - ls));
}

// ---------------------------------------------------------------------------
// Staging helpers.  Tokens s in [s0, s0 + kST) of the chunk; rows past the
// chunk's valid length Lc are written as zeros.
// ---------------------------------------------------------------------------

// xT[p][s - s0] = x[b, t0 + s, h, p]   (transposed: s contiguous)
template <typename TI, int P>
__device__ __forceinline__ void stage_xT(TI* xT, const TI* __restrict__ x, size_t row0,
                                         size_t row_stride, int s0, int Lc) {
  constexpr int XP = kST + Pad<TI>::row;
  if constexpr (std::is_same<TI, uint16_t>::value) {
    // item = (pair of rows, 8 columns); two rows packed per 32-bit LDS write
    constexpr int NPG = P / 8;
    for (int it = threadIdx.x; it < (kST / 2) * NPG; it += kThreads) {
      const int pg = it % NPG, sp = it / NPG;
      const int s = s0 + 2 * sp;
      uint4 r0 = make_uint4(0, 0, 0, 0), r1 = make_uint4(0, 0, 0, 0);
      if (s < Lc) r0 = *reinterpret_cast<const uint4*>(x + row0 + s * row_stride + pg * 8);
      if (s + 1 < Lc)
        r1 = *reinterpret_cast<const uint4*>(x + row0 + (s + 1) * row_stride + pg * 8);
      const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
      const uint32_t b[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo_pair = (a[j] & 0xFFFFu) | (b[j] << 16);
        const uint32_t hi_pair = (a[j] >> 16) | (b[j] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(xT + (pg * 8 + 2 * j) * XP + 2 * sp) = lo_pair;
        *reinterpret_cast<uint32_t*>(xT + (pg * 8 + 2 * j + 1) * XP + 2 * sp) = hi_pair;
      }
    }
  } else {
    constexpr int NPG = P / 4;
    for (int it = threadIdx.x; it < kST * NPG; it += kThreads) {
      const int pg = it % NPG, sl = it / NPG;
      const int s = s0 + sl;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < Lc) v = *reinterpret_cast<const float4*>(x + row0 + s * row_stride + pg * 4);
      xT[(pg * 4 + 0) * XP + sl] = v.x;
      xT[(pg * 4 + 1) * XP + sl] = v.y;
      xT[(pg * 4 + 2) * XP + sl] = v.z;
      xT[(pg * 4 + 3) * XP + sl] = v.w;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 1: chunk-end states from a zero start.
// ---------------------------------------------------------------------------
template <typename TI, bool CPLX, int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const TI* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, float* __restrict__ states, float* __restrict__ decay, int T, int H,
    int G, int Q, int nc) {
  using E = TI;
  constexpr bool BF = std::is_same<E, uint16_t>::value;
  constexpr int KC = CPLX ? 2 * N : N;
  constexpr int XP = kST + Pad<E>::row;
  constexpr int NTILE = (P / 16) * (KC / 16);
  constexpr int TPW = (NTILE + 3) / 4;  // output tiles per wave

  __shared__ __attribute__((aligned(16))) E xT[P * XP];
  __shared__ __attribute__((aligned(16))) E bT[KC * XP];
  __shared__ float dl[256], cs_hi[256], cs_lo[256], cth[256], sth[256];
  __shared__ float wre[256], wim[256];
  __shared__ double wsum[4], tot;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const float a_re = CPLX ? A[2 * h] : A[h];
  const float a_im = CPLX ? A[2 * h + 1] : 0.0f;
  const float bias = dt_bias ? dt_bias[h] : 0.0f;

  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const double cum = chunk_prologue<CPLX>(dt, dt_base, H, Lc, a_re, a_im, bias, dt_min,
                                          dt_max, dl, cs_hi, cs_lo, cth, sth, wsum, &tot, Q);
  // weights of each source token to the chunk end
  const int tid = threadIdx.x;
  const double total = tot;
  if (tid < Q) {
    const double rem = total - cum;  // >= 0 steps (complex) / exponent (real)
    if (CPLX) {
      const float mag = __expf(static_cast<float>(static_cast<double>(a_re) * rem));
      float cr, sr;
      rot_cs(static_cast<double>(a_im) * rem, cr, sr);
      wre[tid] = mag * cr;
      wim[tid] = mag * sr;
    } else {
      wre[tid] = __expf(static_cast<float>(rem)) * dl[tid];
    }
  }
  if (tid == 0) {
    float* dc = decay + ((static_cast<size_t>(b) * H + h) * nc + c) * 2;
    if (CPLX) {
      const float mag = __expf(static_cast<float>(static_cast<double>(a_re) * total));
      float cr, sr;
      rot_cs(static_cast<double>(a_im) * total, cr, sr);
      dc[0] = mag * cr;
      dc[1] = mag * sr;
    } else {
      dc[0] = __expf(static_cast<float>(total));
      dc[1] = 0.0f;
    }
  }
  __syncthreads();

  const int lane = tid & 63, wid = tid >> 6, q = lane >> 4, r16 = lane & 15;
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t x_row0 = (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P;
  const size_t x_rs = static_cast<size_t>(H) * P;
  const size_t b_row0 = (static_cast<size_t>(b) * T + t0) * G * N * (CPLX ? 2 : 1) +
                        static_cast<size_t>(g) * N * (CPLX ? 2 : 1);
  const size_t b_rs = static_cast<size_t>(G) * N * (CPLX ? 2 : 1);

  for (int s0 = 0; s0 < Lc; s0 += kST) {
    __syncthreads();
    stage_xT<E, P>(xT, x, x_row0, x_rs, s0, Lc);
    // bT[k][s - s0] = w_s B_s[k]  (complex: planar re | im of W_s B_s)
    if constexpr (CPLX) {
      constexpr int NG = N / 4;
      for (int it = tid; it < kST * NG; it += kThreads) {
        const int ng = it % NG, sl = it / NG, s = s0 + sl;
        float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
        if (s < Lc) {
          const float4* src = reinterpret_cast<const float4*>(Bm + b_row0 + s * b_rs + ng * 8);
          v0 = src[0];
          v1 = src[1];
        }
        const float wr = wre[s < Q ? s : 0], wi = wim[s < Q ? s : 0];
        const float br[4] = {v0.x, v0.z, v1.x, v1.z}, bi[4] = {v0.y, v0.w, v1.y, v1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bT[(ng * 4 + j) * XP + sl] = wr * br[j] - wi * bi[j];
          bT[(N + ng * 4 + j) * XP + sl] = wr * bi[j] + wi * br[j];
        }
      }
    } else if constexpr (BF) {
      constexpr int NG = N / 8;
      for (int it = tid; it < (kST / 2) * NG; it += kThreads) {
        const int ng = it % NG, sp = it / NG, s = s0 + 2 * sp;
        uint4 r0 = make_uint4(0, 0, 0, 0), r1 = r0;
        if (s < Lc) r0 = *reinterpret_cast<const uint4*>(Bm + b_row0 + s * b_rs + ng * 8);
        if (s + 1 < Lc)
          r1 = *reinterpret_cast<const uint4*>(Bm + b_row0 + (s + 1) * b_rs + ng * 8);
        const float w0 = s < Q ? wre[s] : 0.f, w1 = s + 1 < Q ? wre[s + 1] : 0.f;
        const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
        const uint32_t bb[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a_lo = bf16_bits_to_f32(a[j] & 0xFFFFu) * w0;
          const float a_hi = bf16_bits_to_f32(a[j] >> 16) * w0;
          const float b_lo = bf16_bits_to_f32(bb[j] & 0xFFFFu) * w1;
          const float b_hi = bf16_bits_to_f32(bb[j] >> 16) * w1;
          *reinterpret_cast<uint32_t*>(bT + (ng * 8 + 2 * j) * XP + 2 * sp) = pack_bf16x2(a_lo, b_lo);
          *reinterpret_cast<uint32_t*>(bT + (ng * 8 + 2 * j + 1) * XP + 2 * sp) = pack_bf16x2(a_hi, b_hi);
        }
      }
    } else {
      constexpr int NG = N / 4;
      for (int it = tid; it < kST * NG; it += kThreads) {
        const int ng = it % NG, sl = it / NG, s = s0 + sl;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (s < Lc) v = *reinterpret_cast<const float4*>(Bm + b_row0 + s * b_rs + ng * 4);
        const float w = s < Q ? wre[s] : 0.f;
        bT[(ng * 4 + 0) * XP + sl] = w * v.x;
        bT[(ng * 4 + 1) * XP + sl] = w * v.y;
        bT[(ng * 4 + 2) * XP + sl] = w * v.z;
        bT[(ng * 4 + 3) * XP + sl] = w * v.w;
      }
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wid + 4 * i;
      if (tile >= NTILE) break;
      const int pt = tile / (KC / 16), kt = tile % (KC / 16);
      const E* arow = xT + (pt * 16 + r16) * XP;
      const E* brow = bT + (kt * 16 + r16) * XP;
      if constexpr (BF) {
#pragma unroll
        for (int ss = 0; ss < kST; ss += 32) {
          const uint4 av = *reinterpret_cast<const uint4*>(arow + ss + 8 * q);
          const uint4 bv = *reinterpret_cast<const uint4*>(brow + ss + 8 * q);
          acc[i] = mfma_bf16(as_bf16x8(av), as_bf16x8(bv), acc[i]);
        }
      } else {
#pragma unroll
        for (int ss = 0; ss < kST; ss += 16) {
          const float4 av = *reinterpret_cast<const float4*>(arow + ss + 4 * q);
          const float4 bv = *reinterpret_cast<const float4*>(brow + ss + 4 * q);
          acc[i] = mfma_f32(av.x, bv.x, acc[i]);
          acc[i] = mfma_f32(av.y, bv.y, acc[i]);
          acc[i] = mfma_f32(av.z, bv.z, acc[i]);
          acc[i] = mfma_f32(av.w, bv.w, acc[i]);
        }
      }
    }
  }

  // S[p][k]: accumulator lane holds column k = kt*16 + r16, rows p = pt*16 + 4q + j
  float* dst = states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * KC);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wid + 4 * i;
    if (tile >= NTILE) break;
    const int pt = tile / (KC / 16), kt = tile % (KC / 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[(pt * 16 + 4 * q + j) * KC + kt * 16 + r16] = acc[i][j];
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: inter-chunk scan of states, in place.
//   states[b][c][h] : S_c on entry, h_in(c) on exit.
// Real: one thread per 4 consecutive (p, n).  Complex: one thread per 4
// consecutive n of one p, re and im together (planar re | im in the
// workspace; h0/h_final interleaved (re, im) as complex64).
// ---------------------------------------------------------------------------
template <bool CPLX, int N>
__global__ __launch_bounds__(kThreads) void ssd_pass_kernel(
    float* __restrict__ states, const float* __restrict__ decay, const float* __restrict__ h0,
    float* __restrict__ h_final, int H, int P, int nc) {
  constexpr int KC = CPLX ? 2 * N : N;
  constexpr int PF = 4;  // chunks in flight per thread
  const int h = blockIdx.y, b = blockIdx.z;
  const int e4 = blockIdx.x * kThreads + threadIdx.x;  // group of 4 elements
  const int groups = P * N / 4;
  if (e4 >= groups) return;
  const int p = (e4 * 4) / N, n = (e4 * 4) % N;
  const size_t chunk_stride = static_cast<size_t>(H) * P * KC;
  float* base = states + (static_cast<size_t>(b) * nc * H + h) * (static_cast<size_t>(P) * KC) +
                static_cast<size_t>(p) * KC + n;
  const float* dc = decay + (static_cast<size_t>(b) * H + h) * nc * 2;
  const size_t pub = ((static_cast<size_t>(b) * H + h) * P + p) * N + n;  // public (p, n) index

  float4 hr = make_float4(0.f, 0.f, 0.f, 0.f), hi = hr;
  if (h0) {
    if (CPLX) {
      const float4* src = reinterpret_cast<const float4*>(h0 + pub * 2);
      const float4 u = src[0], v = src[1];
      hr = make_float4(u.x, u.z, v.x, v.z);
      hi = make_float4(u.y, u.w, v.y, v.w);
    } else {
      hr = *reinterpret_cast<const float4*>(h0 + pub);
    }
  }

  float4 cur_r[PF], cur_i[PF];
  float2 cur_d[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    if (j < nc) {
      cur_r[j] = *reinterpret_cast<const float4*>(base + j * chunk_stride);
      if (CPLX) cur_i[j] = *reinterpret_cast<const float4*>(base + j * chunk_stride + N);
      cur_d[j] = *reinterpret_cast<const float2*>(dc + 2 * j);
    }
  }
  for (int c0 = 0; c0 < nc; c0 += PF) {
    float4 nxt_r[PF], nxt_i[PF];
    float2 nxt_d[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cn = c0 + PF + j;
      if (cn < nc) {
        nxt_r[j] = *reinterpret_cast<const float4*>(base + cn * chunk_stride);
        if (CPLX) nxt_i[j] = *reinterpret_cast<const float4*>(base + cn * chunk_stride + N);
        nxt_d[j] = *reinterpret_cast<const float2*>(dc + 2 * cn);
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cc = c0 + j;
      if (cc < nc) {
        float* slot = base + cc * chunk_stride;
        *reinterpret_cast<float4*>(slot) = hr;
        if (CPLX) {
          *reinterpret_cast<float4*>(slot + N) = hi;
          const float dr = cur_d[j].x, di = cur_d[j].y;
          const float4 sr = cur_r[j], si = cur_i[j];
          float4 nr, ni;
          nr.x = dr * hr.x - di * hi.x + sr.x;
          nr.y = dr * hr.y - di * hi.y + sr.y;
          nr.z = dr * hr.z - di * hi.z + sr.z;
          nr.w = dr * hr.w - di * hi.w + sr.w;
          ni.x = dr * hi.x + di * hr.x + si.x;
          ni.y = dr * hi.y + di * hr.y + si.y;
          ni.z = dr * hi.z + di * hr.z + si.z;
          ni.w = dr * hi.w + di * hr.w + si.w;
          hr = nr;
          hi = ni;
        } else {
          const float d = cur_d[j].x;
          const float4 s = cur_r[j];
          hr = make_float4(d * hr.x + s.x, d * hr.y + s.y, d * hr.z + s.z, d * hr.w + s.w);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      cur_r[j] = nxt_r[j];
      if (CPLX) cur_i[j] = nxt_i[j];
      cur_d[j] = nxt_d[j];
    }
  }
  if (h_final) {
    if (CPLX) {
      float4* dst = reinterpret_cast<float4*>(h_final + pub * 2);
      dst[0] = make_float4(hr.x, hi.x, hr.y, hi.y);
      dst[1] = make_float4(hr.z, hi.z, hr.w, hi.w);
    } else {
      *reinterpret_cast<float4*>(h_final + pub) = hr;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: chunk outputs.
// Wave w owns l-tiles (16 output rows each) w, 7-w, 8+w, 15-w (those < Q/16),
// which balances the causal work.  For each owned tile the wave keeps the C
// rows as MFMA operands in registers and accumulates Y (16 x P) over:
//   (1) e^{cs_l} C_l . h_in           (A = scaled C, B = h_in from LDS)
//   (2) for each source sub-tile s <= l: G^T = B_s . C_l^T on MFMA; its
//       accumulator (lane: column l, rows s) is, after the decay/mask
//       multiply, exactly the A operand of  Y += M . X  (B = x^T from LDS).
// ---------------------------------------------------------------------------
template <typename TI, bool CPLX, int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const TI* __restrict__ Bm, const TI* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* __restrict__ hin, TI* __restrict__ y, int T, int H, int G, int Q, int nc) {
  using E = TI;
  constexpr bool BF = std::is_same<E, uint16_t>::value;
  constexpr int KC = CPLX ? 2 * N : N;
  constexpr int XP = kST + Pad<E>::row;  // pitch of xT rows
  constexpr int BP = KC + Pad<E>::row;   // pitch of bt / hT rows
  constexpr int KSTEP = BF ? 32 : 16;    // k covered by one operand register group
  constexpr int NKS = KC / KSTEP;
  constexpr int NPT = P / 16;
  constexpr int MAXR = 4;
  typedef typename std::conditional<BF, uint4, float4>::type CReg;

  __shared__ __attribute__((aligned(16))) E bt[kST * BP];
  __shared__ __attribute__((aligned(16))) E xT[P * XP];
  __shared__ __attribute__((aligned(16))) E hT[P * BP];
  __shared__ float dl[256], cs_hi[256], cs_lo[256], cth[256], sth[256];
  __shared__ double wsum[4], tot;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const float a_re = CPLX ? A[2 * h] : A[h];
  const float a_im = CPLX ? A[2 * h + 1] : 0.0f;
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const int tid = threadIdx.x;

  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  chunk_prologue<CPLX>(dt, dt_base, H, Lc, a_re, a_im, bias, dt_min, dt_max, dl, cs_hi, cs_lo,
                       cth, sth, wsum, &tot, Q);

  // h_in(c) into LDS as the second MFMA operand of e^{cs} C h_in:
  // real hT[p][n] = h[p][n]; complex hT[p][k] = [h_re | -h_im].
  {
    const float* src = hin + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * KC);
    if constexpr (BF) {
      for (int it = tid; it < P * KC / 8; it += kThreads) {
        const int p = (it * 8) / KC, k = (it * 8) % KC;
        const float4 u = *reinterpret_cast<const float4*>(src + p * KC + k);
        const float4 v = *reinterpret_cast<const float4*>(src + p * KC + k + 4);
        uint4 o;
        o.x = pack_bf16x2(u.x, u.y);
        o.y = pack_bf16x2(u.z, u.w);
        o.z = pack_bf16x2(v.x, v.y);
        o.w = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<uint4*>(hT + p * BP + k) = o;
      }
    } else {
      for (int it = tid; it < P * KC / 4; it += kThreads) {
        const int p = (it * 4) / KC, k = (it * 4) % KC;
        float4 u = *reinterpret_cast<const float4*>(src + p * KC + k);
        if (CPLX && k >= N) u = make_float4(-u.x, -u.y, -u.z, -u.w);
        *reinterpret_cast<float4*>(hT + p * BP + k) = u;
      }
    }
  }

  const int lane = tid & 63, wid = tid >> 6, q = lane >> 4, r16 = lane & 15;
  const int ntl = Q / 16;
  int tl[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) tl[r] = (r / 2) * 8 + ((r & 1) ? 7 - wid : wid);

  const size_t cstride = static_cast<size_t>(G) * N * (CPLX ? 2 : 1);
  const size_t c_row0 = (static_cast<size_t>(b) * T + t0) * cstride +
                        static_cast<size_t>(g) * N * (CPLX ? 2 : 1);

  // C rows of the owned tiles, in the operand layout: lane (row r16, group q)
  // holds k = ks*KSTEP + (BF ? 8q .. 8q+7 : 4q .. 4q+3).
  CReg creg[MAXR][NKS];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = tl[r] * 16 + r16;
    const bool ok = tl[r] < ntl && row < Lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int k0 = ks * KSTEP + (BF ? 8 : 4) * q;
      if constexpr (CPLX) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) {
          const int n0 = k0 < N ? k0 : k0 - N;
          const float4* src = reinterpret_cast<const float4*>(Cm + c_row0 + row * cstride + 2 * n0);
          const float4 u = src[0], v = src[1];
          const float cr[4] = {u.x, u.z, v.x, v.z}, ci[4] = {u.y, u.w, v.y, v.w};
          const float co = cth[row], si = sth[row];
          float res[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            res[j] = k0 < N ? cr[j] * co - ci[j] * si : cr[j] * si + ci[j] * co;
          o = make_float4(res[0], res[1], res[2], res[3]);
        }
        creg[r][ks] = o;
      } else if constexpr (BF) {
        uint4 o = make_uint4(0, 0, 0, 0);
        if (ok) o = *reinterpret_cast<const uint4*>(Cm + c_row0 + row * cstride + k0);
        creg[r][ks] = o;
      } else {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) o = *reinterpret_cast<const float4*>(Cm + c_row0 + row * cstride + k0);
        creg[r][ks] = o;
      }
    }
  }

  f32x4 yacc[MAXR][NPT];
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) yacc[r][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // hT, prologue arrays

  // (1) contribution of the state entering the chunk
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (tl[r] >= ntl) continue;
    const int row = tl[r] * 16 + r16;
    const float sc = __expf(cs_hi[row] + cs_lo[row]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (BF) {
        const uint4 cv = creg[r][ks];
        const uint32_t w[4] = {cv.x, cv.y, cv.z, cv.w};
        uint4 a;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_bf16x2(bf16_bits_to_f32(w[j] & 0xFFFFu) * sc, bf16_bits_to_f32(w[j] >> 16) * sc);
        a = make_uint4(o[0], o[1], o[2], o[3]);
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint4 hv = *reinterpret_cast<const uint4*>(hT + (pt * 16 + r16) * BP + ks * KSTEP + 8 * q);
          yacc[r][pt] = mfma_bf16(as_bf16x8(a), as_bf16x8(hv), yacc[r][pt]);
        }
      } else {
        const float4 cv = creg[r][ks];
        const float4 a = make_float4(cv.x * sc, cv.y * sc, cv.z * sc, cv.w * sc);
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const float4 hv = *reinterpret_cast<const float4*>(hT + (pt * 16 + r16) * BP + ks * KSTEP + 4 * q);
          yacc[r][pt] = mfma_f32(a.x, hv.x, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(a.y, hv.y, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(a.z, hv.z, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(a.w, hv.w, yacc[r][pt]);
        }
      }
    }
  }

  const size_t x_row0 = (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P;
  const size_t x_rs = static_cast<size_t>(H) * P;

  // (2) intra-chunk part, source tokens staged kST at a time
  int lmax = 0;
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
    if (tl[r] < ntl) lmax = max(lmax, tl[r] * 16 + 15);
  for (int s0 = 0; s0 < Lc; s0 += kST) {
    __syncthreads();
    // bt[s - s0][k]: real B_s; complex [B'_re | -B'_im], B' = B e^{-i theta_s}
    if constexpr (CPLX) {
      constexpr int NG = N / 4;
      for (int it = tid; it < kST * NG; it += kThreads) {
        const int ng = it % NG, sl = it / NG, s = s0 + sl;
        float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
        if (s < Lc) {
          const float4* src = reinterpret_cast<const float4*>(Bm + c_row0 + s * cstride + ng * 8);
          v0 = src[0];
          v1 = src[1];
        }
        const float co = cth[s < Q ? s : 0], si = sth[s < Q ? s : 0];
        const float br[4] = {v0.x, v0.z, v1.x, v1.z}, bi[4] = {v0.y, v0.w, v1.y, v1.w};
        float re[4], nim[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          re[j] = br[j] * co + bi[j] * si;
          nim[j] = br[j] * si - bi[j] * co;
        }
        *reinterpret_cast<float4*>(bt + sl * BP + ng * 4) = make_float4(re[0], re[1], re[2], re[3]);
        *reinterpret_cast<float4*>(bt + sl * BP + N + ng * 4) = make_float4(nim[0], nim[1], nim[2], nim[3]);
      }
    } else {
      constexpr int V = BF ? 8 : 4;
      constexpr int NG = N / V;
      for (int it = tid; it < kST * NG; it += kThreads) {
        const int ng = it % NG, sl = it / NG, s = s0 + sl;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (s < Lc) v = *reinterpret_cast<const uint4*>(Bm + c_row0 + s * cstride + ng * V);
        *reinterpret_cast<uint4*>(bt + sl * BP + ng * V) = v;
      }
    }
    stage_xT<E, P>(xT, x, x_row0, x_rs, s0, Lc);
    __syncthreads();
    if (s0 > lmax) continue;

#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (tl[r] >= ntl) continue;
      const int lrow = tl[r] * 16 + r16;  // this lane's output row l
      if (s0 > tl[r] * 16 + 15) continue;
      const float lh = cs_hi[lrow], ll = cs_lo[lrow];
      if constexpr (BF) {
#pragma unroll
        for (int ss = 0; ss < kST; ss += 32) {
          const int sb = s0 + ss;
          if (sb > tl[r] * 16 + 15) break;
          f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 va = *reinterpret_cast<const uint4*>(bt + (ss + r16) * BP + ks * 32 + 8 * q);
            const uint4 vb = *reinterpret_cast<const uint4*>(bt + (ss + 16 + r16) * BP + ks * 32 + 8 * q);
            ga = mfma_bf16(as_bf16x8(va), as_bf16x8(creg[r][ks]), ga);
            gb = mfma_bf16(as_bf16x8(vb), as_bf16x8(creg[r][ks]), gb);
          }
          float m[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int sa = sb + 4 * q + j, sbb = sb + 16 + 4 * q + j;
            const float wa = sa <= lrow ? decay_between(lh, ll, cs_hi[sa], cs_lo[sa]) * (CPLX ? 1.f : dl[sa]) : 0.f;
            const float wb = sbb <= lrow ? decay_between(lh, ll, cs_hi[sbb], cs_lo[sbb]) * (CPLX ? 1.f : dl[sbb]) : 0.f;
            m[j] = ga[j] * wa;
            m[4 + j] = gb[j] * wb;
          }
          const uint4 mv = make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]),
                                      pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7]));
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) {
            const E* xr = xT + (pt * 16 + r16) * XP + ss + 4 * q;
            const uint2 x0 = *reinterpret_cast<const uint2*>(xr);
            const uint2 x1 = *reinterpret_cast<const uint2*>(xr + 16);
            const uint4 xv = make_uint4(x0.x, x0.y, x1.x, x1.y);
            yacc[r][pt] = mfma_bf16(as_bf16x8(mv), as_bf16x8(xv), yacc[r][pt]);
          }
        }
      } else {
#pragma unroll
        for (int ss = 0; ss < kST; ss += 16) {
          const int sb = s0 + ss;
          if (sb > tl[r] * 16 + 15) break;
          f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const float4 va = *reinterpret_cast<const float4*>(bt + (ss + r16) * BP + ks * 16 + 4 * q);
            const float4 cv = creg[r][ks];
            ga = mfma_f32(va.x, cv.x, ga);
            ga = mfma_f32(va.y, cv.y, ga);
            ga = mfma_f32(va.z, cv.z, ga);
            ga = mfma_f32(va.w, cv.w, ga);
          }
          float m[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int sa = sb + 4 * q + j;
            const float wa = sa <= lrow ? decay_between(lh, ll, cs_hi[sa], cs_lo[sa]) * (CPLX ? 1.f : dl[sa]) : 0.f;
            m[j] = ga[j] * wa;
          }
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) {
            const float4 xv = *reinterpret_cast<const float4*>(xT + (pt * 16 + r16) * XP + ss + 4 * q);
            yacc[r][pt] = mfma_f32(m[0], xv.x, yacc[r][pt]);
            yacc[r][pt] = mfma_f32(m[1], xv.y, yacc[r][pt]);
            yacc[r][pt] = mfma_f32(m[2], xv.z, yacc[r][pt]);
            yacc[r][pt] = mfma_f32(m[3], xv.w, yacc[r][pt]);
          }
        }
      }
    }
  }

  // epilogue: y[l][p] = acc + D x; lane holds column p = pt*16 + r16, rows
  // l = tile*16 + 4q + j
  const float Dh = (!CPLX && D) ? D[h] : 0.0f;
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (tl[r] >= ntl) continue;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int l = tl[r] * 16 + 4 * q + j;
        if (l < Lc) {
          const size_t idx = x_row0 + l * x_rs + pt * 16 + r16;
          float v = yacc[r][pt][j];
          if (!CPLX && D) v += Dh * load_elem(x, idx);
          store_elem(y, idx, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch of the three kernels for one shape.
// ---------------------------------------------------------------------------
template <typename TI, bool CPLX, int P, int N>
static hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st) {
  constexpr int KC = CPLX ? 2 * N : N;
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  float* states = static_cast<float*>(a.workspace);
  float* decay = states + workspace_state_floats(a.Bsz, nc, a.H, a.P, KC);
  const TI* x = static_cast<const TI*>(a.x);
  const TI* B = static_cast<const TI*>(a.B);
  const TI* C = static_cast<const TI*>(a.C);
  if (a.events) hipEventRecord(a.events[0], st);
  if (nc > 0) {
    dim3 grid(nc, a.H, a.Bsz);
    ssd_state_kernel<TI, CPLX, P, N><<<grid, kThreads, 0, st>>>(
        x, a.dt, a.A, B, a.dt_bias, a.dt_min, a.dt_max, states, decay, a.T, a.H, a.G,
        a.chunk, nc);
  }
  if (a.events) hipEventRecord(a.events[1], st);
  {
    const int groups = P * N / 4;
    dim3 grid((groups + kThreads - 1) / kThreads, a.H, a.Bsz);
    ssd_pass_kernel<CPLX, N><<<grid, kThreads, 0, st>>>(states, decay, a.h0, a.h_final, a.H,
                                                          P, nc);
  }
  if (a.events) hipEventRecord(a.events[2], st);
  if (nc > 0) {
    dim3 grid(nc, a.H, a.Bsz);
    ssd_scan_kernel<TI, CPLX, P, N><<<grid, kThreads, 0, st>>>(
        x, a.dt, a.A, B, C, a.D, a.dt_bias, a.dt_min, a.dt_max, states,
        static_cast<TI*>(a.y), a.T, a.H, a.G, a.chunk, nc);
  }
  if (a.events) hipEventRecord(a.events[3], st);
  return hipGetLastError();
}

template <typename TI, bool CPLX, int P>
static hipError_t dispatch_n(const ChunkArgs& a, hipStream_t st) {
  switch (a.N) {
    case 16: return launch_chunk<TI, CPLX, P, 16>(a, st);
    case 32: return launch_chunk<TI, CPLX, P, 32>(a, st);
    case 64: return launch_chunk<TI, CPLX, P, 64>(a, st);
    case 128:
      if constexpr (!CPLX) return launch_chunk<TI, CPLX, P, 128>(a, st);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename TI, bool CPLX>
static hipError_t dispatch_p(const ChunkArgs& a, hipStream_t st) {
  switch (a.P) {
    case 16: return dispatch_n<TI, CPLX, 16>(a, st);
    case 32: return dispatch_n<TI, CPLX, 32>(a, st);
    case 64: return dispatch_n<TI, CPLX, 64>(a, st);
    case 128: return dispatch_n<TI, CPLX, 128>(a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t run_chunk_real(const ChunkArgs& a, hipStream_t st) {
  if (a.dtype == 1) return dispatch_p<uint16_t, false>(a, st);
  return dispatch_p<float, false>(a, st);
}

hipError_t run_chunk_complex(const ChunkArgs& a, hipStream_t st) {
  return dispatch_p<float, true>(a, st);
}

}  // namespace ssd
