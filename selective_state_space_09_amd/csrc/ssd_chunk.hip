// Chunked SSD forward on gfx950, float32 inputs (real Mamba-2 form): three
// kernels per call.  (bfloat16 inputs run the kernels of ssd_chunk_bf16.hip,
// the complex form those of ssd_chunk_cplx.hip.)
//
//   ssd_state_kernel  one workgroup per (batch b, chunk c, head h): the state a
//                     chunk leaves behind when it starts from zero,
//                     S_c = sum_s w_s x_s (x) B_s  (MFMA, contraction over s),
//                     plus the chunk's total decay factor.
//   ssd_pass_kernel   the inter-chunk recurrence h_in(c+1) = decay_c h_in(c)
//                     + S_c, sequential over chunks and parallel over the
//                     (b, h, p, n) state elements; h_in(c) overwrites S_c.
//   ssd_scan_kernel   one workgroup per (b, c, h): the output of the chunk,
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
// Workgroup order: the 1-D grid is laid out so that the workgroups of one
// (batch, chunk) pair -- all its heads -- fall on the same XCD (consecutive
// workgroup ids rotate over the 8 XCDs), where they share that chunk's B and
// C rows in the XCD's L2.
//
// Latency: the source tokens of a chunk are staged through LDS in stages of
// ST tokens (64, or 32 where two 64-token buffers would not fit in LDS).
// Each stage's global loads are issued into registers one stage ahead, so the
// HBM latency of stage i+1 overlaps the MFMA work of stage i (double-buffered
// LDS, one barrier per stage).

#include <type_traits>

#include "ssd_chunk_common.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Kernel 1: chunk-end states from a zero start.
// ---------------------------------------------------------------------------

// B slab -> bT[k][s - s0] = w_s B_s[k] (transposed, weighted).
template <int ST, int N>
struct StateBSlab : Slab<ST, N / 4, 1> {
  // complex rows: each item's (cos, sin) theta_s, loaded beside the rows
  // (rot[s * stride] for token s; rows past Lc (>= 1) read row Lc - 1, whose
  // weight is zero)
  float2 rc[Slab<ST, N / 4, 1>::PER];
  __device__ __forceinline__ void load_rot(const float2* __restrict__ rot, size_t stride, int s0, int Lc) {
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (this->ITEMS % kThreads == 0 || it < this->ITEMS)
        rc[i] = rot[static_cast<size_t>(min(s0 + it / (N / 4), Lc - 1)) * stride];
    }
  }

  // complex rows (N / 2 values as (re, im) pairs) rotated per token into the
  // N real features [Re | Im] of z e^{-i theta} (CONJ = false: B) or
  // [Re | -Im] of z e^{+i theta} (CONJ = true: C), with the rotations of
  // load_rot
  template <bool CONJ>
  __device__ __forceinline__ void store_rot(float* bT, const float* wre, int s0, int Q) const {
    constexpr int XP = ST + Pad<float>::row;
    constexpr int NH = N / 2;
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % (N / 4), sl = it / (N / 4);
      const int s = s0 + sl;
      const float w = s < Q ? wre[s] : 0.f;
      const float2 r = rc[i];
      const uint4 u = this->v[i][0];
      const float re0 = __uint_as_float(u.x), im0 = __uint_as_float(u.y);
      const float re1 = __uint_as_float(u.z), im1 = __uint_as_float(u.w);
      const int n = 2 * ng;
      if constexpr (!CONJ) {
        bT[(n + 0) * XP + sl] = w * (re0 * r.x + im0 * r.y);
        bT[(n + 1) * XP + sl] = w * (re1 * r.x + im1 * r.y);
        bT[(NH + n + 0) * XP + sl] = w * (im0 * r.x - re0 * r.y);
        bT[(NH + n + 1) * XP + sl] = w * (im1 * r.x - re1 * r.y);
      } else {
        bT[(n + 0) * XP + sl] = w * (re0 * r.x - im0 * r.y);
        bT[(n + 1) * XP + sl] = w * (re1 * r.x - im1 * r.y);
        bT[(NH + n + 0) * XP + sl] = -w * (im0 * r.x + re0 * r.y);
        bT[(NH + n + 1) * XP + sl] = -w * (im1 * r.x + re1 * r.y);
      }
    }
  }

  __device__ __forceinline__ void store(float* bT, const float* wre, int s0, int Q) const {
    constexpr int XP = ST + Pad<float>::row;
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % (N / 4), sl = it / (N / 4);
      const int s = s0 + sl;
      const float w = s < Q ? wre[s] : 0.f;
      const uint4 u = this->v[i][0];
      bT[(ng * 4 + 0) * XP + sl] = w * __uint_as_float(u.x);
      bT[(ng * 4 + 1) * XP + sl] = w * __uint_as_float(u.y);
      bT[(ng * 4 + 2) * XP + sl] = w * __uint_as_float(u.z);
      bT[(ng * 4 + 3) * XP + sl] = w * __uint_as_float(u.w);
    }
  }
};

// MODE kStateFwd: S_c = sum_s e^{tot - cs_s} delta_s x_s (x) B_s and the
// chunk's decay (the forward).  kStateFwdUnit: the same with input scale 1
// (no delta_s on the input term: the rotated-frame form of the complex
// recurrence).  kStateAdj: the adjoint chunk state of the backward,
// G_c = sum_l e^{cs_l} dy_l (x) C_l (x = dy, B = C; no decay written).
// kStateCplxUnit, kStateCplxAdj: kStateFwdUnit and kStateAdj on complex rows
// (B or C as N / 2 (re, im) pairs) rotated into the sequence frame as they are
// staged: features [Re B e^{-i theta} | Im B e^{-i theta}], resp.
// [Re C e^{i theta} | -Im C e^{i theta}], with theta per token from `rot`.
// NBUF = 1: one stage buffer, for chunks of at most one stage (the backward's
// 64-token chunks): half the LDS, so that two workgroups share a CU.
constexpr int kStateFwd = 0, kStateFwdUnit = 1, kStateAdj = 2, kStateCplxUnit = 3, kStateCplxAdj = 4;

template <int P, int N, int MODE = kStateFwd, int NBUF = 2>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    float* __restrict__ states, float* __restrict__ decay, int T, int H, int G, int Q, int nc,
    int npairs, const float2* __restrict__ rot) {
  constexpr bool kCplx = MODE == kStateCplxUnit || MODE == kStateCplxAdj;
  constexpr bool kAdj = MODE == kStateAdj || MODE == kStateCplxAdj;
  constexpr bool kUnit = MODE == kStateFwdUnit || MODE == kStateCplxUnit;
  // stage length: 64 tokens unless two buffers of that size overflow LDS
  constexpr int ST = 2 * (P + N) * (64 + Pad<float>::row) * 4 + 8192 <= kLdsBytes ? 64 : 32;
  constexpr int XP = ST + Pad<float>::row;
  constexpr int NTILE = (P / 16) * (N / 16);
  constexpr int TPW = (NTILE + 3) / 4;  // output tiles per wave

  constexpr int TQ = NBUF == 1 ? 64 : 256;  // longest chunk
  __shared__ __attribute__((aligned(16))) float xT[NBUF][P * XP];
  __shared__ __attribute__((aligned(16))) float bT[NBUF][N * XP];
  __shared__ float dl[TQ], cs_hi[TQ], cs_lo[TQ];
  __shared__ float wre[TQ];
  __shared__ double wsum[4], tot;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const float a_re = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;

  // issue the first global loads before any arithmetic
  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = dt[dt_base + static_cast<size_t>(min(tid, Lc - 1)) * H];  // (ignored past Lc)
  const char* xbase = reinterpret_cast<const char*>(
      x + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P);
  const size_t xrow = static_cast<size_t>(H) * P * sizeof(float);
  const char* bbase = reinterpret_cast<const char*>(
      Bm + (static_cast<size_t>(b) * T + t0) * G * N + static_cast<size_t>(g) * N);
  const size_t brow = static_cast<size_t>(G) * N * sizeof(float);
  // (dt ahead of the slab loads in the issue order: the prologue waits for it,
  // and a wait for a load also waits for every load issued before it)
  __builtin_amdgcn_sched_barrier(0);
  // (rows past the chunk read clamped: their weights w_s are zero)
  XSlabF32<ST, P> xs;
  StateBSlab<ST, N> bs;
  xs.load_clamped(xbase, xrow, 0, Lc);
  bs.load_clamped(bbase, brow, 0, Lc);
  if constexpr (kCplx) {
    static_assert(NBUF == 1, "complex rows: one stage");
    bs.load_rot(rot + dt_base, H, 0, Lc);
  }
  const double cum =
      chunk_prologue(dt_raw, Lc, a_re, bias, dt_min, dt_max, dl, cs_hi, cs_lo, wsum, &tot, Q);
  // weight of each source token to the chunk end (the adjoint: from the chunk start)
  const double total = tot;
  if (tid < Q) {
    if constexpr (kAdj)
      wre[tid] = tid < Lc ? __expf(static_cast<float>(cum)) : 0.0f;  // exponent <= 0
    else if constexpr (kUnit)
      wre[tid] = tid < Lc ? __expf(static_cast<float>(total - cum)) : 0.0f;
    else
      wre[tid] = __expf(static_cast<float>(total - cum)) * dl[tid];
  }
  if (!kAdj && tid == 0) {
    float* dc = decay + ((static_cast<size_t>(b) * H + h) * nc + c) * 2;
    dc[0] = __expf(static_cast<float>(total));
    dc[1] = 0.0f;
  }
  __syncthreads();
  xs.store(xT[0]);
  if constexpr (kCplx)
    bs.template store_rot<MODE == kStateCplxAdj>(bT[0], wre, 0, Q);
  else
    bs.store(bT[0], wre, 0, Q);
  __syncthreads();

  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (Lc + ST - 1) / ST;
  for (int it = 0; it < ntiles; ++it) {
    const int cur = NBUF == 1 ? 0 : it & 1;
    const bool more = NBUF > 1 && it + 1 < ntiles;
    if (more) {
      xs.load_clamped(xbase, xrow, (it + 1) * ST, Lc);
      bs.load_clamped(bbase, brow, (it + 1) * ST, Lc);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wid + 4 * i;
      if (tile >= NTILE) break;
      const int pt = tile / (N / 16), kt = tile % (N / 16);
      const float* arow = xT[cur] + (pt * 16 + r16) * XP;
      const float* brow_l = bT[cur] + (kt * 16 + r16) * XP;
#pragma unroll
      for (int ss = 0; ss < ST; ss += 16) {
        const float4 av = *reinterpret_cast<const float4*>(arow + ss + 4 * q);
        const float4 bv = *reinterpret_cast<const float4*>(brow_l + ss + 4 * q);
        acc[i] = mfma_f32(av.x, bv.x, acc[i]);
        acc[i] = mfma_f32(av.y, bv.y, acc[i]);
        acc[i] = mfma_f32(av.z, bv.z, acc[i]);
        acc[i] = mfma_f32(av.w, bv.w, acc[i]);
      }
    }
    if (more) {
      xs.store(xT[(cur ^ 1) % NBUF]);
      bs.store(bT[(cur ^ 1) % NBUF], wre, (it + 1) * ST, Q);
    }
    __syncthreads();
  }

  // S[p][n]: accumulator lane holds column n = kt*16 + r16, rows p = pt*16 + 4q + j
  float* dst = states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wid + 4 * i;
    if (tile >= NTILE) break;
    const int pt = tile / (N / 16), kt = tile % (N / 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[(pt * 16 + 4 * q + j) * N + kt * 16 + r16] = acc[i][j];
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: chunk outputs.
// ---------------------------------------------------------------------------

// B slab -> bt[s - s0][n] natural layout (a straight copy).
template <int ST, int N, int BP>
struct ScanBSlab : Slab<ST, N / 4, 1> {
  __device__ __forceinline__ void store(float* bt) const {
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % (N / 4), sl = it / (N / 4);
      *reinterpret_cast<uint4*>(bt + sl * BP + ng * 4) = this->v[i][0];
    }
  }
};

// Wave w owns l-tiles (16 output rows each) w, 7-w, 8+w, 15-w (those < Q/16),
// which balances the causal work.  For each owned tile the wave keeps the C
// rows as MFMA operands in registers and accumulates Y (16 x P) over:
//   (1) e^{cs_l} C_l . h_in           (A = scaled C, B = h_in from LDS)
//   (2) for each source sub-tile s <= l: G^T = B_s . C_l^T on MFMA; its
//       accumulator (lane: column l, rows s) is, after the decay/mask
//       multiply, exactly the A operand of  Y += M . X  (B = x^T from LDS).
//   (3) D_h x_l, read from the x^T stage that holds the tile's own rows.
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ Bm, const float* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* __restrict__ hin, float* __restrict__ y, int T, int H, int G, int Q, int nc,
    int npairs) {
  constexpr int BP = N + Pad<float>::row;  // pitch of bt / hT rows
  // stage length: 64 tokens unless two buffers of that size overflow LDS
  constexpr int ST = (2 * (64 * BP + P * (64 + Pad<float>::row)) + P * BP) * 4 + 8192 <= kLdsBytes
                         ? 64 : 32;
  constexpr int XP = ST + Pad<float>::row;  // pitch of xT rows
  constexpr int NKS = N / 16;
  constexpr int NPT = P / 16;
  constexpr int MAXR = 4;

  __shared__ __attribute__((aligned(16))) float bt[2][ST * BP];
  __shared__ __attribute__((aligned(16))) float xT[2][P * XP];
  __shared__ __attribute__((aligned(16))) float hT[P * BP];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs_hi[256];
  __shared__ __attribute__((aligned(16))) float cs_lo[256];
  __shared__ double wsum[4], tot;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar
  const int ntl = Q / 16;
  const float a_re = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const float Dh = D ? D[h] : 0.0f;

  // ---- issue global loads: dt, h_in, C rows, first source stage ----
  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = tid < Lc ? dt[dt_base + static_cast<size_t>(tid) * H] : 0.0f;

  constexpr int HV = P * N / 4;  // float4 vectors of h_in
  constexpr int HPER = (HV + kThreads - 1) / kThreads;
  float4 hreg[HPER];
  {
    const float* src = hin + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N);
#pragma unroll
    for (int i = 0; i < HPER; ++i) {
      const int it = tid + i * kThreads;
      if (it < HV) hreg[i] = *reinterpret_cast<const float4*>(src + it * 4);
    }
  }

  int tl[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) tl[r] = (r / 2) * 8 + ((r & 1) ? 7 - wid : wid);

  const size_t cstride = static_cast<size_t>(G) * N;  // elements between tokens
  const size_t c_row0 = (static_cast<size_t>(b) * T + t0) * cstride + static_cast<size_t>(g) * N;

  // C rows of the owned tiles, in the operand layout: lane (row r16, group q)
  // holds n = ks*16 + 4q .. 4q+3
  float4 creg[MAXR][NKS];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = tl[r] * 16 + r16;
    const bool ok = tl[r] < ntl && row < Lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) o = *reinterpret_cast<const float4*>(Cm + c_row0 + row * cstride + ks * 16 + 4 * q);
      creg[r][ks] = o;
    }
  }

  const char* xbase = reinterpret_cast<const char*>(
      x + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P);
  const size_t xrow = static_cast<size_t>(H) * P * sizeof(float);
  const char* bbase = reinterpret_cast<const char*>(Bm + c_row0);
  const size_t brow = cstride * sizeof(float);
  XSlabF32<ST, P> xs;
  ScanBSlab<ST, N, BP> bs;
  xs.load(xbase, xrow, 0, Lc);
  bs.load(bbase, brow, 0, Lc);

  // ---- prologue ----
  chunk_prologue(dt_raw, Lc, a_re, bias, dt_min, dt_max, dl, cs_hi, cs_lo, wsum, &tot, Q);

  // h_in -> hT[p][n]
#pragma unroll
  for (int i = 0; i < HPER; ++i) {
    const int it = tid + i * kThreads;
    if (it >= HV) break;
    const int p = (it * 4) / N, k = (it * 4) % N;
    *reinterpret_cast<float4*>(hT + p * BP + k) = hreg[i];
  }
  xs.store(xT[0]);
  bs.store(bt[0]);
  __syncthreads();

  f32x4 yacc[MAXR][NPT];
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) yacc[r][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // (1) contribution of the state entering the chunk
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (tl[r] >= ntl) continue;
    const int row = tl[r] * 16 + r16;
    const float sc = __expf(cs_hi[row] + cs_lo[row]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const float4 cv = creg[r][ks];
      const float4 a = make_float4(cv.x * sc, cv.y * sc, cv.z * sc, cv.w * sc);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const float4 hv = *reinterpret_cast<const float4*>(hT + (pt * 16 + r16) * BP + ks * 16 + 4 * q);
        yacc[r][pt] = mfma_f32(a.x, hv.x, yacc[r][pt]);
        yacc[r][pt] = mfma_f32(a.y, hv.y, yacc[r][pt]);
        yacc[r][pt] = mfma_f32(a.z, hv.z, yacc[r][pt]);
        yacc[r][pt] = mfma_f32(a.w, hv.w, yacc[r][pt]);
      }
    }
  }

  // (2) intra-chunk part and (3) the skip term, one stage of ST source tokens at a time
  const int ntiles = (Lc + ST - 1) / ST;
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int s0 = it * ST;
    const bool more = it + 1 < ntiles;
    if (more) {
      xs.load(xbase, xrow, s0 + ST, Lc);
      bs.load(bbase, brow, s0 + ST, Lc);
    }
    const float* btc = bt[cur];
    const float* xTc = xT[cur];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (tl[r] >= ntl) continue;
      const int lfirst = tl[r] * 16, llast = lfirst + 15;
      if (s0 > llast) continue;
      const int lrow = lfirst + r16;  // this lane's output row l (as G^T column)
      const float lh = cs_hi[lrow], ll = cs_lo[lrow];
#pragma unroll
      for (int ss = 0; ss < ST; ss += 16) {
        const int sb = s0 + ss;
        if (sb > llast) break;
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const float4 va = *reinterpret_cast<const float4*>(btc + (ss + r16) * BP + ks * 16 + 4 * q);
          const float4 cv = creg[r][ks];
          ga = mfma_f32(va.x, cv.x, ga);
          ga = mfma_f32(va.y, cv.y, ga);
          ga = mfma_f32(va.z, cv.z, ga);
          ga = mfma_f32(va.w, cv.w, ga);
        }
        const float4 ha = *reinterpret_cast<const float4*>(cs_hi + sb + 4 * q);
        const float4 la = *reinterpret_cast<const float4*>(cs_lo + sb + 4 * q);
        const float4 da = *reinterpret_cast<const float4*>(dl + sb + 4 * q);
        const float hav[4] = {ha.x, ha.y, ha.z, ha.w}, lav[4] = {la.x, la.y, la.z, la.w};
        const float dav[4] = {da.x, da.y, da.z, da.w};
        float m[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int sa = sb + 4 * q + j;
          m[j] = sa <= lrow ? ga[j] * decay_between(lh, ll, hav[j], lav[j]) * dav[j] : 0.f;
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const float4 xv = *reinterpret_cast<const float4*>(xTc + (pt * 16 + r16) * XP + ss + 4 * q);
          yacc[r][pt] = mfma_f32(m[0], xv.x, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(m[1], xv.y, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(m[2], xv.z, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(m[3], xv.w, yacc[r][pt]);
        }
      }
      // (3) D x for the tile's own rows, while they sit in this stage
      if (lfirst >= s0 && lfirst < s0 + ST) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const float4 u = *reinterpret_cast<const float4*>(xTc + (pt * 16 + r16) * XP + (lfirst - s0) + 4 * q);
          yacc[r][pt][0] += Dh * u.x;
          yacc[r][pt][1] += Dh * u.y;
          yacc[r][pt][2] += Dh * u.z;
          yacc[r][pt][3] += Dh * u.w;
        }
      }
    }
    if (more) {
      xs.store(xT[cur ^ 1]);
      bs.store(bt[cur ^ 1]);
    }
    __syncthreads();
  }

  // write y; lane holds column p = pt*16 + r16, rows l = tile*16 + 4q + j
  const size_t x_row0 = (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P;
  const size_t x_rs = static_cast<size_t>(H) * P;
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (tl[r] >= ntl) continue;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int l = tl[r] * 16 + 4 * q + j;
        if (l < Lc) y[x_row0 + l * x_rs + pt * 16 + r16] = yacc[r][pt][j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launch of the three kernels for one shape.
// ---------------------------------------------------------------------------
template <int P, int N>
static hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st) {
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  const int npairs = a.Bsz * nc;
  float* states = static_cast<float*>(a.workspace);
  float* decay = states + workspace_state_floats(a.Bsz, nc, a.H, a.P, N);
  const float* x = static_cast<const float*>(a.x);
  const float* B = static_cast<const float*>(a.B);
  const float* C = static_cast<const float*>(a.C);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  const hipEvent_t* ev = a.events;
  launch_k(nc > 0, ssd_state_kernel<P, N>, dim3(blocks), dim3(kThreads), st, ev, x, a.dt, a.A, B,
           a.dt_bias, a.dt_min, a.dt_max, states, decay, a.T, a.H, a.G, a.chunk, nc, npairs,
           static_cast<const float2*>(nullptr));
  launch_pass<false, N>(states, decay, a.h0, a.h_final, a.Bsz, a.H, P, nc, st,
                        ev ? ev + 2 : nullptr);
  launch_k(nc > 0, ssd_scan_kernel<P, N>, dim3(blocks), dim3(kThreads), st, ev ? ev + 4 : nullptr,
           x, a.dt, a.A, B, C, a.D, a.dt_bias, a.dt_min, a.dt_max,
           static_cast<const float*>(states), static_cast<float*>(a.y), a.T, a.H, a.G, a.chunk, nc,
           npairs);
  return hipGetLastError();
}

template <int P>
static hipError_t dispatch_n(const ChunkArgs& a, hipStream_t st) {
  switch (a.N) {
    case 16: return launch_chunk<P, 16>(a, st);
    case 32: return launch_chunk<P, 32>(a, st);
    case 64: return launch_chunk<P, 64>(a, st);
    case 128: return launch_chunk<P, 128>(a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

// fp32 chunk-state kernel of the backward (see ssd_internal.h)
template <int P, int N>
static hipError_t launch_states_f32(const float* x, const float* dt, const float* A, const float* B,
                                    const float* dt_bias, float dt_min, float dt_max, float* states,
                                    float* decay, int Bsz, int T, int H, int G, int chunk, int mode,
                                    const float2* rot, hipStream_t st, const hipEvent_t* ev) {
  const int nc = (T + chunk - 1) / chunk;
  const int npairs = Bsz * nc;
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * H;
  if (chunk > 64) return hipErrorInvalidValue;  // one stage buffer holds 64 tokens
  auto go = [&](auto m) {
    constexpr int M = decltype(m)::value;
    launch_k(nc > 0, ssd_state_kernel<P, N, M, 1>, dim3(blocks), dim3(kThreads), st, ev, x, dt, A, B, dt_bias,
             dt_min, dt_max, states, decay, T, H, G, chunk, nc, npairs, rot);
  };
  switch (mode) {
    case kStateFwd: go(std::integral_constant<int, kStateFwd>{}); break;
    case kStateFwdUnit: go(std::integral_constant<int, kStateFwdUnit>{}); break;
    case kStateAdj: go(std::integral_constant<int, kStateAdj>{}); break;
    case kStateCplxUnit: go(std::integral_constant<int, kStateCplxUnit>{}); break;
    case kStateCplxAdj: go(std::integral_constant<int, kStateCplxAdj>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t run_states_f32(const float* x, const float* dt, const float* A, const float* B,
                          const float* dt_bias, float dt_min, float dt_max, float* states,
                          float* decay, int Bsz, int T, int H, int P, int G, int N, int chunk,
                          int mode, const float2* rot, hipStream_t st, const hipEvent_t* ev) {
#define SSD_STATES_F32(PP, NN)                                                                     \
  if (P == PP && N == NN)                                                                          \
    return launch_states_f32<PP, NN>(x, dt, A, B, dt_bias, dt_min, dt_max, states, decay, Bsz, T, H, \
                                     G, chunk, mode, rot, st, ev);
  SSD_STATES_F32(32, 32)
  SSD_STATES_F32(32, 64)
  SSD_STATES_F32(32, 128)
  SSD_STATES_F32(64, 32)
  SSD_STATES_F32(64, 64)
  SSD_STATES_F32(64, 128)
#undef SSD_STATES_F32
  return hipErrorInvalidValue;
}

hipError_t run_pass_f32(float* states, const float* decay, const float* h0, float* h_final, int Bsz,
                        int H, int P, int N, int nc, hipStream_t st, const hipEvent_t* ev) {
  switch (N) {
    case 32: launch_pass<false, 32>(states, decay, h0, h_final, Bsz, H, P, nc, st, ev); break;
    case 64: launch_pass<false, 64>(states, decay, h0, h_final, Bsz, H, P, nc, st, ev); break;
    case 128: launch_pass<false, 128>(states, decay, h0, h_final, Bsz, H, P, nc, st, ev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t run_chunk_real(const ChunkArgs& a, hipStream_t st) {
  if (a.dtype == 1) return run_chunk_real_bf16(a, st);
  switch (a.P) {
    case 16: return dispatch_n<16>(a, st);
    case 32: return dispatch_n<32>(a, st);
    case 64: return dispatch_n<64>(a, st);
    case 128: return dispatch_n<128>(a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
