// Chunked SSD forward on gfx950, float32 and complex64 inputs: three kernels
// per call.  (bfloat16 inputs run the kernels of ssd_chunk_bf16.hip.)
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
// Complex form (Mamba-3-Lite): with u_l the cumulative step inside the chunk
// and theta_l = beta u_l, exp(A (u_l - u_s)) = e^{alpha (u_l - u_s)}
// e^{i theta_l} e^{-i theta_s}.  Rotating C'_l = C_l e^{i theta_l} and
// B'_s = B_s e^{-i theta_s} turns the real part of the complex decay-weighted
// product into one real product with K = 2N:
//   Re(C'_l . B'_s) = [C'_re | C'_im] . [B'_re | -B'_im],
// so the complex path is the real kernel with K = 2N and no delta factor.
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

#include "ssd_chunk_common.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Kernel 1: chunk-end states from a zero start.
// ---------------------------------------------------------------------------

// B slab -> bT[k][s - s0] = w_s B_s[k] (transposed, weighted).
template <typename TI, bool CPLX, int ST, int N>
struct StateBSlab;

template <int ST, int N>
struct StateBSlab<uint16_t, false, ST, N> : Slab<ST, N / 8, 2> {
  __device__ __forceinline__ void store(uint16_t* bT, const float* wre, const float*, int s0,
                                        int Q) const {
    constexpr int XP = ST + Pad<uint16_t>::row;
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % (N / 8), sp = it / (N / 8);
      const int s = s0 + 2 * sp;
      const float w0 = s < Q ? wre[s] : 0.f, w1 = s + 1 < Q ? wre[s + 1] : 0.f;
      const uint4 r0 = this->v[i][0], r1 = this->v[i][1];
      const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
      const uint32_t bb[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a_lo = bf16_bits_to_f32(a[j] & 0xFFFFu) * w0;
        const float a_hi = bf16_bits_to_f32(a[j] >> 16) * w0;
        const float b_lo = bf16_bits_to_f32(bb[j] & 0xFFFFu) * w1;
        const float b_hi = bf16_bits_to_f32(bb[j] >> 16) * w1;
        *reinterpret_cast<uint32_t*>(bT + (ng * 8 + 2 * j) * XP + 2 * sp) = pack_bf16x2(a_lo, b_lo);
        *reinterpret_cast<uint32_t*>(bT + (ng * 8 + 2 * j + 1) * XP + 2 * sp) =
            pack_bf16x2(a_hi, b_hi);
      }
    }
  }
};

template <int ST, int N>
struct StateBSlab<float, false, ST, N> : Slab<ST, N / 4, 1> {
  __device__ __forceinline__ void store(float* bT, const float* wre, const float*, int s0,
                                        int Q) const {
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

// complex: a 16-byte vector is 2 complex values; bT rows [0,N) hold the real
// parts and [N,2N) the imaginary parts of W_s B_s.
template <int ST, int N>
struct StateBSlab<float, true, ST, N> : Slab<ST, N / 2, 1> {
  __device__ __forceinline__ void store(float* bT, const float* wre, const float* wim, int s0,
                                        int Q) const {
    constexpr int XP = ST + Pad<float>::row;
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % (N / 2), sl = it / (N / 2);
      const int s = s0 + sl;
      const float wr = s < Q ? wre[s] : 0.f, wi = s < Q ? wim[s] : 0.f;
      const uint4 u = this->v[i][0];
      const float br[2] = {__uint_as_float(u.x), __uint_as_float(u.z)};
      const float bi[2] = {__uint_as_float(u.y), __uint_as_float(u.w)};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bT[(ng * 2 + j) * XP + sl] = wr * br[j] - wi * bi[j];
        bT[(N + ng * 2 + j) * XP + sl] = wr * bi[j] + wi * br[j];
      }
    }
  }
};

template <typename TI, bool CPLX, int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_state_kernel(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const TI* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    float* __restrict__ states, float* __restrict__ decay, int T, int H, int G, int Q, int nc,
    int npairs) {
  using E = TI;
  constexpr bool BF = std::is_same<E, uint16_t>::value;
  constexpr int KC = CPLX ? 2 * N : N;
  // stage length: 64 tokens unless two buffers of that size overflow LDS
  constexpr int ST = 2 * (P + KC) * (64 + Pad<E>::row) * int(sizeof(E)) + 8192 <= kLdsBytes ? 64 : 32;
  constexpr int XP = ST + Pad<E>::row;
  constexpr int NTILE = (P / 16) * (KC / 16);
  constexpr int TPW = (NTILE + 3) / 4;  // output tiles per wave

  __shared__ __attribute__((aligned(16))) E xT[2][P * XP];
  __shared__ __attribute__((aligned(16))) E bT[2][KC * XP];
  __shared__ float dl[256], cs_hi[256], cs_lo[256], cth[256], sth[256];
  __shared__ float wre[256], wim[256];
  __shared__ double wsum[4], tot;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const float a_re = CPLX ? A[2 * h] : A[h];
  const float a_im = CPLX ? A[2 * h + 1] : 0.0f;
  const float bias = dt_bias ? dt_bias[h] : 0.0f;

  // issue the first global loads before any arithmetic
  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = tid < Lc ? dt[dt_base + static_cast<size_t>(tid) * H] : 0.0f;
  constexpr int CW = CPLX ? 2 : 1;
  const char* xbase = reinterpret_cast<const char*>(
      x + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P);
  const size_t xrow = static_cast<size_t>(H) * P * sizeof(E);
  const char* bbase = reinterpret_cast<const char*>(
      Bm + (static_cast<size_t>(b) * T + t0) * G * N * CW + static_cast<size_t>(g) * N * CW);
  const size_t brow = static_cast<size_t>(G) * N * CW * sizeof(E);
  XSlab<E, ST, P> xs;
  StateBSlab<E, CPLX, ST, N> bs;
  xs.load(xbase, xrow, 0, Lc);
  bs.load(bbase, brow, 0, Lc);

  const double cum = chunk_prologue<CPLX>(dt_raw, Lc, a_re, a_im, bias, dt_min, dt_max, dl,
                                          cs_hi, cs_lo, cth, sth, wsum, &tot, Q);
  // weight of each source token to the chunk end
  const double total = tot;
  if (tid < Q) {
    const double rem = total - cum;  // steps left (complex) / exponent <= 0 (real)
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
  xs.store(xT[0]);
  bs.store(bT[0], wre, wim, 0, Q);
  __syncthreads();

  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (Lc + ST - 1) / ST;
  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) {
      xs.load(xbase, xrow, (it + 1) * ST, Lc);
      bs.load(bbase, brow, (it + 1) * ST, Lc);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wid + 4 * i;
      if (tile >= NTILE) break;
      const int pt = tile / (KC / 16), kt = tile % (KC / 16);
      const E* arow = xT[cur] + (pt * 16 + r16) * XP;
      const E* brow_l = bT[cur] + (kt * 16 + r16) * XP;
      if constexpr (BF) {
#pragma unroll
        for (int ss = 0; ss < ST; ss += 32) {
          const uint4 av = *reinterpret_cast<const uint4*>(arow + ss + 8 * q);
          const uint4 bv = *reinterpret_cast<const uint4*>(brow_l + ss + 8 * q);
          acc[i] = mfma_bf16(as_bf16x8(av), as_bf16x8(bv), acc[i]);
        }
      } else {
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
    }
    if (more) {
      xs.store(xT[cur ^ 1]);
      bs.store(bT[cur ^ 1], wre, wim, (it + 1) * ST, Q);
    }
    __syncthreads();
  }

  // S[p][k]: accumulator lane holds column k = kt*16 + r16, rows p = pt*16 + 4q + j
  float* dst = states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * KC);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wid + 4 * i;
    if (tile >= NTILE) break;
    const int pt = tile / (KC / 16), kt = tile % (KC / 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[(pt * 16 + 4 * q + j) * KC + kt * 16 + r16] = acc[i][j];
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: chunk outputs.
// ---------------------------------------------------------------------------

// B slab -> bt[s - s0][k] natural layout.  Real: a straight copy.  Complex:
// [B'_re | -B'_im] with B' = B e^{-i theta_s}.
template <typename TI, bool CPLX, int ST, int N, int BP>
struct ScanBSlab;

template <typename TI, int ST, int N, int BP>
struct ScanBSlab<TI, false, ST, N, BP> : Slab<ST, N * sizeof(TI) / 16, 1> {
  __device__ __forceinline__ void store(TI* bt, const float*, const float*, int) const {
    constexpr int VPR = N * sizeof(TI) / 16, V = 16 / sizeof(TI);
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % VPR, sl = it / VPR;
      *reinterpret_cast<uint4*>(bt + sl * BP + ng * V) = this->v[i][0];
    }
  }
};

template <int ST, int N, int BP>
struct ScanBSlab<float, true, ST, N, BP> : Slab<ST, N / 2, 1> {
  __device__ __forceinline__ void store(float* bt, const float* cth, const float* sth,
                                        int s0) const {
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int ng = it % (N / 2), sl = it / (N / 2);
      const int s = s0 + sl;
      const float co = cth[s < 256 ? s : 0], si = sth[s < 256 ? s : 0];
      const uint4 u = this->v[i][0];
      const float br0 = __uint_as_float(u.x), bi0 = __uint_as_float(u.y);
      const float br1 = __uint_as_float(u.z), bi1 = __uint_as_float(u.w);
      *reinterpret_cast<float2*>(bt + sl * BP + ng * 2) =
          make_float2(br0 * co + bi0 * si, br1 * co + bi1 * si);
      *reinterpret_cast<float2*>(bt + sl * BP + N + ng * 2) =
          make_float2(br0 * si - bi0 * co, br1 * si - bi1 * co);
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
template <typename TI, bool CPLX, int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_kernel(
    const TI* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const TI* __restrict__ Bm, const TI* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* __restrict__ hin, TI* __restrict__ y, int T, int H, int G, int Q, int nc,
    int npairs) {
  using E = TI;
  constexpr bool BF = std::is_same<E, uint16_t>::value;
  constexpr int KC = CPLX ? 2 * N : N;
  constexpr int KSTEP = BF ? 32 : 16;           // k covered by one operand register group
  constexpr int KCP = KC < KSTEP ? KSTEP : KC;  // K padded to whole MFMA steps (zeros)
  constexpr int BP = KCP + Pad<E>::row;         // pitch of bt / hT rows
  // stage length: 64 tokens unless two buffers of that size overflow LDS
  constexpr int ST = (2 * (64 * BP + P * (64 + Pad<E>::row)) + P * BP) * int(sizeof(E)) + 8192 <=
                             kLdsBytes ? 64 : 32;
  constexpr int XP = ST + Pad<E>::row;          // pitch of xT rows
  constexpr int NKS = KCP / KSTEP;
  constexpr int NPT = P / 16;
  constexpr int MAXR = 4;
  constexpr int CW = CPLX ? 2 : 1;
  typedef typename std::conditional<BF, uint4, float4>::type CReg;

  __shared__ __attribute__((aligned(16))) E bt[2][ST * BP];
  __shared__ __attribute__((aligned(16))) E xT[2][P * XP];
  __shared__ __attribute__((aligned(16))) E hT[P * BP];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs_hi[256];
  __shared__ __attribute__((aligned(16))) float cs_lo[256];
  __shared__ __attribute__((aligned(16))) float cth[256];
  __shared__ __attribute__((aligned(16))) float sth[256];
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
  const float a_re = CPLX ? A[2 * h] : A[h];
  const float a_im = CPLX ? A[2 * h + 1] : 0.0f;
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const float Dh = (!CPLX && D) ? D[h] : 0.0f;

  // ---- issue global loads: dt, h_in, C rows, first source stage ----
  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = tid < Lc ? dt[dt_base + static_cast<size_t>(tid) * H] : 0.0f;

  constexpr int HV = P * KC / 4;  // float4 vectors of h_in
  constexpr int HPER = (HV + kThreads - 1) / kThreads;
  float4 hreg[HPER];
  {
    const float* src = hin + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * KC);
#pragma unroll
    for (int i = 0; i < HPER; ++i) {
      const int it = tid + i * kThreads;
      if (it < HV) hreg[i] = *reinterpret_cast<const float4*>(src + it * 4);
    }
  }

  int tl[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) tl[r] = (r / 2) * 8 + ((r & 1) ? 7 - wid : wid);

  const size_t cstride = static_cast<size_t>(G) * N * CW;  // elements between tokens
  const size_t c_row0 = (static_cast<size_t>(b) * T + t0) * cstride + static_cast<size_t>(g) * N * CW;

  // C rows of the owned tiles, in the operand layout: lane (row r16, group q)
  // holds k = ks*KSTEP + (BF ? 8q .. 8q+7 : 4q .. 4q+3).  Complex: raw
  // (re, im) pairs now, rotated once the prologue has the angles.
  CReg creg[MAXR][NKS];
  float4 craw[CPLX ? MAXR : 1][CPLX ? NKS : 1];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = tl[r] * 16 + r16;
    const bool ok = tl[r] < ntl && row < Lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int k0 = ks * KSTEP + (BF ? 8 : 4) * q;
      if constexpr (CPLX) {
        // 4 complex values of n0 .. n0+3 (two float4)
        const int n0 = k0 < N ? k0 : k0 - N;
        float4 u = make_float4(0.f, 0.f, 0.f, 0.f), v = u;
        if (ok) {
          const float4* src = reinterpret_cast<const float4*>(Cm + c_row0 + row * cstride + 2 * n0);
          u = src[0];
          v = src[1];
        }
        creg[r][ks] = u;
        craw[r][ks] = v;
      } else {
        CReg o{};
        if (ok && k0 < KC) o = *reinterpret_cast<const CReg*>(Cm + c_row0 + row * cstride + k0);
        creg[r][ks] = o;
      }
    }
  }

  const char* xbase = reinterpret_cast<const char*>(
      x + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P);
  const size_t xrow = static_cast<size_t>(H) * P * sizeof(E);
  const char* bbase = reinterpret_cast<const char*>(Bm + c_row0);
  const size_t brow = cstride * sizeof(E);
  XSlab<E, ST, P> xs;
  ScanBSlab<E, CPLX, ST, N, BP> bs;
  xs.load(xbase, xrow, 0, Lc);
  bs.load(bbase, brow, 0, Lc);

  // ---- prologue ----
  chunk_prologue<CPLX>(dt_raw, Lc, a_re, a_im, bias, dt_min, dt_max, dl, cs_hi, cs_lo, cth, sth,
                       wsum, &tot, Q);

  if constexpr (KCP > KC) {
    // zero the K padding of both bt buffers and hT (never written by stages)
    for (int it = tid; it < ST + P; it += kThreads) {
      E* row = it < ST ? bt[0] + it * BP : hT + (it - ST) * BP;
      for (int k = KC; k < KCP; ++k) row[k] = E(0);
      if (it < ST)
        for (int k = KC; k < KCP; ++k) bt[1][it * BP + k] = E(0);
    }
  }
  // h_in -> hT: real h[p][n]; complex [h_re | -h_im]
#pragma unroll
  for (int i = 0; i < HPER; ++i) {
    const int it = tid + i * kThreads;
    if (it >= HV) break;
    const int p = (it * 4) / KC, k = (it * 4) % KC;
    float4 u = hreg[i];
    if constexpr (BF) {
      *reinterpret_cast<uint2*>(hT + p * BP + k) =
          make_uint2(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w));
    } else {
      if (CPLX && k >= N) u = make_float4(-u.x, -u.y, -u.z, -u.w);
      *reinterpret_cast<float4*>(hT + p * BP + k) = u;
    }
  }
  xs.store(xT[0]);
  bs.store(bt[0], cth, sth, 0);
  if constexpr (CPLX) {
    // C' = C e^{i theta_l}: lanes with k0 < N keep C'_re, the others C'_im
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int row = tl[r] * 16 + r16;
      const float co = (tl[r] < ntl && row < Q) ? cth[row] : 1.f;
      const float si = (tl[r] < ntl && row < Q) ? sth[row] : 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int k0 = ks * KSTEP + 4 * q;
        const float4 u = creg[r][ks], v = craw[r][ks];
        const float cr[4] = {u.x, u.z, v.x, v.z}, ci[4] = {u.y, u.w, v.y, v.w};
        float res[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          res[j] = k0 < N ? cr[j] * co - ci[j] * si : cr[j] * si + ci[j] * co;
        creg[r][ks] = make_float4(res[0], res[1], res[2], res[3]);
      }
    }
  }
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
      if constexpr (BF) {
        const uint4 cv = creg[r][ks];
        const uint32_t w[4] = {cv.x, cv.y, cv.z, cv.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_bf16x2(bf16_bits_to_f32(w[j] & 0xFFFFu) * sc,
                             bf16_bits_to_f32(w[j] >> 16) * sc);
        const uint4 a = make_uint4(o[0], o[1], o[2], o[3]);
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint4 hv =
              *reinterpret_cast<const uint4*>(hT + (pt * 16 + r16) * BP + ks * KSTEP + 8 * q);
          yacc[r][pt] = mfma_bf16(as_bf16x8(a), as_bf16x8(hv), yacc[r][pt]);
        }
      } else {
        const float4 cv = creg[r][ks];
        const float4 a = make_float4(cv.x * sc, cv.y * sc, cv.z * sc, cv.w * sc);
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const float4 hv =
              *reinterpret_cast<const float4*>(hT + (pt * 16 + r16) * BP + ks * KSTEP + 4 * q);
          yacc[r][pt] = mfma_f32(a.x, hv.x, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(a.y, hv.y, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(a.z, hv.z, yacc[r][pt]);
          yacc[r][pt] = mfma_f32(a.w, hv.w, yacc[r][pt]);
        }
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
    const E* btc = bt[cur];
    const E* xTc = xT[cur];
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (tl[r] >= ntl) continue;
      const int lfirst = tl[r] * 16, llast = lfirst + 15;
      if (s0 > llast) continue;
      const int lrow = lfirst + r16;  // this lane's output row l (as G^T column)
      const float lh = cs_hi[lrow], ll = cs_lo[lrow];
      if constexpr (BF) {
#pragma unroll
        for (int ss = 0; ss < ST; ss += 32) {
          const int sb = s0 + ss;
          if (sb > llast) break;
          const bool need_b = sb + 16 <= llast;  // second 16-row sub-tile not all masked
          f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 va = *reinterpret_cast<const uint4*>(btc + (ss + r16) * BP + ks * 32 + 8 * q);
            ga = mfma_bf16(as_bf16x8(va), as_bf16x8(creg[r][ks]), ga);
          }
          if (need_b) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
              const uint4 vb =
                  *reinterpret_cast<const uint4*>(btc + (ss + 16 + r16) * BP + ks * 32 + 8 * q);
              gb = mfma_bf16(as_bf16x8(vb), as_bf16x8(creg[r][ks]), gb);
            }
          }
          const float4 ha = *reinterpret_cast<const float4*>(cs_hi + sb + 4 * q);
          const float4 la = *reinterpret_cast<const float4*>(cs_lo + sb + 4 * q);
          const float4 hb = *reinterpret_cast<const float4*>(cs_hi + sb + 16 + 4 * q);
          const float4 lb = *reinterpret_cast<const float4*>(cs_lo + sb + 16 + 4 * q);
          const float4 da = *reinterpret_cast<const float4*>(dl + sb + 4 * q);
          const float4 db = *reinterpret_cast<const float4*>(dl + sb + 16 + 4 * q);
          const float hav[4] = {ha.x, ha.y, ha.z, ha.w}, lav[4] = {la.x, la.y, la.z, la.w};
          const float hbv[4] = {hb.x, hb.y, hb.z, hb.w}, lbv[4] = {lb.x, lb.y, lb.z, lb.w};
          const float dav[4] = {da.x, da.y, da.z, da.w}, dbv[4] = {db.x, db.y, db.z, db.w};
          float m[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int sa = sb + 4 * q + j, sbb = sb + 16 + 4 * q + j;
            const float wa = sa <= lrow ? decay_between(lh, ll, hav[j], lav[j]) * (CPLX ? 1.f : dav[j]) : 0.f;
            const float wb = sbb <= lrow ? decay_between(lh, ll, hbv[j], lbv[j]) * (CPLX ? 1.f : dbv[j]) : 0.f;
            m[j] = ga[j] * wa;
            m[4 + j] = gb[j] * wb;
          }
          const uint4 mv = make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]),
                                      pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7]));
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) {
            const E* xr = xTc + (pt * 16 + r16) * XP + ss + 4 * q;
            const uint2 x0 = *reinterpret_cast<const uint2*>(xr);
            const uint2 x1 = *reinterpret_cast<const uint2*>(xr + 16);
            const uint4 xv = make_uint4(x0.x, x0.y, x1.x, x1.y);
            yacc[r][pt] = mfma_bf16(as_bf16x8(mv), as_bf16x8(xv), yacc[r][pt]);
          }
        }
      } else {
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
            const float wa = sa <= lrow ? decay_between(lh, ll, hav[j], lav[j]) * (CPLX ? 1.f : dav[j]) : 0.f;
            m[j] = ga[j] * wa;
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
      }
      // (3) D x for the tile's own rows, while they sit in this stage
      if (!CPLX && lfirst >= s0 && lfirst < s0 + ST) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const E* xr = xTc + (pt * 16 + r16) * XP + (lfirst - s0) + 4 * q;
          float xv[4];
          if constexpr (BF) {
            const uint2 u = *reinterpret_cast<const uint2*>(xr);
            xv[0] = bf16_bits_to_f32(u.x & 0xFFFFu);
            xv[1] = bf16_bits_to_f32(u.x >> 16);
            xv[2] = bf16_bits_to_f32(u.y & 0xFFFFu);
            xv[3] = bf16_bits_to_f32(u.y >> 16);
          } else {
            const float4 u = *reinterpret_cast<const float4*>(xr);
            xv[0] = u.x;
            xv[1] = u.y;
            xv[2] = u.z;
            xv[3] = u.w;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) yacc[r][pt][j] += Dh * xv[j];
        }
      }
    }
    if (more) {
      xs.store(xT[cur ^ 1]);
      bs.store(bt[cur ^ 1], cth, sth, s0 + ST);
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
        if (l < Lc) store_elem(y, x_row0 + l * x_rs + pt * 16 + r16, yacc[r][pt][j]);
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
  const int npairs = a.Bsz * nc;
  float* states = static_cast<float*>(a.workspace);
  float* decay = states + workspace_state_floats(a.Bsz, nc, a.H, a.P, KC);
  const TI* x = static_cast<const TI*>(a.x);
  const TI* B = static_cast<const TI*>(a.B);
  const TI* C = static_cast<const TI*>(a.C);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  const hipEvent_t* ev = a.events;
  launch_k(nc > 0, ssd_state_kernel<TI, CPLX, P, N>, dim3(blocks), dim3(kThreads), st, ev, x,
           a.dt, a.A, B, a.dt_bias, a.dt_min, a.dt_max, states, decay, a.T, a.H, a.G, a.chunk,
           nc, npairs);
  launch_pass<CPLX, N>(states, decay, a.h0, a.h_final, a.Bsz, a.H, P, nc, st,
                       ev ? ev + 2 : nullptr);
  launch_k(nc > 0, ssd_scan_kernel<TI, CPLX, P, N>, dim3(blocks), dim3(kThreads), st,
           ev ? ev + 4 : nullptr, x, a.dt, a.A, B, C, a.D, a.dt_bias, a.dt_min, a.dt_max,
           static_cast<const float*>(states), static_cast<TI*>(a.y), a.T, a.H, a.G, a.chunk, nc,
           npairs);
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
  if (a.dtype == 1) return run_chunk_real_bf16(a, st);
  return dispatch_p<float, false>(a, st);
}


}  // namespace ssd
