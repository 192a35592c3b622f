// Chunked SSD forward on gfx950 for bfloat16 x, B, C (real Mamba-2 form; fp32
// state, fp32 accumulation): the chunk-state and chunk-output kernels.  The
// inter-chunk scan between them is the shared ssd_pass_kernel.
//
// Both kernels stage token rows into LDS in their natural row-major layout
// (plain 16-byte stores) and read MFMA operands whose contraction runs over
// tokens with the gfx950 LDS transpose read ds_read_b64_tr_b16.
//
// Chunk outputs, per (batch, chunk, head) workgroup, Q tokens l, s:
//   y_l = sum_{s<=l} (C_l . B_s) e^{cs_l - cs_s} delta_s x_s   (intra-chunk)
//       + e^{cs_l} C_l . h_in                                  (carried state)
//       + D x_l
// The decay of a source block of 16 tokens ending at r (s in r-15..r) and a
// later output row l factors as e^{cs_l - cs_r} e^{cs_r - cs_s}: both factors
// are <= 1 (no overflow), the second is folded into a scaled copy of x when
// the stage is staged, the first is one exp per lane and block.  Only the
// 16 x 16 blocks on the diagonal (s and l in the same block) take an exp per
// element, with the causal mask, against the unscaled x.
// (Numerical Stability in Mamba-3-Lite, section 4: L[l,s] = exp(cs_l - cs_s)
// 1[l >= s]; the chunk carry by the chunk's total log-decay.)

#include "ssd_chunk_common.h"

namespace ssd {

typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((address_space(3))) short4v lds_short4v;

// LDS transpose read (ds_read_b64_tr_b16) of a row-major bf16 tile; call it
// with all 64 lanes active (wave-uniform control flow only).  Lane i
// of each 16-lane group receives the values of column col0 + (i % 16) in rows
// row0 .. row0+3 (row0 may differ between the four groups of a wave), as four
// bf16 in a uint2, row order.  The instruction hands lane i element (i % 4)
// of the 8 bytes addressed by lanes 4k + i/4 (k = 0..3) of its group, so lane
// m addresses row row0 + m/4, columns col0 + 4(m % 4) .. +3.
__device__ __forceinline__ uint2 lds_tr4(const uint16_t* tile, int pitch, int row0, int col0) {
  const int m = threadIdx.x & 15;
  const uint16_t* a = tile + (row0 + (m >> 2)) * pitch + col0 + 4 * (m & 3);
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(const_cast<uint16_t*>(a)));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float w) {
  const uint32_t a[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = pack_bf16x2(bf16_bits_to_f32(a[j] & 0xFFFFu) * w, bf16_bits_to_f32(a[j] >> 16) * w);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// Chunk-end states from a zero start: S[p][n] = sum_s (w_s x_s[p]) B_s[n],
// w_s = e^{cs_last - cs_s} delta_s.  Each wave owns N/64 of the n tiles (all
// p tiles), so an x fragment is read once per k step and reused over them.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_state_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, float* __restrict__ states, float* __restrict__ decay, int T, int H, int G,
    int Q, int nc, int npairs) {
  constexpr int ST = 64;
  constexpr int XPn = P + 16, BPn = N + 16;  // natural pitches (bf16 elements)
  constexpr int KT = N / 16, PT = P / 16;
  constexpr int KTW = (KT + 3) / 4;          // n tiles per wave

  __shared__ __attribute__((aligned(16))) uint16_t xl[ST * XPn];
  __shared__ __attribute__((aligned(16))) uint16_t bl[ST * BPn];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs_hi[256];
  __shared__ __attribute__((aligned(16))) float cs_lo[256];
  __shared__ __attribute__((aligned(16))) float wsc[256];
  __shared__ double wsum[4], tot;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar

  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = tid < Lc ? dt[dt_base + static_cast<size_t>(tid) * H] : 0.0f;
  const char* xbase = reinterpret_cast<const char*>(
      x + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P);
  const size_t xrow = static_cast<size_t>(H) * P * 2;
  const char* bbase = reinterpret_cast<const char*>(
      Bm + (static_cast<size_t>(b) * T + t0) * G * N + static_cast<size_t>(g) * N);
  const size_t brow = static_cast<size_t>(G) * N * 2;
  Slab<ST, P / 8, 1> xs;
  Slab<ST, N / 8, 1> bs;
  xs.load(xbase, xrow, 0, Lc);
  bs.load(bbase, brow, 0, Lc);

  const float a_re = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const double cum = chunk_prologue<false>(dt_raw, Lc, a_re, 0.0f, bias, dt_min, dt_max, dl,
                                           cs_hi, cs_lo, nullptr, nullptr, wsum, &tot, Q);
  const double total = tot;
  if (tid < Q) wsc[tid] = __expf(static_cast<float>(total - cum)) * dl[tid];
  if (tid == 0) {
    float* dc = decay + ((static_cast<size_t>(b) * H + h) * nc + c) * 2;
    dc[0] = __expf(static_cast<float>(total));
    dc[1] = 0.0f;
  }
  __syncthreads();

  auto store_stage = [&](int s0) {
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (it < xs.ITEMS) {
        const int v = it % (P / 8), sl = it / (P / 8);
        const int s = s0 + sl;
        const float w = s < Q ? wsc[s] : 0.0f;
        *reinterpret_cast<uint4*>(xl + sl * XPn + v * 8) = scale_bf16x8(xs.v[i][0], w);
      }
    }
#pragma unroll
    for (int i = 0; i < bs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (it < bs.ITEMS) {
        const int v = it % (N / 8), sl = it / (N / 8);
        *reinterpret_cast<uint4*>(bl + sl * BPn + v * 8) = bs.v[i][0];
      }
    }
  };
  store_stage(0);
  __syncthreads();

  f32x4 acc[KTW][PT];
#pragma unroll
  for (int i = 0; i < KTW; ++i)
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) acc[i][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (Lc + ST - 1) / ST;
  for (int it = 0; it < ntiles; ++it) {
    const bool more = it + 1 < ntiles;
    if (more) {
      xs.load(xbase, xrow, (it + 1) * ST, Lc);
      bs.load(bbase, brow, (it + 1) * ST, Lc);
    }
#pragma unroll
    for (int ss = 0; ss < ST; ss += 32) {
      uint4 afr[PT];
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        const uint2 lo = lds_tr4(xl, XPn, ss + 8 * q, pt * 16);
        const uint2 hi = lds_tr4(xl, XPn, ss + 8 * q + 4, pt * 16);
        afr[pt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
#pragma unroll
      for (int i = 0; i < KTW; ++i) {
        const int kt = wid * KTW + i;
        if (kt >= KT) break;
        const uint2 lo = lds_tr4(bl, BPn, ss + 8 * q, kt * 16);
        const uint2 hi = lds_tr4(bl, BPn, ss + 8 * q + 4, kt * 16);
        const uint4 bfr = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          acc[i][pt] = mfma_bf16(as_bf16x8(afr[pt]), as_bf16x8(bfr), acc[i][pt]);
      }
    }
    if (more) {
      __syncthreads();
      store_stage((it + 1) * ST);
      __syncthreads();
    }
  }

  // S[p][n]: accumulator lane holds column n = kt*16 + r16, rows p = pt*16 + 4q + j
  float* dst = states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N);
#pragma unroll
  for (int i = 0; i < KTW; ++i) {
    const int kt = wid * KTW + i;
    if (kt >= KT) break;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(pt * 16 + 4 * q + j) * N + kt * 16 + r16] = acc[i][pt][j];
  }
}

// ---------------------------------------------------------------------------
// Chunk outputs.  Wave w owns the 16-row output tiles w, 7-w, 8+w, 15-w (those
// below Q/16), which balances the causal work; it keeps their C rows in
// registers as MFMA operands.  Per 32-token source step the wave reads the B
// fragments and the scaled-x fragments once and applies them to all of its
// tiles:  G^T = B_s . C_l^T (MFMA; lane = column l, rows s), then
// M = G^T x decay, whose accumulator layout is exactly the A operand of
// Y += M . X.  y is staged through LDS and written with 16-byte stores.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* __restrict__ hin, uint16_t* __restrict__ y, int T, int H, int G, int Q, int nc,
    int npairs) {
  constexpr int ST = 64;
  constexpr int KCP = N < 32 ? 32 : N;  // K padded to whole 32-wide MFMA steps (zeros)
  constexpr int BP = KCP + 8;           // pitch of bt / hT rows
  constexpr int XPn = P + 16;           // pitch of the natural x tiles
  constexpr int YP = P + 8;             // pitch of the y staging tile
  constexpr int NKS = KCP / 32;
  constexpr int NPT = P / 16;
  constexpr int MAXR = 4;
  constexpr int STAGE_BYTES = (ST * BP + 2 * ST * XPn) * 2;
  constexpr int YT_BYTES = 256 * YP * 2;
  constexpr int R1 = STAGE_BYTES > YT_BYTES ? STAGE_BYTES : YT_BYTES;

  // stage buffers during the source loop; the y tile afterwards
  __shared__ __attribute__((aligned(16))) uint16_t r1[R1 / 2];
  uint16_t* const bt = r1;
  uint16_t* const xl = r1 + ST * BP;
  uint16_t* const xsl = xl + ST * XPn;
  uint16_t* const yt = r1;
  __shared__ __attribute__((aligned(16))) uint16_t hT[P * BP];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs_hi[256];
  __shared__ __attribute__((aligned(16))) float cs_lo[256];
  __shared__ __attribute__((aligned(16))) float xsc[256];
  __shared__ __attribute__((aligned(16))) float ecs[256];
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

  // ---- global loads first: dt, h_in, C rows, first source stage ----
  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = tid < Lc ? dt[dt_base + static_cast<size_t>(tid) * H] : 0.0f;

  constexpr int HV = P * N / 4;
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
  int lmax = -1;
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
    if (tl[r] < ntl) lmax = max(lmax, tl[r] * 16 + 15);

  const size_t cstride = static_cast<size_t>(G) * N;
  const size_t c_row0 = (static_cast<size_t>(b) * T + t0) * cstride + static_cast<size_t>(g) * N;
  // C rows of the owned tiles: lane (row r16, group q) holds k = ks*32 + 8q .. +7
  uint4 creg[MAXR][NKS];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = tl[r] * 16 + r16;
    const bool ok = tl[r] < ntl && row < Lc;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int k0 = ks * 32 + 8 * q;
      uint4 o = make_uint4(0, 0, 0, 0);
      if (ok && k0 < N) o = *reinterpret_cast<const uint4*>(Cm + c_row0 + row * cstride + k0);
      creg[r][ks] = o;
    }
  }

  const char* xbase = reinterpret_cast<const char*>(
      x + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P);
  const size_t xrow = static_cast<size_t>(H) * P * 2;
  const char* bbase = reinterpret_cast<const char*>(Bm + c_row0);
  const size_t brow = cstride * 2;
  Slab<ST, P / 8, 1> xs;
  Slab<ST, N / 8, 1> bs;
  xs.load(xbase, xrow, 0, Lc);
  bs.load(bbase, brow, 0, Lc);

  // ---- prologue ----
  chunk_prologue<false>(dt_raw, Lc, a_re, 0.0f, bias, dt_min, dt_max, dl, cs_hi, cs_lo, nullptr,
                        nullptr, wsum, &tot, Q);
  if (tid < Q) {
    const int ref = tid | 15;  // last token of this token's 16-block
    const float colf = decay_between(cs_hi[ref], cs_lo[ref], cs_hi[tid], cs_lo[tid]);
    xsc[tid] = colf * dl[tid];
    ecs[tid] = __expf(cs_hi[tid] + cs_lo[tid]);
  }
  if constexpr (KCP > N) {
    // zero the K padding of bt and hT (stage stores never write it)
    for (int it = tid; it < ST + P; it += kThreads) {
      uint16_t* row = it < ST ? bt + it * BP : hT + (it - ST) * BP;
      for (int k = N; k < KCP; ++k) row[k] = 0;
    }
  }
#pragma unroll
  for (int i = 0; i < HPER; ++i) {
    const int it = tid + i * kThreads;
    if (it < HV) {
      const int p = (it * 4) / N, k = (it * 4) % N;
      const float4 u = hreg[i];
      *reinterpret_cast<uint2*>(hT + p * BP + k) =
          make_uint2(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w));
    }
  }
  __syncthreads();

  auto store_stage = [&](int s0) {
#pragma unroll
    for (int i = 0; i < bs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (it < bs.ITEMS) {
        const int v = it % (N / 8), sl = it / (N / 8);
        *reinterpret_cast<uint4*>(bt + sl * BP + v * 8) = bs.v[i][0];
      }
    }
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (it < xs.ITEMS) {
        const int v = it % (P / 8), sl = it / (P / 8);
        const int s = s0 + sl;
        const float w = s < Q ? xsc[s] : 0.0f;
        *reinterpret_cast<uint4*>(xl + sl * XPn + v * 8) = xs.v[i][0];
        *reinterpret_cast<uint4*>(xsl + sl * XPn + v * 8) = scale_bf16x8(xs.v[i][0], w);
      }
    }
  };
  store_stage(0);

  // (1) carried state: Y = (C . h_in) with rows scaled by e^{cs_l} afterwards
  f32x4 yacc[MAXR][NPT];
#pragma unroll
  for (int r = 0; r < MAXR; ++r)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) yacc[r][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (tl[r] >= ntl) continue;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const uint4 hv = *reinterpret_cast<const uint4*>(hT + (pt * 16 + r16) * BP + ks * 32 + 8 * q);
        yacc[r][pt] = mfma_bf16(as_bf16x8(creg[r][ks]), as_bf16x8(hv), yacc[r][pt]);
      }
    }
    const float4 e = *reinterpret_cast<const float4*>(ecs + tl[r] * 16 + 4 * q);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      yacc[r][pt][0] *= e.x;
      yacc[r][pt][1] *= e.y;
      yacc[r][pt][2] *= e.z;
      yacc[r][pt][3] *= e.w;
    }
  }
  __syncthreads();

  // (2) intra-chunk part and (3) the skip term, one stage of ST tokens at a time
  const int ntiles = (Lc + ST - 1) / ST;
  for (int it = 0; it < ntiles; ++it) {
    const int s0 = it * ST;
    const bool more = it + 1 < ntiles;
    if (more) {
      xs.load(xbase, xrow, s0 + ST, Lc);
      bs.load(bbase, brow, s0 + ST, Lc);
    }
#pragma unroll
    for (int ss = 0; ss < ST; ss += 32) {
      const int sb = s0 + ss;
      if (sb > lmax) break;
      uint4 bA[NKS], bB[NKS], xsf[NPT];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        bA[ks] = *reinterpret_cast<const uint4*>(bt + (ss + r16) * BP + ks * 32 + 8 * q);
        bB[ks] = *reinterpret_cast<const uint4*>(bt + (ss + 16 + r16) * BP + ks * 32 + 8 * q);
      }
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const uint2 lo = lds_tr4(xsl, XPn, ss + 4 * q, pt * 16);
        const uint2 hi = lds_tr4(xsl, XPn, ss + 16 + 4 * q, pt * 16);
        xsf[pt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
      // decay exponents at the two block ends (all lanes read the same word)
      const float refa_h = cs_hi[sb + 15], refa_l = cs_lo[sb + 15];
      const float refb_h = cs_hi[sb + 31], refb_l = cs_lo[sb + 31];
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        if (tl[r] >= ntl) continue;
        const int lfirst = tl[r] * 16, llast = lfirst + 15;
        if (sb > llast) continue;
        const bool a_diag = sb == lfirst;        // first 16 sources = this tile's rows
        const bool b_diag = sb + 16 == lfirst;   // second 16 sources = this tile's rows
        const bool b_dead = sb + 16 > llast;     // second 16 sources all after the tile
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ga = mfma_bf16(as_bf16x8(bA[ks]), as_bf16x8(creg[r][ks]), ga);
        if (!b_dead) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            gb = mfma_bf16(as_bf16x8(bB[ks]), as_bf16x8(creg[r][ks]), gb);
        }
        const int lrow = lfirst + r16;
        const float lh = cs_hi[lrow], ll = cs_lo[lrow];
        float m[8];
        if (a_diag) {
          const float4 hs = *reinterpret_cast<const float4*>(cs_hi + sb + 4 * q);
          const float4 ls = *reinterpret_cast<const float4*>(cs_lo + sb + 4 * q);
          const float4 ds = *reinterpret_cast<const float4*>(dl + sb + 4 * q);
          const float hv[4] = {hs.x, hs.y, hs.z, hs.w}, lv[4] = {ls.x, ls.y, ls.z, ls.w};
          const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            m[j] = sb + 4 * q + j <= lrow ? ga[j] * decay_between(lh, ll, hv[j], lv[j]) * dv[j] : 0.f;
        } else {
          const float rf = decay_between(lh, ll, refa_h, refa_l);
#pragma unroll
          for (int j = 0; j < 4; ++j) m[j] = ga[j] * rf;
        }
        if (b_dead) {
#pragma unroll
          for (int j = 0; j < 4; ++j) m[4 + j] = 0.f;
        } else if (b_diag) {
          const float4 hs = *reinterpret_cast<const float4*>(cs_hi + sb + 16 + 4 * q);
          const float4 ls = *reinterpret_cast<const float4*>(cs_lo + sb + 16 + 4 * q);
          const float4 ds = *reinterpret_cast<const float4*>(dl + sb + 16 + 4 * q);
          const float hv[4] = {hs.x, hs.y, hs.z, hs.w}, lv[4] = {ls.x, ls.y, ls.z, ls.w};
          const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            m[4 + j] =
                sb + 16 + 4 * q + j <= lrow ? gb[j] * decay_between(lh, ll, hv[j], lv[j]) * dv[j] : 0.f;
        } else {
          const float rf = decay_between(lh, ll, refb_h, refb_l);
#pragma unroll
          for (int j = 0; j < 4; ++j) m[4 + j] = gb[j] * rf;
        }
        const uint4 mv = make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]),
                                    pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7]));
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          uint4 xv = xsf[pt];
          if (a_diag) {
            const uint2 raw = lds_tr4(xl, XPn, ss + 4 * q, pt * 16);
            xv.x = raw.x;
            xv.y = raw.y;
          }
          if (b_diag) {
            const uint2 raw = lds_tr4(xl, XPn, ss + 16 + 4 * q, pt * 16);
            xv.z = raw.x;
            xv.w = raw.y;
          }
          yacc[r][pt] = mfma_bf16(as_bf16x8(mv), as_bf16x8(xv), yacc[r][pt]);
        }
      }
    }
    // (3) D x for the tiles whose rows sit in this stage
    if (D) {
#pragma unroll
      for (int r = 0; r < MAXR; ++r) {
        if (tl[r] >= ntl) continue;
        const int lfirst = tl[r] * 16;
        if (lfirst < s0 || lfirst >= s0 + ST) continue;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 u = lds_tr4(xl, XPn, lfirst - s0 + 4 * q, pt * 16);
          yacc[r][pt][0] += Dh * bf16_bits_to_f32(u.x & 0xFFFFu);
          yacc[r][pt][1] += Dh * bf16_bits_to_f32(u.x >> 16);
          yacc[r][pt][2] += Dh * bf16_bits_to_f32(u.y & 0xFFFFu);
          yacc[r][pt][3] += Dh * bf16_bits_to_f32(u.y >> 16);
        }
      }
    }
    if (more) {
      __syncthreads();
      store_stage(s0 + ST);
      __syncthreads();
    }
  }

  // y: through LDS (row-major tile, reusing the stage buffers) to 16-byte stores
  __syncthreads();
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    if (tl[r] >= ntl) continue;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        yt[(tl[r] * 16 + 4 * q + j) * YP + pt * 16 + r16] = f32_to_bf16_bits(yacc[r][pt][j]);
  }
  __syncthreads();
  {
    uint16_t* ybase = y + (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P;
    const size_t yrow = static_cast<size_t>(H) * P;
    for (int it = tid; it < Lc * (P / 8); it += kThreads) {
      const int l = it / (P / 8), v = it % (P / 8);
      *reinterpret_cast<uint4*>(ybase + l * yrow + v * 8) =
          *reinterpret_cast<const uint4*>(yt + l * YP + v * 8);
    }
  }
}

// ---------------------------------------------------------------------------
template <int P, int N>
static hipError_t launch_bf16(const ChunkArgs& a, hipStream_t st) {
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  const int npairs = a.Bsz * nc;
  float* states = static_cast<float*>(a.workspace);
  float* decay = states + workspace_state_floats(a.Bsz, nc, a.H, a.P, N);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const uint16_t* C = static_cast<const uint16_t*>(a.C);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  if (a.events) (void)hipEventRecord(a.events[0], st);
  if (nc > 0)
    ssd_state_bf16_kernel<P, N><<<blocks, kThreads, 0, st>>>(
        x, a.dt, a.A, B, a.dt_bias, a.dt_min, a.dt_max, states, decay, a.T, a.H, a.G, a.chunk,
        nc, npairs);
  if (a.events) (void)hipEventRecord(a.events[1], st);
  launch_pass<false, N>(states, decay, a.h0, a.h_final, a.Bsz, a.H, P, nc, st);
  if (a.events) (void)hipEventRecord(a.events[2], st);
  if (nc > 0)
    ssd_scan_bf16_kernel<P, N><<<blocks, kThreads, 0, st>>>(
        x, a.dt, a.A, B, C, a.D, a.dt_bias, a.dt_min, a.dt_max, states,
        static_cast<uint16_t*>(a.y), a.T, a.H, a.G, a.chunk, nc, npairs);
  if (a.events) (void)hipEventRecord(a.events[3], st);
  return hipGetLastError();
}

template <int P>
static hipError_t dispatch_bf16_n(const ChunkArgs& a, hipStream_t st) {
  switch (a.N) {
    case 16: return launch_bf16<P, 16>(a, st);
    case 32: return launch_bf16<P, 32>(a, st);
    case 64: return launch_bf16<P, 64>(a, st);
    case 128: return launch_bf16<P, 128>(a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t run_chunk_real_bf16(const ChunkArgs& a, hipStream_t st) {
  switch (a.P) {
    case 16: return dispatch_bf16_n<16>(a, st);
    case 32: return dispatch_bf16_n<32>(a, st);
    case 64: return dispatch_bf16_n<64>(a, st);
    case 128: return dispatch_bf16_n<128>(a, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
