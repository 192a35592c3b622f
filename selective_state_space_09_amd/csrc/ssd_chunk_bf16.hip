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
// Chunk outputs.  The workgroup walks its chunk in sub-chunks of QS = 64
// tokens and carries the state across them in MFMA accumulators; for
// sub-chunk j (tokens j0..j1, state h_j at its start, h_0 = h_in(c)):
//   y_l     = e^{cs_l - cs_{j0-1}} C_l . h_j                      (carried)
//           + sum_{j0 <= s <= l} (C_l . B_s) e^{cs_l - cs_s} delta_s x_s
//           + D x_l
//   h_{j+1} = e^{cs_j1 - cs_{j0-1}} h_j + sum_s e^{cs_j1 - cs_s} delta_s x_s B_s^T
// (the chunkwise identity applied once more inside the chunk: the quadratic
// part shrinks to 64 x 64 blocks at the price of a small state update per
// sub-chunk).
//
// Decay factoring.  With the pivot m = j0 + QS/2 - 1 of the sub-chunk,
// e^{cs_l - cs_s} = e^{cs_l - cs_m} e^{cs_m - cs_s}: the first factor scales
// C_l once (C~), the second scales x_s once (x^ = x e^{cs_m - cs_s} delta), and
// the intra-chunk matrix is just (B_s . C~_l) under the causal mask -- no
// per-element exponentials.  The same C~ serves the carried term if the state
// is kept as H = e^{cs_m - cs_{j0-1}} h_j (scaled by one factor per
// sub-chunk), and the state update accumulates x^ B^T into it.  The factors
// stay below e^60 when every half sub-chunk decays by at most e^60; when a
// chunk breaks that bound the workgroup switches to exact mode (per-element
// exponentials, unscaled C in the intra products, state kept unscaled).
//
// Wave w produces output rows 16w .. 16w+15 of each sub-chunk (C rows in
// registers, prefetched a sub-chunk ahead): G^T = B_s . C_l^T on MFMA per 32
// source tokens; its accumulator (lane = column l, rows s) is, after the mask,
// the A operand of Y += M . X.  For the state update wave w owns n tiles
// w, w+4, ..: H^T[n][p] += sum_s B_s[n] x^_s[p] (both operands from LDS with
// the transpose read), so a lane holds 4 consecutive n of one p and writes the
// bf16 state tile with 8-byte stores.  y leaves through an LDS tile.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* __restrict__ hin, uint16_t* __restrict__ y, int T, int H, int G, int Q, int nc,
    int npairs) {
  constexpr int QSM = 64;               // sub-chunk length (Q >= 64); Q = 32 runs one of 32
  constexpr int KCP = N < 32 ? 32 : N;  // K of G^T padded to whole 32-wide MFMA steps (zeros)
  constexpr int BP = KCP + 8;           // pitch of bt / hT rows (bf16)
  constexpr int XPn = P + 16;           // pitch of the x tiles
  constexpr int YP = P + 8;             // pitch of the y tile
  constexpr int NKS = KCP / 32;
  constexpr int NPT = P / 16;
  constexpr int KT = N / 16;            // n tiles of the state
  constexpr int KTW = (KT + 3) / 4;     // n tiles per wave in the state update
  constexpr float kMaxHalfSpread = 60.0f;

  __shared__ __attribute__((aligned(16))) uint16_t bt[QSM * BP];
  __shared__ __attribute__((aligned(16))) uint16_t xl[QSM * XPn];  // raw x
  __shared__ __attribute__((aligned(16))) uint16_t xh[QSM * XPn];  // x * xsc
  __shared__ __attribute__((aligned(16))) uint16_t hT[P * BP];
  __shared__ __attribute__((aligned(16))) uint16_t yt[QSM * YP];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs_hi[256];
  __shared__ __attribute__((aligned(16))) float cs_lo[256];
  __shared__ __attribute__((aligned(16))) float csc[256];  // C row scale
  __shared__ __attribute__((aligned(16))) float xsc[256];  // x row scale
  __shared__ float kpre[4], kpost[4];                       // state factors per sub-chunk
  __shared__ int exact_flag;
  __shared__ double wsum[4], tot;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar
  const int QS = Q < QSM ? Q : QSM;
  const int nsub = Q / QS;
  const bool has_rows = 16 * wid < QS;  // waves without output rows (Q = 32) only help stage
  const float a_re = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const float Dh = D ? D[h] : 0.0f;
  if (tid == 0) exact_flag = 0;

  // ---- buffer descriptors of this chunk's slices (rows >= Lc read as zero) ----
  const size_t xy0 = (static_cast<size_t>(b) * T + t0) * H * P + static_cast<size_t>(h) * P;
  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2;
  const uint32_t xbytes = Lc > 0 ? static_cast<uint32_t>(Lc - 1) * xrow + P * 2 : 0;
  const buf_t xbuf = make_buf(x + xy0, xbytes);
  const buf_t ybuf = make_buf(y + xy0, xbytes);
  const size_t bc0 = (static_cast<size_t>(b) * T + t0) * G * N + static_cast<size_t>(g) * N;
  const uint32_t brow = static_cast<uint32_t>(G) * N * 2;
  const uint32_t bbytes = Lc > 0 ? static_cast<uint32_t>(Lc - 1) * brow + N * 2 : 0;
  const buf_t bbuf = make_buf(Bm + bc0, bbytes);
  const buf_t cbuf = make_buf(Cm + bc0, bbytes);
  const buf_t hbuf = make_buf(hin + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N),
                              P * N * 4);

  // ---- global loads first: dt, h_in, C rows and x/B of sub-chunk 0 ----
  const size_t dt_base = (static_cast<size_t>(b) * T + t0) * H + h;
  const float dt_raw = tid < Lc ? dt[dt_base + static_cast<size_t>(tid) * H] : 0.0f;

  // state tiles, transposed: lane holds column p = pt*16 + r16, rows n = nt*16 + 4q + j
  f32x4 hacc[KTW][NPT];
#pragma unroll
  for (int i = 0; i < KTW; ++i) {
    const int nt = wid + 4 * i;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      const uint4 v = buf_load16(hbuf, ((pt * 16 + r16) * N + nt * 16 + 4 * q) * 4);
      hacc[i][pt] = nt < KT ? __builtin_bit_cast(f32x4, v) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // C rows of this wave's output tile in sub-chunk j: lane (row r16, group q)
  // holds k = ks*32 + 8q .. +7
  auto load_c = [&](uint4 (&cr)[NKS], int j) {
    const uint32_t row = j * QS + 16 * wid + r16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int k0 = ks * 32 + 8 * q;
      const uint4 v = buf_load16(cbuf, row * brow + k0 * 2);
      cr[ks] = (has_rows && k0 < N) ? v : make_uint4(0, 0, 0, 0);
    }
  };
  uint4 creg[NKS], cnext[NKS];
  load_c(creg, 0);

  BufSlab<QSM, P / 8> xs;
  BufSlab<QSM, N / 8> bs;
  xs.load(xbuf, xrow, 0);
  bs.load(bbuf, brow, 0);

  // ---- prologue: step sizes, cumulative exponents, per-sub-chunk factors ----
  chunk_prologue<false>(dt_raw, Lc, a_re, 0.0f, bias, dt_min, dt_max, dl, cs_hi, cs_lo, nullptr,
                        nullptr, wsum, &tot, Q);
  // exponent of token t as a double (t = -1: 0)
  auto csd = [&](int t) -> double {
    return t < 0 ? 0.0 : static_cast<double>(cs_hi[t]) + static_cast<double>(cs_lo[t]);
  };
  if (tid < nsub) {
    const int j0 = tid * QS, m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    if (csd(j0 - 1) - csd(m) > kMaxHalfSpread || csd(m) - csd(j1) > kMaxHalfSpread)
      atomicOr(&exact_flag, 1);
  }
  __syncthreads();
  const bool exact = exact_flag != 0;  // uniform over the workgroup
  if (tid < Q) {
    const int j0 = tid & ~(QS - 1), m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    const double e = csd(tid);
    if (exact) {
      csc[tid] = __expf(static_cast<float>(e - csd(j0 - 1)));
      xsc[tid] = __expf(static_cast<float>(csd(j1) - e)) * dl[tid];
    } else {
      csc[tid] = __expf(static_cast<float>(e - csd(m)));
      xsc[tid] = __expf(static_cast<float>(csd(m) - e)) * dl[tid];
    }
    if (tid == j1) {
      const int j = tid / QS;
      if (exact) {
        kpre[j] = 1.0f;
        kpost[j] = __expf(static_cast<float>(csd(j1) - csd(j0 - 1)));
      } else {
        kpre[j] = __expf(static_cast<float>(csd(m) - (j0 > 0 ? csd(m - QS) : 0.0)));
        kpost[j] = 1.0f;
      }
    }
  }
  if constexpr (KCP > N) {
    // zero the K padding of bt and hT (stage stores never write it)
    for (int it = tid; it < QSM + P; it += kThreads) {
      uint16_t* row = it < QSM ? bt + it * BP : hT + (it - QSM) * BP;
      for (int k = N; k < KCP; ++k) row[k] = 0;
    }
  }
  __syncthreads();

  auto store_stage = [&](int j) {
#pragma unroll
    for (int i = 0; i < bs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (bs.ITEMS % kThreads == 0 || it < bs.ITEMS) {
        const int v = it % (N / 8), sl = it / (N / 8);
        *reinterpret_cast<uint4*>(bt + sl * BP + v * 8) = bs.v[i];
      }
    }
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (xs.ITEMS % kThreads == 0 || it < xs.ITEMS) {
        const int v = it % (P / 8), sl = it / (P / 8);
        const int s = j * QS + sl;
        const float w = (sl < QS && s < Q) ? xsc[s] : 0.0f;
        *reinterpret_cast<uint4*>(xl + sl * XPn + v * 8) = xs.v[i];
        *reinterpret_cast<uint4*>(xh + sl * XPn + v * 8) = scale_bf16x8(xs.v[i], w);
      }
    }
  };
  // scale the state by kpre[j] and write its bf16 copy hT[p][n]
  auto store_state = [&](int j) {
    const float k = kpre[j];
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
      const int nt = wid + 4 * i;
      if (nt >= KT) break;
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        hacc[i][pt] = hacc[i][pt] * k;
        *reinterpret_cast<uint2*>(hT + (pt * 16 + r16) * BP + nt * 16 + 4 * q) =
            make_uint2(pack_bf16x2(hacc[i][pt][0], hacc[i][pt][1]),
                       pack_bf16x2(hacc[i][pt][2], hacc[i][pt][3]));
      }
    }
  };
  store_stage(0);
  store_state(0);
  __syncthreads();

  for (int j = 0; j < nsub; ++j) {
    const int sj = j * QS;  // first token of the sub-chunk
    const bool more = j + 1 < nsub;
    if (more) {
      xs.load(xbuf, xrow, sj + QS);
      bs.load(bbuf, brow, sj + QS);
      load_c(cnext, j + 1);
    }

    // ---- outputs of rows sj + 16 wid .. +15 ----
    if (has_rows) {
      const int lrow = sj + 16 * wid + r16;  // this lane's output row (as G^T column)
      uint4 ct[NKS];                          // C~ rows
      {
        const float sc = csc[lrow];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) ct[ks] = scale_bf16x8(creg[ks], sc);
      }
      f32x4 yacc[NPT];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) yacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint4 hv = *reinterpret_cast<const uint4*>(hT + (pt * 16 + r16) * BP + ks * 32 + 8 * q);
          yacc[pt] = mfma_bf16(as_bf16x8(ct[ks]), as_bf16x8(hv), yacc[pt]);
        }
      }
      // intra-chunk: source blocks b0 = 2k2, b1 = 2k2+1 (16 tokens each)
      for (int k2 = 0; 2 * k2 <= wid; ++k2) {
        const int b0 = 2 * k2, b1 = 2 * k2 + 1;
        const bool live1 = b1 <= wid;
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 va = *reinterpret_cast<const uint4*>(bt + (b0 * 16 + r16) * BP + ks * 32 + 8 * q);
          ga = mfma_bf16(as_bf16x8(va), as_bf16x8(exact ? creg[ks] : ct[ks]), ga);
        }
        if (live1) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 vb = *reinterpret_cast<const uint4*>(bt + (b1 * 16 + r16) * BP + ks * 32 + 8 * q);
            gb = mfma_bf16(as_bf16x8(vb), as_bf16x8(exact ? creg[ks] : ct[ks]), gb);
          }
        }
        float m[8];
        if (!exact) {
          // causal mask only: the decay sits in C~ and x^
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            m[jj] = sj + b0 * 16 + 4 * q + jj <= lrow ? ga[jj] : 0.f;
            m[4 + jj] = sj + b1 * 16 + 4 * q + jj <= lrow ? gb[jj] : 0.f;
          }
        } else {
          const float lh = cs_hi[lrow], ll = cs_lo[lrow];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int s0 = sj + (b0 + half) * 16 + 4 * q;
            const f32x4 gv = half ? gb : ga;
            const float4 hs = *reinterpret_cast<const float4*>(cs_hi + s0);
            const float4 ls = *reinterpret_cast<const float4*>(cs_lo + s0);
            const float4 ds = *reinterpret_cast<const float4*>(dl + s0);
            const float hv[4] = {hs.x, hs.y, hs.z, hs.w}, lv[4] = {ls.x, ls.y, ls.z, ls.w};
            const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              m[4 * half + jj] =
                  s0 + jj <= lrow ? gv[jj] * decay_between(lh, ll, hv[jj], lv[jj]) * dv[jj] : 0.f;
          }
        }
        const uint4 mv = make_uint4(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]),
                                    pack_bf16x2(m[4], m[5]), pack_bf16x2(m[6], m[7]));
        const uint16_t* xs_tile = exact ? xl : xh;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = lds_tr4(xs_tile, XPn, b0 * 16 + 4 * q, pt * 16);
          const uint2 hi = lds_tr4(xs_tile, XPn, b1 * 16 + 4 * q, pt * 16);
          yacc[pt] = mfma_bf16(as_bf16x8(mv), as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)),
                               yacc[pt]);
        }
      }
      // + D x_l, then the rows into the LDS y tile (lane: column pt*16 + r16, rows 4q + jj)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const uint2 u = lds_tr4(xl, XPn, 16 * wid + 4 * q, pt * 16);
        const float xv[4] = {bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                             bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16)};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          yt[(16 * wid + 4 * q + jj) * YP + pt * 16 + r16] = f32_to_bf16_bits(yacc[pt][jj] + Dh * xv[jj]);
      }
    }

    // ---- state update to the start of the next sub-chunk ----
    if (more) {
      const float kp = kpost[j];
      if (exact) {
#pragma unroll
        for (int i = 0; i < KTW; ++i)
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) hacc[i][pt] = hacc[i][pt] * kp;
      }
      for (int k = 0; k < QS; k += 32) {
        uint4 bfr[KTW];
#pragma unroll
        for (int i = 0; i < KTW; ++i) {
          const int nt = wid + 4 * i;
          const uint2 lo = lds_tr4(bt, BP, k + 8 * q, (nt < KT ? nt : 0) * 16);
          const uint2 hi = lds_tr4(bt, BP, k + 8 * q + 4, (nt < KT ? nt : 0) * 16);
          bfr[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = lds_tr4(xh, XPn, k + 8 * q, pt * 16);
          const uint2 hi = lds_tr4(xh, XPn, k + 8 * q + 4, pt * 16);
          const uint4 afr = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int i = 0; i < KTW; ++i)
            if (wid + 4 * i < KT)
              hacc[i][pt] = mfma_bf16(as_bf16x8(bfr[i]), as_bf16x8(afr), hacc[i][pt]);
        }
      }
    }
    __syncthreads();
    // y rows of this sub-chunk out with 16-byte stores (rows past Lc are dropped)
    for (int it = tid; it < QS * (P / 8); it += kThreads) {
      const int l = it / (P / 8), v = it % (P / 8);
      buf_store16(ybuf, static_cast<uint32_t>(sj + l) * xrow + v * 16,
                  *reinterpret_cast<const uint4*>(yt + l * YP + v * 8));
    }
    if (more) {
      store_stage(j + 1);
      store_state(j + 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) creg[ks] = cnext[ks];
    }
    __syncthreads();
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
