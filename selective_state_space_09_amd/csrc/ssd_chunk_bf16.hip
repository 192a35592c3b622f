// Chunked SSD forward on gfx950 for bfloat16 x, B, C (real Mamba-2 form; fp32
// state and accumulation), in two kernels:
//   ssd_walk_bf16_kernel  chunk-boundary states h_in(c) and the final state:
//                         each workgroup walks the chunks of one (batch, head,
//                         state-column group) in order;
//   ssd_scan_bf16_kernel  chunk outputs from h_in(c), per (batch, chunk, head).
// (Numerical Stability in Mamba-3-Lite, section 4: the chunkwise form with
// L[l,s] = exp(cs_l - cs_s) 1[l >= s] inside a chunk and the chunk's total
// log-decay carrying the state from one chunk to the next.)
//
// Both kernels stage token rows into LDS in their natural row-major layout
// (16-byte stores) and read MFMA operands whose contraction runs over tokens
// with the gfx950 LDS transpose read ds_read_b64_tr_b16.

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
// Chunk-boundary states, walked.  One workgroup per (batch, head, group of NG
// state columns) runs through the chunks in order with the running state in
// MFMA accumulators; for chunk c it writes h_in(c) and then advances
//   h <- e^{A u_c} h + sum_s x_s (e^{A (u_c - u_s)} delta_s B_s)^T,
// u_s = delta_1 + .. + delta_s, u_c the chunk total (the chunk's state from a
// zero start on MFMA, contraction over the chunk's tokens, plus the decayed
// carry: the chunkwise recurrence of the state-passing step).  After the
// last chunk it writes the final state (fp32).  Chunk c+1's x, B and dt are
// in flight while chunk c computes.  The column groups of one (batch, head)
// are dispatched to one XCD, so x comes from HBM once and from that XCD's L2
// for the other groups; the decay weights go onto this group's B columns,
// so no group rescales the shared x.
//
// The exponent sums here are fp32 (a wave DPP scan): a sum of at most 256
// positive steps carries a relative error of ~1e-6, far below the bf16
// rounding of the weighted B.  The boundary states are stored as bf16: the
// output kernel rounds the carried state to bf16 for its MFMA in any case.
//
// Tiles are transposed (D[n][p] = sum_s B~_s[n] x_s[p]): an accumulator lane
// holds column p and four consecutive n, which is one 8-byte store of the
// [p][n] state layout.
// ---------------------------------------------------------------------------
template <int P, int N, int NG>
__global__ __launch_bounds__(kThreads) void ssd_walk_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, const float* __restrict__ h0, uint16_t* __restrict__ hin,
    float* __restrict__ h_final, int Bsz, int T, int H, int G, int Q, int nc) {
  constexpr int NGRP = N / NG;
  constexpr int QM = 256;               // largest chunk
  constexpr int XPn = P + 16, BPn = NG + 16;
  constexpr int PT = P / 16, NT = NG / 16;
  constexpr int TILES = PT * NT;
  constexpr int TPW = (TILES + 3) / 4;  // tiles per wave: tile = wave + 4 i

  __shared__ __attribute__((aligned(16))) uint16_t xt[QM * XPn];  // x_s
  __shared__ __attribute__((aligned(16))) uint16_t bq[QM * BPn];  // w_s B_s, this column group
  __shared__ __attribute__((aligned(16))) float wsc[QM];
  __shared__ float wpart[4];

  // workgroup -> (b, h, column group): groups of one (b, h) on one XCD
  const int id = blockIdx.x;
  const int k = id / kXCD;
  const int unit = (id % kXCD) + kXCD * (k / NGRP);
  const int gn = k % NGRP;
  if (unit >= Bsz * H) return;
  const int b = unit / H, h = unit % H;
  const int g = h / (H / G);
  const int n0 = gn * NG;
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const float a_re = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;

  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2;
  const uint32_t brow = static_cast<uint32_t>(G) * N * 2;
  BufSlab<QM, P / 8> xs;
  BufSlab<QM, NG / 8> bs;
  float dtv = 0.0f;
  // chunk c's rows into registers (rows at or past the chunk's end read 0)
  // (dt first: the next chunk's scan waits for it alone, the in-order load
  // counter then leaves x and B in flight)
  auto prefetch = [&](int c) {
    const int t0 = c * Q, Lc = min(Q, T - t0);
    const size_t r0 = static_cast<size_t>(b) * T + t0;
    dtv = tid < Lc ? dt[(r0 + tid) * H + h] : 0.0f;
    xs.load(make_buf(x + r0 * H * P + static_cast<size_t>(h) * P,
                     static_cast<uint32_t>(Lc - 1) * xrow + P * 2), xrow, 0);
    bs.load(make_buf(Bm + r0 * G * N + static_cast<size_t>(g) * N + n0,
                     static_cast<uint32_t>(Lc - 1) * brow + NG * 2), brow, 0);
  };

  // running state: lane holds column p = pt*16 + r16, rows n = n0 + nt*16 + 4q + j
  const size_t pub = (static_cast<size_t>(b) * H + h) * P * N;  // h0 / h_final slice
  f32x4 hacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wid + 4 * i;
    const int nt = tile % NT, pt = tile / NT;
    hacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (h0 && tile < TILES)
      hacc[i] = *reinterpret_cast<const f32x4*>(h0 + pub + (pt * 16 + r16) * N + n0 + nt * 16 + 4 * q);
  }

  // rows Q..127 of the tiles stay zero (the MFMA groups run over 128 rows)
  for (int it = tid; it < (128 - min(Q, 128)) * (XPn + BPn) / 8; it += kThreads) {
    const int r = it / ((XPn + BPn) / 8), v = it % ((XPn + BPn) / 8);
    uint16_t* row = v < XPn / 8 ? xt + (Q + r) * XPn + v * 8 : bq + (Q + r) * BPn + (v - XPn / 8) * 8;
    *reinterpret_cast<uint4*>(row) = make_uint4(0, 0, 0, 0);
  }

  if (nc > 0) prefetch(0);
  for (int c = 0; c < nc; ++c) {
    const int Lc = min(Q, T - c * Q);
    // step sizes and their running sums u_s over the chunk (thread s = token s)
    const float d = tid < Lc ? step_size(dtv, bias, dt_min, dt_max) : 0.0f;
    float u = wave_inclusive_sum(d);
    if (lane == kWave - 1) wpart[wid] = u;
    __syncthreads();  // (also: every wave is done with the previous chunk's tiles)
    float before = 0.0f, total = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float pw = wpart[w];
      before += w < wid ? pw : 0.0f;
      total += pw;
    }
    u += before;
    wsc[tid] = __expf(a_re * (total - u)) * d;
    const float lam = __expf(a_re * total);
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * kThreads;
      const int v = it % (P / 8), s = it / (P / 8);
      if ((xs.ITEMS % kThreads == 0 || it < xs.ITEMS) && s < Q)
        *reinterpret_cast<uint4*>(xt + s * XPn + v * 8) = xs.v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < bs.PER; ++i) {
      const int it = tid + i * kThreads;
      const int v = it % (NG / 8), s = it / (NG / 8);
      if ((bs.ITEMS % kThreads == 0 || it < bs.ITEMS) && s < Q)
        *reinterpret_cast<uint4*>(bq + s * BPn + v * 8) = scale_bf16x8(bs.v[i], wsc[s]);
    }
    // h_in(c), bf16 -- issued after this chunk's loads are consumed and before
    // the next chunk's are issued: the in-order load/store counter then never
    // holds a prefetch behind a wait on these stores
    uint16_t* dst = hin + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wid + 4 * i;
      if (tile >= TILES) break;
      const int nt = tile % NT, pt = tile / NT;
      *reinterpret_cast<uint2*>(dst + (pt * 16 + r16) * N + n0 + nt * 16 + 4 * q) =
          make_uint2(pack_bf16x2(hacc[i][0], hacc[i][1]), pack_bf16x2(hacc[i][2], hacc[i][3]));
    }
    if (c + 1 < nc) prefetch(c + 1);
    __syncthreads();

    // chunk state on MFMA, 128 tokens (4 k-steps) per group: every operand
    // read of a group is issued before its MFMAs (rows Q..127 are zero)
    f32x4 sacc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) sacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < Q; kb += 128) {
      uint4 af[4][TPW], bf[4][TPW];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ks = kb + 32 * kk;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
          const int tile = wid + 4 * i;
          const int nt = (tile < TILES ? tile : 0) % NT, pt = (tile < TILES ? tile : 0) / NT;
          const uint2 alo = lds_tr4(bq, BPn, ks + 8 * q, nt * 16);
          const uint2 ahi = lds_tr4(bq, BPn, ks + 8 * q + 4, nt * 16);
          const uint2 blo = lds_tr4(xt, XPn, ks + 8 * q, pt * 16);
          const uint2 bhi = lds_tr4(xt, XPn, ks + 8 * q + 4, pt * 16);
          af[kk][i] = make_uint4(alo.x, alo.y, ahi.x, ahi.y);
          bf[kk][i] = make_uint4(blo.x, blo.y, bhi.x, bhi.y);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < TPW; ++i)
          if (wid + 4 * i < TILES)
            sacc[i] = mfma_bf16(as_bf16x8(af[kk][i]), as_bf16x8(bf[kk][i]), sacc[i]);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) hacc[i] = hacc[i] * lam + sacc[i];
  }
  if (h_final) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wid + 4 * i;
      if (tile >= TILES) break;
      const int nt = tile % NT, pt = tile / NT;
      *reinterpret_cast<f32x4*>(h_final + pub + (pt * 16 + r16) * N + n0 + nt * 16 + 4 * q) = hacc[i];
    }
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
// e^{cs_l - cs_s} = e^{cs_l - cs_m} e^{cs_m - cs_s}.  The second factor scales
// x_s once when the sub-chunk is staged (x^ = x e^{cs_m - cs_s} delta); the
// first is common to every term of output row l, carried one included when
// the state is kept as H = e^{cs_m - cs_{j0-1}} h_j (one factor per
// sub-chunk), so
//   y_l = e^{cs_l - cs_m} (C_l . H + sum_{s <= l} (C_l . B_s) x^_s) + D x_l
// -- raw C everywhere, the causal mask only on diagonal blocks, one scale per
// output row at the end.  The state update accumulates x^ B^T into H.  The
// factors stay below e^60 when every half sub-chunk decays by at most e^60;
// when a chunk breaks that bound the workgroup switches to exact mode
// (per-element exponentials against raw x, the carried term scaled by
// e^{cs_l - cs_{j0-1}}, the state kept unscaled).
//
// The output tile is computed transposed, Y^T[p][l]: wave w owns output rows
// l = 16w .. 16w+15 of each sub-chunk as accumulator columns, so a lane holds
// one row l (one scale factor) and four consecutive p (one 8-byte store of y).
// Per 32 source tokens, G^T = B_s . C_l^T on MFMA (C rows in registers,
// prefetched a sub-chunk ahead) leaves column l in the lane, which after the
// mask is the B operand of Y^T += X^T M^T.  For the state update wave w owns
// n tiles w, w+4, ..: H^T[n][p] += sum_s B_s[n] x^_s[p] (operands from LDS by
// the transpose read); a lane holds 4 consecutive n of one p and writes the
// bf16 state tile with 8-byte stores.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const uint16_t* __restrict__ hin, uint16_t* __restrict__ y, int T, int H, int G, int Q, int nc,
    int npairs) {
  constexpr int QSM = 64;               // sub-chunk length (Q >= 64); Q = 32 runs one of 32
  constexpr int KCP = N < 32 ? 32 : N;  // K of G^T padded to whole 32-wide MFMA steps (zeros)
  constexpr int BP = KCP + 8;           // pitch of bt / hT rows (bf16)
  constexpr int XPn = P + 16;           // pitch of the x tiles
  constexpr int NKS = KCP / 32;
  constexpr int NPT = P / 16;
  constexpr int KT = N / 16;            // n tiles of the state
  constexpr int KTW = (KT + 3) / 4;     // n tiles per wave in the state update
  constexpr float kMaxHalfSpread = 60.0f;

  __shared__ __attribute__((aligned(16))) uint16_t bt[QSM * BP];
  __shared__ __attribute__((aligned(16))) uint16_t xl[QSM * XPn];  // raw x
  __shared__ __attribute__((aligned(16))) uint16_t xh[QSM * XPn];  // x * xsc
  __shared__ __attribute__((aligned(16))) uint16_t hT[P * BP];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs_hi[256];
  __shared__ __attribute__((aligned(16))) float cs_lo[256];
  __shared__ __attribute__((aligned(16))) float csc[256];  // output row scale
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
                              P * N * 2);

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
      const uint2 v = buf_load8(hbuf, ((pt * 16 + r16) * N + nt * 16 + 4 * q) * 2);
      hacc[i][pt] = nt < KT ? f32x4{bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16),
                                    bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16)}
                            : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // C rows of this wave's output tile in sub-chunk j: lane (row r16, group q)
  // holds k = ks*32 + 8q .. +7.  Rows past the chunk (and every row of the
  // waves without output rows, Q = 32) read as zero through the descriptor;
  // the K padding (N = 16) is zeroed by an out-of-range offset, not by a
  // select on the loaded value, so the prefetch is not waited for here.
  auto load_c = [&](uint4 (&cr)[NKS], int j) {
    const uint32_t row = j * QS + 16 * wid + r16;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int k0 = ks * 32 + 8 * q;
      const uint32_t off = (KCP == N || k0 < N) ? row * brow + k0 * 2 : 0xFFFFFFF0u;
      cr[ks] = buf_load16(cbuf, off);
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
  // uniform over the workgroup; scalar so that its branches keep EXEC whole
  const bool exact = __builtin_amdgcn_readfirstlane(exact_flag) != 0;
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

    // ---- outputs of rows sj + 16 wid .. +15 (accumulator columns) ----
    if (has_rows) {
      const int lrow = sj + 16 * wid + r16;  // this lane's output row
      f32x4 yacc[NPT];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) yacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // carried: Y^T[p][l] += sum_n H[p][n] C_l[n]
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint4 hv = *reinterpret_cast<const uint4*>(hT + (pt * 16 + r16) * BP + ks * 32 + 8 * q);
          yacc[pt] = mfma_bf16(as_bf16x8(hv), as_bf16x8(creg[ks]), yacc[pt]);
        }
      }
      if (exact) {
        const float s1 = csc[lrow];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) yacc[pt] = yacc[pt] * s1;
      }
      // intra-chunk: source blocks b0 = 2k2, b1 = 2k2+1 (16 tokens each);
      // block wid is the diagonal one
      for (int k2 = 0; 2 * k2 <= wid; ++k2) {
        const int b0 = 2 * k2, b1 = 2 * k2 + 1;
        const bool live1 = b1 <= wid;
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 va = *reinterpret_cast<const uint4*>(bt + (b0 * 16 + r16) * BP + ks * 32 + 8 * q);
          ga = mfma_bf16(as_bf16x8(va), as_bf16x8(creg[ks]), ga);
        }
        if (live1) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 vb = *reinterpret_cast<const uint4*>(bt + (b1 * 16 + r16) * BP + ks * 32 + 8 * q);
            gb = mfma_bf16(as_bf16x8(vb), as_bf16x8(creg[ks]), gb);
          }
        }
        // lane: column l = r16 (+16 wid), rows s = 4q + jj of blocks b0, b1
        if (!exact) {
          if (b0 == wid) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ga[jj] = 4 * q + jj <= r16 ? ga[jj] : 0.f;
          }
          if (b1 == wid) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) gb[jj] = 4 * q + jj <= r16 ? gb[jj] : 0.f;
          }
        } else {
          const float lh = cs_hi[lrow], ll = cs_lo[lrow];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int s0 = sj + (b0 + half) * 16 + 4 * q;
            f32x4& gv = half ? gb : ga;
            const float4 hs = *reinterpret_cast<const float4*>(cs_hi + s0);
            const float4 ls = *reinterpret_cast<const float4*>(cs_lo + s0);
            const float4 ds = *reinterpret_cast<const float4*>(dl + s0);
            const float hv[4] = {hs.x, hs.y, hs.z, hs.w}, lv[4] = {ls.x, ls.y, ls.z, ls.w};
            const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              gv[jj] = s0 + jj <= lrow ? gv[jj] * decay_between(lh, ll, hv[jj], lv[jj]) * dv[jj] : 0.f;
          }
        }
        const uint4 mv = make_uint4(pack_bf16x2(ga[0], ga[1]), pack_bf16x2(ga[2], ga[3]),
                                    pack_bf16x2(gb[0], gb[1]), pack_bf16x2(gb[2], gb[3]));
        const uint16_t* xs_tile = exact ? xl : xh;
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = lds_tr4(xs_tile, XPn, b0 * 16 + 4 * q, pt * 16);
          const uint2 hi = lds_tr4(xs_tile, XPn, b1 * 16 + 4 * q, pt * 16);
          yacc[pt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(mv),
                               yacc[pt]);
        }
      }
      // row scale, + D x_l, y rows out (lane: row lrow, columns pt*16 + 4q .. +3;
      // rows past Lc are dropped by the descriptor)
      const float s2 = exact ? 1.0f : csc[lrow];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const uint2 u = *reinterpret_cast<const uint2*>(xl + (16 * wid + r16) * XPn + pt * 16 + 4 * q);
        const float o0 = yacc[pt][0] * s2 + Dh * bf16_bits_to_f32(u.x & 0xFFFFu);
        const float o1 = yacc[pt][1] * s2 + Dh * bf16_bits_to_f32(u.x >> 16);
        const float o2 = yacc[pt][2] * s2 + Dh * bf16_bits_to_f32(u.y & 0xFFFFu);
        const float o3 = yacc[pt][3] * s2 + Dh * bf16_bits_to_f32(u.y >> 16);
        buf_store8(ybuf, static_cast<uint32_t>(lrow) * xrow + (pt * 16 + 4 * q) * 2,
                   make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)));
      }
    }

    // ---- state update to the start of the next sub-chunk ----
    if (more) {
      if (exact) {
        const float kp = kpost[j];
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
      __syncthreads();  // every wave is done with this sub-chunk's tiles
      store_stage(j + 1);
      store_state(j + 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) creg[ks] = cnext[ks];
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
template <int P, int N>
static hipError_t launch_bf16(const ChunkArgs& a, hipStream_t st) {
  constexpr int NG = N < 32 ? N : 32;  // state columns per walking workgroup
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  const int npairs = a.Bsz * nc;
  uint16_t* hin = static_cast<uint16_t*>(a.workspace);  // (Bsz, nc, H, P, N) bf16
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const uint16_t* C = static_cast<const uint16_t*>(a.C);
  const unsigned walkers = static_cast<unsigned>((a.Bsz * a.H + kXCD - 1) / kXCD) * kXCD * (N / NG);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  if (a.events) (void)hipEventRecord(a.events[0], st);
  // the walk also runs for T = 0: it writes h_final = h0 (or zeros)
  if (nc > 0 || a.h_final)
    ssd_walk_bf16_kernel<P, N, NG><<<walkers, kThreads, 0, st>>>(
        x, a.dt, a.A, B, a.dt_bias, a.dt_min, a.dt_max, a.h0, hin, a.h_final, a.Bsz, a.T, a.H,
        a.G, a.chunk, nc);
  if (a.events) {
    (void)hipEventRecord(a.events[1], st);
    (void)hipEventRecord(a.events[2], st);
  }
  if (nc > 0)
    ssd_scan_bf16_kernel<P, N><<<blocks, kThreads, 0, st>>>(
        x, a.dt, a.A, B, C, a.D, a.dt_bias, a.dt_min, a.dt_max, hin,
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
