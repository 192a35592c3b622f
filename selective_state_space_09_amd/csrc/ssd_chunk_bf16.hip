// Chunked SSD forward on gfx950 for bfloat16 x, B, C (real Mamba-2 form; fp32
// state and accumulation), in three kernels:
//   ssd_state_bf16_kernel  each chunk's own state S_c and decay, per (batch,
//                          chunk, head);
//   ssd_pass_bf16_kernel   the boundary states h_in(c) and the final state;
//   ssd_scan_bf16_kernel   chunk outputs from h_in(c), per (batch, chunk, head).
// (Numerical Stability in Mamba-3-Lite, section 4: the chunkwise form with
// L[l,s] = exp(cs_l - cs_s) 1[l >= s] inside a chunk and the chunk's total
// log-decay carrying the state from one chunk to the next.)
//
// Both kernels stage token rows into LDS in their natural row-major layout
// (16-byte stores) and read MFMA operands whose contraction runs over tokens
// with the gfx950 LDS transpose read ds_read_b64_tr_b16.

#include "ssd_chunk_common.h"

namespace ssd {

// eight bf16 scaled by eight factors (element i by w[i]), rounded back to bf16
__device__ __forceinline__ uint4 scale_bf16x8_each(uint4 v, float4 w0, float4 w1) {
  return make_uint4(pack_bf16x2(bf16_bits_to_f32(v.x & 0xFFFFu) * w0.x, bf16_bits_to_f32(v.x >> 16) * w0.y),
                    pack_bf16x2(bf16_bits_to_f32(v.y & 0xFFFFu) * w0.z, bf16_bits_to_f32(v.y >> 16) * w0.w),
                    pack_bf16x2(bf16_bits_to_f32(v.z & 0xFFFFu) * w1.x, bf16_bits_to_f32(v.z >> 16) * w1.y),
                    pack_bf16x2(bf16_bits_to_f32(v.w & 0xFFFFu) * w1.z, bf16_bits_to_f32(v.w >> 16) * w1.w));
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
// Chunk states from a zero start, one workgroup per (batch, chunk, HPW heads
// of one group):
//   S_c[p][n] = sum_s x_s[p] e^{A (u_c - u_s)} delta_s B_s[n],
//   lambda_c  = e^{A u_c},
// u_s = delta_1 + .. + delta_s over the chunk and u_c its total (the chunk's
// own contribution to the state at its end, and its decay; the state-passing
// kernel chains them).  The heads of a workgroup share their B rows: B is
// staged once and its MFMA operands are read once for all of them (HPW = 2
// when the heads of a group pair up, which also halves the grid so that one
// round of workgroups covers it at the BitMamba shape).  The chunk is staged
// through LDS in quarters of up to 64 tokens, loaded into registers two
// quarters ahead.  The decay weight goes onto x (P columns) as it is staged.
// Eight waves; wave w owns n tiles 2(w%4), 2(w%4)+1 and p tiles 2(w/4),
// 2(w/4)+1 of the transposed product D[n][p] = sum_s B_s[n] (w_s x_s[p]) of
// every head, so an accumulator lane holds one p and four consecutive n: one
// 8-byte store of S_c (bf16; the output kernel rounds the carried state to
// bf16 for its MFMA in any case).  The exponent sums are fp32 (a wave DPP
// scan): a sum of at most 256 positive steps carries a relative error of ~1e-6.
// ---------------------------------------------------------------------------
template <int P, int N, int HPW>
__global__ __launch_bounds__(512) void ssd_state_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, uint16_t* __restrict__ states, float* __restrict__ decay,
    float2* __restrict__ tok, int T, int H, int G, int Q, int nc, int npairs) {
  constexpr int NTHR = 512, WW = 8;
  constexpr int HS = 64;                    // tokens per staged quarter
  constexpr int XPn = P + 16, BPn = N + 16;  // pitches (bf16 elements)
  constexpr int PT = P / 16, NT = N / 16;
  // wave tile block: NTW n tiles x PTW p tiles
  constexpr int NTW = NT >= 8 ? NT / 4 : (NT >= 2 ? 2 : 1);
  constexpr int NGW = NT / NTW;             // wave groups along n
  constexpr int PGW = WW / NGW;             // wave groups along p
  constexpr int PTW = (PT + PGW - 1) / PGW;
  // a wave's n tiles in pairs (NTW even): tile (pair m, half) covers n = 32 m +
  // 4 half + 8 (r / 4) + r % 4 for its MFMA row r, so a lane's rows of the pair
  // are 8 consecutive n (one 16-byte store of S_c)
  constexpr bool kPairN = NTW % 2 == 0;

  __shared__ __attribute__((aligned(16))) uint16_t xl[HPW][HS * XPn];  // w_s x_s per head
  __shared__ __attribute__((aligned(16))) uint16_t bl[HS * BPn];       // B_s
  __shared__ __attribute__((aligned(16))) float wsc[HPW][256];
  __shared__ float wpart[HPW][WW];

  int b, c, hp;
  if (!unit_of_block(H / HPW, nc, npairs, b, c, hp)) return;
  const int h0 = hp * HPW;  // first head of the workgroup
  const int g = h0 / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const int ng = wid % NGW, pg = wid / NGW;

  // ---- loads: dt first, then the first two quarters of x and B ----
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  float dtv[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) dtv[e] = tid < Lc ? dt[(r0 + tid) * H + h0 + e] : 0.0f;
  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2;
  const uint32_t brow = static_cast<uint32_t>(G) * N * 2;
  buf_t xbuf[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e)
    xbuf[e] = make_buf(x + r0 * H * P + static_cast<size_t>(h0 + e) * P,
                       static_cast<uint32_t>(Lc - 1) * xrow + P * 2);
  const buf_t bbuf = make_buf(Bm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Lc - 1) * brow + N * 2);
  BufSlab<HS, P / 8, NTHR> xs[2][HPW];
  BufSlab<HS, N / 8, NTHR> bs[2];
  const int nq = (Q + HS - 1) / HS;  // quarters of the chunk
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (i < nq) {
#pragma unroll
      for (int e = 0; e < HPW; ++e) xs[i][e].load(xbuf[e], xrow, i * HS);
      bs[i].load(bbuf, brow, i * HS);
    }

  // ---- step sizes and running sums (thread s = token s), per head ----
  float dd[HPW], uu[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    const float bias = dt_bias ? dt_bias[h0 + e] : 0.0f;
    dd[e] = tid < Lc ? step_size(dtv[e], bias, dt_min, dt_max) : 0.0f;
    uu[e] = wave_inclusive_sum(dd[e]);
    if (lane == kWave - 1) wpart[e][wid] = uu[e];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    const int h = h0 + e;
    const float a_re = A[h];
    float before = 0.0f, total = 0.0f;
#pragma unroll
    for (int w = 0; w < WW; ++w) {
      const float pw = wpart[e][w];
      before += w < wid ? pw : 0.0f;
      total += pw;
    }
    const float u = uu[e] + before;
    if (tid < 256) wsc[e][tid] = __expf(a_re * (total - u)) * dd[e];
    if (tid == 0) decay[(static_cast<size_t>(b) * H + h) * nc + c] = __expf(a_re * total);
    // (A u_l, delta_l) of every token for the output kernel (padding: delta 0)
    if (tid < Q) tok[((static_cast<size_t>(b) * nc + c) * H + h) * Q + tid] = make_float2(a_re * u, dd[e]);
  }
  __syncthreads();

  // quarter -> LDS (x scaled by w_s; rows past the chunk are zero)
  auto stage = [&](const BufSlab<HS, P / 8, NTHR> (&xsq)[HPW], const BufSlab<HS, N / 8, NTHR>& bsq,
                   int s0) {
#pragma unroll
    for (int e = 0; e < HPW; ++e)
#pragma unroll
      for (int i = 0; i < xsq[e].PER; ++i) {
        const int it = tid + i * NTHR;
        const int v = it % (P / 8), sl = it / (P / 8);
        if (xsq[e].ITEMS % NTHR == 0 || it < xsq[e].ITEMS)
          *reinterpret_cast<uint4*>(xl[e] + sl * XPn + v * 8) =
              scale_bf16x8(xsq[e].v[i], s0 + sl < Q ? wsc[e][s0 + sl] : 0.0f);
      }
#pragma unroll
    for (int i = 0; i < bsq.PER; ++i) {
      const int it = tid + i * NTHR;
      const int v = it % (N / 8), sl = it / (N / 8);
      if (bsq.ITEMS % NTHR == 0 || it < bsq.ITEMS)
        *reinterpret_cast<uint4*>(bl + sl * BPn + v * 8) = bsq.v[i];
    }
  };

  f32x4 acc[HPW][NTW][PTW];
#pragma unroll
  for (int e = 0; e < HPW; ++e)
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int j = 0; j < PTW; ++j) acc[e][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one quarter on MFMA: contraction over its tokens, all operand reads of a
  // 32-token step issued before the step's MFMAs; the B operands serve every head
  auto mma = [&](int rows) {
    for (int ks = 0; ks < rows; ks += 32) {
      uint4 af[NTW], bf[HPW][PTW];
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int nt = ng * NTW + i;
        const int c0 = kPairN ? 32 * (nt >> 1) + 4 * (nt & 1) : nt * 16;
        const uint2 lo = kPairN ? lds_tr4s<8>(bl, BPn, ks + 8 * q, c0) : lds_tr4(bl, BPn, ks + 8 * q, c0);
        const uint2 hi = kPairN ? lds_tr4s<8>(bl, BPn, ks + 8 * q + 4, c0) : lds_tr4(bl, BPn, ks + 8 * q + 4, c0);
        af[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
#pragma unroll
      for (int e = 0; e < HPW; ++e)
#pragma unroll
        for (int j = 0; j < PTW; ++j) {
          const int pt = pg * PTW + j < PT ? pg * PTW + j : 0;
          const uint2 lo = lds_tr4(xl[e], XPn, ks + 8 * q, pt * 16);
          const uint2 hi = lds_tr4(xl[e], XPn, ks + 8 * q + 4, pt * 16);
          bf[e][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
      for (int e = 0; e < HPW; ++e)
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
          for (int j = 0; j < PTW; ++j)
            if (pg * PTW + j < PT)
              acc[e][i][j] = mfma_bf16(as_bf16x8(af[i]), as_bf16x8(bf[e][j]), acc[e][i][j]);
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nq) {
      if (i > 0) __syncthreads();
      stage(xs[i & 1], bs[i & 1], i * HS);
      if (i + 2 < nq) {
#pragma unroll
        for (int e = 0; e < HPW; ++e) xs[i & 1][e].load(xbuf[e], xrow, (i + 2) * HS);
        bs[i & 1].load(bbuf, brow, (i + 2) * HS);
      }
      __syncthreads();
      mma(Q - i * HS < HS ? Q - i * HS : HS);
    }

  // S_c: lane holds p = pt*16 + r16 and, per pair of n tiles, n = 32 m + 8q .. +7
  // (else per tile n = nt*16 + 4q .. +3)
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    uint16_t* dst = states + ((static_cast<size_t>(b) * nc + c) * H + h0 + e) * (static_cast<size_t>(P) * N);
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int pt = pg * PTW + j;
      if (pt >= PT) continue;
      if constexpr (kPairN) {
#pragma unroll
        for (int i = 0; i < NTW; i += 2) {
          const int m = (ng * NTW + i) >> 1;
          *reinterpret_cast<uint4*>(dst + (pt * 16 + r16) * N + 32 * m + 8 * q) =
              make_uint4(pack_bf16x2(acc[e][i][j][0], acc[e][i][j][1]),
                         pack_bf16x2(acc[e][i][j][2], acc[e][i][j][3]),
                         pack_bf16x2(acc[e][i + 1][j][0], acc[e][i + 1][j][1]),
                         pack_bf16x2(acc[e][i + 1][j][2], acc[e][i + 1][j][3]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const int nt = ng * NTW + i;
          *reinterpret_cast<uint2*>(dst + (pt * 16 + r16) * N + nt * 16 + 4 * q) =
              make_uint2(pack_bf16x2(acc[e][i][j][0], acc[e][i][j][1]),
                         pack_bf16x2(acc[e][i][j][2], acc[e][i][j][3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk state passing (bf16 chunk states in, bf16 boundary states out):
//   h_in(0) = h0,  h_in(c+1) = lambda_c h_in(c) + S_c,  h_final = h_in(nc)
// (the chunkwise recurrence of the state across chunks), fp32 running state.
// One thread per 8 consecutive n of one p of one (batch, head) (16-byte
// accesses); PF chunks in flight.  h_in(c) overwrites S_c in place (S_c is
// read before it).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ssd_pass_bf16_kernel(
    uint16_t* __restrict__ states, const float* __restrict__ decay, const float* __restrict__ h0,
    float* __restrict__ h_final, int H, int PN, int nc) {
  constexpr int PF = 8;
  const int h = blockIdx.y, b = blockIdx.z;
  const int e8 = blockIdx.x * kThreads + threadIdx.x;  // group of 8 elements
  if (e8 * 8 >= PN) return;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t cstride = static_cast<size_t>(H) * PN;  // between chunks of one (b, h)
  uint16_t* base = states + static_cast<size_t>(b) * nc * cstride + h * static_cast<size_t>(PN) + e8 * 8;
  const float* dc = decay + bh * nc;
  float hv[8];
  if (h0) {
    const float4 a = *reinterpret_cast<const float4*>(h0 + bh * PN + e8 * 8);
    const float4 c4 = *reinterpret_cast<const float4*>(h0 + bh * PN + e8 * 8 + 4);
    hv[0] = a.x; hv[1] = a.y; hv[2] = a.z; hv[3] = a.w;
    hv[4] = c4.x; hv[5] = c4.y; hv[6] = c4.z; hv[7] = c4.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) hv[k] = 0.0f;
  }

  uint4 cur[PF];
  float cd[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (j < nc) {
      cur[j] = *reinterpret_cast<const uint4*>(base + j * cstride);
      cd[j] = dc[j];
    }
  for (int c0 = 0; c0 < nc; c0 += PF) {
    uint4 nxt[PF];
    float nd[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cn = c0 + PF + j;
      if (cn < nc) {
        nxt[j] = *reinterpret_cast<const uint4*>(base + cn * cstride);
        nd[j] = dc[cn];
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cc = c0 + j;
      if (cc < nc) {
        *reinterpret_cast<uint4*>(base + cc * cstride) =
            make_uint4(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                       pack_bf16x2(hv[6], hv[7]));
        const float l = cd[j];
        const uint32_t sw[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hv[2 * k] = l * hv[2 * k] + bf16_bits_to_f32(sw[k] & 0xFFFFu);
          hv[2 * k + 1] = l * hv[2 * k + 1] + bf16_bits_to_f32(sw[k] >> 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      cur[j] = nxt[j];
      cd[j] = nd[j];
    }
  }
  if (h_final) {
    *reinterpret_cast<float4*>(h_final + bh * PN + e8 * 8) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<float4*>(h_final + bh * PN + e8 * 8 + 4) = make_float4(hv[4], hv[5], hv[6], hv[7]);
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
// e^{cs_l - cs_s} = e^{cs_l - cs_m} e^{cs_m - cs_s}.  The second factor (times
// delta_s) is one weight w_s per source token; the first is common to every
// term of output row l, carried one included when the state is kept as
// H = e^{cs_m - cs_{j0-1}} h_j (one factor per sub-chunk), so
//   y_l = e^{cs_l - cs_m} (C_l . H + sum_{s <= l} (C_l . B_s) w_s x_s) + D x_l
// -- raw C and raw x everywhere, the causal mask only on diagonal blocks, w_s
// on the columns of the masked (C_l . B_s) block before it is rounded to bf16,
// one scale per output row at the end.  The state update accumulates
// (w_s B_s) x_s^T into H, w_s applied to the B operand in registers.  Only
// raw x is staged, one tile that also supplies D x_l.  The
// factors stay below e^60 when every half sub-chunk decays by at most e^60;
// when a chunk breaks that bound the workgroup switches to exact mode
// (per-element exponentials against raw x, the carried term scaled by
// e^{cs_l - cs_{j0-1}}, the state kept unscaled, w_s = e^{cs_j1 - cs_s} delta_s).
//
// The output tile is computed transposed, Y^T[p][l]: wave w owns output rows
// l = 16w .. 16w+15 of each sub-chunk as accumulator columns, so a lane holds
// one row l (one scale factor) and four consecutive p of each tile; the
// tiles go in pairs with permuted p (P >= 32), so a lane holds 8 consecutive p
// of a pair: one 16-byte store of y.
// Per 32 source tokens, G^T = B_s . C_l^T on MFMA (C rows in registers,
// prefetched a sub-chunk ahead) leaves column l in the lane, which after the
// mask and the weights is the B operand of Y^T += X^T M^T.  For the state
// update wave w owns n tiles 2w, 2w+1 with N = 128 (paired, permuted n), else
// w, w+4, ..: H^T[n][p] += sum_s (w_s B_s[n]) x_s[p]
// (operands from LDS by the transpose read); a lane holds 4 consecutive n of
// one p and writes the bf16 state tile with 8-byte stores.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_scan_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm, const float* __restrict__ D,
    const float2* __restrict__ tok, const uint16_t* __restrict__ hin, uint16_t* __restrict__ y,
    int T, int H, int G, int Q, int nc, int npairs) {
  constexpr int QSM = 64;               // sub-chunk length (Q >= 64); Q = 32 runs one of 32
  constexpr int KCP = N < 32 ? 32 : N;  // K of G^T padded to whole 32-wide MFMA steps (zeros)
  // row pitches (bf16): the B tile is read by rows (16 bytes a lane) and by the
  // transpose read (4 rows x 32 bytes a 16-lane group), so its rows start 8
  // banks apart; the state tile is read by rows only (4 banks apart suffice)
  constexpr int BTP = KCP + 16;
  constexpr int HTP = KCP + 8;
  constexpr int XPn = P + 16;           // pitch of the x tiles
  constexpr int NKS = KCP / 32;
  constexpr int NPT = P / 16;
  constexpr int KT = N / 16;            // n tiles of the state
  constexpr int KTW = (KT + 3) / 4;     // n tiles per wave in the state update
  constexpr float kMaxHalfSpread = 60.0f;
  // Output tiles in pairs (P >= 32): tile pt covers p = 32 (pt / 2) + 4 (pt % 2)
  // + 8 (r / 4) + r % 4 for its MFMA row r, so that a lane's accumulator rows of
  // the two tiles of a pair are 8 consecutive p (one 16-byte y store)
  constexpr bool kPairP = NPT % 2 == 0;
  auto prow = [](int pt, int r) {
    return kPairP ? 32 * (pt >> 1) + 4 * (pt & 1) + 8 * (r >> 2) + (r & 3) : pt * 16 + r;
  };
  // State tiles of a wave: n tiles 2w, 2w+1 paired with permuted n when there
  // are eight (N = 128; a lane's rows of the pair are the 8 consecutive
  // n = 32w + 8q .. +7: 16-byte loads of h_in and stores of its bf16 copy),
  // else n tiles w, w + 4, ..
  constexpr bool kPairS = KT == 8;

  __shared__ __attribute__((aligned(16))) uint16_t bt[QSM * BTP];
  __shared__ __attribute__((aligned(16))) uint16_t xl[QSM * XPn];  // raw x
  __shared__ __attribute__((aligned(16))) uint16_t hT[P * HTP];
  __shared__ __attribute__((aligned(16))) float dl[256];
  __shared__ __attribute__((aligned(16))) float cs[256];   // A u_l
  __shared__ __attribute__((aligned(16))) float csc[256];  // output row scale
  __shared__ __attribute__((aligned(16))) float xsc[256];  // source token weight w_s
  __shared__ float kpre[4], kpost[4];                       // state factors per sub-chunk
  __shared__ int exact_flag;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar
  // the output row tile of this wave, rotated by the workgroup index: the tiles
  // late in a sub-chunk carry more of the causal block, and rotation spreads
  // them over the SIMDs of a CU instead of loading one SIMD in every workgroup
  const int rw = __builtin_amdgcn_readfirstlane((wid + static_cast<int>(blockIdx.x)) & 3);
  const int QS = Q < QSM ? Q : QSM;
  const int nsub = Q / QS;
  const bool has_rows = 16 * rw < QS;  // waves without output rows (Q = 32) only help stage
  // per-token exponents and step sizes (from the chunk-state kernel), first
  const float2 tv = tid < Q ? tok[((static_cast<size_t>(b) * nc + c) * H + h) * Q + tid]
                            : make_float2(0.f, 0.f);
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

  // ---- global loads: h_in, C rows and x/B of sub-chunk 0 ----

  // h_in tiles (bf16, converted after the prologue so that nothing waits for
  // them before every other load is in flight)
  uint2 hv[KTW][NPT];
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) {
    if constexpr (kPairS) {
      const uint4 u = buf_load16(hbuf, ((pt * 16 + r16) * N + 32 * wid + 8 * q) * 2);
      hv[0][pt] = make_uint2(u.x, u.y);
      hv[1][pt] = make_uint2(u.z, u.w);
    } else {
#pragma unroll
      for (int i = 0; i < KTW; ++i)
        hv[i][pt] = buf_load8(hbuf, ((pt * 16 + r16) * N + (wid + 4 * i) * 16 + 4 * q) * 2);
    }
  }

  // C rows of this wave's output tile in sub-chunk j: lane (row r16, group q)
  // holds k = ks*32 + 8q .. +7.  Rows past the chunk (and every row of the
  // waves without output rows, Q = 32) read as zero through the descriptor;
  // the K padding (N = 16) is zeroed by an out-of-range offset, not by a
  // select on the loaded value, so the prefetch is not waited for here.
  auto load_c = [&](uint4 (&cr)[NKS], int j) {
    const uint32_t row = j * QS + 16 * rw + r16;
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

  // ---- prologue: per-token values, per-sub-chunk factors ----
  // (entries past the chunk are zero: with chunk 16 the diagonal block pair
  // reads the weights of tokens 16..31 into a product it then discards)
  cs[tid] = tid < Q ? tv.x : 0.0f;
  dl[tid] = tid < Q ? tv.y : 0.0f;
  __syncthreads();
  // exponent of token t (t = -1: 0)
  auto csd = [&](int t) -> float { return t < 0 ? 0.0f : cs[t]; };
  if (tid < nsub) {
    const int j0 = tid * QS, m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    if (csd(j0 - 1) - csd(m) > kMaxHalfSpread || csd(m) - csd(j1) > kMaxHalfSpread)
      atomicOr(&exact_flag, 1);
  }
  __syncthreads();
  // uniform over the workgroup; scalar so that its branches keep EXEC whole
  const bool exact = __builtin_amdgcn_readfirstlane(exact_flag) != 0;
  csc[tid] = 0.0f;
  xsc[tid] = 0.0f;
  if (tid < Q) {
    const int j0 = tid & ~(QS - 1), m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    const float e = csd(tid);
    if (exact) {
      csc[tid] = __expf(e - csd(j0 - 1));
      xsc[tid] = __expf(csd(j1) - e) * dl[tid];
    } else {
      csc[tid] = __expf(e - csd(m));
      xsc[tid] = __expf(csd(m) - e) * dl[tid];
    }
    if (tid == j1) {
      const int j = tid / QS;
      if (exact) {
        kpre[j] = 1.0f;
        kpost[j] = __expf(csd(j1) - csd(j0 - 1));
      } else {
        kpre[j] = __expf(csd(m) - (j0 > 0 ? csd(m - QS) : 0.0f));
        kpost[j] = 1.0f;
      }
    }
  }
  // state tiles, transposed: lane holds column p = pt*16 + r16, rows n = nt*16 + 4q + j
  f32x4 hacc[KTW][NPT];
#pragma unroll
  for (int i = 0; i < KTW; ++i)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      const uint2 v = hv[i][pt];
      hacc[i][pt] = kPairS || wid + 4 * i < KT
                        ? f32x4{bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16),
                                bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16)}
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  if constexpr (KCP > N) {
    // zero the K padding of bt and hT (stage stores never write it)
    for (int it = tid; it < QSM + P; it += kThreads) {
      uint16_t* row = it < QSM ? bt + it * BTP : hT + (it - QSM) * HTP;
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
        *reinterpret_cast<uint4*>(bt + sl * BTP + v * 8) = bs.v[i];
      }
    }
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (xs.ITEMS % kThreads == 0 || it < xs.ITEMS) {
        const int v = it % (P / 8), sl = it / (P / 8);
        *reinterpret_cast<uint4*>(xl + sl * XPn + v * 8) = xs.v[i];
      }
    }
  };
  // scale the state by kpre[j] and write its bf16 copy hT[p][n]
  auto store_state = [&](int j) {
    const float k = kpre[j];
    if constexpr (kPairS) {
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        hacc[0][pt] = hacc[0][pt] * k;
        hacc[1][pt] = hacc[1][pt] * k;
        *reinterpret_cast<uint4*>(hT + (pt * 16 + r16) * HTP + 32 * wid + 8 * q) =
            make_uint4(pack_bf16x2(hacc[0][pt][0], hacc[0][pt][1]), pack_bf16x2(hacc[0][pt][2], hacc[0][pt][3]),
                       pack_bf16x2(hacc[1][pt][0], hacc[1][pt][1]), pack_bf16x2(hacc[1][pt][2], hacc[1][pt][3]));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
      const int nt = wid + 4 * i;
      if (nt >= KT) break;
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        hacc[i][pt] = hacc[i][pt] * k;
        *reinterpret_cast<uint2*>(hT + (pt * 16 + r16) * HTP + nt * 16 + 4 * q) =
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

    // ---- outputs of rows sj + 16 rw .. +15 (accumulator columns) ----
    if (has_rows) {
      const int lrow = sj + 16 * rw + r16;  // this lane's output row
      f32x4 yacc[NPT];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) yacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // carried: Y^T[p][l] += sum_n H[p][n] C_l[n]
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint4 hv = *reinterpret_cast<const uint4*>(hT + prow(pt, r16) * HTP + ks * 32 + 8 * q);
          yacc[pt] = mfma_bf16(as_bf16x8(hv), as_bf16x8(creg[ks]), yacc[pt]);
        }
      }
      if (exact) {
        const float s1 = csc[lrow];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) yacc[pt] = yacc[pt] * s1;
      }
      // intra-chunk: source blocks b0 = 2k2, b1 = 2k2+1 (16 tokens each);
      // block rw is the diagonal one
      for (int k2 = 0; 2 * k2 <= rw; ++k2) {
        const int b0 = 2 * k2, b1 = 2 * k2 + 1;
        const bool live1 = b1 <= rw;
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 va = *reinterpret_cast<const uint4*>(bt + (b0 * 16 + r16) * BTP + ks * 32 + 8 * q);
          ga = mfma_bf16(as_bf16x8(va), as_bf16x8(creg[ks]), ga);
        }
        if (live1) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 vb = *reinterpret_cast<const uint4*>(bt + (b1 * 16 + r16) * BTP + ks * 32 + 8 * q);
            gb = mfma_bf16(as_bf16x8(vb), as_bf16x8(creg[ks]), gb);
          }
        }
        // lane: column l = r16 (+16 rw), rows s = 4q + jj of blocks b0, b1
        if (!exact) {
          const float4 wa = *reinterpret_cast<const float4*>(xsc + sj + b0 * 16 + 4 * q);
          const float4 wb = *reinterpret_cast<const float4*>(xsc + sj + b1 * 16 + 4 * q);
          ga = ga * f32x4{wa.x, wa.y, wa.z, wa.w};
          gb = gb * f32x4{wb.x, wb.y, wb.z, wb.w};
          if (b0 == rw) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ga[jj] = 4 * q + jj <= r16 ? ga[jj] : 0.f;
          }
          if (b1 == rw) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) gb[jj] = 4 * q + jj <= r16 ? gb[jj] : 0.f;
          }
        } else {
          const float lh = cs[lrow];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int s0 = sj + (b0 + half) * 16 + 4 * q;
            f32x4& gv = half ? gb : ga;
            const float4 hs = *reinterpret_cast<const float4*>(cs + s0);
            const float4 ds = *reinterpret_cast<const float4*>(dl + s0);
            const float hv[4] = {hs.x, hs.y, hs.z, hs.w};
            const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              gv[jj] = s0 + jj <= lrow ? gv[jj] * __expf(lh - hv[jj]) * dv[jj] : 0.f;
          }
        }
        const uint4 mv = make_uint4(pack_bf16x2(ga[0], ga[1]), pack_bf16x2(ga[2], ga[3]),
                                    pack_bf16x2(gb[0], gb[1]), pack_bf16x2(gb[2], gb[3]));
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = kPairP ? lds_tr4s<8>(xl, XPn, b0 * 16 + 4 * q, 32 * (pt >> 1) + 4 * (pt & 1))
                                  : lds_tr4(xl, XPn, b0 * 16 + 4 * q, pt * 16);
          const uint2 hi = kPairP ? lds_tr4s<8>(xl, XPn, b1 * 16 + 4 * q, 32 * (pt >> 1) + 4 * (pt & 1))
                                  : lds_tr4(xl, XPn, b1 * 16 + 4 * q, pt * 16);
          yacc[pt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(mv),
                               yacc[pt]);
        }
      }
      // row scale, + D x_l, y rows out (lane: row lrow; rows past Lc are dropped
      // by the descriptor).  Paired tiles: columns 32 hh + 8q .. +7, one 16-byte
      // store per pair; else columns pt*16 + 4q .. +3
      const float s2 = exact ? 1.0f : csc[lrow];
      if constexpr (kPairP) {
#pragma unroll
        for (int hh = 0; hh < NPT / 2; ++hh) {
          const uint4 u = *reinterpret_cast<const uint4*>(xl + (16 * rw + r16) * XPn + hh * 32 + 8 * q);
          const uint32_t xw[4] = {u.x, u.y, u.z, u.w};
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w2 = xw[e >> 1];
            const float xv = bf16_bits_to_f32((e & 1) ? (w2 >> 16) : (w2 & 0xFFFFu));
            o[e] = yacc[2 * hh + (e >> 2)][e & 3] * s2 + Dh * xv;
          }
          buf_store16(ybuf, static_cast<uint32_t>(lrow) * xrow + (hh * 32 + 8 * q) * 2,
                      make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                 pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])));
        }
      } else {
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const uint2 u = *reinterpret_cast<const uint2*>(xl + (16 * rw + r16) * XPn + pt * 16 + 4 * q);
        const float o0 = yacc[pt][0] * s2 + Dh * bf16_bits_to_f32(u.x & 0xFFFFu);
        const float o1 = yacc[pt][1] * s2 + Dh * bf16_bits_to_f32(u.x >> 16);
        const float o2 = yacc[pt][2] * s2 + Dh * bf16_bits_to_f32(u.y & 0xFFFFu);
        const float o3 = yacc[pt][3] * s2 + Dh * bf16_bits_to_f32(u.y >> 16);
        buf_store8(ybuf, static_cast<uint32_t>(lrow) * xrow + (pt * 16 + 4 * q) * 2,
                   make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)));
      }
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
        // weights of this lane's source tokens sj + k + 8q .. +7
        const float4 w0 = *reinterpret_cast<const float4*>(xsc + sj + k + 8 * q);
        const float4 w1 = *reinterpret_cast<const float4*>(xsc + sj + k + 8 * q + 4);
        uint4 bfr[KTW];
#pragma unroll
        for (int i = 0; i < KTW; ++i) {
          const int nt = wid + 4 * i;
          const uint2 lo = kPairS ? lds_tr4s<8>(bt, BTP, k + 8 * q, 32 * wid + 4 * i)
                                  : lds_tr4(bt, BTP, k + 8 * q, (nt < KT ? nt : 0) * 16);
          const uint2 hi = kPairS ? lds_tr4s<8>(bt, BTP, k + 8 * q + 4, 32 * wid + 4 * i)
                                  : lds_tr4(bt, BTP, k + 8 * q + 4, (nt < KT ? nt : 0) * 16);
          bfr[i] = scale_bf16x8_each(make_uint4(lo.x, lo.y, hi.x, hi.y), w0, w1);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = lds_tr4(xl, XPn, k + 8 * q, pt * 16);
          const uint2 hi = lds_tr4(xl, XPn, k + 8 * q + 4, pt * 16);
          const uint4 afr = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int i = 0; i < KTW; ++i)
            if (kPairS || wid + 4 * i < KT)
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
static hipError_t launch_bf16(const ChunkArgs& a, hipStream_t st, bool with_output = true) {
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  const int npairs = a.Bsz * nc;
  // workspace: bf16 chunk states (Bsz, nc, H, P, N), overwritten in place by
  // the boundary states; fp32 chunk decays (Bsz, H, nc) after the room an
  // fp32 copy of the states would take
  // (Bsz, nc, H, Q) (exponent, step size) pairs after the decays
  uint16_t* states = static_cast<uint16_t*>(a.workspace);
  float* decay = static_cast<float*>(a.workspace) + workspace_state_floats(a.Bsz, nc, a.H, P, N);
  float2* tok = reinterpret_cast<float2*>(decay + workspace_decay_floats(a.Bsz, nc, a.H));
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const uint16_t* C = static_cast<const uint16_t*>(a.C);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  const hipEvent_t* ev = a.events;
  // chunk states: two heads per workgroup when the heads of a group pair up
  if ((a.H / a.G) % 2 == 0)
    launch_k(nc > 0, ssd_state_bf16_kernel<P, N, 2>, dim3(blocks / 2), dim3(512), st, ev, x, a.dt,
             a.A, B, a.dt_bias, a.dt_min, a.dt_max, states, decay, tok, a.T, a.H, a.G, a.chunk,
             nc, npairs);
  else
    launch_k(nc > 0, ssd_state_bf16_kernel<P, N, 1>, dim3(blocks), dim3(512), st, ev, x, a.dt,
             a.A, B, a.dt_bias, a.dt_min, a.dt_max, states, decay, tok, a.T, a.H, a.G, a.chunk,
             nc, npairs);
  launch_k(nc > 0 || a.h_final, ssd_pass_bf16_kernel,
           dim3((P * N / 8 + kThreads - 1) / kThreads, a.H, a.Bsz), dim3(kThreads), st,
           ev ? ev + 2 : nullptr, states, static_cast<const float*>(decay), a.h0, a.h_final, a.H,
           P * N, nc);
  if (!with_output) return hipGetLastError();
  launch_k(nc > 0, ssd_scan_bf16_kernel<P, N>, dim3(blocks), dim3(kThreads), st,
           ev ? ev + 4 : nullptr, x, B, C, a.D, static_cast<const float2*>(tok),
           static_cast<const uint16_t*>(states), static_cast<uint16_t*>(a.y), a.T, a.H, a.G,
           a.chunk, nc, npairs);
  return hipGetLastError();
}

template <int P>
static hipError_t dispatch_bf16_n(const ChunkArgs& a, hipStream_t st, bool with_output) {
  switch (a.N) {
    case 16: return launch_bf16<P, 16>(a, st, with_output);
    case 32: return launch_bf16<P, 32>(a, st, with_output);
    case 64: return launch_bf16<P, 64>(a, st, with_output);
    case 128: return launch_bf16<P, 128>(a, st, with_output);
    default: break;
  }
  return hipErrorInvalidValue;
}

static hipError_t dispatch_bf16(const ChunkArgs& a, hipStream_t st, bool with_output) {
  switch (a.P) {
    case 16: return dispatch_bf16_n<16>(a, st, with_output);
    case 32: return dispatch_bf16_n<32>(a, st, with_output);
    case 64: return dispatch_bf16_n<64>(a, st, with_output);
    case 128: return dispatch_bf16_n<128>(a, st, with_output);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t run_chunk_real_bf16(const ChunkArgs& a, hipStream_t st) { return dispatch_bf16(a, st, true); }

// the chunk states, boundary states, decays, token table and h_final of a
// forward call without its outputs (the backward recomputes these)
hipError_t run_chunk_states_bf16(const ChunkArgs& a, hipStream_t st) { return dispatch_bf16(a, st, false); }

}  // namespace ssd
