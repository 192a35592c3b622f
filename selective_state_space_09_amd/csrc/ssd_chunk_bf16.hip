// Chunked SSD forward on gfx950 for bfloat16 x, B, C (real Mamba-2 form; fp32
// state and accumulation), in three kernels:
//   ssd_state_bf16_kernel  the end state of each segment of K chunks from a
//                          zero start, and its decay, per (batch, segment,
//                          head pair);
//   ssd_pass_bf16_kernel   the states entering each segment and the final
//                          state;
//   ssd_scan_bf16_kernel   the outputs of a segment from the state entering
//                          it, per (batch, segment, head).
// (Numerical Stability in Mamba-3-Lite, section 4: the chunkwise form with
// L[l,s] = exp(cs_l - cs_s) 1[l >= s] inside a chunk and the chunk's total
// log-decay carrying the state from one chunk to the next.)
//
// A segment is K consecutive chunks of one (batch, head) (the workspace
// layout and the choice of K are in ssd_internal.h): both chunk kernels walk
// its chunks in order and carry the state between them in fp32 matrix-core
// accumulators, so states go through memory only at segment ends.  Cumulative
// decay exponents restart at every chunk (each exponent difference the
// kernels form lies inside one chunk, or is a chunk total), so K does not
// change the arithmetic's accuracy; results equal those of K = 1 up to
// rounding order.
//
// Token rows are staged into LDS in their natural row-major layout (16-byte
// stores); matrix-core operands whose contraction runs over tokens are read
// with the gfx950 LDS transpose read ds_read_b64_tr_b16.

#include <type_traits>

#include <vector>

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

template <int S>
using Slot = std::integral_constant<int, S>;

// The k slots of a 32-token step of an MFMA contraction over tokens whose two
// operands both come from the LDS transpose read: lane group q takes the rows
// (tokens) kSlotRow(q, 0) .. +3 and kSlotRow(q, 1) .. +3.  S4: rows 4q and
// 16 + 4q, so that the four groups of a half-wave read 8 consecutive rows,
// which the transpose read serves without bank conflicts at these pitches;
// otherwise rows 8q and 8q + 4 (groups 8 rows apart: 2-way conflicts), which
// the single-chunk builds keep: measured faster there (the other form made
// the single-chunk output kernel spill at its 168-register bound).
template <bool S4>
__host__ __device__ constexpr int kSlotRow(int q, int half) {
  return S4 ? 4 * q + 16 * half : 8 * q + 4 * half;
}

#ifndef SSD_STATE_PAIR_HEADS
#define SSD_STATE_PAIR_HEADS 1
#endif
constexpr bool kStatePairHeads = SSD_STATE_PAIR_HEADS;

// ---------------------------------------------------------------------------
// Segment end states from a zero start, one workgroup per (batch, segment,
// HPW heads of one group).  For each chunk c of the segment, with u_s = delta_1
// + .. + delta_s over the chunk and u_c its total:
//   S_c[p][n] = sum_s x_s[p] e^{A (u_c - u_s)} delta_s B_s[n],  lambda_c = e^{A u_c}
// and the segment's state S = lambda_c S + S_c chunk by chunk (fp32, in the
// accumulators), its decay the product of the lambda_c.  The heads of a
// workgroup share their B rows: B is staged once and its MFMA operands are
// read once for all of them (HPW = 2 when the heads of a group pair up).  The
// segment is staged through LDS in quarters of up to 64 tokens (a quarter
// never spans two chunks), loaded into registers two quarters ahead.  The
// decay weight goes onto x (P columns) as it is staged.  Eight waves; wave w
// owns n tiles 2(w%4), 2(w%4)+1 and p tiles 2(w/4), 2(w/4)+1 of the
// transposed product D[n][p] = sum_s B_s[n] (w_s x_s[p]) of every head, so an
// accumulator lane holds one p and, per pair of n tiles, 8 consecutive n (two
// 16-byte stores of the fp32 state).  The exponent sums are fp32 (a wave DPP
// scan): a sum of at most 256 positive steps carries a relative error of
// ~1e-6.  Each chunk's (A u_l, delta_l) per token goes to the token table.
// ---------------------------------------------------------------------------
// S4: the k slots of the contraction over tokens (see kSlotRow)
template <int P, int N, int HPW, bool S4>
__global__ __launch_bounds__(512, 4) void ssd_state_bf16_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, float* __restrict__ states, float* __restrict__ decay,
    float2* __restrict__ tok, int T, int H, int G, int Q, int nc, int K, int nseg, int npairs,
    VarLen vl) {
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
  // are 8 consecutive n
  constexpr bool kPairN = NTW % 2 == 0;

  __shared__ __attribute__((aligned(16))) uint16_t xl[HPW][HS * XPn];  // w_s x_s per head
  __shared__ __attribute__((aligned(16))) uint16_t bl[HS * BPn];       // B_s
  __shared__ __attribute__((aligned(16))) float wsc[HPW][256];
  __shared__ float wpart[HPW][WW];

  SegView sv;
  if (!seg_of_block(vl, H / HPW, T, nseg, npairs, sv)) return;
  const int b = sv.b, sg = sv.sg;
  const int h0 = sv.h * HPW;  // first head of the workgroup
  const int g = h0 / (H / G);
  const int ncb = (sv.T + Q - 1) / Q;       // chunks of the sequence
  const int c0 = sg * K;                    // first chunk of the segment
  const int nck = min(K, ncb - c0);         // chunks of the segment
  const int ts = c0 * Q;                    // first token
  const int Ls = min(nck * Q, sv.T - ts);   // tokens of the segment
  // token-table chunk of the segment's first chunk (variable lengths: K slots
  // per global segment)
  const size_t tokc0 = vl.cu ? static_cast<size_t>(sv.gs) * K : static_cast<size_t>(b) * nc + c0;
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const int ng = wid % NGW, pg = wid / NGW;

  // ---- loads: the heads' A and dt bias, dt of the first chunk, then the
  // first two quarters (the per-head values loaded once, first: a wait for a
  // load also waits for every load issued before it) ----
  const size_t r0 = sv.row0 + ts;
  float a_h[HPW], bias_h[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    a_h[e] = A[h0 + e];
    bias_h[e] = dt_bias ? dt_bias[h0 + e] : 0.0f;
  }
  float dtv[HPW];
  auto load_dt = [&](int kc) {
    const int lc = min(Q, Ls - kc * Q);
#pragma unroll
    for (int e = 0; e < HPW; ++e)
      dtv[e] = tid < lc ? dt[(r0 + static_cast<size_t>(kc) * Q + tid) * H + h0 + e] : 0.0f;
  };
  load_dt(0);
  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2;
  const uint32_t brow = static_cast<uint32_t>(G) * N * 2;
  buf_t xbuf[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e)
    xbuf[e] = make_buf(x + r0 * H * P + static_cast<size_t>(h0 + e) * P,
                       static_cast<uint32_t>(Ls - 1) * xrow + P * 2);
  const buf_t bbuf = make_buf(Bm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Ls - 1) * brow + N * 2);
  BufSlab<HS, P / 8, NTHR> xs[2][HPW];
  BufSlab<HS, N / 8, NTHR> bs[2];
  // quarters: Q >= 64 splits every chunk into Q / 64 of them; a shorter chunk
  // is one quarter (its segment has one chunk)
  const int QR = Q < HS ? Q : HS;           // tokens per quarter
  const int nqc = Q < HS ? 1 : Q / HS;      // quarters per chunk
  const int nq = nck * nqc;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (i < nq) {
#pragma unroll
      for (int e = 0; e < HPW; ++e) xs[i][e].load(xbuf[e], xrow, i * QR);
      bs[i].load(bbuf, brow, i * QR);
    }

  f32x4 acc[HPW][NTW][PTW];
#pragma unroll
  for (int e = 0; e < HPW; ++e)
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int j = 0; j < PTW; ++j) acc[e][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float lam_seg[HPW];
#pragma unroll
  for (int e = 0; e < HPW; ++e) lam_seg[e] = 1.0f;

  // ---- chunk kc: step sizes, running sums (thread s = token s), weights to
  // the chunk end, token table, decay; the carried state decays over the chunk
  auto chunk_start = [&](int kc) {
    const int lc = min(Q, Ls - kc * Q);
    float dd[HPW], uu[HPW];
#pragma unroll
    for (int e = 0; e < HPW; ++e) {
      dd[e] = tid < lc ? step_size(dtv[e], bias_h[e], dt_min, dt_max) : 0.0f;
      uu[e] = wave_inclusive_sum(dd[e]);
      if (lane == kWave - 1) wpart[e][wid] = uu[e];
    }
    if (kc + 1 < nck) load_dt(kc + 1);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < HPW; ++e) {
      const int h = h0 + e;
      const float a_re = a_h[e];
      float before = 0.0f, total = 0.0f;
#pragma unroll
      for (int w = 0; w < WW; ++w) {
        const float pw = wpart[e][w];
        before += w < wid ? pw : 0.0f;
        total += pw;
      }
      const float u = uu[e] + before;
      if (tid < 256) wsc[e][tid] = __expf(a_re * (total - u)) * dd[e];
      const float lam = __expf(a_re * total);
      lam_seg[e] *= lam;
      // (A u_l, delta_l) of every token for the output kernel (padding: delta 0)
      if (tid < Q)
        tok[((tokc0 + kc) * H + h) * Q + tid] = make_float2(a_re * u, dd[e]);
      if (kc > 0) {
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
          for (int j = 0; j < PTW; ++j) acc[e][i][j] = acc[e][i][j] * lam;
      }
    }
    __syncthreads();
  };

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

  // one quarter on MFMA: contraction over its tokens, all operand reads of a
  // 32-token step issued before the step's MFMAs; the B operands serve every head
  auto mma = [&](int rows) {
    for (int ks = 0; ks < rows; ks += 32) {
      uint4 af[NTW], bf[HPW][PTW];
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int nt = ng * NTW + i;
        const int cc = kPairN ? 32 * (nt >> 1) + 4 * (nt & 1) : nt * 16;
        const int r0 = ks + kSlotRow<S4>(q, 0), r1 = ks + kSlotRow<S4>(q, 1);
        const uint2 lo = kPairN ? lds_tr4s<8>(bl, BPn, r0, cc) : lds_tr4(bl, BPn, r0, cc);
        const uint2 hi = kPairN ? lds_tr4s<8>(bl, BPn, r1, cc) : lds_tr4(bl, BPn, r1, cc);
        af[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
#pragma unroll
      for (int e = 0; e < HPW; ++e)
#pragma unroll
        for (int j = 0; j < PTW; ++j) {
          const int pt = pg * PTW + j < PT ? pg * PTW + j : 0;
          const uint2 lo = lds_tr4(xl[e], XPn, ks + kSlotRow<S4>(q, 0), pt * 16);
          const uint2 hi = lds_tr4(xl[e], XPn, ks + kSlotRow<S4>(q, 1), pt * 16);
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

  // quarter gi of the segment through register slot S of the ring
  auto quarter = [&](auto slot, int gi) {
    constexpr int S = decltype(slot)::value;
    const int kc = gi / nqc, qi = gi - kc * nqc;
    if (qi == 0)
      chunk_start(kc);  // its barriers also end the previous quarter's use of the tiles
    else
      __syncthreads();
    stage(xs[S], bs[S], qi * HS);
    if (gi + 2 < nq) {
#pragma unroll
      for (int e = 0; e < HPW; ++e) xs[S][e].load(xbuf[e], xrow, (gi + 2) * QR);
      bs[S].load(bbuf, brow, (gi + 2) * QR);
    }
    __syncthreads();
    mma(QR);
  };
  for (int gi = 0; gi < nq; gi += 2) {
    quarter(Slot<0>{}, gi);
    if (gi + 1 < nq) quarter(Slot<1>{}, gi + 1);
  }

  // segment state: lane holds p = pt*16 + r16 and, per pair of n tiles,
  // n = 32 m + 8q .. +7 (else per tile n = nt*16 + 4q .. +3)
#pragma unroll
  for (int e = 0; e < HPW; ++e) {
    float* dst = states + (static_cast<size_t>(sv.gs) * H + h0 + e) * (static_cast<size_t>(P) * N);
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int pt = pg * PTW + j;
      if (pt >= PT) continue;
      if constexpr (kPairN) {
#pragma unroll
        for (int i = 0; i < NTW; i += 2) {
          const int m = (ng * NTW + i) >> 1;
          float* o = dst + (pt * 16 + r16) * N + 32 * m + 8 * q;
          *reinterpret_cast<float4*>(o) = __builtin_bit_cast(float4, acc[e][i][j]);
          *reinterpret_cast<float4*>(o + 4) = __builtin_bit_cast(float4, acc[e][i + 1][j]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const int nt = ng * NTW + i;
          *reinterpret_cast<float4*>(dst + (pt * 16 + r16) * N + nt * 16 + 4 * q) =
              __builtin_bit_cast(float4, acc[e][i][j]);
        }
      }
    }
    if (tid == 0)
      decay[vl.cu ? static_cast<size_t>(sv.gs) * H + h0 + e : (static_cast<size_t>(b) * H + h0 + e) * nseg + sg] =
          lam_seg[e];
  }
}

// ---------------------------------------------------------------------------
// State passing between segments (fp32 segment states in, boundary states
// out):
//   h_in(0) = h0,  h_in(s+1) = lambda_s h_in(s) + S_s,  h_final = h_in(nseg)
// (the chunkwise recurrence of the state across chunks, applied to segments),
// fp32 running state.  The boundary states go out as the bf16 copy the output
// kernel multiplies with (KEEP32 = false), or in fp32 over the segment states
// they were made from (KEEP32 = true: for consumers that need them exact).
// One thread per 8 consecutive n of one p of one (batch, head): 32-byte reads
// of S, 16-byte writes of the bf16 copy; PF segments in flight.
// ---------------------------------------------------------------------------
template <bool KEEP32>
__global__ __launch_bounds__(kThreads) void ssd_pass_bf16_kernel(
    float* __restrict__ S, uint16_t* __restrict__ hin, const float* __restrict__ decay,
    const float* __restrict__ h0, float* __restrict__ h_final, int H, int PN, int nseg_all,
    const int* __restrict__ segstart) {
  constexpr int PF = 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int e8 = blockIdx.x * kThreads + threadIdx.x;  // group of 8 elements
  if (e8 * 8 >= PN) return;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t sstride = static_cast<size_t>(H) * PN;  // between segments of one (b, h)
  // the sequence's segments: nseg_all each, or (variable lengths) its range of
  // global segments, whose decays are stored segment-major
  const size_t gs0 = segstart ? static_cast<size_t>(segstart[b]) : static_cast<size_t>(b) * nseg_all;
  const int nseg = segstart ? segstart[b + 1] - segstart[b] : nseg_all;
  const size_t off = gs0 * sstride + h * static_cast<size_t>(PN) + e8 * 8;
  float* sp = S + off;
  uint16_t* hp = hin + off;
  const float* dc = segstart ? decay + gs0 * H + h : decay + bh * nseg;
  const int dstr = segstart ? H : 1;
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

  float4 cur[PF][2];
  float cd[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (j < nseg) {
      cur[j][0] = *reinterpret_cast<const float4*>(sp + j * sstride);
      cur[j][1] = *reinterpret_cast<const float4*>(sp + j * sstride + 4);
      cd[j] = dc[j * dstr];
    }
  for (int s0 = 0; s0 < nseg; s0 += PF) {
    float4 nxt[PF][2];
    float nd[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int sn = s0 + PF + j;
      if (sn < nseg) {
        nxt[j][0] = *reinterpret_cast<const float4*>(sp + sn * sstride);
        nxt[j][1] = *reinterpret_cast<const float4*>(sp + sn * sstride + 4);
        nd[j] = dc[sn * dstr];
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int ss = s0 + j;
      if (ss < nseg) {
        if constexpr (!KEEP32)
          *reinterpret_cast<uint4*>(hp + ss * sstride) =
              make_uint4(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                         pack_bf16x2(hv[6], hv[7]));
        const float l = cd[j];
        const float sv[8] = {cur[j][0].x, cur[j][0].y, cur[j][0].z, cur[j][0].w,
                             cur[j][1].x, cur[j][1].y, cur[j][1].z, cur[j][1].w};
        float hold[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          hold[k] = hv[k];
          hv[k] = l * hv[k] + sv[k];
        }
        if constexpr (KEEP32) {
          // the fp32 state entering segment ss over its own S (already consumed)
          *reinterpret_cast<float4*>(sp + ss * sstride) = make_float4(hold[0], hold[1], hold[2], hold[3]);
          *reinterpret_cast<float4*>(sp + ss * sstride + 4) = make_float4(hold[4], hold[5], hold[6], hold[7]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      cur[j][0] = nxt[j][0];
      cur[j][1] = nxt[j][1];
      cd[j] = nd[j];
    }
  }
  if (h_final) {
    *reinterpret_cast<float4*>(h_final + bh * PN + e8 * 8) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    *reinterpret_cast<float4*>(h_final + bh * PN + e8 * 8 + 4) = make_float4(hv[4], hv[5], hv[6], hv[7]);
  }
}

// ---------------------------------------------------------------------------
// Segment outputs.  The workgroup walks its segment in sub-chunks of QS = 64
// tokens (QS = chunk for chunks below 64; a sub-chunk never spans two chunks)
// and carries the state across them -- and across the chunk boundaries inside
// the segment -- in MFMA accumulators; for sub-chunk j (tokens j0..j1 of its
// chunk, state h_j at its start, h_0 = the state entering the segment, cs the
// cumulative decay exponent of the chunk, cs_{j0-1} = 0 at a chunk start):
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
// H_j = sigma_j h_j with sigma_j = e^{cs_m - cs_{j0-1}}, so
//   y_l = e^{cs_l - cs_m} (C_l . H_j + sum_{s <= l} (C_l . B_s) w_s x_s
//                          + D e^{cs_m - cs_l} x_l)
// -- raw C and raw x everywhere, the causal mask only on diagonal blocks, w_s
// on the columns of the masked (C_l . B_s) block before it is rounded to bf16,
// D x_l as one more term on the block's diagonal, one scale per output row at
// the end.  The state update accumulates (w_s B_s) x_s^T into H, w_s applied
// to the B operand in registers, which leaves tau_j h_{j+1} with tau_j =
// e^{cs_m - cs_j1}; the next sub-chunk starts by scaling the accumulators by
// sigma_{j+1} / tau_j (<= 1, the decay from one pivot to the next).  The
// factors stay below e^60 when every half sub-chunk decays by at most e^60; a
// sub-chunk that breaks this runs in exact mode (per-element exponentials
// against raw x, the carried term scaled by e^{cs_l - cs_{j0-1}}, the state
// unscaled: sigma = tau = 1, w_s = e^{cs_j1 - cs_s} delta_s, the state scaled
// by e^{cs_j1 - cs_{j0-1}} before its update).  The pivot-to-pivot factor
// sigma_{j+1} / tau_j can be as small as e^-120, below fp32's range, while the
// state it produces is not: it is applied as its two factors in turn when
// their product would underflow.  Wave 0 computes each
// sub-chunk's factors from the token table one sub-chunk ahead, into one of
// two LDS sets.
//
// The output tile is computed transposed, Y^T[p][l]: wave w owns output rows
// l = 16w .. 16w+15 of each sub-chunk (rotated by workgroup) as accumulator
// columns, so a lane holds one row l (one scale factor) and four consecutive p
// of each tile; the tiles go in pairs with permuted p (P >= 32), so a lane
// holds 8 consecutive p of a pair: one 16-byte store of y.
// Per 32 source tokens, G^T = B_s . C_l^T on MFMA (C rows in registers,
// prefetched a sub-chunk ahead) leaves column l in the lane, which after the
// mask and the weights is the B operand of Y^T += X^T M^T.  For the state
// update wave w owns n tiles 2w, 2w+1 with N = 128 (paired, permuted n), else
// w, w+4, ..: H^T[n][p] += sum_s (w_s B_s[n]) x_s[p] (operands from LDS by the
// transpose read); a lane holds 4 consecutive n of one p.
// ---------------------------------------------------------------------------
// MULTI: the segment may hold several chunks (K > 1).  The single-chunk build
// keeps three workgroups per CU (<= 168 VGPRs); the per-chunk factor step in
// the loop of the multi-chunk build needs more registers, and it runs at two
// per CU rather than spill (T65536: 454 us against 488 us spilled at three).
template <int P, int N, bool MULTI>
__global__ __launch_bounds__(kThreads, MULTI ? 2 : 3) void ssd_scan_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ D, const float2* __restrict__ tok, const uint16_t* __restrict__ hin,
    uint16_t* __restrict__ y, int T, int H, int G, int Q, int nc, int K, int nseg, int npairs, VarLen vl) {
  constexpr int QSM = 64;               // sub-chunk length (Q >= 64); a shorter chunk is one
  constexpr int KCP = N < 32 ? 32 : N;  // K of G^T padded to whole 32-wide MFMA steps (zeros)
  // row pitches (bf16): the B tile is read by rows (16 bytes a lane) and by the
  // transpose read (4 rows x 32 bytes a 16-lane group), so its rows start 8
  // banks apart; the state tile is read by rows only (4 banks apart suffice)
  constexpr int BTP = KCP + 16;
  constexpr int HTP = KCP + 8;
  constexpr int XPn = P + 16;           // pitch of the x tile
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
  // per token of the current chunk: exponent, step size, output row scale,
  // source weight, diagonal D term; per sub-chunk of the chunk: the state's two
  // scale factors before it and its scale before the update, exact mode; the
  // scale the state carries after the chunk's last update
  __shared__ __attribute__((aligned(16))) float tcs[256];
  __shared__ __attribute__((aligned(16))) float tdl[256];
  __shared__ __attribute__((aligned(16))) float tcsc[256];
  __shared__ __attribute__((aligned(16))) float txsc[256];
  __shared__ __attribute__((aligned(16))) float tdsc[256];
  __shared__ float skp1[256 / QSM], skp2[256 / QSM], skpost[256 / QSM];
  __shared__ int sexact[256 / QSM];
  __shared__ float stau_last;

  SegView sv;
  if (!seg_of_block(vl, H, T, nseg, npairs, sv)) return;
  const int b = sv.b, sg = sv.sg, h = sv.h;
  const int g = h / (H / G);
  const int c0 = sg * K;
  const int nck = min(K, (sv.T + Q - 1) / Q - c0);
  const int ts = c0 * Q;
  const int Ls = min(nck * Q, sv.T - ts);
  const size_t tokc0 = vl.cu ? static_cast<size_t>(sv.gs) * K : static_cast<size_t>(b) * nc + c0;
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();  // wave-uniform (SGPR): tile branches stay scalar
  // the output row tile of this wave, rotated by the workgroup index: the tiles
  // late in a sub-chunk carry more of the causal block, and rotation spreads
  // them over the SIMDs of a CU instead of loading one SIMD in every workgroup
  const int rw = __builtin_amdgcn_readfirstlane((wid + static_cast<int>(blockIdx.x)) & 3);
  const int QS = Q < QSM ? Q : QSM;
  const int nsc = Q / QS;               // sub-chunks per chunk
  const int nsub = nck * nsc;
  const bool has_rows = 16 * rw < QS;   // waves without output rows (Q < 64) only help stage
  const float Dh = D ? D[h] : 0.0f;

  // ---- buffer descriptors of this segment's slices (rows >= Ls read as zero) ----
  const size_t xy0 = (sv.row0 + ts) * H * P + static_cast<size_t>(h) * P;
  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2;
  const uint32_t xbytes = Ls > 0 ? static_cast<uint32_t>(Ls - 1) * xrow + P * 2 : 0;
  const buf_t xbuf = make_buf(x + xy0, xbytes);
  const buf_t ybuf = make_buf(y + xy0, xbytes);
  const size_t bc0 = (sv.row0 + ts) * G * N + static_cast<size_t>(g) * N;
  const uint32_t brow = static_cast<uint32_t>(G) * N * 2;
  const uint32_t bbytes = Ls > 0 ? static_cast<uint32_t>(Ls - 1) * brow + N * 2 : 0;
  const buf_t bbuf = make_buf(Bm + bc0, bbytes);
  const buf_t cbuf = make_buf(Cm + bc0, bbytes);
  const buf_t hbuf = make_buf(hin + (static_cast<size_t>(sv.gs) * H + h) * (static_cast<size_t>(P) * N),
                              P * N * 2);
  // token table entry of token tid of chunk kc of the segment
  auto load_tok = [&](int kc) -> float2 {
    return tid < Q ? tok[((tokc0 + kc) * H + h) * Q + tid]
                   : make_float2(0.f, 0.f);
  };

  // ---- global loads: token table, h_in, C rows and x/B of sub-chunk 0 ----
  float2 tv = load_tok(0);

  // h_in tiles (bf16, converted after the first factors so that nothing waits
  // for them before every other load is in flight)
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
  // holds k = ks*32 + 8q .. +7.  Rows past the segment (and every row of the
  // waves without output rows, Q < 64) read as zero through the descriptor;
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
  // x, B and C rows of the sub-chunks ahead, in registers.  The single-chunk
  // build loads one sub-chunk ahead (slot 0 for x and B; C in creg, the next
  // in cnext).  The multi-chunk build runs at two workgroups per CU with
  // registers to spare and loads two ahead through a two-slot ring: sub-chunk
  // j's x, B and C in slot j % 2 (C rows of the sub-chunk being computed stay
  // in its slot until its outputs are done).
  constexpr int NSLOT = MULTI ? 2 : 1;
  uint4 creg[NKS], cnext[NKS];
  uint4 cslot[NSLOT][NKS];
  BufSlab<QSM, P / 8> xsl[NSLOT];
  BufSlab<QSM, N / 8> bsl[NSLOT];
  if constexpr (MULTI) {
    load_c(cslot[0], 0);
    xsl[0].load(xbuf, xrow, 0);
    bsl[0].load(bbuf, brow, 0);
    if (nsub > 1) {
      load_c(cslot[1], 1);
      xsl[1].load(xbuf, xrow, QS);
      bsl[1].load(bbuf, brow, QS);
    }
  } else {
    load_c(creg, 0);
    xsl[0].load(xbuf, xrow, 0);
    bsl[0].load(bbuf, brow, 0);
  }

  // ---- factors of chunk kc's tokens and sub-chunks (every thread; t: token
  // tid's table entry).  Contains two barriers; the first also ends every
  // use of the previous chunk's factors.
  auto chunk_factors = [&](float2 t, bool first) {
    // scale after the previous chunk's last update (the segment's entering
    // state is unscaled)
    const float tau_in = first ? 1.0f : stau_last;
    tcs[tid] = tid < Q ? t.x : 0.0f;
    tdl[tid] = tid < Q ? t.y : 0.0f;
    __syncthreads();
    const int jl = tid / QS, j0 = jl * QS, m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    // exponents around sub-chunk jb (in the chunk's frame): before its first
    // token, at its pivot, at its last token; and whether it runs exact
    auto sub_exps = [&](int jb, float& st, float& cm, float& ce) {
      st = jb > 0 ? tcs[jb * QS - 1] : 0.0f;
      cm = tcs[jb * QS + QS / 2 - 1];
      ce = tcs[jb * QS + QS - 1];
      return st - cm > kMaxHalfSpread || cm - ce > kMaxHalfSpread;
    };
    if (tid < Q) {
      float start, cm, ce;
      const bool exact = sub_exps(jl, start, cm, ce);
      const float e = t.x;
      float sigma, tau, kpost;
      if (!exact) {
        const float w = __expf(cm - e);
        tcsc[tid] = __expf(e - cm);
        txsc[tid] = w * t.y;
        tdsc[tid] = Dh * w;
        sigma = __expf(cm - start);
        tau = __expf(cm - ce);
        kpost = 1.0f;
      } else {
        tcsc[tid] = __expf(e - start);
        txsc[tid] = __expf(ce - e) * t.y;
        tdsc[tid] = Dh;
        sigma = 1.0f;
        tau = 1.0f;
        kpost = __expf(ce - start);
      }
      if (tid == j1) {
        float tau_prev = tau_in;
        if (jl > 0) {
          float s1, m1, e1;
          tau_prev = sub_exps(jl - 1, s1, m1, e1) ? 1.0f : __expf(m1 - e1);
        }
        // sigma / tau_prev, as two factors each >= e^-60: their product (the
        // decay from one pivot to the next) can fall below fp32's range while
        // the state it scales to stays representable
        skp1[jl] = 1.0f / tau_prev;
        skp2[jl] = sigma;
        skpost[jl] = kpost;
        sexact[jl] = exact ? 1 : 0;
        if (jl == nsc - 1) stau_last = tau;
      }
    } else {
      tcsc[tid] = 0.0f;
      txsc[tid] = 0.0f;
      tdsc[tid] = 0.0f;
    }
    __syncthreads();
  };
  chunk_factors(tv, true);

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

  // x and B rows of a slot into the LDS tiles
  auto store_stage = [&](const BufSlab<QSM, P / 8>& xs, const BufSlab<QSM, N / 8>& bs) {
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
  // scale the state by the sub-chunk's factors and write its bf16 copy hT[p][n]
  auto store_state = [&](int jl) {
    const float k1 = skp1[jl], k2 = skp2[jl];
    const float k12 = k1 * k2;
    if (k12 < 0x1p-100f) {  // uniform: the two factors one after the other
#pragma unroll
      for (int i = 0; i < KTW; ++i)
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) hacc[i][pt] = hacc[i][pt] * k1;
    }
    const float k = k12 < 0x1p-100f ? k2 : k12;
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
  store_stage(xsl[0], bsl[0]);
  store_state(0);
  __syncthreads();

  // one sub-chunk: its outputs, then (unless it is the last) the state update
  // and the staging of the next sub-chunk.  S: the slot of sub-chunk j.
  auto step = [&](auto S, int j) {
    constexpr int slot = decltype(S)::value;
    const int kc = j / nsc, jl = j - kc * nsc;  // chunk, sub-chunk within it
    const int sl0 = jl * QS;                    // its first token in the chunk
    const int sj = j * QS;                      // its first token in the segment
    const bool more = j + 1 < nsub;
    const bool next_chunk = more && jl == nsc - 1;
    // uniform over the workgroup; scalar so that its branches keep EXEC whole
    const bool exact = __builtin_amdgcn_readfirstlane(sexact[jl]) != 0;
    float2 tvn = make_float2(0.f, 0.f);
    if constexpr (MULTI) {
      if (j + 2 < nsub) {
        xsl[slot].load(xbuf, xrow, sj + 2 * QS);
        bsl[slot].load(bbuf, brow, sj + 2 * QS);
      }
      if (next_chunk) tvn = load_tok(kc + 1);
    } else {
      if (more) {
        xsl[0].load(xbuf, xrow, sj + QS);
        bsl[0].load(bbuf, brow, sj + QS);
        load_c(cnext, j + 1);
      }
    }
    // C rows of this sub-chunk
    auto& cr = [&]() -> uint4(&)[NKS] {
      if constexpr (MULTI)
        return cslot[slot];
      else
        return creg;
    }();

    // ---- outputs of rows sj + 16 rw .. +15 (accumulator columns) ----
    if (has_rows) {
      const int lr = 16 * rw + r16;  // this lane's output row in the sub-chunk
      f32x4 yacc[NPT];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) yacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // carried: Y^T[p][l] += sum_n H[p][n] C_l[n]
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint4 hvv = *reinterpret_cast<const uint4*>(hT + prow(pt, r16) * HTP + ks * 32 + 8 * q);
          yacc[pt] = mfma_bf16(as_bf16x8(hvv), as_bf16x8(cr[ks]), yacc[pt]);
        }
      }
      const float rsc = tcsc[sl0 + lr];  // row scale (exact mode: the carried term's)
      if (exact) {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) yacc[pt] = yacc[pt] * rsc;
      }
      const float dterm = tdsc[sl0 + lr];
      // intra-chunk: source blocks b0 = 2k2, b1 = 2k2+1 (16 tokens each);
      // block rw is the diagonal one
      for (int k2 = 0; 2 * k2 <= rw; ++k2) {
        const int b0 = 2 * k2, b1 = 2 * k2 + 1;
        const bool live1 = b1 <= rw;
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 va = *reinterpret_cast<const uint4*>(bt + (b0 * 16 + r16) * BTP + ks * 32 + 8 * q);
          ga = mfma_bf16(as_bf16x8(va), as_bf16x8(cr[ks]), ga);
        }
        if (live1) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 vb = *reinterpret_cast<const uint4*>(bt + (b1 * 16 + r16) * BTP + ks * 32 + 8 * q);
            gb = mfma_bf16(as_bf16x8(vb), as_bf16x8(cr[ks]), gb);
          }
        }
        // lane: column l = r16 (+16 rw), rows s = 4q + jj of blocks b0, b1; on
        // the diagonal block the mask, and the D term on its diagonal
        if (!exact) {
          const float4 wa = *reinterpret_cast<const float4*>(&txsc[sl0 + b0 * 16 + 4 * q]);
          const float4 wb = *reinterpret_cast<const float4*>(&txsc[sl0 + b1 * 16 + 4 * q]);
          ga = ga * f32x4{wa.x, wa.y, wa.z, wa.w};
          gb = gb * f32x4{wb.x, wb.y, wb.z, wb.w};
        } else {
          const float lh = tcs[sl0 + lr];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int s0 = (b0 + half) * 16 + 4 * q;
            f32x4& gv = half ? gb : ga;
            const float4 hs = *reinterpret_cast<const float4*>(&tcs[sl0 + s0]);
            const float4 ds = *reinterpret_cast<const float4*>(&tdl[sl0 + s0]);
            const float hsv[4] = {hs.x, hs.y, hs.z, hs.w};
            const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              gv[jj] = s0 + jj <= lr ? gv[jj] * __expf(lh - hsv[jj]) * dv[jj] : 0.f;
          }
        }
        // (selects and an add, no per-lane branches)
        if (b0 == rw) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float keep = 4 * q + jj <= r16 ? ga[jj] : 0.f;
            ga[jj] = keep + (4 * q + jj == r16 ? dterm : 0.f);
          }
        }
        if (b1 == rw) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float keep = 4 * q + jj <= r16 ? gb[jj] : 0.f;
            gb[jj] = keep + (4 * q + jj == r16 ? dterm : 0.f);
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
      // row scale, y rows out (lane: row sj + lr; rows past Ls are dropped by
      // the descriptor).  Paired tiles: columns 32 hh + 8q .. +7, one 16-byte
      // store per pair; else columns pt*16 + 4q .. +3
      const float s2 = exact ? 1.0f : rsc;
      const uint32_t yoff = static_cast<uint32_t>(sj + lr) * xrow;
      if constexpr (kPairP) {
#pragma unroll
        for (int hh = 0; hh < NPT / 2; ++hh) {
          const f32x4 o0 = yacc[2 * hh] * s2, o1 = yacc[2 * hh + 1] * s2;
          buf_store16(ybuf, yoff + (hh * 32 + 8 * q) * 2,
                      make_uint4(pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3]),
                                 pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])));
        }
      } else {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const f32x4 o = yacc[pt] * s2;
          buf_store8(ybuf, yoff + (pt * 16 + 4 * q) * 2,
                     make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])));
        }
      }
    }

    if constexpr (MULTI) {
      if (j + 2 < nsub) load_c(cslot[slot], j + 2);
    }

    // ---- state update to the start of the next sub-chunk ----
    if (more) {
      if (exact) {
        const float kp = skpost[jl];
#pragma unroll
        for (int i = 0; i < KTW; ++i)
#pragma unroll
          for (int pt = 0; pt < NPT; ++pt) hacc[i][pt] = hacc[i][pt] * kp;
      }
      // (only chunks of 64 tokens and more have a next sub-chunk: QS = QSM)
#pragma unroll
      for (int k = 0; k < QSM; k += 32) {
        // weights of this lane's source tokens (its two k slots, kSlotRow)
        constexpr int kHalf = kSlotRow<MULTI>(0, 1);  // row offset of the second half
        const int r0 = k + kSlotRow<MULTI>(q, 0), r1 = r0 + kHalf;
        const float4 w0 = *reinterpret_cast<const float4*>(&txsc[sl0 + k + kSlotRow<MULTI>(q, 0)]);
        const float4 w1 = *reinterpret_cast<const float4*>(&txsc[sl0 + k + kSlotRow<MULTI>(q, 0) + kHalf]);
        uint4 bfr[KTW];
#pragma unroll
        for (int i = 0; i < KTW; ++i) {
          const int nt = wid + 4 * i;
          const uint2 lo = kPairS ? lds_tr4s<8>(bt, BTP, r0, 32 * wid + 4 * i)
                                  : lds_tr4(bt, BTP, r0, (nt < KT ? nt : 0) * 16);
          const uint2 hi = kPairS ? lds_tr4s<8>(bt, BTP, r1, 32 * wid + 4 * i)
                                  : lds_tr4(bt, BTP, r1, (nt < KT ? nt : 0) * 16);
          bfr[i] = scale_bf16x8_each(make_uint4(lo.x, lo.y, hi.x, hi.y), w0, w1);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = lds_tr4(xl, XPn, r0, pt * 16);
          const uint2 hi = lds_tr4(xl, XPn, r1, pt * 16);
          const uint4 afr = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
          for (int i = 0; i < KTW; ++i)
            if (kPairS || wid + 4 * i < KT)
              hacc[i][pt] = mfma_bf16(as_bf16x8(bfr[i]), as_bf16x8(afr), hacc[i][pt]);
        }
      }
      __syncthreads();  // every wave is done with this sub-chunk's tiles
      store_stage(xsl[MULTI ? 1 - slot : 0], bsl[MULTI ? 1 - slot : 0]);
      if constexpr (MULTI) {
        if (next_chunk) chunk_factors(tvn, false);  // the chunk's factors replace the last one's
      }
      store_state(next_chunk ? 0 : jl + 1);
      if constexpr (!MULTI) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) creg[ks] = cnext[ks];
      }
      __syncthreads();
    }
  };
  if constexpr (MULTI) {
    for (int j = 0; j < nsub; j += 2) {
      step(Slot<0>{}, j);
      if (j + 1 < nsub) step(Slot<1>{}, j + 1);
    }
  } else {
    for (int j = 0; j < nsub; ++j) step(Slot<0>{}, j);
  }
}

// ---------------------------------------------------------------------------
// variable lengths: the plan's segment count, the workspace layout and the
// device copies of the tables
struct VarSetup {
  int npairs;
  Bf16FwdLayout L;
  VarLen vl;
};

template <int P, int N>
static hipError_t launch_bf16(const ChunkArgs& a, hipStream_t st, bool with_output, int K,
                              const VarSetup* vs = nullptr) {
  // uniform: nc chunks and nseg segments per sequence; variable lengths: the
  // global segments of the plan (nc, nseg unused by the kernels)
  const int nc = vs ? 0 : (a.T + a.chunk - 1) / a.chunk;
  const int nseg = vs ? 0 : (nc + K - 1) / K;
  const int npairs = vs ? vs->npairs : a.Bsz * nseg;
  const Bf16FwdLayout L = vs ? vs->L : bf16_fwd_layout(a.Bsz, nc, a.H, P, N, a.chunk, K);
  const VarLen vl = vs ? vs->vl : VarLen{nullptr, nullptr, nullptr};
  const bool any = npairs > 0;
  char* ws = static_cast<char*>(a.workspace);
  float* S = reinterpret_cast<float*>(ws + L.S);
  uint16_t* hin = reinterpret_cast<uint16_t*>(ws + L.Hin);
  float* decay = reinterpret_cast<float*>(ws + L.decay);
  float2* tok = reinterpret_cast<float2*>(ws + L.tok);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const uint16_t* C = static_cast<const uint16_t*>(a.C);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  const hipEvent_t* ev = a.events;
  // segment states: two heads per workgroup when the heads of a group pair up
  auto state = [&](auto hpw, auto s4) {
    constexpr int HPW = decltype(hpw)::value;
    launch_k(any, ssd_state_bf16_kernel<P, N, HPW, decltype(s4)::value>, dim3(blocks / HPW), dim3(512),
             st, ev, x, a.dt, a.A, B, a.dt_bias, a.dt_min, a.dt_max, S, decay, tok, a.T, a.H, a.G,
             a.chunk, nc, K, nseg, npairs, vl);
  };
  const bool pair = kStatePairHeads && (a.H / a.G) % 2 == 0;
  if (pair && K > 1)
    state(Slot<2>{}, std::true_type{});
  else if (pair)
    state(Slot<2>{}, std::false_type{});
  else if (K > 1)
    state(Slot<1>{}, std::true_type{});
  else
    state(Slot<1>{}, std::false_type{});
  // without the outputs (the backward's recompute, K = 1) the fp32 boundary
  // states are kept too, over the chunk states
  if (with_output)
    launch_k(any || a.h_final, ssd_pass_bf16_kernel<false>,
             dim3((P * N / 8 + kThreads - 1) / kThreads, a.H, a.Bsz), dim3(kThreads), st,
             ev ? ev + 2 : nullptr, S, hin, static_cast<const float*>(decay), a.h0, a.h_final, a.H,
             P * N, nseg, vl.segstart);
  else
    launch_k(any || a.h_final, ssd_pass_bf16_kernel<true>,
             dim3((P * N / 8 + kThreads - 1) / kThreads, a.H, a.Bsz), dim3(kThreads), st,
             ev ? ev + 2 : nullptr, S, hin, static_cast<const float*>(decay), a.h0, a.h_final, a.H,
             P * N, nseg, vl.segstart);
  if (!with_output) return hipGetLastError();
  // the kernel walks several chunks only when K > 1 (a separate build: the
  // per-chunk factor step inside its loop costs registers)
  if (K > 1)
    launch_k(any, ssd_scan_bf16_kernel<P, N, true>, dim3(blocks), dim3(kThreads), st,
             ev ? ev + 4 : nullptr, x, B, C, a.D, static_cast<const float2*>(tok),
             static_cast<const uint16_t*>(hin), static_cast<uint16_t*>(a.y), a.T, a.H, a.G,
             a.chunk, nc, K, nseg, npairs, vl);
  else
    launch_k(any, ssd_scan_bf16_kernel<P, N, false>, dim3(blocks), dim3(kThreads), st,
             ev ? ev + 4 : nullptr, x, B, C, a.D, static_cast<const float2*>(tok),
             static_cast<const uint16_t*>(hin), static_cast<uint16_t*>(a.y), a.T, a.H, a.G,
             a.chunk, nc, K, nseg, npairs, vl);
  return hipGetLastError();
}

template <int P>
static hipError_t dispatch_bf16_n(const ChunkArgs& a, hipStream_t st, bool with_output, int K,
                                  const VarSetup* vs = nullptr) {
  switch (a.N) {
    case 16: return launch_bf16<P, 16>(a, st, with_output, K, vs);
    case 32: return launch_bf16<P, 32>(a, st, with_output, K, vs);
    case 64: return launch_bf16<P, 64>(a, st, with_output, K, vs);
    case 128: return launch_bf16<P, 128>(a, st, with_output, K, vs);
    default: break;
  }
  return hipErrorInvalidValue;
}

static hipError_t dispatch_bf16(const ChunkArgs& a, hipStream_t st, bool with_output, int K,
                                const VarSetup* vs = nullptr) {
  switch (a.P) {
    case 16: return dispatch_bf16_n<16>(a, st, with_output, K, vs);
    case 32: return dispatch_bf16_n<32>(a, st, with_output, K, vs);
    case 64: return dispatch_bf16_n<64>(a, st, with_output, K, vs);
    case 128: return dispatch_bf16_n<128>(a, st, with_output, K, vs);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t run_chunk_real_bf16(const ChunkArgs& a, hipStream_t st) {
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  return dispatch_bf16(a, st, true, bf16_segment_chunks(a.Bsz, nc, a.H, a.chunk));
}

// the per-chunk boundary states (fp32 over S, and their bf16 copies), decays,
// token table and h_final of a forward call without its outputs (the backward
// recomputes these)
hipError_t run_chunk_states_bf16(const ChunkArgs& a, hipStream_t st) { return dispatch_bf16(a, st, false, 1); }

// ---- variable-length batches ----

bool varlen_plan(const int* cu, int nseq, int H, int chunk, VarlenPlan& p, const char** why) {
  if (nseq <= 0 || nseq > 65535) {
    *why = "nseq must be in [1, 65535]";
    return false;
  }
  if (cu[0] != 0) {
    *why = "cu_seqlens[0] must be 0";
    return false;
  }
  long long nc_tot = 0;
  int max_nc = 0;
  for (int b = 0; b < nseq; ++b) {
    if (cu[b + 1] < cu[b]) {
      *why = "cu_seqlens must be non-decreasing";
      return false;
    }
    const int nc = (cu[b + 1] - cu[b] + chunk - 1) / chunk;
    nc_tot += nc;
    max_nc = nc > max_nc ? nc : max_nc;
  }
  p.nseq = nseq;
  p.Ttot = cu[nseq];
  p.nc_tot = nc_tot;
  p.max_nc = max_nc;
  // the rule over all chunks (the variable-length target), then no longer than
  // the longest sequence
  int K = nc_tot > 2147483647LL
              ? 16
              : bf16_segment_chunks(1, static_cast<int>(nc_tot), H, chunk, kSegTargetUnitsVarlen);
  while (K > 1 && K > max_nc) K /= 2;
  p.K = K;
  long long npairs = 0;
  for (int b = 0; b < nseq; ++b) {
    const int nc = (cu[b + 1] - cu[b] + chunk - 1) / chunk;
    npairs += (nc + K - 1) / K;
  }
  if ((npairs + kXCD - 1) / kXCD * kXCD * H > 2147483647LL) {
    *why = "grid too large: the segments times H exceed 2^31 - 1 workgroups";
    return false;
  }
  p.npairs = static_cast<int>(npairs);
  return true;
}

Bf16FwdLayout bf16_varlen_layout(const VarlenPlan& p, int H, int P, int N, int chunk) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t np = static_cast<size_t>(p.npairs);
  const size_t st = np * H * P * N;
  Bf16FwdLayout L{};
  size_t o = 0;
  L.S = o;
  o += up(st * 4);
  L.Hin = o;
  o += up(st * 2);
  L.decay = o;
  o += up(np * H * 4);
  L.tok = o;
  o += up(np * p.K * H * chunk * 8);
  L.table = o;
  o += up(np * 8 + 2 * (static_cast<size_t>(p.nseq) + 1) * 4);
  L.total = o;
  return L;
}

hipError_t run_chunk_varlen_bf16(const ChunkArgs& a, const VarlenPlan& p, const int* cu, hipStream_t st) {
  const Bf16FwdLayout L = bf16_varlen_layout(p, a.H, a.P, a.N, a.chunk);
  // the table, built here and copied into the workspace (the call returns
  // once the copy has taken the host data)
  std::vector<int> t(static_cast<size_t>(p.npairs) * 2 + 2 * (static_cast<size_t>(p.nseq) + 1));
  int* seg = t.data();
  int* segstart = seg + static_cast<size_t>(p.npairs) * 2;
  int* cud = segstart + p.nseq + 1;
  int j = 0;
  for (int b = 0; b < p.nseq; ++b) {
    segstart[b] = j;
    const int nc = (cu[b + 1] - cu[b] + a.chunk - 1) / a.chunk;
    for (int sg = 0; sg < (nc + p.K - 1) / p.K; ++sg, ++j) {
      seg[2 * j] = b;
      seg[2 * j + 1] = sg;
    }
  }
  segstart[p.nseq] = j;
  for (int b = 0; b <= p.nseq; ++b) cud[b] = cu[b];
  char* ws = static_cast<char*>(a.workspace);
  hipError_t e = hipMemcpyAsync(ws + L.table, t.data(), t.size() * sizeof(int), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return e;
  const char* tb = ws + L.table;
  const VarSetup vs{p.npairs, L,
                    VarLen{reinterpret_cast<const int*>(tb + (static_cast<size_t>(p.npairs) * 2 + p.nseq + 1) * 4),
                           reinterpret_cast<const int2*>(tb),
                           reinterpret_cast<const int*>(tb + static_cast<size_t>(p.npairs) * 8)}};
  return dispatch_bf16(a, st, true, p.K, &vs);
}

}  // namespace ssd
