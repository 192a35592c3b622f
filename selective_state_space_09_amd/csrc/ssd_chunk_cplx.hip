// Chunked SSD forward on gfx950, complex form (Mamba-3-Lite): fp32 x,
// complex64 A, B, C, complex64 state, y = Re(h C).
//
// Rotation factoring (Numerical Stability in Mamba-3-Lite, section 3.3 expands
// the complex product into real ones).  Inside a chunk, with u_l the cumulative
// step from the chunk start and theta_l = beta u_l,
//   e^{A (u_l - u_s)} = e^{alpha (u_l - u_s)} e^{i theta_l} e^{-i theta_s}.
// With B'_s = B_s e^{-i theta_s}, C'_l = C_l e^{i theta_l} and the state kept
// in the frame of the chunk start (h~ = e^{-i theta} h, equal to h_in at the
// start), the chunk evolves with real decays only:
//   h~ <- e^{alpha delta} h~ + x B',   y_l = Re(C'_l . h~)
// and everything is a real product with K = 2N features:
//   B features [B'_re | B'_im], C features [C'_re | -C'_im], state [h~_re | h~_im].
//
// Products run on bf16 MFMA with each fp32 operand split into bf16 hi + lo
// (a b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi, relative error ~2^-16 per
// product, fp32 accumulation): five times the fp32 MFMA rate.
//
// Kernels: ssd_state_cplx_kernel (chunk states, decays and the per-token
// table), the shared ssd_pass_kernel<true> (state passing), and the output
// kernel.

#include "ssd_chunk_common.h"

namespace ssd {

// Where a token row's inputs live.  Separate arrays: x (Bsz,T,H,P), B and C
// (Bsz,T,G,N) of (re, im) pairs, dt (Bsz,T,H).  Packed (PACKED = true): one
// row of the in_proj output per token, `ld` floats apart, head-major slices
// [x | B_re | B_im | C_re | C_im | dt] of widths H*P, H*N (x4) and H (the
// Mamba-3-Lite block page, section 4.2), G = H.
struct CplxRows {
  const float* x;   // x of token 0, head 0 (separate: x; packed: the row base)
  const float* B;   // separate: B; packed: the B_re slice (B_im at +im_off)
  const float* C;   // separate: C; packed: the C_re slice (C_im at +im_off)
  const float* dt;  // separate: dt; packed: the dt slice
  int ld;           // packed: floats between token rows
  int im_off;       // packed: floats from a re slice to its im slice (H*N)
};

// ---------------------------------------------------------------------------
// Chunk states from a zero start, one workgroup (8 waves) per (batch, chunk,
// head):
//   S~_c[p][k] = sum_s w_s x_s[p] Bfeat_s[k],  w_s = e^{alpha (u_c - u_s)}
// (no step factor on the complex input), then S_c = e^{i theta_c} S~_c in the
// frame of the chunk end, written as fp32 (re | im) rows for the state
// passing; lambda_c = e^{A u_c}.  Also writes, per token, (alpha u_l,
// cos theta_l, sin theta_l) for the output kernel.  The chunk is staged
// through LDS in quarters of up to 64 tokens, loaded into registers two
// quarters ahead.  The step prefix sums are double (a DPP wave scan), so the
// rotation angles (up to ~100 rad over a chunk) keep fp32 accuracy; they are
// reduced modulo 2 pi in double.
//
// Wave w owns the k tile pair (kp, kp + N/16) -- real and imaginary parts of
// the same 16 state columns -- for kp = w % NKP, and p tiles pg*PTW ..
// pg*PTW + PTW-1 for pg = w / NKP, so that an accumulator lane holds both
// parts of 4 consecutive n of one p for the final rotation.
// ---------------------------------------------------------------------------
template <int P, int N, bool PACKED>
__global__ __launch_bounds__(512) void ssd_state_cplx_kernel(
    CplxRows in, const float* __restrict__ A, const float* __restrict__ dt_bias, float dt_min,
    float dt_max, float* __restrict__ states, float* __restrict__ decay, float4* __restrict__ tok,
    int T, int H, int G, int Q, int nc, int npairs) {
  constexpr int NTHR = 512, WW = 8;
  constexpr int K = 2 * N;
  constexpr int HS = 64;                     // tokens per staged quarter
  constexpr int XPn = P + 16, BPn = K + 16;  // pitches (bf16 elements)
  constexpr int PT = P / 16;
  constexpr int NKP = N / 16;                // k tile pairs (re, im)
  constexpr int WPK = WW / NKP;              // waves per pair (N <= 128)
  constexpr int PTW = (PT + WPK - 1) / WPK;  // p tiles per wave

  __shared__ __attribute__((aligned(16))) uint16_t xh[2][HS * XPn];  // w x, hi / lo
  __shared__ __attribute__((aligned(16))) uint16_t bh[2][HS * BPn];  // Bfeat, hi / lo
  __shared__ __attribute__((aligned(16))) float wsc[256], cth[256], sth[256];
  __shared__ double wpart[WW];

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const int kp = wid % NKP, pg = wid / NKP;

  // ---- loads: dt first, then the first two quarters of x and B ----
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  const size_t drow = PACKED ? static_cast<size_t>(in.ld) : static_cast<size_t>(H);
  const float dtv = tid < Lc ? in.dt[(r0 + tid) * drow + h] : 0.0f;
  const uint32_t xrow = PACKED ? static_cast<uint32_t>(in.ld) * 4 : static_cast<uint32_t>(H) * P * 4;
  const uint32_t brow = PACKED ? static_cast<uint32_t>(in.ld) * 4 : static_cast<uint32_t>(G) * N * 8;
  const buf_t xbuf = make_buf(in.x + r0 * (xrow / 4) + static_cast<size_t>(h) * P,
                              static_cast<uint32_t>(Lc - 1) * xrow + P * 4);
  // separate: (re, im) pairs, 16 bytes = 2 complex; packed: the re slice (and
  // the im slice in bbi), 16 bytes = 4 parts
  const size_t bcol = PACKED ? static_cast<size_t>(g) * N : static_cast<size_t>(g) * N * 2;
  const buf_t bbuf = make_buf(in.B + r0 * (brow / 4) + bcol,
                              static_cast<uint32_t>(Lc - 1) * brow + N * (PACKED ? 4 : 8));
  const buf_t bbi = make_buf(in.B + (PACKED ? in.im_off : 0) + r0 * (brow / 4) + bcol,
                             static_cast<uint32_t>(Lc - 1) * brow + N * 4);
  constexpr int BV = PACKED ? N / 4 : N / 2;  // 16-byte vectors per row (per part if packed)
  // two register slots: quarters 0 and 1 now, quarter i+2 once quarter i is staged
  BufSlab<HS, P / 4, NTHR> xs[2];
  BufSlab<HS, BV, NTHR> bs[2], bsi[PACKED ? 2 : 1];
  const int nq = (Q + HS - 1) / HS;  // quarters of the chunk
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (i < nq) {
      xs[i].load(xbuf, xrow, i * HS);
      bs[i].load(bbuf, brow, i * HS);
      if constexpr (PACKED) bsi[i].load(bbi, brow, i * HS);
    }
  const float a_re = A[2 * h], a_im = A[2 * h + 1];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;

  // ---- steps, their running sums u (double), weights, angles ----
  const float d = tid < Lc ? step_size(dtv, bias, dt_min, dt_max) : 0.0f;
  double u = wave_inclusive_sum_d(static_cast<double>(d));
  if (lane == kWave - 1) wpart[wid] = u;
  __syncthreads();
  double before = 0.0, total = 0.0;
#pragma unroll
  for (int w = 0; w < WW; ++w) {
    const double pw = wpart[w];
    before += w < wid ? pw : 0.0;
    total += pw;
  }
  u += before;
  if (tid < Q) {
    float co, si;
    rot_cs(static_cast<double>(a_im) * u, co, si);
    cth[tid] = co;
    sth[tid] = si;
    wsc[tid] = __expf(static_cast<float>(static_cast<double>(a_re) * (total - u)));
    tok[((static_cast<size_t>(b) * nc + c) * H + h) * Q + tid] =
        make_float4(static_cast<float>(static_cast<double>(a_re) * u), co, si, 0.0f);
  }
  float ce, se;  // rotation to the chunk end
  rot_cs(static_cast<double>(a_im) * total, ce, se);
  if (tid == 0) {
    const float mag = __expf(static_cast<float>(static_cast<double>(a_re) * total));
    float* dc = decay + ((static_cast<size_t>(b) * H + h) * nc + c) * 2;
    dc[0] = mag * ce;
    dc[1] = mag * se;
  }
  __syncthreads();

  // quarter -> LDS: x scaled by w and split; B rotated by e^{-i theta}, split
  auto stage = [&](const BufSlab<HS, P / 4, NTHR>& xs, const BufSlab<HS, BV, NTHR>& bs,
                   const BufSlab<HS, BV, NTHR>& bsi, int s0) {
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * NTHR;
      const int v = it % (P / 4), sl = it / (P / 4);
      if (xs.ITEMS % NTHR == 0 || it < xs.ITEMS) {
        const float w = s0 + sl < Q ? wsc[s0 + sl] : 0.0f;
        const uint4 r = xs.v[i];
        uint32_t h0, l0, h1, l1;
        split_bf16x2(__uint_as_float(r.x) * w, __uint_as_float(r.y) * w, h0, l0);
        split_bf16x2(__uint_as_float(r.z) * w, __uint_as_float(r.w) * w, h1, l1);
        *reinterpret_cast<uint2*>(xh[0] + sl * XPn + v * 4) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(xh[1] + sl * XPn + v * 4) = make_uint2(l0, l1);
      }
    }
#pragma unroll
    for (int i = 0; i < bs.PER; ++i) {
      const int it = tid + i * NTHR;
      const int v = it % BV, sl = it / BV;
      if (bs.ITEMS % NTHR == 0 || it < bs.ITEMS) {
        const int s = s0 + sl < Q ? s0 + sl : 0;
        const float co = cth[s], si = sth[s];
        if constexpr (PACKED) {
          const uint4 r = bs.v[i], m = bsi.v[i];  // re and im of n = 4v .. 4v+3
          const float br[4] = {__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                               __uint_as_float(r.w)};
          const float bi[4] = {__uint_as_float(m.x), __uint_as_float(m.y), __uint_as_float(m.z),
                               __uint_as_float(m.w)};
          uint32_t rh[2], rl[2], ih[2], il[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            split_bf16x2(br[2 * k] * co + bi[2 * k] * si, br[2 * k + 1] * co + bi[2 * k + 1] * si,
                         rh[k], rl[k]);  // B'_re
            split_bf16x2(bi[2 * k] * co - br[2 * k] * si, bi[2 * k + 1] * co - br[2 * k + 1] * si,
                         ih[k], il[k]);  // B'_im
          }
          *reinterpret_cast<uint2*>(bh[0] + sl * BPn + 4 * v) = make_uint2(rh[0], rh[1]);
          *reinterpret_cast<uint2*>(bh[1] + sl * BPn + 4 * v) = make_uint2(rl[0], rl[1]);
          *reinterpret_cast<uint2*>(bh[0] + sl * BPn + N + 4 * v) = make_uint2(ih[0], ih[1]);
          *reinterpret_cast<uint2*>(bh[1] + sl * BPn + N + 4 * v) = make_uint2(il[0], il[1]);
        } else {
          const uint4 r = bs.v[i];  // (re, im) of n = 2v, 2v+1
          const float b0r = __uint_as_float(r.x), b0i = __uint_as_float(r.y);
          const float b1r = __uint_as_float(r.z), b1i = __uint_as_float(r.w);
          uint32_t rh, rl, ih, il;
          split_bf16x2(b0r * co + b0i * si, b1r * co + b1i * si, rh, rl);  // B'_re
          split_bf16x2(b0i * co - b0r * si, b1i * co - b1r * si, ih, il);  // B'_im
          *reinterpret_cast<uint32_t*>(bh[0] + sl * BPn + 2 * v) = rh;
          *reinterpret_cast<uint32_t*>(bh[1] + sl * BPn + 2 * v) = rl;
          *reinterpret_cast<uint32_t*>(bh[0] + sl * BPn + N + 2 * v) = ih;
          *reinterpret_cast<uint32_t*>(bh[1] + sl * BPn + N + 2 * v) = il;
        }
      }
    }
  };

  // acc[0][j]: real k tile kp, acc[1][j]: imaginary k tile kp + NKP; p tile pg*PTW + j
  f32x4 acc[2][PTW];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < PTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int rows) {
    for (int ks = 0; ks < rows; ks += 32) {
      uint4 af[2][2], bf[PTW][2];  // [tile][hi/lo]
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          const int kt = kp + i * NKP;
          const uint2 lo = lds_tr4(bh[hl], BPn, ks + 8 * q, kt * 16);
          const uint2 hi = lds_tr4(bh[hl], BPn, ks + 8 * q + 4, kt * 16);
          af[i][hl] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
      for (int j = 0; j < PTW; ++j) {
        const int pt = pg * PTW + j < PT ? pg * PTW + j : 0;
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          const uint2 lo = lds_tr4(xh[hl], XPn, ks + 8 * q, pt * 16);
          const uint2 hi = lds_tr4(xh[hl], XPn, ks + 8 * q + 4, pt * 16);
          bf[j][hl] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < PTW; ++j)
          if (pg * PTW + j < PT) {
            acc[i][j] = mfma_bf16(as_bf16x8(af[i][0]), as_bf16x8(bf[j][0]), acc[i][j]);
            acc[i][j] = mfma_bf16(as_bf16x8(af[i][0]), as_bf16x8(bf[j][1]), acc[i][j]);
            acc[i][j] = mfma_bf16(as_bf16x8(af[i][1]), as_bf16x8(bf[j][0]), acc[i][j]);
          }
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nq) {
      if (i > 0) __syncthreads();
      stage(xs[i & 1], bs[i & 1], bsi[PACKED ? (i & 1) : 0], i * HS);
      if (i + 2 < nq) {
        xs[i & 1].load(xbuf, xrow, (i + 2) * HS);
        bs[i & 1].load(bbuf, brow, (i + 2) * HS);
        if constexpr (PACKED) bsi[i & 1].load(bbi, brow, (i + 2) * HS);
      }
      __syncthreads();
      mma(Q - i * HS < HS ? Q - i * HS : HS);
    }

  // S_c = e^{i theta_c} S~_c; lane: p = pt*16 + r16, n = kp*16 + 4q .. +3
  float* dst = states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * K);
#pragma unroll
  for (int j = 0; j < PTW; ++j) {
    const int pt = pg * PTW + j;
    if (pt >= PT) break;
    float4 sr, si;
    sr.x = ce * acc[0][j][0] - se * acc[1][j][0];
    sr.y = ce * acc[0][j][1] - se * acc[1][j][1];
    sr.z = ce * acc[0][j][2] - se * acc[1][j][2];
    sr.w = ce * acc[0][j][3] - se * acc[1][j][3];
    si.x = se * acc[0][j][0] + ce * acc[1][j][0];
    si.y = se * acc[0][j][1] + ce * acc[1][j][1];
    si.z = se * acc[0][j][2] + ce * acc[1][j][2];
    si.w = se * acc[0][j][3] + ce * acc[1][j][3];
    float* row = dst + (pt * 16 + r16) * K + kp * 16 + 4 * q;
    *reinterpret_cast<float4*>(row) = sr;
    *reinterpret_cast<float4*>(row + N) = si;
  }
}

// ---------------------------------------------------------------------------
// Chunk outputs, one workgroup (4 waves) per (batch, chunk, head), in the
// rotated frame of the chunk start (see the top of this file): the bf16
// output kernel's scheme with K = 2N real features, no step factor on the
// input, no D, fp32 y, every product as three split-bf16 MFMAs.  The
// workgroup walks its chunk in sub-chunks of QS = 64 tokens and carries the
// state H (fp32, real and imaginary halves) across them in MFMA accumulators:
//   y_l = e^{cs_l - cs_m} (Cfeat_l . H + sum_{s<=l} (Cfeat_l . Bfeat_s) x^_s)
// with cs = alpha u, the pivot m = j0 + QS/2 - 1, x^_s = x_s e^{cs_m - cs_s},
// H = e^{cs_m - cs_{j0-1}} h~_j, and H updated by Bfeat^T x^ between
// sub-chunks; exact mode (per-element exponentials, raw x, unscaled state)
// when a half sub-chunk decays by more than e^60.  Each 16-row block of a
// sub-chunk is produced by 4 / (QS/16) waves, each over its share of the p
// tiles (C features in registers, loaded a sub-chunk ahead and rotated once
// the angles are known); for the state update wave w owns k tiles w, w+4, ...
// ---------------------------------------------------------------------------
template <int P, int N, bool PACKED>
__global__ __launch_bounds__(kThreads) void ssd_scan_cplx_kernel(
    CplxRows in, const float4* __restrict__ tok, const float* __restrict__ hin,
    float* __restrict__ y, int T, int H, int G, int Q, int nc, int npairs) {
  constexpr int K = 2 * N;              // real features
  // sub-chunk length: 64 tokens unless the hi / lo tiles then overflow LDS
  constexpr int QSM = (2 * 64 * (K + 8) + 4 * 64 * (P + 16) + 2 * P * (K + 8)) * 2 + 6 * 1024 <=
                              kLdsBytes / 2 ? 64 : 32;
  constexpr int BP = K + 8;             // pitch of bt / hT rows (bf16)
  constexpr int XPn = P + 16;           // pitch of the x tiles
  constexpr int NKS = K / 32;
  constexpr int NCG = N >= 32 ? N / 32 : 1;  // complex groups of 8 per lane in a C row
  constexpr int NPT = P / 16;
  constexpr int KT = K / 16;
  constexpr int KTW = (KT + 3) / 4;
  constexpr int NRB = QSM / 16;                 // row blocks of a sub-chunk
  constexpr int WPR = 4 / NRB;                  // waves per row block (p tiles split)
  constexpr int NPW = (NPT + WPR - 1) / WPR;    // p tiles per wave in the outputs
  constexpr float kMaxHalfSpread = 60.0f;

  __shared__ __attribute__((aligned(16))) uint16_t bt[2][QSM * BP];   // Bfeat hi / lo
  __shared__ __attribute__((aligned(16))) uint16_t xh[2][QSM * XPn];  // x^ hi / lo
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][QSM * XPn];  // raw x hi / lo (exact mode)
  __shared__ __attribute__((aligned(16))) uint16_t hT[2][P * BP];     // H hi / lo
  __shared__ __attribute__((aligned(16))) float cs[256], cth[256], sth[256], csc[256], xsc[256];
  __shared__ float kpre[256 / QSM], kpre2[256 / QSM], kpost[256 / QSM];
  __shared__ int exact_flag;

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const int rb = wid / WPR, ph = wid % WPR;     // row block, p part
  const int QS = Q < QSM ? Q : QSM;
  const int nsub = Q / QS;
  const bool has_rows = 16 * rb < QS;
  const size_t unit = (static_cast<size_t>(b) * nc + c) * H + h;
  const float4 tv = tid < Q ? tok[unit * Q + tid] : make_float4(0.f, 1.f, 0.f, 0.f);
  if (tid == 0) exact_flag = 0;

  // ---- buffer descriptors (rows >= Lc read as zero, stores there dropped) ----
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  const size_t xy0 = r0 * H * P + static_cast<size_t>(h) * P;
  const uint32_t yrow = static_cast<uint32_t>(H) * P * 4;
  const uint32_t xrow = PACKED ? static_cast<uint32_t>(in.ld) * 4 : yrow;
  const buf_t xbuf = make_buf(in.x + r0 * (xrow / 4) + static_cast<size_t>(h) * P,
                              static_cast<uint32_t>(Lc - 1) * xrow + P * 4);
  const buf_t ybuf = make_buf(y + xy0, static_cast<uint32_t>(Lc - 1) * yrow + P * 4);
  // separate: (re, im) pairs; packed: the re slices (im slices in bbi, cbi)
  const uint32_t brow = PACKED ? static_cast<uint32_t>(in.ld) * 4 : static_cast<uint32_t>(G) * N * 8;
  const size_t bc0 = r0 * (brow / 4) + (PACKED ? static_cast<size_t>(g) * N : static_cast<size_t>(g) * N * 2);
  const uint32_t bbytes = static_cast<uint32_t>(Lc - 1) * brow + N * (PACKED ? 4 : 8);
  const buf_t bbuf = make_buf(in.B + bc0, bbytes);
  const buf_t cbuf = make_buf(in.C + bc0, bbytes);
  const buf_t bbi = make_buf(in.B + (PACKED ? in.im_off : 0) + bc0, bbytes);
  const buf_t cbi = make_buf(in.C + (PACKED ? in.im_off : 0) + bc0, bbytes);
  constexpr int BV = PACKED ? N / 4 : N / 2;  // 16-byte vectors per row (per part if packed)
  const buf_t hbuf = make_buf(hin + unit * (static_cast<size_t>(P) * K), P * K * 4);

  // ---- every load first: h_in tiles, C rows, x / B of sub-chunk 0 ----
  uint4 hv[KTW][NPT];  // fp32 x 4: k = nt*16 + 4q .. +3 of p = pt*16 + r16
#pragma unroll
  for (int i = 0; i < KTW; ++i)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
      hv[i][pt] = buf_load16(hbuf, ((pt * 16 + r16) * K + (wid + 4 * i) * 16 + 4 * q) * 4);

  // C row of this lane's output row in sub-chunk j: complex group cg holds
  // n0 .. n0+7 with n0 = cg*32 + 8q (N >= 32) or 8q mod 16 (N = 16); as four
  // (re, im) pair vectors (separate) or two re and two im vectors (packed)
  auto load_c = [&](uint4 (&cr)[NCG][4], int j) {
    const uint32_t row = j * QS + 16 * rb + r16;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int n0 = N >= 32 ? cg * 32 + 8 * q : (8 * q) % 16;
      if constexpr (PACKED) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          cr[cg][v] = buf_load16(cbuf, row * brow + (n0 + 4 * v) * 4);
          cr[cg][2 + v] = buf_load16(cbi, row * brow + (n0 + 4 * v) * 4);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) cr[cg][v] = buf_load16(cbuf, row * brow + (n0 + 2 * v) * 8);
      }
    }
  };
  uint4 craw[NCG][4];
  load_c(craw, 0);
  BufSlab<QSM, P / 4> xs;
  BufSlab<QSM, BV> bs, bsi;
  xs.load(xbuf, xrow, 0);
  bs.load(bbuf, brow, 0);
  if constexpr (PACKED) bsi.load(bbi, brow, 0);

  // ---- prologue: per-token values, per-sub-chunk factors ----
  if (tid < Q) {
    cs[tid] = tv.x;
    cth[tid] = tv.y;
    sth[tid] = tv.z;
  }
  __syncthreads();
  auto csd = [&](int t) -> float { return t < 0 ? 0.0f : cs[t]; };
  if (tid < nsub) {
    const int j0 = tid * QS, m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    if (csd(j0 - 1) - csd(m) > kMaxHalfSpread || csd(m) - csd(j1) > kMaxHalfSpread)
      atomicOr(&exact_flag, 1);
  }
  __syncthreads();
  const bool exact = __builtin_amdgcn_readfirstlane(exact_flag) != 0;
  if (tid < Q) {
    const int j0 = tid & ~(QS - 1), m = j0 + QS / 2 - 1, j1 = j0 + QS - 1;
    const float e = csd(tid);
    if (exact) {
      csc[tid] = __expf(e - csd(j0 - 1));
      xsc[tid] = __expf(csd(j1) - e);
    } else {
      csc[tid] = __expf(e - csd(m));
      xsc[tid] = __expf(csd(m) - e);
    }
    if (tid == j1) {
      const int j = tid / QS;
      if (exact) {
        kpre[j] = 1.0f;
        kpre2[j] = 1.0f;
        kpost[j] = __expf(csd(j1) - csd(j0 - 1));
      } else {
        // e^{cs_m - cs_{m-QS}} as two factors each >= e^-60 (before and after
        // the sub-chunk boundary): their product can fall below fp32's range
        // while the state it scales to stays representable
        kpre[j] = j0 > 0 ? __expf(csd(j0 - 1) - csd(m - QS)) : 1.0f;
        kpre2[j] = __expf(csd(m) - csd(j0 - 1));
        kpost[j] = 1.0f;
      }
    }
  }
  f32x4 hacc[KTW][NPT];  // lane: p = pt*16 + r16, k = nt*16 + 4q + j
#pragma unroll
  for (int i = 0; i < KTW; ++i)
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
      hacc[i][pt] = wid + 4 * i < KT ? __builtin_bit_cast(f32x4, hv[i][pt]) : f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  // C features of the lane's row (rotated by e^{i theta_l}), split, as MFMA
  // operands: k = ks*32 + 8q .. +7 is the real part (C'_re) for k < N and
  // the negated imaginary part for k >= N
  uint4 ch[NKS], cl[NKS];
  auto make_c = [&](const uint4 (&cr)[NCG][4], int lrow) {
    const float co = cth[lrow], si = sth[lrow];
    float re[NCG][8], im[NCG][8];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float a[8], bi[8];  // C re and im of n0 .. n0+7
      if constexpr (PACKED) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const uint4 r = cr[cg][v], m = cr[cg][2 + v];
          a[4 * v] = __uint_as_float(r.x);
          a[4 * v + 1] = __uint_as_float(r.y);
          a[4 * v + 2] = __uint_as_float(r.z);
          a[4 * v + 3] = __uint_as_float(r.w);
          bi[4 * v] = __uint_as_float(m.x);
          bi[4 * v + 1] = __uint_as_float(m.y);
          bi[4 * v + 2] = __uint_as_float(m.z);
          bi[4 * v + 3] = __uint_as_float(m.w);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint4 r = cr[cg][v];
          a[2 * v] = __uint_as_float(r.x);
          bi[2 * v] = __uint_as_float(r.y);
          a[2 * v + 1] = __uint_as_float(r.z);
          bi[2 * v + 1] = __uint_as_float(r.w);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        re[cg][e] = a[e] * co - bi[e] * si;
        im[cg][e] = -(a[e] * si + bi[e] * co);
      }
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int cg = N >= 32 ? ks % NCG : 0;
      const bool imag = N >= 32 ? ks >= NCG : q >= 2;
      uint32_t hh[4], ll[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f0 = imag ? im[cg][2 * e] : re[cg][2 * e];
        const float f1 = imag ? im[cg][2 * e + 1] : re[cg][2 * e + 1];
        split_bf16x2(f0, f1, hh[e], ll[e]);
      }
      ch[ks] = make_uint4(hh[0], hh[1], hh[2], hh[3]);
      cl[ks] = make_uint4(ll[0], ll[1], ll[2], ll[3]);
    }
  };

  auto store_stage = [&](int j) {
#pragma unroll
    for (int i = 0; i < bs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (bs.ITEMS % kThreads == 0 || it < bs.ITEMS) {
        const int v = it % BV, sl = it / BV;
        const int s = j * QS + sl < Q ? j * QS + sl : 0;
        const float co = cth[s], si = sth[s];
        if constexpr (PACKED) {
          const uint4 r = bs.v[i], m = bsi.v[i];  // re and im of n = 4v .. 4v+3
          const float br[4] = {__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                               __uint_as_float(r.w)};
          const float bi[4] = {__uint_as_float(m.x), __uint_as_float(m.y), __uint_as_float(m.z),
                               __uint_as_float(m.w)};
          uint32_t rh[2], rl[2], ih[2], il[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            split_bf16x2(br[2 * k] * co + bi[2 * k] * si, br[2 * k + 1] * co + bi[2 * k + 1] * si,
                         rh[k], rl[k]);
            split_bf16x2(bi[2 * k] * co - br[2 * k] * si, bi[2 * k + 1] * co - br[2 * k + 1] * si,
                         ih[k], il[k]);
          }
          *reinterpret_cast<uint2*>(bt[0] + sl * BP + 4 * v) = make_uint2(rh[0], rh[1]);
          *reinterpret_cast<uint2*>(bt[1] + sl * BP + 4 * v) = make_uint2(rl[0], rl[1]);
          *reinterpret_cast<uint2*>(bt[0] + sl * BP + N + 4 * v) = make_uint2(ih[0], ih[1]);
          *reinterpret_cast<uint2*>(bt[1] + sl * BP + N + 4 * v) = make_uint2(il[0], il[1]);
        } else {
          const uint4 r = bs.v[i];
          const float b0r = __uint_as_float(r.x), b0i = __uint_as_float(r.y);
          const float b1r = __uint_as_float(r.z), b1i = __uint_as_float(r.w);
          uint32_t rh, rl, ih, il;
          split_bf16x2(b0r * co + b0i * si, b1r * co + b1i * si, rh, rl);
          split_bf16x2(b0i * co - b0r * si, b1i * co - b1r * si, ih, il);
          *reinterpret_cast<uint32_t*>(bt[0] + sl * BP + 2 * v) = rh;
          *reinterpret_cast<uint32_t*>(bt[1] + sl * BP + 2 * v) = rl;
          *reinterpret_cast<uint32_t*>(bt[0] + sl * BP + N + 2 * v) = ih;
          *reinterpret_cast<uint32_t*>(bt[1] + sl * BP + N + 2 * v) = il;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < xs.PER; ++i) {
      const int it = tid + i * kThreads;
      if (xs.ITEMS % kThreads == 0 || it < xs.ITEMS) {
        const int v = it % (P / 4), sl = it / (P / 4);
        const int s = j * QS + sl;
        const float w = (sl < QS && s < Q) ? xsc[s] : 0.0f;
        const uint4 r = xs.v[i];
        const float f[4] = {__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                            __uint_as_float(r.w)};
        uint32_t h0, l0, h1, l1;
        split_bf16x2(f[0] * w, f[1] * w, h0, l0);
        split_bf16x2(f[2] * w, f[3] * w, h1, l1);
        *reinterpret_cast<uint2*>(xh[0] + sl * XPn + v * 4) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(xh[1] + sl * XPn + v * 4) = make_uint2(l0, l1);
        if (exact) {
          split_bf16x2(f[0], f[1], h0, l0);
          split_bf16x2(f[2], f[3], h1, l1);
          *reinterpret_cast<uint2*>(xl[0] + sl * XPn + v * 4) = make_uint2(h0, h1);
          *reinterpret_cast<uint2*>(xl[1] + sl * XPn + v * 4) = make_uint2(l0, l1);
        }
      }
    }
  };
  // scale the state by kpre[j] and write its split copy hT[p][k]
  auto store_state = [&](int j) {
    const float k1 = kpre[j], k2 = kpre2[j];
    const bool two = k1 * k2 < 0x1p-100f;  // uniform: the factors one after the other
    const float kk = two ? k2 : k1 * k2;
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
      const int nt = wid + 4 * i;
      if (nt >= KT) break;
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        if (two) hacc[i][pt] = hacc[i][pt] * k1;
        hacc[i][pt] = hacc[i][pt] * kk;
        uint32_t h0, l0, h1, l1;
        split_bf16x2(hacc[i][pt][0], hacc[i][pt][1], h0, l0);
        split_bf16x2(hacc[i][pt][2], hacc[i][pt][3], h1, l1);
        *reinterpret_cast<uint2*>(hT[0] + (pt * 16 + r16) * BP + nt * 16 + 4 * q) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(hT[1] + (pt * 16 + r16) * BP + nt * 16 + 4 * q) = make_uint2(l0, l1);
      }
    }
  };
  store_stage(0);
  store_state(0);
  make_c(craw, 16 * rb + r16);
  __syncthreads();

  // three split-bf16 products: (ah + al)(bh + bl) without al*bl
  auto mma3 = [](uint4 ah, uint4 al, uint4 bh_, uint4 bl_, f32x4 acc) {
    acc = mfma_bf16(as_bf16x8(ah), as_bf16x8(bh_), acc);
    acc = mfma_bf16(as_bf16x8(ah), as_bf16x8(bl_), acc);
    return mfma_bf16(as_bf16x8(al), as_bf16x8(bh_), acc);
  };

  for (int j = 0; j < nsub; ++j) {
    const int sj = j * QS;
    const bool more = j + 1 < nsub;
    if (more) {
      xs.load(xbuf, xrow, sj + QS);
      bs.load(bbuf, brow, sj + QS);
      if constexpr (PACKED) bsi.load(bbi, brow, sj + QS);
      load_c(craw, j + 1);
    }

    // ---- outputs of rows sj + 16 rb .. +15 (accumulator columns), p tiles
    // ph*NPW .. +NPW-1 ----
    if (has_rows) {
      const int lrow = sj + 16 * rb + r16;
      f32x4 yacc[NPW];
#pragma unroll
      for (int i = 0; i < NPW; ++i) yacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
          const int pt = ph * NPW + i < NPT ? ph * NPW + i : 0;
          const uint4 h_h = *reinterpret_cast<const uint4*>(hT[0] + (pt * 16 + r16) * BP + ks * 32 + 8 * q);
          const uint4 h_l = *reinterpret_cast<const uint4*>(hT[1] + (pt * 16 + r16) * BP + ks * 32 + 8 * q);
          yacc[i] = mma3(h_h, h_l, ch[ks], cl[ks], yacc[i]);
        }
      if (exact) {
        const float s1 = csc[lrow];
#pragma unroll
        for (int i = 0; i < NPW; ++i) yacc[i] = yacc[i] * s1;
      }
      for (int k2 = 0; 2 * k2 <= rb; ++k2) {
        const int b0 = 2 * k2, b1 = 2 * k2 + 1;
        const bool live1 = b1 <= rb;
        f32x4 ga = f32x4{0.f, 0.f, 0.f, 0.f}, gb = ga;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const uint4 va = *reinterpret_cast<const uint4*>(bt[0] + (b0 * 16 + r16) * BP + ks * 32 + 8 * q);
          const uint4 wa = *reinterpret_cast<const uint4*>(bt[1] + (b0 * 16 + r16) * BP + ks * 32 + 8 * q);
          ga = mma3(va, wa, ch[ks], cl[ks], ga);
        }
        if (live1) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const uint4 vb = *reinterpret_cast<const uint4*>(bt[0] + (b1 * 16 + r16) * BP + ks * 32 + 8 * q);
            const uint4 wb = *reinterpret_cast<const uint4*>(bt[1] + (b1 * 16 + r16) * BP + ks * 32 + 8 * q);
            gb = mma3(vb, wb, ch[ks], cl[ks], gb);
          }
        }
        if (!exact) {
          if (b0 == rb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ga[jj] = 4 * q + jj <= r16 ? ga[jj] : 0.f;
          }
          if (b1 == rb) {
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
            const float ev[4] = {hs.x, hs.y, hs.z, hs.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              gv[jj] = s0 + jj <= lrow ? gv[jj] * __expf(lh - ev[jj]) : 0.f;
          }
        }
        uint32_t mh[4], ml[4];
        split_bf16x2(ga[0], ga[1], mh[0], ml[0]);
        split_bf16x2(ga[2], ga[3], mh[1], ml[1]);
        split_bf16x2(gb[0], gb[1], mh[2], ml[2]);
        split_bf16x2(gb[2], gb[3], mh[3], ml[3]);
        const uint4 mvh = make_uint4(mh[0], mh[1], mh[2], mh[3]);
        const uint4 mvl = make_uint4(ml[0], ml[1], ml[2], ml[3]);
        const uint16_t* xt0 = exact ? xl[0] : xh[0];
        const uint16_t* xt1 = exact ? xl[1] : xh[1];
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
          const int pt = ph * NPW + i < NPT ? ph * NPW + i : 0;
          const uint2 lo0 = lds_tr4(xt0, XPn, b0 * 16 + 4 * q, pt * 16);
          const uint2 hi0 = lds_tr4(xt0, XPn, b1 * 16 + 4 * q, pt * 16);
          const uint2 lo1 = lds_tr4(xt1, XPn, b0 * 16 + 4 * q, pt * 16);
          const uint2 hi1 = lds_tr4(xt1, XPn, b1 * 16 + 4 * q, pt * 16);
          yacc[i] = mma3(make_uint4(lo0.x, lo0.y, hi0.x, hi0.y), make_uint4(lo1.x, lo1.y, hi1.x, hi1.y),
                         mvh, mvl, yacc[i]);
        }
      }
      // row scale, y rows out (lane: row lrow, p = pt*16 + 4q .. +3)
      const float s2 = exact ? 1.0f : csc[lrow];
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int pt = ph * NPW + i;
        if (pt >= NPT) break;
        const f32x4 o = yacc[i] * s2;
        buf_store16(ybuf, static_cast<uint32_t>(lrow) * yrow + (pt * 16 + 4 * q) * 4,
                       __builtin_bit_cast(uint4, o));
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
        uint4 bfh[KTW], bfl[KTW];
#pragma unroll
        for (int i = 0; i < KTW; ++i) {
          const int nt = (wid + 4 * i < KT ? wid + 4 * i : 0);
          const uint2 lo = lds_tr4(bt[0], BP, k + 8 * q, nt * 16);
          const uint2 hi = lds_tr4(bt[0], BP, k + 8 * q + 4, nt * 16);
          const uint2 lo1 = lds_tr4(bt[1], BP, k + 8 * q, nt * 16);
          const uint2 hi1 = lds_tr4(bt[1], BP, k + 8 * q + 4, nt * 16);
          bfh[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          bfl[i] = make_uint4(lo1.x, lo1.y, hi1.x, hi1.y);
        }
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
          const uint2 lo = lds_tr4(xh[0], XPn, k + 8 * q, pt * 16);
          const uint2 hi = lds_tr4(xh[0], XPn, k + 8 * q + 4, pt * 16);
          const uint2 lo1 = lds_tr4(xh[1], XPn, k + 8 * q, pt * 16);
          const uint2 hi1 = lds_tr4(xh[1], XPn, k + 8 * q + 4, pt * 16);
          const uint4 ah = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const uint4 al = make_uint4(lo1.x, lo1.y, hi1.x, hi1.y);
#pragma unroll
          for (int i = 0; i < KTW; ++i)
            if (wid + 4 * i < KT) hacc[i][pt] = mma3(bfh[i], bfl[i], ah, al, hacc[i][pt]);
        }
      }
      __syncthreads();  // every wave is done with this sub-chunk's tiles
      store_stage(j + 1);
      store_state(j + 1);
      __syncthreads();
      make_c(craw, (j + 1) * QS + 16 * rb + r16);
    }
  }
}

// ---------------------------------------------------------------------------
template <int P, int N, bool PACKED>
static hipError_t launch_cplx(const ChunkArgs& a, const CplxRows& in, hipStream_t st) {
  constexpr int K = 2 * N;
  const int nc = (a.T + a.chunk - 1) / a.chunk;
  const int npairs = a.Bsz * nc;
  // workspace: chunk states (Bsz, nc, H, P, 2N) fp32 (overwritten in place by
  // the boundary states), decays (Bsz, H, nc) complex, then the per-token
  // table (Bsz, nc, H, chunk) float4 on a 16-byte boundary
  float* states = static_cast<float*>(a.workspace);
  float* decay = states + workspace_state_floats(a.Bsz, nc, a.H, P, K);
  float4* tok = reinterpret_cast<float4*>(decay + (workspace_decay_floats(a.Bsz, nc, a.H) + 3) / 4 * 4);
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  const hipEvent_t* ev = a.events;
  launch_k(nc > 0, ssd_state_cplx_kernel<P, N, PACKED>, dim3(blocks), dim3(512), st, ev, in, a.A,
           a.dt_bias, a.dt_min, a.dt_max, states, decay, tok, a.T, a.H, a.G, a.chunk, nc, npairs);
  launch_pass<true, N>(states, decay, a.h0, a.h_final, a.Bsz, a.H, P, nc, st, ev ? ev + 2 : nullptr);
  launch_k(nc > 0, ssd_scan_cplx_kernel<P, N, PACKED>, dim3(blocks), dim3(kThreads), st,
           ev ? ev + 4 : nullptr, in, static_cast<const float4*>(tok),
           static_cast<const float*>(states), static_cast<float*>(a.y), a.T, a.H, a.G, a.chunk, nc,
           npairs);
  return hipGetLastError();
}

template <int P, bool PACKED>
static hipError_t dispatch_cplx_n(const ChunkArgs& a, const CplxRows& in, hipStream_t st) {
  switch (a.N) {
    case 16: return launch_cplx<P, 16, PACKED>(a, in, st);
    case 32: return launch_cplx<P, 32, PACKED>(a, in, st);
    case 64: return launch_cplx<P, 64, PACKED>(a, in, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

template <bool PACKED>
static hipError_t dispatch_cplx(const ChunkArgs& a, const CplxRows& in, hipStream_t st) {
  switch (a.P) {
    case 16: return dispatch_cplx_n<16, PACKED>(a, in, st);
    case 32: return dispatch_cplx_n<32, PACKED>(a, in, st);
    case 64: return dispatch_cplx_n<64, PACKED>(a, in, st);
    case 128: return dispatch_cplx_n<128, PACKED>(a, in, st);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t run_chunk_complex(const ChunkArgs& a, hipStream_t st) {
  const CplxRows in{static_cast<const float*>(a.x), static_cast<const float*>(a.B),
                    static_cast<const float*>(a.C), a.dt, 0, 0};
  return dispatch_cplx<false>(a, in, st);
}

// Packed rows: a.x is the in_proj output (Bsz, T, ld) of head-major slices
// [x | B_re | B_im | C_re | C_im | dt]; G = H.
hipError_t run_chunk_complex_packed(const ChunkArgs& a, int ld, hipStream_t st) {
  const float* base = static_cast<const float*>(a.x);
  const size_t HP = static_cast<size_t>(a.H) * a.P, HN = static_cast<size_t>(a.H) * a.N;
  const CplxRows in{base, base + HP, base + HP + 2 * HN, base + HP + 4 * HN, ld,
                    static_cast<int>(HN)};
  return dispatch_cplx<true>(a, in, st);
}

}  // namespace ssd
