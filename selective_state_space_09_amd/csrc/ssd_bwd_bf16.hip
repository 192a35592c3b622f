// Backward of the chunked SSD, real Mamba-2 form, bfloat16 x, B, C and dy
// (fp32 accumulation, fp32 gradients except dx), on gfx950.
//
// Gradient of  loss = sum_t dy_t . y_t + <dh_final, h_final>  for
//   h_t = e^{A delta_t} h_{t-1} + delta_t x_t B_t^T,  y_t = h_t C_t + D x_t
// (the classical Mamba-2 recurrence of the Mamba-3-Lite README, evaluated
// chunkwise as in Numerical Stability in Mamba-3-Lite, section 4).  Inside a
// chunk (cs_l the inclusive cumulative log-decay, tot its total) the adjoint
// of the state is
//   dh_s = sum_{l >= s} e^{cs_l - cs_s} C_l^T dy_l + e^{tot - cs_s} R_c,
// R_c the adjoint at the chunk's end (from the later chunks and dh_final),
// carried across chunks by R_{c-1} = e^{tot_c} R_c + G_c with
// G_c = sum_l e^{cs_l} C_l^T dy_l.  Then, per head,
//   v_s   = dh_s B_s       = sum_{l>=s} e^{cs_l-cs_s} (C_l.B_s) dy_l + e^{tot-cs_s} R_c B_s
//   dx_s  = delta_s v_s + D dy_s
//   dB_s += delta_s dh_s^T x_s
//         = delta_s [ sum_{l>=s} e^{cs_l-cs_s} (dy_l.x_s) C_l + e^{tot-cs_s} R_c^T x_s ]
//   dC_l += h_l^T dy_l     = sum_{s<=l} e^{cs_l-cs_s} delta_s (dy_l.x_s) B_s + e^{cs_l} H_in^T dy_l
// (dB and dC summed over the heads of a group), and for the step sizes
//   ddelta_t = A da_t + x_t . v_t,   dA = sum_t delta_t da_t,   dD = sum_t dy_t . x_t,
// with da_t = <dh_t, e^{A delta_t} h_{t-1}> the gradient of the step's
// log-decay, taken apart inside the chunk into terms that each decay away
// from t (so that none of them is a long sum of terms that cancel):
//   da_t = sum_{s < t <= l} E[l][s]                                       (box)
//        + sum_{l >= t} e^{cs_l} C_l . (H_in^T dy_l)                      (f1)
//        + sum_{s < t} e^{tot-cs_s} delta_s x_s . (R_c B_s)               (f2)
//        + e^{tot} <R_c, H_in>,
// E[l][s] = e^{cs_l-cs_s} delta_s (C_l.B_s)(dy_l.x_s).  Stepping t by one
// moves column t into the box and row t out of it, so that
//   box_t = sum_{u < t} (col_u - row_u),  col_u = sum_{l > u} E[l][u],
//   row_u = sum_{s < u} E[u][s]
// (strictly below the diagonal; each of col_u, row_u and their difference
// is made of the terms next to the diagonal, so the scan stays well scaled).
// The terms of da_t and x_t . v_t cancel (their magnitudes can sum to tens
// of times the result), so everything that feeds them is fp32-accurate: the
// boundary states h_in(c), G_c and R_c are fp32, and a product of an fp32
// operand with bf16 data is taken as two bf16 products (the operand split
// into bf16 hi + lo).  Only dx, dB and dC's own products, which no gradient
// subtracts from, use single bf16 operands.
// The pieces:
//   forward recompute   chunk states, boundary states h_in(c) (fp32) and the
//                       per-token (cs, delta) table (the forward's kernels)
//   ssd_adj_state       G_c per (batch, chunk, head), MFMA over tokens
//   ssd_adj_pass        R_c in place over G_c, dh0, and the chunk constants
//                       e^{tot} <R_c, H_in(c)> as fp64 shares
//   ssd_bwd_dxdb        per (batch, chunk, 64-token column block s, head
//                       group): v, dx, x.v, dy.x, f2, col, the block's
//                       share of row, and dB summed over the group
//   ssd_bwd_dc          per (batch, chunk, 64-token row block l, head group):
//                       dC summed over the group, f1 per head
//   ssd_bwd_dt          per (chunk, head, batch): the prefix / suffix sums of
//                       col - row, f2 / f1 inside the chunk (fp64), da, ddt, the chunk's
//                       shares of dA, ddt_bias, dD
//   ssd_bwd_reduce      sums of the head-group partials of dB and dC, and
//                       dA, ddt_bias, dD as the sums of the chunk shares.
// Every factor e^{cs_l - cs_s} (l >= s), e^{cs_l} and e^{tot - cs_s} is at
// most 1 (A < 0), so each is evaluated directly per element.

#include "ssd_chunk_common.h"

namespace ssd {

namespace {

constexpr int kBlk = 64;  // tokens per row / column block
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte LDS row read (8 bf16): an MFMA A or B operand whose k runs along a row
__device__ __forceinline__ uint4 lds_row8(const uint16_t* tile, int pitch, int row, int col) {
  return *reinterpret_cast<const uint4*>(tile + row * pitch + col);
}

// The 8 bf16 of v times f as an unevaluated pair of bf16 vectors hi + lo
// (hi = f v rounded, lo = the rest rounded): ~2^-17 relative, so that a
// matrix product with an exact bf16 operand, taken as two products, is
// accurate to fp32 level.
__device__ __forceinline__ void split8(uint4 v, float f, uint4& hi, uint4& lo) {
  const uint32_t a[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split_bf16x2(bf16_bits_to_f32(a[j] & 0xFFFFu) * f, bf16_bits_to_f32(a[j] >> 16) * f, h[j], l[j]);
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// writes rows held in registers (a BufSlab of the same shape) into an LDS tile
template <int ROWS, int VPR>
__device__ __forceinline__ void put_rows(uint16_t* tile, int pitch, const BufSlab<ROWS, VPR, kThreads>& q) {
#pragma unroll
  for (int i = 0; i < q.PER; ++i) {
    const int it = static_cast<int>(threadIdx.x) + i * kThreads;
    if (q.ITEMS % kThreads == 0 || it < q.ITEMS)
      *reinterpret_cast<uint4*>(tile + (it / VPR) * pitch + (it % VPR) * 8) = q.v[i];
  }
}

// writes fp32 rows held in registers (a BufSlab of 4-float pieces) into two
// LDS bf16 tiles of pitch `pitch`: the leading part round(v) into `hi` and the
// remainder round(v - round(v)) into `lo`
template <int ROWS, int VPR>
__device__ __forceinline__ void put_rows_split(uint16_t* hi, uint16_t* lo, int pitch,
                                               const BufSlab<ROWS, VPR, kThreads>& q) {
#pragma unroll
  for (int i = 0; i < q.PER; ++i) {
    const int it = static_cast<int>(threadIdx.x) + i * kThreads;
    if (q.ITEMS % kThreads == 0 || it < q.ITEMS) {
      const int v = it % VPR, r = it / VPR;
      const uint4 u = q.v[i];
      uint32_t h0, l0, h1, l1;
      split_bf16x2(__uint_as_float(u.x), __uint_as_float(u.y), h0, l0);
      split_bf16x2(__uint_as_float(u.z), __uint_as_float(u.w), h1, l1);
      *reinterpret_cast<uint2*>(hi + r * pitch + v * 4) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lo + r * pitch + v * 4) = make_uint2(l0, l1);
    }
  }
}

// Per column r16, the sum of the values of the four lane groups (rows of 16
// lanes), in every lane.  The gfx950 row swaps exchange rows 2m <-> 2m+1
// (permlane16) and the wave's halves (permlane32); each returns the even
// (first) and the odd (second) side.
__device__ __forceinline__ float group_total(float a) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  const float pair = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// lane permutation inside rows of 16 by DPP (every source lane valid)
template <int CTRL>
__device__ __forceinline__ float dperm(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sixteen values per lane, summed over the 16 lanes of each lane group: lane
// r16 returns the sum of value k = r16.  Butterfly over the partners r ^ 8,
// r ^ 4, r ^ 2, r ^ 1 (row_ror:8; quad_perm [3,2,1,0] then row_half_mirror;
// quad_perm [2,3,0,1]; quad_perm [1,0,3,2]): at each step a lane keeps the
// half of its values whose index bit equals its own lane bit and adds the
// partner's copy of that half.
__device__ __forceinline__ float transpose_sum16(const float (&v)[16]) {
  const int r = threadIdx.x & 15;
  float a[8], c[4], e[2];
  const bool b3 = r & 8, b2 = r & 4, b1 = r & 2, b0 = r & 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = (b3 ? v[k + 8] : v[k]) + dperm<0x128>(b3 ? v[k] : v[k + 8]);
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = (b2 ? a[k + 4] : a[k]) + dperm<0x141>(dperm<0x1B>(b2 ? a[k] : a[k + 4]));
#pragma unroll
  for (int k = 0; k < 2; ++k) e[k] = (b1 ? c[k + 2] : c[k]) + dperm<0x4E>(b1 ? c[k] : c[k + 2]);
  return (b0 ? e[1] : e[0]) + dperm<0xB1>(b0 ? e[0] : e[1]);
}

}  // namespace

// ---------------------------------------------------------------------------
// G_c[p][n] = sum_l e^{cs_l} dy_l[p] C_l[n] (fp32), one workgroup per (batch,
// chunk, head), computed transposed (D[n][p], contraction over tokens on MFMA
// with operands from the LDS transpose read) so that a lane holds one p and
// four consecutive n.  The weighted rows e^{cs_l} dy_l are split into bf16
// hi + lo (two products with the exact bf16 C): G and the adjoint states
// built from it feed the step-size gradient, whose terms cancel (the sum of
// their magnitudes is tens of times the result), so they are kept to fp32
// accuracy.  With two n tiles per wave they go in pairs with permuted n (the
// transpose read's 4-column pieces 8 apart): 8 consecutive n, 32-byte stores.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_adj_state_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ Cm,
    const float2* __restrict__ tok, float* __restrict__ adj, int T, int H, int G, int Q, int nc,
    int npairs) {
  constexpr int YP = P + 16, CP = N + 16;
  constexpr int PT = P / 16, NT = N / 16, NTW = NT / 4;  // n tiles per wave
  constexpr bool kPairN = NTW % 2 == 0;  // wave w: n tiles NTW w + i (paired), else w, w + 4, ..
  __shared__ __attribute__((aligned(16))) uint16_t yl[kBlk * YP];  // e^{cs_l} dy_l, hi
  __shared__ __attribute__((aligned(16))) uint16_t ylo[kBlk * YP];  // and lo
  __shared__ __attribute__((aligned(16))) uint16_t cl[kBlk * CP];  // C_l
  __shared__ float wl[256];

  int b, c, h;
  if (!unit_of_block(H, nc, npairs, b, c, h)) return;
  const int g = h / (H / G);
  const int t0 = c * Q;
  const int Lc = min(Q, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  const float2* tk = tok + ((static_cast<size_t>(b) * nc + c) * H + h) * Q;
  const uint32_t yrow = static_cast<uint32_t>(H) * P * 2, crow = static_cast<uint32_t>(G) * N * 2;
  const buf_t ybuf = make_buf(dy + r0 * H * P + static_cast<size_t>(h) * P,
                              static_cast<uint32_t>(Lc - 1) * yrow + P * 2);
  const buf_t cbuf = make_buf(Cm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Lc - 1) * crow + N * 2);
  // the C and dy rows of the next block, loaded one block ahead
  BufSlab<kBlk, N / 8, kThreads> cq;
  BufSlab<kBlk, P / 8, kThreads> yq;
  cq.load(cbuf, crow, 0);
  yq.load(ybuf, yrow, 0);
  if (tid < Q) wl[tid] = tid < Lc ? __expf(tk[tid].x) : 0.0f;
  f32x4 acc[NTW][PT];
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int j = 0; j < PT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int l0 = 0; l0 < Lc; l0 += kBlk) {
    __syncthreads();  // wl written / previous block consumed
    put_rows(cl, CP, cq);
    // dy rows scaled by e^{cs_l}
#pragma unroll
    for (int i = 0; i < yq.PER; ++i) {
      const int it = tid + i * kThreads;
      if (yq.ITEMS % kThreads == 0 || it < yq.ITEMS) {
        const int v = it % (P / 8), r = it / (P / 8);
        const float w = l0 + r < Q ? wl[l0 + r] : 0.0f;
        uint4 hi, lo;
        split8(yq.v[i], w, hi, lo);
        *reinterpret_cast<uint4*>(yl + r * YP + v * 8) = hi;
        *reinterpret_cast<uint4*>(ylo + r * YP + v * 8) = lo;
      }
    }
    if (l0 + kBlk < Lc) {
      cq.load(cbuf, crow, l0 + kBlk);
      yq.load(ybuf, yrow, l0 + kBlk);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBlk; ks += 32) {
      uint4 af[NTW], bf[PT], bfl[PT];
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int nt = kPairN ? NTW * wid + i : wid + 4 * i;
        const int c0 = kPairN ? 32 * (nt >> 1) + 4 * (nt & 1) : nt * 16;
        const uint2 lo = kPairN ? lds_tr4s<8>(cl, CP, ks + 8 * q, c0) : lds_tr4(cl, CP, ks + 8 * q, c0);
        const uint2 hi = kPairN ? lds_tr4s<8>(cl, CP, ks + 8 * q + 4, c0) : lds_tr4(cl, CP, ks + 8 * q + 4, c0);
        af[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const uint2 lo = lds_tr4(yl, YP, ks + 8 * q, j * 16);
        const uint2 hi = lds_tr4(yl, YP, ks + 8 * q + 4, j * 16);
        bf[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const uint2 lo2 = lds_tr4(ylo, YP, ks + 8 * q, j * 16);
        const uint2 hi2 = lds_tr4(ylo, YP, ks + 8 * q + 4, j * 16);
        bfl[j] = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
      }
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int j = 0; j < PT; ++j) {
          acc[i][j] = mfma_bf16(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j]);
          acc[i][j] = mfma_bf16(as_bf16x8(af[i]), as_bf16x8(bfl[j]), acc[i][j]);
        }
    }
  }
  float* dst = adj + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N);
  if constexpr (kPairN) {
#pragma unroll
    for (int i = 0; i < NTW; i += 2)
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int m = (NTW * wid + i) >> 1;  // n = 32 m + 8q .. +7
        float* o = dst + (j * 16 + r16) * N + 32 * m + 8 * q;
        *reinterpret_cast<f32x4*>(o) = acc[i][j];
        *reinterpret_cast<f32x4*>(o + 4) = acc[i + 1][j];
      }
  } else {
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
      for (int j = 0; j < PT; ++j) {
        const int nt = wid + 4 * i;
        *reinterpret_cast<f32x4*>(dst + (j * 16 + r16) * N + nt * 16 + 4 * q) = acc[i][j];
      }
  }
}

// ---------------------------------------------------------------------------
// Adjoint passing, last chunk first:  R_{nc-1} = dh_final,
// R_{c-1} = lambda_c R_c + G_c,  dh0 = R_{-1}.  R_c overwrites G_c in place
// (fp32, after G_c is consumed).  One thread per 4 consecutive n; the chunks
// in groups of 8 whose loads are issued together.  Beside it, the chunk
// constants of da, e^{tot_c} <R_c, H_in(c)> (the term shared by every step of
// chunk c): each workgroup reads H_in(c) with R_c and writes its fp64 share
// of the inner product per chunk, cpart[(b, h, c) * nblk + block], which the
// step-size kernel sums and scales.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ssd_adj_pass_kernel(
    float* __restrict__ adj, const float* __restrict__ decay, const float* __restrict__ dh_final,
    float* __restrict__ dh0, const float* __restrict__ states, double* __restrict__ cpart, int H, int PN,
    int nc) {
  constexpr int PF = 8;
  __shared__ double ws[PF][kThreads / kWave];
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
  const int e4 = blockIdx.x * kThreads + tid;
  const bool in = e4 * 4 < PN;
  const int nblk = gridDim.x;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t cstride = static_cast<size_t>(H) * PN;
  const size_t off = static_cast<size_t>(b) * nc * cstride + h * static_cast<size_t>(PN) + (in ? e4 * 4 : 0);
  float* base = adj + off;
  const float* hb = states + off;
  const float* dc = decay + bh * nc;
  float4 r = in && dh_final ? *reinterpret_cast<const float4*>(dh_final + bh * PN + e4 * 4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c1 = nc; c1 > 0; c1 -= PF) {  // chunks c1-1 down to c1-PF
    float4 gv[PF], hv[PF];
    float ld[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cc = c1 - 1 - j;
      gv[j] = hv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      ld[j] = 0.0f;
      if (cc >= 0 && in) {
        gv[j] = *reinterpret_cast<const float4*>(base + cc * cstride);
        hv[j] = *reinterpret_cast<const float4*>(hb + cc * cstride);
      }
      if (cc >= 0) ld[j] = dc[cc];
    }
    double part[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cc = c1 - 1 - j;
      // R_c = r here: its share of <R_c, H_in(c)>, then the update
      part[j] = static_cast<double>(r.x * hv[j].x + r.y * hv[j].y) +
                static_cast<double>(r.z * hv[j].z + r.w * hv[j].w);
      if (cc >= 0) {
        if (in) *reinterpret_cast<float4*>(base + cc * cstride) = r;
        const float l = ld[j];
        r = make_float4(l * r.x + gv[j].x, l * r.y + gv[j].y, l * r.z + gv[j].z, l * r.w + gv[j].w);
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      double v = part[j];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
      if (lane == 0) ws[j][wid] = v;
    }
    __syncthreads();
    if (tid < PF && c1 - 1 - tid >= 0)
      cpart[(bh * nc + (c1 - 1 - tid)) * nblk + blockIdx.x] = (ws[tid][0] + ws[tid][1]) + (ws[tid][2] + ws[tid][3]);
    __syncthreads();  // (ws is rewritten by the next group of chunks)
  }
  if (in && dh0) *reinterpret_cast<float4*>(dh0 + bh * PN + e4 * 4) = r;
}

// Work unit of the two block kernels: (b, chunk, 64-token block, head group).
// A unit's work grows with its block's distance from the chunk's end (column
// blocks) or start (row blocks), so the workgroups go out heaviest block
// first (the longest-first order keeps the tail short); inside one block
// rank, the XCD-grouped order of the forward (the head groups of one (b,
// chunk, block) share an XCD and its L2, which serves their common B and C
// rows).  `units_per_rank` workgroups per block rank.
struct BlockUnit {
  int b, c, blk, hg;
};
__host__ __device__ inline int units_per_rank(int ngroups, int nc, int Bsz) {
  return (Bsz * nc + kXCD - 1) / kXCD * kXCD * ngroups;
}
__device__ __forceinline__ bool block_unit(int ngroups, int nc, int nb, int Bsz, bool heavy_last_block,
                                           BlockUnit& u) {
  const int per = units_per_rank(ngroups, nc, Bsz);
  const int rank = static_cast<int>(blockIdx.x) / per;
  int b, c, hg;
  if (rank >= nb || !unit_coords(static_cast<int>(blockIdx.x) % per, ngroups, nc, Bsz * nc, b, c, hg))
    return false;
  u.b = b;
  u.c = c;
  u.blk = heavy_last_block ? nb - 1 - rank : rank;
  u.hg = hg;
  return true;
}

// ---------------------------------------------------------------------------
// Column blocks: per (batch, chunk, block j of source tokens s, group of HPG
// heads of one B/C group).  Wave w owns the 16 tokens s of tile w of the block
// and, per head, accumulates
//   v[s][p]  = e^{tot-cs_s} (B_s . R_c[p]) + sum_{l >= s} M[l][s] dy_l[p]
//   dB[s][n] += delta_s e^{tot-cs_s} (x_s R_c)[n] + sum_{l >= s} W[l][s] C_l[n]
// with M[l][s] = e^{cs_l-cs_s} (C_l.B_s) and W[l][s] = e^{cs_l-cs_s} delta_s
// (dy_l.x_s) for l >= s.  The rows l run over 64-token blocks, last first
// (the diagonal block last, so that its dy rows are in LDS for dx); C_l.B_s
// and dy_l.x_s are MFMA tiles whose lane holds one s and four l, which after
// the mask and decay are the B operands (columns s, contraction over l) of the
// transposed products v^T += dy^T M and dB^T += C^T W, whose A operands (dy and
// C) come from LDS by the transpose read: a lane ends with one s of v and dB
// and runs of consecutive p or n (16-byte stores of dx and the dB partials).
// v feeds x.v and f2, which enter the step-size gradient where its terms cancel,
// so its products are fp32-accurate: R_c (fp32) is staged as bf16 hi + lo and
// M as hi + lo, each product taken twice; W (which only reaches dB) is one bf16
// operand.  The same
// fp32 tiles give the box terms E[l][s] (l > s): each lane sums its column
// over the l blocks (col_s, once per head), and a transposing reduction over
// the 16 columns of each lane group gives the rows' sums (the block's share of
// row_l).  Blocks off the diagonal and inside the chunk need no mask.  Per
// head: dx (bf16), x.v, dy.x, f2, col and the row shares; after the group: dB.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_bwd_dxdb_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dy, const float* __restrict__ D, const float2* __restrict__ tok,
    const float* __restrict__ adj, uint16_t* __restrict__ dx, float* __restrict__ xv,
    float* __restrict__ dyx, float* __restrict__ f2o, float* __restrict__ colp,
    float* __restrict__ rowp, float* __restrict__ dBp, int Bsz, int T, int H, int G, int Q, int nc,
    int HPG) {
  constexpr int XP = P + 16, NP = N + 16;
  constexpr int PT = P / 16, NT = N / 16;
  static_assert(P % 32 == 0, "v tiles go in pairs of 16 p");
  static_assert(P <= kBlk, "R_c's lo part is staged in the C tile");
  // C rows of the l block; before the l blocks of a head, the lo part of R_c
  __shared__ __attribute__((aligned(16))) uint16_t Cs[kBlk * NP];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kBlk * XP];  // dy rows of the l block
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBlk * NP];  // B rows of the s block
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kBlk * XP];  // x rows of the s block
  __shared__ __attribute__((aligned(16))) uint16_t Rs[P * NP];     // R_c of the head, hi part
  __shared__ __attribute__((aligned(16))) float cs2[256];  // cs_l log2(e) of the chunk's tokens
  __shared__ float dlt[256];                               // delta_l
  __shared__ float rows[2][4][kBlk];  // per l-block parity and wave: row share of each row l
  __shared__ float dsh;                // D of the head

  const int nb = (Q + kBlk - 1) / kBlk;
  const int hpg = H / G;
  BlockUnit u;
  if (!block_unit(H / HPG, nc, nb, Bsz, false, u)) return;  // column block 0 carries the most rows
  const int b = u.b, c = u.c, j = u.blk;
  const size_t BTH = static_cast<size_t>(Bsz) * T * H;
  const int h0 = u.hg * HPG, g = h0 / hpg, hgl = (h0 % hpg) / HPG;
  const int t0 = c * Q, Lc = min(Q, T - t0), s0 = j * kBlk;
  if (s0 >= Lc) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int w = wave_id();
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  // per-token values for the step-size kernel: token-contiguous per (batch, head)
  auto head_row = [&](int hh) { return (static_cast<size_t>(b) * H + hh) * T + t0; };
  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2, brow = static_cast<uint32_t>(G) * N * 2;
  const buf_t bbuf = make_buf(Bm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Lc - 1) * brow + N * 2);
  const buf_t cbuf = make_buf(Cm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Lc - 1) * brow + N * 2);
  const int nlb = (Lc - s0 + kBlk - 1) / kBlk;
  auto rows_of = [&](const uint16_t* base, int hh) {
    return make_buf(base + r0 * H * P + static_cast<size_t>(hh) * P, static_cast<uint32_t>(Lc - 1) * xrow + P * 2);
  };
  // Each step's tiles pass through registers: all of its loads are issued
  // before the barrier that frees their LDS tiles, and stored after it.
  // (Loading them one step ahead instead costs the 36 registers that keep a
  // second wave on each SIMD: 150 against 95 us at the BitMamba shape.)
  BufSlab<kBlk, P / 8, kThreads> xq;
  BufSlab<P, N / 4, kThreads> rq;
  BufSlab<kBlk, N / 8, kThreads> cq;
  BufSlab<kBlk, P / 8, kThreads> yq;
  float2 tq = make_float2(0.f, 0.f);
  float dq = 0.0f;
  auto load_head = [&](int hh) {
    xq.load(rows_of(x, hh), xrow, s0);
    rq.load(make_buf(adj + ((static_cast<size_t>(b) * nc + c) * H + hh) * (static_cast<size_t>(P) * N),
                     static_cast<uint32_t>(P) * N * 4),
            N * 4, 0);
    if (tid < Q) tq = tok[((static_cast<size_t>(b) * nc + c) * H + hh) * Q + tid];
    if (D != nullptr && tid == 0) dq = D[hh];
  };
  auto load_lblock = [&](int hh, int lb) {
    cq.load(cbuf, brow, s0 + lb * kBlk);
    yq.load(rows_of(dy, hh), xrow, s0 + lb * kBlk);
  };
  {
    BufSlab<kBlk, N / 8, kThreads> bq;
    bq.load(bbuf, brow, s0);
    put_rows(Bs, NP, bq);
  }

  f32x4 dB[NT];  // dB^T[n][s]: lane holds column s = sl, rows n = 16 nt + 4q + i
#pragma unroll
  for (int i = 0; i < NT; ++i) dB[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sl = s0 + 16 * w + r16;  // this lane's source token (score, v^T and dB^T columns)

  for (int e = 0; e < HPG; ++e) {
    const int h = h0 + e;
    load_head(h);
    __syncthreads();  // previous head done with Xs, Rs, cs2, dlt, Ys, Cs
    put_rows(Xs, XP, xq);
    put_rows_split(Rs, Cs, NP, rq);
    if (tid < Q) {
      cs2[tid] = tq.x * kLog2e;
      dlt[tid] = tq.y;
    }
    if (tid == 0) dsh = dq;
    __syncthreads();
    // every decay factor below is 2^(cs2_l - cs2_s) <= 1 (l >= s)
    const float tot = cs2[Q - 1];
    const float cs_s = cs2[sl], dl_s = dlt[sl];

    // v transposed, v^T[p][s]: a lane holds column s = sl and, per tile pt, the
    // rows p = vp(pt, 4q + i).  The tiles go in pairs with permuted p (the pair
    // hh covers p = 32 hh .. 32 hh + 31; MFMA row r of its tile (hh, half) is
    // p = 32 hh + 4 half + 8 (r / 4) + r % 4), so that a lane's rows of a pair
    // are the 8 consecutive p = 32 hh + 8q .. +7: 16-byte accesses of dx, x, dy.
    auto vp = [](int pt, int r) { return 32 * (pt >> 1) + 4 * (pt & 1) + 8 * (r >> 2) + (r & 3); };
    const int sr = 16 * w + r16;  // this lane's row s within the block
    // boundary part: e^{tot-cs_s} R_c[p] . B_s
    f32x4 v[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) v[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N; ks += 32) {
      const uint4 bb = lds_row8(Bs, NP, sr, ks + 8 * q);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) {
        v[pt] = mfma_bf16(as_bf16x8(lds_row8(Rs, NP, vp(pt, r16), ks + 8 * q)), as_bf16x8(bb), v[pt]);
        v[pt] = mfma_bf16(as_bf16x8(lds_row8(Cs, NP, vp(pt, r16), ks + 8 * q)), as_bf16x8(bb), v[pt]);
      }
    }
    {
      const float fr = __builtin_amdgcn_exp2f(tot - cs_s);
#pragma unroll
      for (int pt = 0; pt < PT; ++pt) v[pt] = v[pt] * fr;
    }
    // x_s . v_s over this lane's 8 p of pair hh (x . the R part of v: f2; later x . v)
    auto xdot = [&](const uint16_t* rowp) {
      float part = 0.0f;
#pragma unroll
      for (int hh = 0; hh < PT / 2; ++hh) {
        const uint4 u = *reinterpret_cast<const uint4*>(rowp + hh * 32 + 8 * q);
        const uint32_t xw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part += bf16_bits_to_f32((e & 1) ? (xw[e >> 1] >> 16) : (xw[e >> 1] & 0xFFFFu)) *
                  v[2 * hh + (e >> 2)][e & 3];
      }
      return part;
    };
    // f2_s = delta_s x_s . (e^{tot-cs_s} R_c B_s): the R part of x.v, before the rest
    {
      const float part = group_total(xdot(Xs + sr * XP));
      if (q == 0 && sl < Lc) f2o[head_row(h) + sl] = dl_s * part;
    }
    // boundary part of dB: delta_s e^{tot-cs_s} (x_s R)[n] (B columns s = this lane's sl),
    // x_s R from the exact x rows and both parts of R, scaled in fp32
    {
      f32x4 xr[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) xr[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < P; ks += 32) {
        const uint4 a = lds_row8(Xs, XP, 16 * w + r16, ks + 8 * q);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 lo = lds_tr4(Rs, NP, ks + 8 * q, nt * 16);
          const uint2 hi = lds_tr4(Rs, NP, ks + 8 * q + 4, nt * 16);
          xr[nt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(a), xr[nt]);
          const uint2 lo2 = lds_tr4(Cs, NP, ks + 8 * q, nt * 16);
          const uint2 hi2 = lds_tr4(Cs, NP, ks + 8 * q + 4, nt * 16);
          xr[nt] = mfma_bf16(as_bf16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y)), as_bf16x8(a), xr[nt]);
        }
      }
      const float f2 = dl_s * __builtin_amdgcn_exp2f(tot - cs_s);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) dB[nt] += xr[nt] * f2;
    }

    float col = 0.0f;  // this lane's rows of sum_{l > s} E[l][s], column s = sl
    // the four waves' shares of row_l of l block lb, summed into the block's
    // share (once every wave has written rows[lb & 1], i.e. after the next barrier)
    auto flush_rows = [&](int lb) {
      const int l0 = s0 + lb * kBlk;
      const float(*rw)[kBlk] = rows[lb & 1];
      if (tid < kBlk && l0 + tid < Lc)
        rowp[static_cast<size_t>(j) * BTH + head_row(h) + l0 + tid] = rw[0][tid] + rw[1][tid] + rw[2][tid] + rw[3][tid];
    };
    for (int lb = nlb - 1; lb >= 0; --lb) {
      const int l0 = s0 + lb * kBlk;
      load_lblock(h, lb);
      __syncthreads();
      put_rows(Cs, NP, cq);
      put_rows(Ys, XP, yq);
      // (after the waits for this block's rows: a store before them would be waited for too)
      if (lb + 1 < nlb) flush_rows(lb + 1);
      __syncthreads();
      // score tiles of this wave's 16 columns s: lane holds s = sl, l = l0 + 16 lt + 4q + i
      f32x4 s1[4], s2[4];
#pragma unroll
      for (int lt = 0; lt < 4; ++lt) {
        s1[lt] = f32x4{0.f, 0.f, 0.f, 0.f};
        s2[lt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < N; ks += 32) {
        const uint4 bb = lds_row8(Bs, NP, 16 * w + r16, ks + 8 * q);
#pragma unroll
        for (int lt = 0; lt < 4; ++lt)
          s1[lt] = mfma_bf16(as_bf16x8(lds_row8(Cs, NP, lt * 16 + r16, ks + 8 * q)), as_bf16x8(bb), s1[lt]);
      }
#pragma unroll
      for (int ks = 0; ks < P; ks += 32) {
        const uint4 xx = lds_row8(Xs, XP, 16 * w + r16, ks + 8 * q);
#pragma unroll
        for (int lt = 0; lt < 4; ++lt)
          s2[lt] = mfma_bf16(as_bf16x8(lds_row8(Ys, XP, lt * 16 + r16, ks + 8 * q)), as_bf16x8(xx), s2[lt]);
      }
      // mask and decay -> bf16 A operands (k slot of lane group q: l = 16 lt + 4q + i)
      // and the fp32 box terms E[l][s] (l > s only)
      uint32_t am[4][2], aml[4][2], aw[4][2];
      float ee[16];
      auto decay = [&](auto masked) {
#pragma unroll
        for (int lt = 0; lt < 4; ++lt) {
          const int lb4 = l0 + 16 * lt + 4 * q;
          float mv[4], wv[4];
          if constexpr (decltype(masked)::value) {
            // lb4 + 3 < 256: in the table; entries past the chunk are selected away
            const float4 c4 = *reinterpret_cast<const float4*>(cs2 + lb4);
            const float cl[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int l = lb4 + i;
              const bool ok = l >= sl && l < Lc;
              const float d = ok ? __builtin_amdgcn_exp2f(cl[i] - cs_s) : 0.0f;
              mv[i] = d * s1[lt][i];
              wv[i] = d * dl_s * s2[lt][i];
              ee[4 * lt + i] = l > sl ? wv[i] * s1[lt][i] : 0.0f;
            }
          } else {
            const float4 c4 = *reinterpret_cast<const float4*>(cs2 + lb4);
            const float cl[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float d = __builtin_amdgcn_exp2f(cl[i] - cs_s);
              mv[i] = d * s1[lt][i];
              wv[i] = d * dl_s * s2[lt][i];
              ee[4 * lt + i] = wv[i] * s1[lt][i];
            }
          }
          split_bf16x2(mv[0], mv[1], am[lt][0], aml[lt][0]);
          split_bf16x2(mv[2], mv[3], am[lt][1], aml[lt][1]);
          aw[lt][0] = pack_bf16x2(wv[0], wv[1]);
          aw[lt][1] = pack_bf16x2(wv[2], wv[3]);
        }
      };
      // off the diagonal block (every l > every s) and inside the chunk: no mask
      if (lb > 0 && l0 + kBlk <= Lc)
        decay(std::false_type{});
      else
        decay(std::true_type{});
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 Am = make_uint4(am[2 * kk][0], am[2 * kk][1], am[2 * kk + 1][0], am[2 * kk + 1][1]);
        const uint4 Aml = make_uint4(aml[2 * kk][0], aml[2 * kk][1], aml[2 * kk + 1][0], aml[2 * kk + 1][1]);
        const uint4 Aw = make_uint4(aw[2 * kk][0], aw[2 * kk][1], aw[2 * kk + 1][0], aw[2 * kk + 1][1]);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
          const int c0 = 32 * (pt >> 1) + 4 * (pt & 1);
          const uint2 lo = lds_tr4s<8>(Ys, XP, 32 * kk + 4 * q, c0);
          const uint2 hi = lds_tr4s<8>(Ys, XP, 32 * kk + 16 + 4 * q, c0);
          const bf16x8 yt = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          v[pt] = mfma_bf16(yt, as_bf16x8(Am), v[pt]);
          v[pt] = mfma_bf16(yt, as_bf16x8(Aml), v[pt]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 lo = lds_tr4(Cs, NP, 32 * kk + 4 * q, nt * 16);
          const uint2 hi = lds_tr4(Cs, NP, 32 * kk + 16 + 4 * q, nt * 16);
          dB[nt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(Aw), dB[nt]);
        }
      }
      // column sums (per lane) and the rows' sums over the 16 columns of the
      // lane group: lane r16 gets value 4 lt + i = r16, i.e. row 16 (r16 / 4) + 4q + r16 % 4
      {
        float cp[4];
#pragma unroll
        for (int lt = 0; lt < 4; ++lt) cp[lt] = (ee[4 * lt] + ee[4 * lt + 1]) + (ee[4 * lt + 2] + ee[4 * lt + 3]);
        col += (cp[0] + cp[1]) + (cp[2] + cp[3]);
      }
      rows[lb & 1][w][16 * (r16 >> 2) + 4 * q + (r16 & 3)] = transpose_sum16(ee);
    }
    __syncthreads();
    flush_rows(0);
    {
      const float ct = group_total(col);
      if (q == 0 && sl < Lc) colp[head_row(h) + sl] = ct;
    }

    // outputs of head h: lane holds row s = sl, p = 32 hh + 8q .. +7 of each pair;
    // Ys now holds the dy rows of the s block (the last l block was the diagonal)
    const float Dh = dsh;  // (the D load went with the head's other loads)
    const buf_t dxbuf = make_buf(dx + r0 * H * P + static_cast<size_t>(h) * P,
                                 static_cast<uint32_t>(Lc - 1) * xrow + P * 2);
    {
      float pxv = 0.0f, pdx = 0.0f;
#pragma unroll
      for (int hh = 0; hh < PT / 2; ++hh) {
        const uint4 ux = *reinterpret_cast<const uint4*>(Xs + sr * XP + hh * 32 + 8 * q);
        const uint4 uy = *reinterpret_cast<const uint4*>(Ys + sr * XP + hh * 32 + 8 * q);
        const uint32_t xw[4] = {ux.x, ux.y, ux.z, ux.w}, yw[4] = {uy.x, uy.y, uy.z, uy.w};
        float gx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xe = bf16_bits_to_f32((e & 1) ? (xw[e >> 1] >> 16) : (xw[e >> 1] & 0xFFFFu));
          const float ye = bf16_bits_to_f32((e & 1) ? (yw[e >> 1] >> 16) : (yw[e >> 1] & 0xFFFFu));
          const float ve = v[2 * hh + (e >> 2)][e & 3];
          pxv += xe * ve;
          pdx += xe * ye;
          gx[e] = dl_s * ve + Dh * ye;
        }
        buf_store16(dxbuf, static_cast<uint32_t>(sl) * xrow + (hh * 32 + 8 * q) * 2,
                    make_uint4(pack_bf16x2(gx[0], gx[1]), pack_bf16x2(gx[2], gx[3]),
                               pack_bf16x2(gx[4], gx[5]), pack_bf16x2(gx[6], gx[7])));
      }
      pxv = group_total(pxv);
      pdx = group_total(pdx);
      if (q == 0 && sl < Lc) {
        xv[head_row(h) + sl] = pxv;
        dyx[head_row(h) + sl] = pdx;
      }
    }
  }

  // dB of the head group, computed transposed: lane holds row s = sl and
  // n = 16 nt + 4q .. +3 (one 16-byte store per tile)
  float* dst = dBp + ((static_cast<size_t>(hgl) * Bsz + b) * T + t0) * G * N + static_cast<size_t>(g) * N;
  if (sl < Lc) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(dst + static_cast<size_t>(sl) * G * N + nt * 16 + 4 * q) = dB[nt];
  }
}

// ---------------------------------------------------------------------------
// Row blocks: per (batch, chunk, block i of target tokens l, group of HPG
// heads).  Wave w owns the 16 tokens l of tile w and, per head, accumulates
//   dC_h[l][n] = e^{cs_l} (dy_l H_in)[n] + sum_{s <= l} W[l][s] B_s[n],
//   W[l][s] = e^{cs_l - cs_s} delta_s (dy_l . x_s),
// the scores computed transposed (x_s . dy_l: a lane holds one l and four s),
// which after the decay are the B operand of dC^T += B^T W^T, so that a lane
// ends with one row l of dC and 4 consecutive n per tile (16-byte stores).
// Per head: f1_l = C_l . (the H_in part of dC_h[l]); after the group: dC.
// f1 enters the step-size gradient where its terms cancel, so the H_in part
// is fp32-accurate: H_in (fp32) is staged as bf16 hi + lo, multiplied by the
// exact dy rows, and the product scaled by e^{cs_l} in fp32.
// ---------------------------------------------------------------------------
template <int P, int N>
__global__ __launch_bounds__(kThreads) void ssd_bwd_dc_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dy, const float2* __restrict__ tok,
    const float* __restrict__ states, float* __restrict__ f1o, float* __restrict__ dCp, int Bsz,
    int T, int H, int G, int Q, int nc, int HPG) {
  constexpr int XP = P + 16, NP = N + 16;
  constexpr int NT = N / 16;
  static_assert(P <= kBlk, "h_in's lo part is staged in the B tile");
  __shared__ __attribute__((aligned(16))) uint16_t Xs[kBlk * XP];  // x rows of the s block
  // B rows of the s block; before the s blocks of a head, the lo part of h_in(c)
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBlk * NP];
  __shared__ __attribute__((aligned(16))) uint16_t Ys[kBlk * XP];  // dy rows of the l block
  __shared__ __attribute__((aligned(16))) uint16_t Hs[P * NP];     // h_in(c) of the head, hi part
  __shared__ __attribute__((aligned(16))) uint16_t Cs[kBlk * NP];  // C rows of the l block
  __shared__ __attribute__((aligned(16))) float cs2[256];  // cs_s log2(e) of the chunk's tokens
  __shared__ __attribute__((aligned(16))) float dlt[256];  // delta_s

  const int nb = (Q + kBlk - 1) / kBlk;
  const int hpg = H / G;
  BlockUnit u;
  if (!block_unit(H / HPG, nc, nb, Bsz, true, u)) return;  // the last row block carries the most columns
  const int b = u.b, c = u.c, ib = u.blk;
  const int h0 = u.hg * HPG, g = h0 / hpg, hgl = (h0 % hpg) / HPG;
  const int t0 = c * Q, Lc = min(Q, T - t0), l0 = ib * kBlk;
  if (l0 >= Lc) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int w = wave_id();
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  // per-token values for the step-size kernel: token-contiguous per (batch, head)
  auto head_row = [&](int hh) { return (static_cast<size_t>(b) * H + hh) * T + t0; };
  const uint32_t xrow = static_cast<uint32_t>(H) * P * 2, brow = static_cast<uint32_t>(G) * N * 2;
  const buf_t bbuf = make_buf(Bm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Lc - 1) * brow + N * 2);
  const buf_t cbuf = make_buf(Cm + r0 * G * N + static_cast<size_t>(g) * N,
                              static_cast<uint32_t>(Lc - 1) * brow + N * 2);

  f32x4 dCg[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) dCg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ll = l0 + 16 * w + r16;  // this lane's target token (score and dC^T columns)
  auto xbufh = [&](int hh) {
    return make_buf(x + r0 * H * P + static_cast<size_t>(hh) * P,
                    static_cast<uint32_t>(Lc - 1) * xrow + P * 2);
  };
  // the x and B rows of the next s block, loaded one block ahead (the last
  // block of a head loads the first block of the next head)
  BufSlab<kBlk, P / 8, kThreads> xq;
  BufSlab<kBlk, N / 8, kThreads> bq;
  xq.load(xbufh(h0), xrow, 0);
  bq.load(bbuf, brow, 0);
  {
    BufSlab<kBlk, N / 8, kThreads> cq;
    cq.load(cbuf, brow, l0);
    put_rows(Cs, NP, cq);
  }

  for (int e = 0; e < HPG; ++e) {
    const int h = h0 + e;
    {
      // the head's dy rows, h_in(c) and token table: every load issued before
      // the barrier that frees their tiles
      BufSlab<kBlk, P / 8, kThreads> yq;
      BufSlab<P, N / 4, kThreads> hq;
      float2 t2 = make_float2(0.f, 0.f);
      if (tid < Q) t2 = tok[((static_cast<size_t>(b) * nc + c) * H + h) * Q + tid];
      yq.load(make_buf(dy + r0 * H * P + static_cast<size_t>(h) * P, static_cast<uint32_t>(Lc - 1) * xrow + P * 2),
              xrow, l0);
      hq.load(make_buf(states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * N),
                       static_cast<uint32_t>(P) * N * 4),
              N * 4, 0);
      __syncthreads();
      put_rows(Ys, XP, yq);
      put_rows_split(Hs, Bs, NP, hq);
      if (tid < Q) {
        cs2[tid] = t2.x * kLog2e;
        dlt[tid] = t2.y;
      }
    }
    __syncthreads();
    // every decay factor below is 2^(cs2_l - cs2_s) <= 1 (s <= l)
    const float cs_l = cs2[ll < Lc ? ll : Lc - 1];

    // dC_h computed transposed, dC^T[n][l]: lane holds column l = ll, rows
    // n = 16 nt + 4q + i.  Boundary: e^{cs_l} (dy_l H_in)[n] (B columns l = ll)
    f32x4 dC[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dC[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int ks = 0; ks < P; ks += 32) {
        const uint4 a = lds_row8(Ys, XP, 16 * w + r16, ks + 8 * q);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 lo = lds_tr4(Hs, NP, ks + 8 * q, nt * 16);
          const uint2 hi = lds_tr4(Hs, NP, ks + 8 * q + 4, nt * 16);
          dC[nt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(a), dC[nt]);
          const uint2 lo2 = lds_tr4(Bs, NP, ks + 8 * q, nt * 16);
          const uint2 hi2 = lds_tr4(Bs, NP, ks + 8 * q + 4, nt * 16);
          dC[nt] = mfma_bf16(as_bf16x8(make_uint4(lo2.x, lo2.y, hi2.x, hi2.y)), as_bf16x8(a), dC[nt]);
        }
      }
      const float f = __builtin_amdgcn_exp2f(cs_l);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) dC[nt] = dC[nt] * f;
    }
    // f1_l = e^{cs_l} C_l . (H_in^T dy_l): the H_in part of C_l . dC_h[l]
    {
      float pd = 0.0f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint2 cc = *reinterpret_cast<const uint2*>(Cs + (16 * w + r16) * NP + nt * 16 + 4 * q);
        pd += bf16_bits_to_f32(cc.x & 0xFFFFu) * dC[nt][0] + bf16_bits_to_f32(cc.x >> 16) * dC[nt][1] +
              bf16_bits_to_f32(cc.y & 0xFFFFu) * dC[nt][2] + bf16_bits_to_f32(cc.y >> 16) * dC[nt][3];
      }
      pd = group_total(pd);
      if (q == 0 && ll < Lc) f1o[head_row(h) + ll] = pd;
    }
    for (int sb = 0; sb <= ib; ++sb) {
      const int s0 = sb * kBlk;
      __syncthreads();
      put_rows(Xs, XP, xq);
      put_rows(Bs, NP, bq);
      if (sb < ib) {
        xq.load(xbufh(h), xrow, s0 + kBlk);
        bq.load(bbuf, brow, s0 + kBlk);
      } else if (e + 1 < HPG) {
        xq.load(xbufh(h + 1), xrow, 0);
        bq.load(bbuf, brow, 0);
      }
      __syncthreads();
      // transposed scores: lane holds l = ll, s = s0 + 16 st + 4q + i
      f32x4 st2[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) st2[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < P; ks += 32) {
        const uint4 yy = lds_row8(Ys, XP, 16 * w + r16, ks + 8 * q);
#pragma unroll
        for (int st = 0; st < 4; ++st)
          st2[st] = mfma_bf16(as_bf16x8(lds_row8(Xs, XP, st * 16 + r16, ks + 8 * q)), as_bf16x8(yy), st2[st]);
      }
      uint32_t aw[4][2];
      auto decay = [&](auto masked) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const int sb4 = s0 + 16 * st + 4 * q;
          const float4 c4 = *reinterpret_cast<const float4*>(cs2 + sb4);
          const float4 d4 = *reinterpret_cast<const float4*>(dlt + sb4);
          const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
          float wv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = __builtin_amdgcn_exp2f(cs_l - cv[i]) * dv[i] * st2[st][i];
            if constexpr (decltype(masked)::value) {
              const int s = sb4 + i;
              wv[i] = (ll >= s && ll < Lc && s < Lc) ? v : 0.0f;
            } else {
              wv[i] = v;
            }
          }
          aw[st][0] = pack_bf16x2(wv[0], wv[1]);
          aw[st][1] = pack_bf16x2(wv[2], wv[3]);
        }
      };
      // blocks below the diagonal: every s < every l, no mask (rows l past
      // the chunk's end hold zero dy, so their scores are zero, and are not stored)
      if (sb < ib)
        decay(std::false_type{});
      else
        decay(std::true_type{});
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 Aw = make_uint4(aw[2 * kk][0], aw[2 * kk][1], aw[2 * kk + 1][0], aw[2 * kk + 1][1]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 lo = lds_tr4(Bs, NP, 32 * kk + 4 * q, nt * 16);
          const uint2 hi = lds_tr4(Bs, NP, 32 * kk + 16 + 4 * q, nt * 16);
          dC[nt] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), as_bf16x8(Aw), dC[nt]);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dCg[nt][i] += dC[nt][i];
  }

  // lane holds row l = ll, n = 16 nt + 4q .. +3: one 16-byte store per tile
  float* dst = dCp + ((static_cast<size_t>(hgl) * Bsz + b) * T + t0) * G * N + static_cast<size_t>(g) * N;
  if (ll < Lc) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(dst + static_cast<size_t>(ll) * G * N + nt * 16 + 4 * q) = dCg[nt];
  }
}

// ---------------------------------------------------------------------------
// Step-size gradients, one workgroup per (chunk, head, batch), thread l =
// token l of the chunk:
//   da_l = box_l + sum_{l' >= l} f1_l' + sum_{s < l} f2_s + e^{tot} <R_c, H_in>,
//   box_l = sum_{u < l} (col_u - row_u)
// (fp64 block scans: f1 summed from the chunk's end, f2 and col - row from its
// start; row_u is the sum of the column blocks' shares), then
// ddelta_l = A da_l + x_l.v_l, ddt_l = ddelta_l sigmoid(z_l) [lo <= sp <= hi];
// the chunk's shares of dA, ddt_bias and dD go to `part` (fp64).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ssd_bwd_dt_kernel(
    const float* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ dt_bias,
    float dt_min, float dt_max, const float* __restrict__ f1, const float* __restrict__ f2,
    const float* __restrict__ colp, const float* __restrict__ rowp, const float* __restrict__ xv,
    const float* __restrict__ dyx, const double* __restrict__ cpart, const float* __restrict__ decay,
    int nblk, float* __restrict__ ddt, double* __restrict__ part, int Bsz, int T, int H, int Q, int nc) {
  __shared__ double wsum[3][4];
  __shared__ double red[3][4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid / kWave;
  const float a_re = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const size_t BTH = static_cast<size_t>(Bsz) * T * H;
  const size_t bhc = (static_cast<size_t>(b) * H + h) * nc + c;
  // the chunk constant e^{tot_c} <R_c, H_in(c)>: the adjoint passing's shares
  double cst = 0.0;
  for (int k = 0; k < nblk; ++k) cst += cpart[bhc * nblk + k];
  cst *= static_cast<double>(decay[bhc]);
  const int t = c * Q + tid;
  const bool in = tid < Q && t < T;
  const size_t row = (static_cast<size_t>(b) * T + (in ? t : 0)) * H + h;  // dt, ddt: (B, T, H)
  // the kernels' per-token values: token-contiguous per (batch, head)
  const size_t hrow = (static_cast<size_t>(b) * H + h) * T + (in ? t : 0);
  const double f1v = in ? static_cast<double>(f1[hrow]) : 0.0;
  const double f2v = in ? static_cast<double>(f2[hrow]) : 0.0;
  double gv = 0.0;  // col_u - row_u of this token
  if (in) {
    // the shares of the column blocks jb <= this token's block (at most 4:
    // Q <= 256), all loads issued together
    float rs[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) rs[jb] = jb <= tid / kBlk ? rowp[static_cast<size_t>(jb) * BTH + hrow] : 0.0f;
    gv = static_cast<double>(colp[hrow]);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) gv -= rs[jb];
  }
  // one fp64 block scan of (f1, f2, col - row): DPP wave scans, then the
  // preceding waves' totals; f1's suffix is its total less the prefix before l
  double sc[3] = {f1v, f2v, gv};
#pragma unroll
  for (int k = 0; k < 3; ++k) sc[k] = wave_inclusive_sum_d(sc[k]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int k = 0; k < 3; ++k) wsum[k][wid] = sc[k];
  }
  __syncthreads();
  double before[3] = {0.0, 0.0, 0.0};
  for (int w = 0; w < wid; ++w) {
#pragma unroll
    for (int k = 0; k < 3; ++k) before[k] += wsum[k][w];
  }
  const double f1_total = (wsum[0][0] + wsum[0][1]) + (wsum[0][2] + wsum[0][3]);
  const double f1_suffix = f1_total - (sc[0] + before[0]) + f1v;
  const double f2_prefix = sc[1] + before[1] - f2v;
  const double box = sc[2] + before[2] - gv;
  double sA = 0.0, sBias = 0.0, sD = 0.0;
  if (in) {
    const double da = box + f1_suffix + f2_prefix + cst;
    const float z = dt[row] + bias;
    const float d = step_size(dt[row], bias, dt_min, dt_max);
    const float xvt = xv[hrow];
    const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
    const bool pass = sp >= dt_min && sp <= dt_max;
    const double dd = static_cast<double>(a_re) * da + xvt;
    const double gz = pass ? dd / (1.0 + exp(-static_cast<double>(z))) : 0.0;
    ddt[row] = static_cast<float>(gz);
    sA = static_cast<double>(d) * da;
    sBias = gz;
    sD = dyx[hrow];
  }
  // wave sums by DPP scans (the total lands in the last lane)
  sA = wave_inclusive_sum_d(sA);
  sBias = wave_inclusive_sum_d(sBias);
  sD = wave_inclusive_sum_d(sD);
  if (lane == kWave - 1) {
    red[0][wid] = sA;
    red[1][wid] = sBias;
    red[2][wid] = sD;
  }
  __syncthreads();
  if (tid < 3) part[bhc * 3 + tid] = red[tid][0] + red[tid][1] + red[tid][2] + red[tid][3];
}

// The sums after the step-size kernel, one launch: blockIdx.y 0 and 1, dB and
// dC as the sums of their nparts head-group partials, float4 at a time; 2, per
// head, dA, ddt_bias and dD as the sums of the chunk shares over batch and
// chunks (fp64)
__global__ __launch_bounds__(kThreads) void ssd_bwd_reduce_kernel(
    const float* __restrict__ partB, float* __restrict__ outB, const float* __restrict__ partC,
    float* __restrict__ outC, size_t n4, int nparts, const double* __restrict__ dtp,
    float* __restrict__ dA, float* __restrict__ ddt_bias, float* __restrict__ dD, int Bsz, int H,
    int nc) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (blockIdx.y == 2) {
    if (i >= static_cast<size_t>(H)) return;
    double s[3] = {0.0, 0.0, 0.0};
    for (int b = 0; b < Bsz; ++b)
      for (int c = 0; c < nc; ++c)
#pragma unroll
        for (int k = 0; k < 3; ++k) s[k] += dtp[(((static_cast<size_t>(b) * H + i) * nc + c) * 3) + k];
    dA[i] = static_cast<float>(s[0]);
    ddt_bias[i] = static_cast<float>(s[1]);
    dD[i] = static_cast<float>(s[2]);
    return;
  }
  if (i >= n4) return;
  const float* part = blockIdx.y == 0 ? partB : partC;
  float* out = blockIdx.y == 0 ? outB : outC;
  const float4* p = reinterpret_cast<const float4*>(part);
  float4 s = p[i];
  for (int k = 1; k < nparts; ++k) {
    const float4 v = p[i + k * n4];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  reinterpret_cast<float4*>(out)[i] = s;
}

// An event slot with no kernel of its own: its pair recorded back to back.
inline void empty_slot(hipStream_t st, const hipEvent_t* ev) {
  if (ev) {
    (void)hipEventRecord(ev[0], st);
    (void)hipEventRecord(ev[1], st);
  }
}

// heads per workgroup of the block kernels: the largest divisor of H/G up to
// 4 (1024 workgroups per block kernel at the BitMamba shape; more heads per
// workgroup share staging but leave too few workgroups to fill the CUs)
constexpr int kMaxHeadsPerWG = 4;
int bwd_heads_per_group(int H, int G) {
  const int hpg = H / G;
  for (int d = hpg < kMaxHeadsPerWG ? hpg : kMaxHeadsPerWG; d >= 1; --d)
    if (hpg % d == 0) return d;
  return 1;
}

// workspace layout of the backward, after the forward's own (states, decays,
// token table): the adjoint states (fp32); f1, f2, x.v, dy.x, col (fp32 per
// token and head); the row shares of the column blocks (fp32, one per block); the
// chunk constants of da and the chunk shares of dA, ddt_bias, dD (fp64); the
// dB and dC partials (fp32)
struct BwdLayout {
  size_t fwd, adj, f1, f2, xv, dyx, col, row, cst, dtp, dBp, dCp, total;
};
static BwdLayout bwd_layout(int Bsz, int T, int H, int P, int G, int N, int chunk) {
  const int nc = (T + chunk - 1) / chunk;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  BwdLayout L{};
  size_t o = up(bf16_fwd_layout(Bsz, nc, H, P, N, chunk, 1).total);
  L.fwd = 0;
  L.adj = o;
  o += up(static_cast<size_t>(Bsz) * nc * H * P * N * 4);
  const size_t tok = static_cast<size_t>(Bsz) * T * H * 4;
  L.f1 = o;
  o += up(tok);
  L.f2 = o;
  o += up(tok);
  L.xv = o;
  o += up(tok);
  L.dyx = o;
  o += up(tok);
  L.col = o;
  o += up(tok);
  L.row = o;
  o += up(tok * ((chunk + kBlk - 1) / kBlk));
  L.cst = o;  // the adjoint passing's shares of the chunk constants, per workgroup
  o += up(static_cast<size_t>(Bsz) * H * nc * 8 * ((P * N / 4 + kThreads - 1) / kThreads));
  L.dtp = o;
  o += up(static_cast<size_t>(Bsz) * H * nc * 3 * 8);
  const int nparts = (H / G) / bwd_heads_per_group(H, G);
  const size_t part = static_cast<size_t>(nparts) * Bsz * T * G * N * 4;
  L.dBp = o;
  o += up(part);
  L.dCp = o;
  o += up(part);
  L.total = o + 256;
  return L;
}

size_t bwd_workspace_bytes(int Bsz, int T, int H, int P, int G, int N, int chunk) {
  return bwd_layout(Bsz, T, H, P, G, N, chunk).total;
}

template <int P, int N>
static hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
  const int Q = a.chunk;
  const int nc = (a.T + Q - 1) / Q;
  const BwdLayout L = bwd_layout(a.Bsz, a.T, a.H, P, a.G, N, Q);
  char* ws = static_cast<char*>(a.workspace);
  const hipEvent_t* ev = a.events;
  // forward recompute: chunk states -> boundary states, decays, token table
  ChunkArgs f{};
  f.x = a.x;
  f.dt = a.dt;
  f.A = a.A;
  f.B = a.B;
  f.C = a.C;
  f.dt_bias = a.dt_bias;
  f.dt_min = a.dt_min;
  f.dt_max = a.dt_max;
  f.h0 = a.h0;
  f.Bsz = a.Bsz;
  f.T = a.T;
  f.H = a.H;
  f.P = P;
  f.G = a.G;
  f.N = N;
  f.chunk = Q;
  f.dtype = 1;
  f.workspace = ws;
  f.events = const_cast<hipEvent_t*>(ev);
  hipError_t e = run_chunk_states_bf16(f, st);
  if (e != hipSuccess) return e;
  const Bf16FwdLayout FL = bf16_fwd_layout(a.Bsz, nc, a.H, P, N, Q, 1);
  // h_in(c) in fp32 (the recompute leaves it over the chunk states)
  const float* states = reinterpret_cast<const float*>(ws + FL.S);
  const float* decay = reinterpret_cast<const float*>(ws + FL.decay);
  const float2* tok = reinterpret_cast<const float2*>(ws + FL.tok);
  float* adj = reinterpret_cast<float*>(ws + L.adj);
  float* f1 = reinterpret_cast<float*>(ws + L.f1);
  float* f2 = reinterpret_cast<float*>(ws + L.f2);
  float* col = reinterpret_cast<float*>(ws + L.col);
  float* rowp = reinterpret_cast<float*>(ws + L.row);
  float* xv = reinterpret_cast<float*>(ws + L.xv);
  float* dyx = reinterpret_cast<float*>(ws + L.dyx);
  float* dBp = reinterpret_cast<float*>(ws + L.dBp);
  float* dCp = reinterpret_cast<float*>(ws + L.dCp);
  const uint16_t* x = static_cast<const uint16_t*>(a.x);
  const uint16_t* B = static_cast<const uint16_t*>(a.B);
  const uint16_t* C = static_cast<const uint16_t*>(a.C);
  const uint16_t* dy = static_cast<const uint16_t*>(a.dy);
  const int npairs = a.Bsz * nc;
  const unsigned blocks = static_cast<unsigned>((npairs + kXCD - 1) / kXCD) * kXCD * a.H;
  launch_k(nc > 0, ssd_adj_state_kernel<P, N>, dim3(blocks), dim3(kThreads), st, ev ? ev + 4 : nullptr,
           dy, C, tok, adj, a.T, a.H, a.G, Q, nc, npairs);
  // the adjoint passing also forms each chunk's constant, as per-workgroup shares
  const int nblk = (P * N / 4 + kThreads - 1) / kThreads;
  double* cpart = reinterpret_cast<double*>(ws + L.cst);
  launch_k(true, ssd_adj_pass_kernel, dim3(nblk, a.H, a.Bsz), dim3(kThreads), st, ev ? ev + 6 : nullptr, adj,
           decay, a.dh_final, a.dh0, states, cpart, a.H, P * N, nc);
  const int HPG = bwd_heads_per_group(a.H, a.G);
  const int nb = (Q + kBlk - 1) / kBlk;
  const unsigned bblocks = static_cast<unsigned>(nb) * units_per_rank(a.H / HPG, nc, a.Bsz);
  launch_k(nc > 0, ssd_bwd_dxdb_kernel<P, N>, dim3(bblocks), dim3(kThreads), st, ev ? ev + 8 : nullptr,
           x, B, C, dy, a.D, tok, static_cast<const float*>(adj), static_cast<uint16_t*>(a.dx), xv,
           dyx, f2, col, rowp, dBp, a.Bsz, a.T, a.H, a.G, Q, nc, HPG);
  launch_k(nc > 0, ssd_bwd_dc_kernel<P, N>, dim3(bblocks), dim3(kThreads), st, ev ? ev + 10 : nullptr,
           x, B, C, dy, tok, states, f1, dCp, a.Bsz, a.T, a.H, a.G, Q, nc, HPG);
  // (the chunk constants' slot: an empty pair, recorded back to back)
  empty_slot(st, ev ? ev + 12 : nullptr);
  double* dtp = reinterpret_cast<double*>(ws + L.dtp);
  launch_k(nc > 0, ssd_bwd_dt_kernel, dim3(nc > 0 ? nc : 1, a.H, a.Bsz), dim3(kThreads), st,
           ev ? ev + 14 : nullptr, a.dt, a.A, a.dt_bias, a.dt_min, a.dt_max, static_cast<const float*>(f1),
           static_cast<const float*>(f2), static_cast<const float*>(col), static_cast<const float*>(rowp),
           static_cast<const float*>(xv),
           static_cast<const float*>(dyx), static_cast<const double*>(cpart), decay, nblk, a.ddt, dtp, a.Bsz,
           a.T, a.H, Q, nc);
  // (the per-head sums' slot: an empty pair; they run in the launch below)
  const size_t n4 = static_cast<size_t>(a.Bsz) * a.T * a.G * N / 4;
  const int nparts = (a.H / a.G) / HPG;
  empty_slot(st, ev ? ev + 16 : nullptr);
  // dB, dC and the per-head sums in one launch (slot 9; slot 10: an empty pair)
  const size_t rblocks = std::max((n4 + kThreads - 1) / kThreads,
                                  static_cast<size_t>((a.H + kThreads - 1) / kThreads));
  launch_k(true, ssd_bwd_reduce_kernel, dim3(static_cast<unsigned>(rblocks), 3), dim3(kThreads), st,
           ev ? ev + 18 : nullptr, static_cast<const float*>(dBp), a.dB, static_cast<const float*>(dCp), a.dC,
           n4, nparts, static_cast<const double*>(dtp), a.dA, a.ddt_bias, a.dD, a.Bsz, a.H, nc);
  empty_slot(st, ev ? ev + 20 : nullptr);
  return hipGetLastError();
}

hipError_t run_chunk_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  if (a.P == 64 && a.N == 128) return launch_bwd<64, 128>(a, st);
  if (a.P == 64 && a.N == 64) return launch_bwd<64, 64>(a, st);
  if (a.P == 32 && a.N == 64) return launch_bwd<32, 64>(a, st);
  if (a.P == 32 && a.N == 128) return launch_bwd<32, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ssd
