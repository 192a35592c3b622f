// Backward of the chunked SSD for float32 inputs on gfx950 (fp32 matrix
// cores, v_mfma_f32_16x16x4_f32): the real Mamba-2 form with float32 x, B, C,
// dy, and the complex Mamba-3-Lite form through its rotated-frame real form.
//
// Real form.  The gradient of loss = sum_t dy_t . y_t + <dh_final, h_final>
// for h_t = e^{A delta_t} h_{t-1} + s_t x_t B_t^T, y_t = h_t C_t + D x_t, with
// input scale s_t = delta_t (the Mamba-2 discretisation).  The chunkwise
// adjoint is the one of the bf16 backward (ssd_bwd_bf16.hip, which states the
// formulas): inside a chunk of 64 tokens (cs_l the inclusive cumulative
// log-decay, tot its total, R_c the adjoint at the chunk end)
//   v_s   = sum_{l>=s} e^{cs_l-cs_s} (C_l.B_s) dy_l + e^{tot-cs_s} R_c B_s
//   dx_s  = s_s v_s + D dy_s
//   dB_s  = sum_{l>=s} e^{cs_l-cs_s} s_s (dy_l.x_s) C_l + s_s e^{tot-cs_s} R_c^T x_s
//   dC_l  = sum_{s<=l} e^{cs_l-cs_s} s_s (dy_l.x_s) B_s + e^{cs_l} H_in^T dy_l
//   da_t  = sum_{s<t<=l} E[l][s] + sum_{l>=t} f1_l + sum_{s<t} f2_s + e^{tot}<R_c, H_in>,
//   E[l][s] = e^{cs_l-cs_s} s_s (C_l.B_s)(dy_l.x_s),  f1_l = e^{cs_l} C_l.(H_in^T dy_l),
//   f2_s = e^{tot-cs_s} s_s x_s.(R_c B_s),
//   d delta_t = A da_t + [s = delta] x_t.v_t,  dA = sum delta_t da_t,  dD = sum dy.x.
// (Numerical Stability in Mamba-3-Lite, section 4, for the chunkwise form; the
// backward is the plain reverse-mode derivative of the recurrence.)
//
// Complex form.  With u_t = delta_1 + .. + delta_t over the sequence and
// theta_t = beta u_t, the state in the rotated frame h~_t = e^{-i theta_t} h_t
// obeys h~_t = e^{alpha delta_t} h~_{t-1} + x_t B'_t with B' = B e^{-i theta},
// and y_t = Re(C'_t h~_t) with C' = C e^{i theta}: two real recurrences (the
// real and imaginary parts of h~) with one real decay, i.e. the real form
// with 2N features B_eff = [Re B' | Im B'], C_eff = [Re C' | -Im C'], decay
// alpha and input scale 1 (Mamba-3-Lite README, the complex recurrence; the
// rotation is the factoring the complex forward kernels use inside a chunk,
// here over the whole sequence).  The complex gradients follow from the real
// ones:  dB = e^{i theta} (dB_eff[n] + i dB_eff[N+n]),
// dC = e^{-i theta} (dC_eff[n] - i dC_eff[N+n]), dh0 = (R[p][n], R[p][N+n])
// after the first chunk, d alpha = sum delta da; and the rotations themselves
// depend on u_t, hence on every earlier step size and on beta:
//   rho_t = sum_n Im(conj(dB'_n) B'_n) - Im(conj(dC'_n) C'_n)  (dL/du_t / beta),
//   plus -Im<dh~_final, h~_final> at the last token (h_final = e^{i theta} h~_final),
//   d delta_t += beta sum_{j>=t} rho_j,   d beta = sum_t u_t rho_t.
// The angles theta_t are reduced modulo 2 pi in double precision.
//
// Kernels (one workgroup per (chunk, head, batch) unless noted):
//   ssd_cplx_frame      (complex; one workgroup per (head, batch)) u and theta
//                         over the sequence (an fp64 scan), (cos, sin) theta per
//                         token, the rotated h0 and dh_final; B_eff and C_eff are
//                         never stored: the chunk-state and block kernels form them
//                         from B and C as they stage them
//   chunk states, state passing, adjoint chunk states: ssd_chunk.hip's fp32
//                         kernels (run_states_f32, run_pass_f32)
//   ssd_f32_adj_pass      R_c in place over G_c, last chunk first; dh0; the
//                         shares of the chunk constants <R_c, H_in(c)>
//   ssd_f32_col           v, dx, dB (per head), f2, col, x.v, dy.x [, rho_B]
//   ssd_f32_row           dC (per head), f1, row [, rho_C]
//   ssd_cplx_tau          (complex) the last token's rho term of h_final
//   ssd_cplx_rho_total    (complex) rho summed over each chunk
//   ssd_f32_dt            fp64 scans of f1, f2, col - row [, rho]: da, ddt and
//                         the chunk's shares of dA, ddt_bias, dD [, d beta]
//   ssd_f32_dt_sum        per head: the sums of the shares
//   ssd_f32_group_sum     dB, dC: the heads of each group summed (complex:
//                         rotated back first); complex dh0 interleaved.  When
//                         each head has its own group the block kernels write
//                         dB and dC directly (complex: rotated back) instead
// With measurement events, pair k (events 2k, 2k+1) is bound to: 0 rotation
// (from the start of the u sums to the end of the rotation),
// 1 chunk states, 2 state passing, 3 adjoint chunk states, 4 adjoint passing,
// 5 column side, 6 row side, 7 chunk constants (formed inside the adjoint
// passing: recorded back to back), 8 tau, 9 rho totals,
// 10 step sizes, 11 their sums, 12 group sums, 13 dh0 (a kernel a form does
// not run records its pair back to back).
//
// MFMA operands: 16x16x4 fp32, lane i holding A[i%16][k] and B[k][i%16] of
// one k per instruction.  A run of four instructions takes k = 4q + j
// (q = i / 16, j = 0..3), so both operands come as one float4 per lane from
// LDS rows; and a product whose B operand is an accumulator tile (lane:
// column i%16, rows 4q + j) takes k = that row, so the tile feeds the next
// product in registers with no exchange between lanes.

#include "ssd_chunk_common.h"

namespace ssd {

namespace {

constexpr int kQ = 64;  // tokens per chunk of the fp32 backward

// sum over the 4 lane groups of the lanes that share i % 16
__device__ __forceinline__ float qsum(float a) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  const float pair = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// A tile of ROWS rows of W floats (source row stride `ld` floats) staged in two
// phases, so that every load of a workgroup's tiles is in flight before the
// first wait: load() into registers, then store() into LDS at `pitch`, rows at
// or past `valid` (>= 1) as zeros.  The loads are unconditional (a row past
// `valid` reads row valid - 1, zeroed at the store): a load under a branch
// ends in a wait for it where the branch joins.  For complex rows (W/2 (re, im) pairs per row),
// load_rot() fetches each row's (cos, sin) theta and store_rot() writes the W
// real features [Re | Im] of z e^{-i theta} (CONJ = false) or [Re | -Im] of
// z e^{+i theta} (CONJ = true).
template <int W, int ROWS, int NTHR>
struct TileRegs {
  static constexpr int VPR = W / 4;
  static constexpr int ITEMS = ROWS * VPR;
  static constexpr int PER = (ITEMS + NTHR - 1) / NTHR;
  float4 v[PER];
  float2 cs[PER];
  int valid_;
  __device__ __forceinline__ float4 val(int i) const {
    return (threadIdx.x + i * NTHR) / VPR < valid_ ? v[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ __forceinline__ void load(const float* __restrict__ src, size_t ld, int valid) {
    valid_ = valid;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NTHR;
      const int r = min(it / VPR, valid - 1), c4 = it % VPR;
      if (ITEMS % NTHR == 0 || it < ITEMS) v[i] = *reinterpret_cast<const float4*>(src + r * ld + c4 * 4);
    }
  }
  __device__ __forceinline__ void load_rot(const float2* __restrict__ rc, size_t rstride, int valid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NTHR;
      const int r = min(it / VPR, valid - 1);
      if (ITEMS % NTHR == 0 || it < ITEMS) cs[i] = rc[r * rstride];
    }
  }
  __device__ __forceinline__ void store(float* tile, int pitch) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NTHR;
      if (ITEMS % NTHR == 0 || it < ITEMS)
        *reinterpret_cast<float4*>(tile + (it / VPR) * pitch + (it % VPR) * 4) = val(i);
    }
  }
  template <bool CONJ>
  __device__ __forceinline__ void store_rot(float* tile, int pitch, const float2 (&rcs)[PER]) const {
    constexpr int NH = W / 2;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NTHR;
      if (!(ITEMS % NTHR == 0 || it < ITEMS)) continue;
      const float4 val = this->val(i);  // zero past `valid`, whatever its rotation
      const float2 c = rcs[i];
      float* t = tile + (it / VPR) * pitch + 2 * (it % VPR);
      if constexpr (!CONJ) {
        *reinterpret_cast<float2*>(t) = make_float2(val.x * c.x + val.y * c.y, val.z * c.x + val.w * c.y);
        *reinterpret_cast<float2*>(t + NH) = make_float2(val.y * c.x - val.x * c.y, val.w * c.x - val.z * c.y);
      } else {
        *reinterpret_cast<float2*>(t) = make_float2(val.x * c.x - val.y * c.y, val.z * c.x - val.w * c.y);
        *reinterpret_cast<float2*>(t + NH) =
            make_float2(-(val.y * c.x + val.x * c.y), -(val.w * c.x + val.z * c.y));
      }
    }
  }
};

// acc += A . B over k in [0, K): A rows `arow` (k contiguous), B rows `brow`
// (k contiguous), 4 k per lane group per float4
template <int K>
__device__ __forceinline__ f32x4 dot_rows(const float* arow, const float* brow, f32x4 acc) {
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 a = *reinterpret_cast<const float4*>(arow + k0 + 4 * q);
    const float4 b = *reinterpret_cast<const float4*>(brow + k0 + 4 * q);
    acc = mfma_f32(a.x, b.x, acc);
    acc = mfma_f32(a.y, b.y, acc);
    acc = mfma_f32(a.z, b.z, acc);
    acc = mfma_f32(a.w, b.w, acc);
  }
  return acc;
}

}  // namespace

// ---------------------------------------------------------------------------
// Both block kernels run eight waves (two per SIMD: the 137 KB of LDS of the
// widest tiles leave room for one workgroup per CU), in two roles of four
// waves; in each role wave w owns the 16 tokens 16 (w % 4) .. +15 of the
// chunk as MFMA columns.
// ---------------------------------------------------------------------------
constexpr int kT8 = 512;

// Column side, source token s = 16 (w % 4) + lane % 16.  Scores S = C.B^T and
// W0 = dy.x^T (rows l, columns s), masked and decayed into M and W.
//   role 0:  v^T[p][s] = e^{tot-cs_s} (R B_s)[p] + sum_l dy^T[p][l] M[l][s];
//            dx, f2, col (the box terms), x.v, dy.x
//   role 1:  dB^T[n][s] = s_s e^{tot-cs_s} (R^T x_s)[n] + sum_l C^T[n][l] W[l][s];
//            rho_B (complex)
// ---------------------------------------------------------------------------
template <int P, int NE, bool SCALE, bool CPLX>
__global__ __launch_bounds__(kT8) void ssd_f32_col_kernel(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ dt_bias, float dt_min, float dt_max, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ dy, const float* __restrict__ D,
    const float* __restrict__ adj, float* __restrict__ dx, float* __restrict__ dBh,
    float* __restrict__ f2o, float* __restrict__ colo, float* __restrict__ xvo,
    float* __restrict__ dyxo, float* __restrict__ rhoB, const float2* __restrict__ rot,
    float* __restrict__ dBo, int T, int H, int G, int nc) {
  constexpr int XP = P + 4, NP = NE + 4;
  constexpr int PT = P / 16, NT = NE / 16;
  __shared__ __attribute__((aligned(16))) float Xs[kQ * XP];
  __shared__ __attribute__((aligned(16))) float Ys[kQ * XP];
  __shared__ __attribute__((aligned(16))) float Bs[kQ * NP];
  __shared__ __attribute__((aligned(16))) float Cs[kQ * NP];
  __shared__ __attribute__((aligned(16))) float Rs[P * NP];
  __shared__ float Ws[4][16][kWave];  // role 1's W tiles, per wave (w % 4), value and lane
  __shared__ float dl[kQ], cs_hi[kQ], cs_lo[kQ];
  __shared__ double wsum[kT8 / kWave], tot;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int t0 = c * kQ, Lc = min(kQ, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int w = wave_id(), role = w >> 2;
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  const int s = 16 * (w & 3) + r16;  // this lane's source token
  const size_t row = (r0 + s) * H + h;
  // The loads come in the order they are waited for (a wait for one load also
  // waits for those issued before it): the step sizes and per-head values the
  // prologue needs, this lane's rotation (the complex dB), then every tile
  // into registers; the prologue's scans run while the tiles arrive.
  // (unconditional loads of clamped rows: the prologue ignores dt past Lc, and
  // the rotation is used only for s < Lc)
  const float dt_raw = dt[(r0 + min(tid, Lc - 1)) * H + h];
  const float a_h = A[h], bias_h = dt_bias ? dt_bias[h] : 0.0f;
  const float Dh = D ? D[h] : 0.0f;
  float2 rs = make_float2(1.0f, 0.0f);
  if (CPLX && dBo != nullptr) rs = rot[(r0 + min(s, Lc - 1)) * H + h];
  {
    TileRegs<P, kQ, kT8> tx, ty;
    TileRegs<NE, kQ, kT8> tb, tc;
    TileRegs<NE, P, kT8> tr;
    tx.load(x + (r0 * H + h) * P, static_cast<size_t>(H) * P, Lc);
    ty.load(dy + (r0 * H + h) * P, static_cast<size_t>(H) * P, Lc);
    tb.load(Bm + (r0 * G + g) * NE, static_cast<size_t>(G) * NE, Lc);
    tc.load(Cm + (r0 * G + g) * NE, static_cast<size_t>(G) * NE, Lc);
    tr.load(adj + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * NE), NE, P);
    if constexpr (CPLX) tb.load_rot(rot + r0 * H + h, H, Lc);
    chunk_prologue(dt_raw, Lc, a_h, bias_h, dt_min, dt_max, dl, cs_hi, cs_lo, wsum, &tot, kQ);
    tx.store(Xs, XP);
    ty.store(Ys, XP);
    if constexpr (CPLX) {
      tb.template store_rot<false>(Bs, NP, tb.cs);
      tc.template store_rot<true>(Cs, NP, tb.cs);
    } else {
      tb.store(Bs, NP);
      tc.store(Cs, NP);
    }
    tr.store(Rs, NP);
  }
  __syncthreads();

  const float hs = cs_hi[s], ls = cs_lo[s];
  const float sc = SCALE ? dl[s] : (s < Lc ? 1.0f : 0.0f);
  const float fr = s < Lc ? __expf(static_cast<float>((tot - static_cast<double>(hs)) - static_cast<double>(ls)))
                          : 0.0f;  // e^{tot - cs_s} <= 1

  float dd[4][4];  // decay of (l, s), 0 off the causal block
#pragma unroll
  for (int lt = 0; lt < 4; ++lt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = 16 * lt + 4 * q + i;
      const bool ok = l >= s && l < Lc && s < Lc;
      dd[lt][i] = ok ? decay_between(cs_hi[l], cs_lo[l], hs, ls) : 0.0f;
    }
  // W0 = dy.x^T, rows l = 16 lt + 4q + i, masked, decayed and scaled into W:
  // role 1 forms it and hands it to role 0 through LDS (one barrier, each role
  // reaching it after its first products)
  f32x4 sW[4];
  if (role == 1) {
#pragma unroll
    for (int lt = 0; lt < 4; ++lt)
      sW[lt] = dot_rows<P>(Ys + (16 * lt + r16) * XP, Xs + s * XP, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int lt = 0; lt < 4; ++lt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sW[lt][i] = dd[lt][i] * sc * sW[lt][i];
        Ws[w & 3][4 * lt + i][lane] = sW[lt][i];
      }
  }

  if (role == 0) {
    // scores S = C.B^T; the box terms; M = decayed S
    f32x4 sS[4];
#pragma unroll
    for (int lt = 0; lt < 4; ++lt)
      sS[lt] = dot_rows<NE>(Cs + (16 * lt + r16) * NP, Bs + s * NP, f32x4{0.f, 0.f, 0.f, 0.f});
    __syncthreads();  // (the W tiles of role 1)
    float col = 0.0f;
#pragma unroll
    for (int lt = 0; lt < 4; ++lt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int l = 16 * lt + 4 * q + i;
        col += l > s ? Ws[w & 3][4 * lt + i][lane] * sS[lt][i] : 0.0f;
        sS[lt][i] = dd[lt][i] * sS[lt][i];
      }
    col = qsum(col);
    // v: boundary (R B_s), then f2, then the intra-chunk part
    f32x4 v[PT];
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      v[pt] = dot_rows<NE>(Rs + (16 * pt + r16) * NP, Bs + s * NP, f32x4{0.f, 0.f, 0.f, 0.f});
      v[pt] = v[pt] * fr;
    }
    float f2 = 0.0f;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) f2 += Xs[s * XP + 16 * pt + 4 * q + i] * v[pt][i];
    f2 = sc * qsum(f2);
#pragma unroll
    for (int lt = 0; lt < 4; ++lt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
          v[pt] = mfma_f32(Ys[(16 * lt + 4 * q + j) * XP + 16 * pt + r16], sS[lt][j], v[pt]);
    float xv = 0.0f, dyx = 0.0f;
    float* dxr = dx + row * P;
#pragma unroll
    for (int pt = 0; pt < PT; ++pt) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 16 * pt + 4 * q + i;
        const float xe = Xs[s * XP + p], ye = Ys[s * XP + p];
        xv += xe * v[pt][i];
        dyx += xe * ye;
        o[i] = sc * v[pt][i] + Dh * ye;
      }
      if (s < Lc) *reinterpret_cast<float4*>(dxr + 16 * pt + 4 * q) = make_float4(o[0], o[1], o[2], o[3]);
    }
    xv = qsum(xv);
    dyx = qsum(dyx);
    if (q == 0 && s < Lc) {
      f2o[row] = f2;
      colo[row] = col;
      xvo[row] = xv;
      dyxo[row] = dyx;
    }
    return;
  }

  // role 1 -- dB: boundary (R^T x_s), scaled, then the intra-chunk part
  f32x4 db[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < P; k0 += 16) {
      const float4 xb = *reinterpret_cast<const float4*>(Xs + s * XP + k0 + 4 * q);
      acc = mfma_f32(Rs[(k0 + 4 * q + 0) * NP + 16 * nt + r16], xb.x, acc);
      acc = mfma_f32(Rs[(k0 + 4 * q + 1) * NP + 16 * nt + r16], xb.y, acc);
      acc = mfma_f32(Rs[(k0 + 4 * q + 2) * NP + 16 * nt + r16], xb.z, acc);
      acc = mfma_f32(Rs[(k0 + 4 * q + 3) * NP + 16 * nt + r16], xb.w, acc);
    }
    db[nt] = acc * (sc * fr);
  }
  __syncthreads();  // (role 0 takes the W tiles)
#pragma unroll
  for (int lt = 0; lt < 4; ++lt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        db[nt] = mfma_f32(Cs[(16 * lt + 4 * q + j) * NP + 16 * nt + r16], sW[lt][j], db[nt]);
  if (s < Lc) {
    if (CPLX && dBo) {
      // each head its own group: dB = e^{i theta} (dB_eff[n] + i dB_eff[N+n]) straight out
      const float2 r = rs;
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xr = db[nt][i], xi = db[nt + NT / 2][i];
          o[2 * i] = xr * r.x - xi * r.y;
          o[2 * i + 1] = xr * r.y + xi * r.x;
        }
        float* dst = dBo + (row * (NE / 2) + 16 * nt + 4 * q) * 2;
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4*>(dBh + row * NE + 16 * nt + 4 * q) = db[nt];
    }
  }
  if constexpr (CPLX) {
    // Im(conj(dB') B') = dB_eff[n] B_eff[N+n] - dB_eff[N+n] B_eff[n]
    constexpr int HT = NT / 2;
    float rb = 0.0f;
#pragma unroll
    for (int nt = 0; nt < HT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * nt + 4 * q + i;
        rb += db[nt][i] * Bs[s * NP + NE / 2 + n] - db[nt + HT][i] * Bs[s * NP + n];
      }
    rb = qsum(rb);
    if (q == 0 && s < Lc) rhoB[row] = rb;
  }
}

// ---------------------------------------------------------------------------
// Row side, target token l = 16 (w % 4) + lane % 16.  Transposed scores
// S^T = B.C^T and W0^T = x.dy^T (rows s, columns l), masked and decayed.
//   role 0:  the boundary part of dC^T[n][l], e^{cs_l} (H_in^T dy_l)[n]; f1;
//            row (the box terms); after the exchange the whole dC, rho_C
//   role 1:  the intra-chunk part sum_s B^T[n][s] W^T[s][l], handed to role 0
//            through LDS (over the B tile, once every wave is done with it)
// ---------------------------------------------------------------------------
template <int P, int NE, bool SCALE, bool CPLX>
__global__ __launch_bounds__(kT8) void ssd_f32_row_kernel(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ dt_bias, float dt_min, float dt_max, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ dy, const float* __restrict__ states,
    float* __restrict__ dCh, float* __restrict__ f1o, float* __restrict__ rowo,
    float* __restrict__ rhoC, const float2* __restrict__ rot, float* __restrict__ dCo, int T, int H,
    int G, int nc) {
  constexpr int XP = P + 4, NP = NE + 4;
  constexpr int NT = NE / 16;
  __shared__ __attribute__((aligned(16))) float Xs[kQ * XP];
  __shared__ __attribute__((aligned(16))) float Ys[kQ * XP];
  __shared__ __attribute__((aligned(16))) float Bs[kQ * NP];
  __shared__ __attribute__((aligned(16))) float Cs[kQ * NP];
  __shared__ __attribute__((aligned(16))) float Hs[P * NP];
  __shared__ float Ws[4][16][kWave];  // role 1's W^T tiles, per wave (w % 4), value and lane
  __shared__ float dl[kQ], cs_hi[kQ], cs_lo[kQ];
  __shared__ double wsum[kT8 / kWave], tot;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int t0 = c * kQ, Lc = min(kQ, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int w = wave_id(), role = w >> 2;
  const size_t r0 = static_cast<size_t>(b) * T + t0;
  const int l = 16 * (w & 3) + r16;  // this lane's target token
  const size_t row = (r0 + l) * H + h;
  // loads in the order they are waited for, as in the column kernel
  const float dt_raw = dt[(r0 + min(tid, Lc - 1)) * H + h];
  const float a_h = A[h], bias_h = dt_bias ? dt_bias[h] : 0.0f;
  float2 rl = make_float2(1.0f, 0.0f);
  if (CPLX && dCo != nullptr) rl = rot[(r0 + min(l, Lc - 1)) * H + h];
  {
    TileRegs<P, kQ, kT8> tx, ty;
    TileRegs<NE, kQ, kT8> tb, tc;
    TileRegs<NE, P, kT8> th;
    tx.load(x + (r0 * H + h) * P, static_cast<size_t>(H) * P, Lc);
    ty.load(dy + (r0 * H + h) * P, static_cast<size_t>(H) * P, Lc);
    tb.load(Bm + (r0 * G + g) * NE, static_cast<size_t>(G) * NE, Lc);
    tc.load(Cm + (r0 * G + g) * NE, static_cast<size_t>(G) * NE, Lc);
    th.load(states + ((static_cast<size_t>(b) * nc + c) * H + h) * (static_cast<size_t>(P) * NE), NE, P);
    if constexpr (CPLX) tb.load_rot(rot + r0 * H + h, H, Lc);
    chunk_prologue(dt_raw, Lc, a_h, bias_h, dt_min, dt_max, dl, cs_hi, cs_lo, wsum, &tot, kQ);
    tx.store(Xs, XP);
    ty.store(Ys, XP);
    if constexpr (CPLX) {
      tb.template store_rot<false>(Bs, NP, tb.cs);
      tc.template store_rot<true>(Cs, NP, tb.cs);
    } else {
      tb.store(Bs, NP);
      tc.store(Cs, NP);
    }
    th.store(Hs, NP);
  }
  __syncthreads();

  const float hl = cs_hi[l], ll = cs_lo[l];

  // W0^T = x.dy^T, rows s = 16 st + 4q + i, masked, decayed and scaled: role 1
  // forms it and hands it to role 0 through LDS (one barrier, each role
  // reaching it after its first products)
  f32x4 sW[4];
  if (role == 1) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
      sW[st] = dot_rows<P>(Xs + (16 * st + r16) * XP, Ys + l * XP, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * st + 4 * q + i;
        const bool ok = s <= l && l < Lc && s < Lc;
        const float d = ok ? decay_between(hl, ll, cs_hi[s], cs_lo[s]) : 0.0f;
        const float sc = SCALE ? dl[s] : 1.0f;
        sW[st][i] = d * sc * sW[st][i];
        Ws[w & 3][4 * st + i][lane] = sW[st][i];
      }
  }

  f32x4 dc[NT];
  float f1 = 0.0f, rw = 0.0f;
  if (role == 0) {
    f32x4 sS[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      sS[st] = dot_rows<NE>(Bs + (16 * st + r16) * NP, Cs + l * NP, f32x4{0.f, 0.f, 0.f, 0.f});
    __syncthreads();  // (the W^T tiles of role 1)
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 16 * st + 4 * q + i;
        rw += s < l ? Ws[w & 3][4 * st + i][lane] * sS[st][i] : 0.0f;
      }
    rw = qsum(rw);
    // boundary (H_in^T dy_l) scaled by e^{cs_l}, and f1
    const float fl = l < Lc ? __expf(hl + ll) : 0.0f;  // e^{cs_l} <= 1
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < P; k0 += 16) {
        const float4 yb = *reinterpret_cast<const float4*>(Ys + l * XP + k0 + 4 * q);
        acc = mfma_f32(Hs[(k0 + 4 * q + 0) * NP + 16 * nt + r16], yb.x, acc);
        acc = mfma_f32(Hs[(k0 + 4 * q + 1) * NP + 16 * nt + r16], yb.y, acc);
        acc = mfma_f32(Hs[(k0 + 4 * q + 2) * NP + 16 * nt + r16], yb.z, acc);
        acc = mfma_f32(Hs[(k0 + 4 * q + 3) * NP + 16 * nt + r16], yb.w, acc);
      }
      dc[nt] = acc * fl;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) f1 += Cs[l * NP + 16 * nt + 4 * q + i] * dc[nt][i];
    f1 = qsum(f1);
  } else {
    __syncthreads();  // (role 0 takes the W^T tiles)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          dc[nt] = mfma_f32(Bs[(16 * st + 4 * q + j) * NP + 16 * nt + r16], sW[st][j], dc[nt]);
  }
  __syncthreads();  // every wave is done with the B tile
  float* part = Bs;  // role 1's part of dC, [l][n] at the B tile's pitch
  if (role == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(part + l * NP + 16 * nt + 4 * q) = dc[nt];
  }
  __syncthreads();
  if (role == 1) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) dc[nt] = dc[nt] + *reinterpret_cast<const f32x4*>(part + l * NP + 16 * nt + 4 * q);
  if (l < Lc) {
    if (CPLX && dCo) {
      // each head its own group: dC = e^{-i theta} (dC_eff[n] - i dC_eff[N+n]) straight out
      const float2 r = rl;
#pragma unroll
      for (int nt = 0; nt < NT / 2; ++nt) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float yr = dc[nt][i], yi = -dc[nt + NT / 2][i];
          o[2 * i] = yr * r.x + yi * r.y;
          o[2 * i + 1] = yi * r.x - yr * r.y;
        }
        float* dst = dCo + (row * (NE / 2) + 16 * nt + 4 * q) * 2;
        *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<f32x4*>(dCh + row * NE + 16 * nt + 4 * q) = dc[nt];
    }
  }
  float rc = 0.0f;
  if constexpr (CPLX) {
    // Im(conj(dC') C') = dC_eff[N+n] C_eff[n] - dC_eff[n] C_eff[N+n]
    constexpr int HT = NT / 2;
#pragma unroll
    for (int nt = 0; nt < HT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * nt + 4 * q + i;
        rc += dc[nt + HT][i] * Cs[l * NP + n] - dc[nt][i] * Cs[l * NP + NE / 2 + n];
      }
    rc = qsum(rc);
  }
  if (q == 0 && l < Lc) {
    f1o[row] = f1;
    rowo[row] = rw;
    if constexpr (CPLX) rhoC[row] = rc;
  }
}

// ---------------------------------------------------------------------------
// Adjoint passing, last chunk first: R_{nc-1} = dh_final, R_{c-1} = lambda_c
// R_c + G_c, dh0 = R_{-1}; R_c over G_c.  One thread per 4 elements, a
// workgroup per 1024 elements of one (batch, head), the chunks in groups of 8
// whose loads are issued together.  On the way it forms its
// share of each chunk's constant <R_c, H_in(c)> (H_in over the forward states,
// fp64 sums): cpart[(b, h, c) * nblk + block], summed and scaled by e^{tot}
// where the step-size gradients use them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ssd_f32_adj_pass_kernel(
    float* __restrict__ adj, const float* __restrict__ decay, const float* __restrict__ dh_final,
    float* __restrict__ dh0, const float* __restrict__ states, double* __restrict__ cpart, int H, int PN,
    int nc) {
  constexpr int PF = 8;  // chunks whose loads are issued together
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
  const float* dc = decay + bh * nc * 2;
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
      if (cc >= 0) ld[j] = dc[2 * cc];
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

// ---------------------------------------------------------------------------
// Complex: the sequence frame, one workgroup per (head, batch).  u_t =
// delta_1 + .. + delta_t over the sequence (fp64: each of 1024 threads sums 2
// consecutive tokens, one block scan per 2048 tokens, carried from block to
// block) and (cos, sin) theta_t, theta_t = beta u_t mod 2 pi, per token
// and head (the kernels that read B and C rotate them by it as they stage
// them); then h0 as [Re | Im] rows and dh_final, rotated by -theta at the last
// token, likewise; the decay alpha of each head.
// ---------------------------------------------------------------------------
constexpr int kFrameThreads = 1024;
__global__ __launch_bounds__(kFrameThreads) void ssd_cplx_frame_kernel(
    const float* __restrict__ dt, const float* __restrict__ dt_bias, float dt_min, float dt_max,
    const float* __restrict__ A, const float* __restrict__ h0, const float* __restrict__ dh_final,
    double* __restrict__ uo, float2* __restrict__ rot, float* __restrict__ alpha, float* __restrict__ h0e,
    float* __restrict__ dhfe, int T, int H, int P, int N) {
  constexpr int TPT = 2;  // consecutive tokens per thread in a block of kFrameThreads * TPT
  __shared__ double wtot[kFrameThreads / kWave];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid / kWave;
  const float be = A[2 * h + 1];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  if (tid == 0 && b == 0) alpha[h] = A[2 * h];
  const size_t bh = static_cast<size_t>(b) * H + h;
  double carry = 0.0;  // u of the tokens before the block
  for (int tb = 0; tb < T; tb += TPT * kFrameThreads) {
    const int t0 = tb + TPT * tid;  // this thread's first token
    float dv[TPT];
#pragma unroll
    for (int r = 0; r < TPT; ++r)  // (clamped rows: no load under a branch)
      dv[r] = dt[(static_cast<size_t>(b) * T + min(t0 + r, T - 1)) * H + h];
    double us[TPT], run = 0.0;  // this thread's inclusive sums
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      run += t0 + r < T ? static_cast<double>(step_size(dv[r], bias, dt_min, dt_max)) : 0.0;
      us[r] = run;
    }
    const double incl = wave_inclusive_sum_d(run);
    if (lane == kWave - 1) wtot[wid] = incl;
    __syncthreads();
    double before = carry + (incl - run), total = carry;
#pragma unroll
    for (int w = 0; w < kFrameThreads / kWave; ++w) {
      const double pw = wtot[w];
      before += w < wid ? pw : 0.0;
      total += pw;
    }
    __syncthreads();  // (wtot is rewritten by the next block)
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      if (t0 + r < T) {
        const double u = before + us[r];
        const size_t row = (static_cast<size_t>(b) * T + t0 + r) * H + h;
        uo[row] = u;
        float cs, sn;
        rot_cs(static_cast<double>(be) * u, cs, sn);
        rot[row] = make_float2(cs, sn);
      }
    }
    carry = total;
  }
  // h0 -> [Re | Im] rows; dh_final -> e^{-i theta_{T-1}} dh_final as [Re | Im]
  float cl = 1.0f, sl = 0.0f;
  if (T > 0) rot_cs(static_cast<double>(be) * carry, cl, sl);
  const int NE = 2 * N;
  for (int i = tid; i < P * N; i += kFrameThreads) {
    const int p = i / N, n = i % N;
    const size_t src = (bh * P * N + i) * 2;
    const size_t dst = bh * P * NE + static_cast<size_t>(p) * NE;
    const float2 hv = h0 ? *reinterpret_cast<const float2*>(h0 + src) : make_float2(0.f, 0.f);
    h0e[dst + n] = hv.x;
    h0e[dst + N + n] = hv.y;
    const float2 dv = dh_final ? *reinterpret_cast<const float2*>(dh_final + src) : make_float2(0.f, 0.f);
    dhfe[dst + n] = dv.x * cl + dv.y * sl;
    dhfe[dst + N + n] = dv.y * cl - dv.x * sl;
  }
}

// Complex: the last token's rho term, -Im <dh~_final, h~_final>, added to
// rho_B of that token (one workgroup per (batch, head)).
__global__ __launch_bounds__(kThreads) void ssd_cplx_tau_kernel(
    const float* __restrict__ dhfe, const float* __restrict__ hfe, float* __restrict__ rhoB, int T,
    int H, int P, int N) {
  __shared__ double ws4[4];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid / kWave;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int NE = 2 * N;
  double sum = 0.0;
  for (int i = tid; i < P * N; i += kThreads) {
    const int p = i / N, n = i % N;
    const size_t o = bh * P * NE + static_cast<size_t>(p) * NE;
    sum += static_cast<double>(dhfe[o + n]) * hfe[o + N + n] - static_cast<double>(dhfe[o + N + n]) * hfe[o + n];
  }
  sum = wave_inclusive_sum_d(sum);
  if (lane == kWave - 1) ws4[wid] = sum;
  __syncthreads();
  if (tid == 0 && T > 0) {
    const size_t row = (static_cast<size_t>(b) * T + T - 1) * H + h;
    rhoB[row] = static_cast<float>(static_cast<double>(rhoB[row]) - ((ws4[0] + ws4[1]) + (ws4[2] + ws4[3])));
  }
}

// Complex: rho = rho_B - rho_C summed over each chunk (fp64)
__global__ __launch_bounds__(kQ) void ssd_cplx_rho_total_kernel(
    const float* __restrict__ rhoB, const float* __restrict__ rhoC, double* __restrict__ rtot, int T,
    int H, int nc) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = c * kQ + threadIdx.x;
  const size_t row = (static_cast<size_t>(b) * T + (t < T ? t : 0)) * H + h;
  double v = t < T ? static_cast<double>(rhoB[row]) - rhoC[row] : 0.0;
  v = wave_inclusive_sum_d(v);
  if (threadIdx.x == kQ - 1) rtot[(static_cast<size_t>(b) * H + h) * nc + c] = v;
}

// ---------------------------------------------------------------------------
// Step-size gradients of one chunk (64 tokens, one wave): fp64 scans of f1
// (suffix), f2 (exclusive prefix) and col - row (exclusive prefix, the box),
// da_t, then d delta_t = A da_t + x.v (real) or alpha da_t + beta (the suffix
// of rho over the rest of the sequence) (complex), ddt through the clamp and
// the softplus, and the chunk's shares of dA (or d alpha), ddt_bias, dD,
// d beta.
// ---------------------------------------------------------------------------
template <bool CPLX>
__global__ __launch_bounds__(kQ) void ssd_f32_dt_kernel(
    const float* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ dt_bias,
    float dt_min, float dt_max, const float* __restrict__ f1, const float* __restrict__ f2,
    const float* __restrict__ colp, const float* __restrict__ rowp, const float* __restrict__ xv,
    const float* __restrict__ dyx, const double* __restrict__ cpart, const float* __restrict__ decay,
    int nblk, const float* __restrict__ rhoB, const float* __restrict__ rhoC, const double* __restrict__ rtot,
    const double* __restrict__ u, float* __restrict__ ddt, double* __restrict__ part, int T, int H, int nc) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t bhc = bh * nc + c;
  // the chunk constant e^{tot} <R_c, H_in(c)> from the adjoint passing's shares
  double cst_c = 0.0;
  for (int k = 0; k < nblk; ++k) cst_c += cpart[bhc * nblk + k];
  cst_c *= static_cast<double>(decay[bhc * 2]);
  const int t = c * kQ + lane;
  const bool in = t < T;
  const size_t row = (static_cast<size_t>(b) * T + (in ? t : 0)) * H + h;
  const float a_re = CPLX ? A[2 * h] : A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  const double f1v = in ? static_cast<double>(f1[row]) : 0.0;
  const double f2v = in ? static_cast<double>(f2[row]) : 0.0;
  const double gv = in ? static_cast<double>(colp[row]) - rowp[row] : 0.0;
  const double rv = CPLX && in ? static_cast<double>(rhoB[row]) - rhoC[row] : 0.0;
  const double s1 = wave_inclusive_sum_d(f1v), s2 = wave_inclusive_sum_d(f2v);
  const double s3 = wave_inclusive_sum_d(gv), s4 = wave_inclusive_sum_d(rv);
  const double f1_total = __shfl(s1, kQ - 1), r_total = __shfl(s4, kQ - 1);
  const double f1_suffix = f1_total - s1 + f1v;
  const double f2_prefix = s2 - f2v;
  const double box = s3 - gv;
  double after = 0.0;  // rho of the later chunks
  if constexpr (CPLX) {
    for (int cc = c + 1 + lane; cc < nc; cc += kQ) after += rtot[bh * nc + cc];
    after = __shfl(wave_inclusive_sum_d(after), kQ - 1);
  }
  double sA = 0.0, sBias = 0.0, sD = 0.0, sBeta = 0.0;
  if (in) {
    const double da = box + f1_suffix + f2_prefix + cst_c;
    const float z = dt[row] + bias;
    const float d = step_size(dt[row], bias, dt_min, dt_max);
    const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
    const bool pass = sp >= dt_min && sp <= dt_max;
    double dd = static_cast<double>(a_re) * da;
    if constexpr (CPLX)
      dd += static_cast<double>(A[2 * h + 1]) * (r_total - s4 + rv + after);
    else
      dd += xv[row];
    const double gz = pass ? dd / (1.0 + exp(-static_cast<double>(z))) : 0.0;
    ddt[row] = static_cast<float>(gz);
    sA = static_cast<double>(d) * da;
    sBias = gz;
    if constexpr (CPLX)
      sBeta = u[row] * rv;
    else
      sD = dyx[row];
  }
  sA = wave_inclusive_sum_d(sA);
  sBias = wave_inclusive_sum_d(sBias);
  sD = wave_inclusive_sum_d(sD);
  sBeta = wave_inclusive_sum_d(sBeta);
  if (lane == kQ - 1) {
    part[bhc * 4 + 0] = sA;
    part[bhc * 4 + 1] = sBias;
    part[bhc * 4 + 2] = sD;
    part[bhc * 4 + 3] = sBeta;
  }
}

// per head (one workgroup each): dA (complex: (d alpha, d beta)), ddt_bias, dD
// from the chunk shares of every sequence (fp64)
template <bool CPLX>
__global__ __launch_bounds__(kThreads) void ssd_f32_dt_sum_kernel(
    const double* __restrict__ part, float* __restrict__ dA, float* __restrict__ ddt_bias,
    float* __restrict__ dD, int Bsz, int H, int nc) {
  __shared__ double ws4[4][4];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid / kWave;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int i = tid; i < Bsz * nc; i += kThreads) {
    const int b = i / nc, c = i % nc;
    const double2* pp = reinterpret_cast<const double2*>(part + ((static_cast<size_t>(b) * H + h) * nc + c) * 4);
    const double2 lo = pp[0], hi = pp[1];
    s[0] += lo.x;
    s[1] += lo.y;
    s[2] += hi.x;
    s[3] += hi.y;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s[k] = wave_inclusive_sum_d(s[k]);
    if (lane == kWave - 1) ws4[wid][k] = s[k];
  }
  __syncthreads();
  if (tid != 0) return;
#pragma unroll
  for (int k = 0; k < 4; ++k) s[k] = (ws4[0][k] + ws4[1][k]) + (ws4[2][k] + ws4[3][k]);
  if constexpr (CPLX) {
    dA[2 * h] = static_cast<float>(s[0]);
    dA[2 * h + 1] = static_cast<float>(s[3]);
  } else {
    dA[h] = static_cast<float>(s[0]);
    if (dD) dD[h] = static_cast<float>(s[2]);
  }
  ddt_bias[h] = static_cast<float>(s[1]);
}

// dB, dC of each group: the sum over its heads of the per-head gradients
// (complex: each head's rotated back to the original frame first, out as
// (re, im) pairs).  One thread per (b, t, g, n) (real: 4 n).
template <bool CPLX>
__global__ __launch_bounds__(kThreads) void ssd_f32_group_sum_kernel(
    const float* __restrict__ dBh, const float* __restrict__ dCh, const float2* __restrict__ rot,
    float* __restrict__ dB, float* __restrict__ dC, size_t rows, int H, int G, int N) {
  const int hpg = H / G;
  const int NE = CPLX ? 2 * N : N;
  const int per = CPLX ? N : N / 4;  // threads per (b, t, g) row
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= rows * G * per) return;
  const size_t bt = i / (static_cast<size_t>(G) * per);
  const int g = static_cast<int>((i / per) % G), k = static_cast<int>(i % per);
  if constexpr (CPLX) {
    float br = 0.f, bi = 0.f, cr = 0.f, ci = 0.f;
    for (int e = 0; e < hpg; ++e) {
      const int h = g * hpg + e;
      const size_t hr = (bt * H + h) * NE;
      const float2 r = rot[bt * H + h];
      const float co = r.x, si = r.y;
      // dB = e^{i theta} (dB_eff[n] + i dB_eff[N+n]); dC = e^{-i theta} (dC_eff[n] - i dC_eff[N+n])
      const float xr = dBh[hr + k], xi = dBh[hr + N + k];
      br += xr * co - xi * si;
      bi += xr * si + xi * co;
      const float yr = dCh[hr + k], yi = -dCh[hr + N + k];
      cr += yr * co + yi * si;
      ci += yi * co - yr * si;
    }
    const size_t o = ((bt * G + g) * N + k) * 2;
    dB[o] = br;
    dB[o + 1] = bi;
    dC[o] = cr;
    dC[o + 1] = ci;
  } else {
    float4 sb = make_float4(0.f, 0.f, 0.f, 0.f), sc = sb;
    for (int e = 0; e < hpg; ++e) {
      const size_t hr = (bt * H + g * hpg + e) * NE + 4 * k;
      const float4 vb = *reinterpret_cast<const float4*>(dBh + hr);
      const float4 vc = *reinterpret_cast<const float4*>(dCh + hr);
      sb = make_float4(sb.x + vb.x, sb.y + vb.y, sb.z + vb.z, sb.w + vb.w);
      sc = make_float4(sc.x + vc.x, sc.y + vc.y, sc.z + vc.z, sc.w + vc.w);
    }
    const size_t o = (bt * G + g) * N + 4 * k;
    *reinterpret_cast<float4*>(dB + o) = sb;
    *reinterpret_cast<float4*>(dC + o) = sc;
  }
}

// complex dh0 from the rotated-frame [Re | Im] rows
__global__ __launch_bounds__(kThreads) void ssd_cplx_dh0_kernel(const float* __restrict__ dh0e,
                                                                 float* __restrict__ dh0, size_t total,
                                                                 int N) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;  // (b, h, p, n)
  if (i >= total) return;
  const size_t bhp = i / N;
  const int n = static_cast<int>(i % N);
  dh0[i * 2] = dh0e[bhp * 2 * N + n];
  dh0[i * 2 + 1] = dh0e[bhp * 2 * N + N + n];
}

// ---------------------------------------------------------------------------
// Workspace of the fp32 backward (256-byte aligned regions): chunk states
// (recomputed; h_in over them), decays, adjoint states (R over G), per-head
// dB and dC, per-token values (f1, f2, col, row, x.v, dy.x, rho_B, rho_C),
// chunk constants and shares; complex: u, (cos, sin) theta, alpha, rotated h0,
// dh_final and h_final, rho chunk totals.
// ---------------------------------------------------------------------------
struct F32BwdLayout {
  size_t S, dec, adj, dBh, dCh, tokv, cst, part, u, rot, alpha, h0e, dhfe, hfe, rtot, dh0e, total;
};
static F32BwdLayout f32_layout(int Bsz, int T, int H, int P, int N, bool cplx) {
  const int NE = cplx ? 2 * N : N;
  const int nc = (T + kQ - 1) / kQ;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  F32BwdLayout L{};
  size_t o = 0;
  const size_t st = static_cast<size_t>(Bsz) * nc * H * P * NE * 4;
  const size_t tok = static_cast<size_t>(Bsz) * T * H;
  L.S = o;    o += up(st);
  L.dec = o;  o += up(static_cast<size_t>(Bsz) * H * nc * 8);
  L.adj = o;  o += up(st);
  L.dBh = o;  o += up(tok * NE * 4);
  L.dCh = o;  o += up(tok * NE * 4);
  L.tokv = o; o += up(tok * 4 * 8);
  L.cst = o;  o += up(static_cast<size_t>(Bsz) * H * nc * 8 * ((P * NE / 4 + kThreads - 1) / kThreads));
  L.part = o; o += up(static_cast<size_t>(Bsz) * H * nc * 32);
  if (cplx) {
    const size_t hs = static_cast<size_t>(Bsz) * H * P * NE * 4;
    L.u = o;     o += up(tok * 8);
    L.rot = o;   o += up(tok * 8);
    L.alpha = o; o += up(static_cast<size_t>(H) * 4);
    L.h0e = o;   o += up(hs);
    L.dhfe = o;  o += up(hs);
    L.hfe = o;   o += up(hs);
    L.dh0e = o;  o += up(hs);
    L.rtot = o;  o += up(static_cast<size_t>(Bsz) * H * nc * 8);
  }
  L.total = o + 256;
  return L;
}

size_t bwd_f32_workspace_bytes(int Bsz, int T, int H, int P, int G, int N, bool cplx) {
  (void)G;
  return f32_layout(Bsz, T, H, P, N, cplx).total;
}

namespace {

// the chunk-local part shared by both forms: block kernels, chunk constants,
// step sizes, their sums
template <int P, int NE, bool CPLX>
hipError_t launch_f32_core(const float* x, const float* dt, const float* A_dec, const float* A_dt,
                           const float* dt_bias, float dt_min, float dt_max, const float* Bin,
                           const float* Cin, int Geff, const float* dy, const float* D,
                           float* dx, float* ddt, float* dA, float* dD, float* ddt_bias, float* dBh,
                           float* dCh, const float2* rot, float* dBo, float* dCo, char* ws,
                           const F32BwdLayout& L, int Bsz, int T, int H, hipStream_t st,
                           const hipEvent_t* ev) {
  auto E = [&](int k) { return ev ? ev + 2 * k : nullptr; };
  const int nc = (T + kQ - 1) / kQ;
  const size_t tok = static_cast<size_t>(Bsz) * T * H;
  float* tv = reinterpret_cast<float*>(ws + L.tokv);
  float *f1 = tv, *f2 = tv + tok, *col = tv + 2 * tok, *rw = tv + 3 * tok, *xv = tv + 4 * tok,
        *dyx = tv + 5 * tok, *rhoB = tv + 6 * tok, *rhoC = tv + 7 * tok;
  const float* S = reinterpret_cast<const float*>(ws + L.S);
  const float* dec = reinterpret_cast<const float*>(ws + L.dec);
  const float* adj = reinterpret_cast<const float*>(ws + L.adj);
  double* cst = reinterpret_cast<double*>(ws + L.cst);
  double* part = reinterpret_cast<double*>(ws + L.part);
  const dim3 grid(nc > 0 ? nc : 1, H, Bsz);
  constexpr bool SCALE = !CPLX;
  const bool run = nc > 0;
  launch_k(run, ssd_f32_col_kernel<P, NE, SCALE, CPLX>, grid, dim3(kT8), st, E(5), x, dt, A_dec,
           dt_bias, dt_min, dt_max, Bin, Cin, dy, D, adj, dx, dBh, f2, col, xv, dyx, rhoB, rot, dBo, T, H,
           Geff, nc);
  launch_k(run, ssd_f32_row_kernel<P, NE, SCALE, CPLX>, grid, dim3(kT8), st, E(6), x, dt, A_dec,
           dt_bias, dt_min, dt_max, Bin, Cin, dy, S, dCh, f1, rw, rhoC, rot, dCo, T, H, Geff,
           nc);
  // (the chunk constants come from the adjoint passing: slot 7 records back to back)
  launch_k(false, ssd_f32_dt_sum_kernel<CPLX>, dim3(1), dim3(kThreads), st, E(7), nullptr, nullptr, nullptr,
           nullptr, 0, 0, 0);
  launch_k(CPLX, ssd_cplx_tau_kernel, dim3(H, Bsz), dim3(kThreads), st, E(8),
           reinterpret_cast<const float*>(ws + L.dhfe), reinterpret_cast<const float*>(ws + L.hfe), rhoB,
           T, H, P, NE / 2);
  launch_k(CPLX && run, ssd_cplx_rho_total_kernel, grid, dim3(kQ), st, E(9), static_cast<const float*>(rhoB),
           static_cast<const float*>(rhoC), reinterpret_cast<double*>(ws + L.rtot), T, H, nc);
  launch_k(run, ssd_f32_dt_kernel<CPLX>, grid, dim3(kQ), st, E(10), dt, A_dt, dt_bias, dt_min, dt_max,
           static_cast<const float*>(f1), static_cast<const float*>(f2), static_cast<const float*>(col),
           static_cast<const float*>(rw), static_cast<const float*>(xv), static_cast<const float*>(dyx),
           static_cast<const double*>(cst), dec, (P * NE / 4 + kThreads - 1) / kThreads,
           static_cast<const float*>(rhoB), static_cast<const float*>(rhoC),
           CPLX ? reinterpret_cast<const double*>(ws + L.rtot) : nullptr,
           CPLX ? reinterpret_cast<const double*>(ws + L.u) : nullptr, ddt, part, T, H, nc);
  launch_k(true, ssd_f32_dt_sum_kernel<CPLX>, dim3(H), dim3(kThreads), st, E(11), static_cast<const double*>(part), dA, ddt_bias, dD, Bsz, H, nc);
  return hipGetLastError();
}

}  // namespace

template <int P, int N>
static hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st) {
  const int nc = (a.T + kQ - 1) / kQ;
  const hipEvent_t* ev = a.events;
  auto E = [&](int k) { return ev ? ev + 2 * k : nullptr; };
  launch_k(false, ssd_cplx_dh0_kernel, dim3(1), dim3(kThreads), st, E(0), nullptr, nullptr, size_t{0}, 0);
  const F32BwdLayout L = f32_layout(a.Bsz, a.T, a.H, P, N, false);
  char* ws = static_cast<char*>(a.workspace);
  float* S = reinterpret_cast<float*>(ws + L.S);
  float* dec = reinterpret_cast<float*>(ws + L.dec);
  float* adj = reinterpret_cast<float*>(ws + L.adj);
  const float* x = static_cast<const float*>(a.x);
  const float* B = static_cast<const float*>(a.B);
  const float* C = static_cast<const float*>(a.C);
  const float* dy = static_cast<const float*>(a.dy);
  hipError_t e = run_states_f32(x, a.dt, a.A, B, a.dt_bias, a.dt_min, a.dt_max, S, dec, a.Bsz, a.T, a.H,
                                P, a.G, N, kQ, 0, nullptr, st, E(1));
  if (e == hipSuccess) e = run_pass_f32(S, dec, a.h0, nullptr, a.Bsz, a.H, P, N, nc, st, E(2));
  if (e == hipSuccess)
    e = run_states_f32(dy, a.dt, a.A, C, a.dt_bias, a.dt_min, a.dt_max, adj, nullptr, a.Bsz, a.T, a.H, P,
                       a.G, N, kQ, 2, nullptr, st, E(3));
  if (e != hipSuccess) return e;
  launch_k(true, ssd_f32_adj_pass_kernel, dim3((P * N / 4 + kThreads - 1) / kThreads, a.H, a.Bsz),
           dim3(kThreads), st, E(4), adj, static_cast<const float*>(dec), a.dh_final, a.dh0,
           static_cast<const float*>(S), reinterpret_cast<double*>(ws + L.cst), a.H, P * N, nc);
  // each head its own group: the per-head gradients are the outputs
  const bool direct = a.G == a.H;
  float* dBh = direct ? a.dB : reinterpret_cast<float*>(ws + L.dBh);
  float* dCh = direct ? a.dC : reinterpret_cast<float*>(ws + L.dCh);
  e = launch_f32_core<P, N, false>(x, a.dt, a.A, a.A, a.dt_bias, a.dt_min, a.dt_max, B, C, a.G, dy, a.D,
                                   static_cast<float*>(a.dx), a.ddt, a.dA, a.dD, a.ddt_bias, dBh, dCh,
                                   nullptr, nullptr, nullptr, ws, L, a.Bsz, a.T, a.H, st, ev);
  if (e != hipSuccess) return e;
  const size_t rows = static_cast<size_t>(a.Bsz) * a.T;
  const size_t nthreads = direct ? 0 : rows * a.G * (N / 4);
  launch_k(false, ssd_cplx_dh0_kernel, dim3(1), dim3(kThreads), st, E(13), nullptr, nullptr, size_t{0}, 0);
  launch_k(nthreads > 0, ssd_f32_group_sum_kernel<false>,
           dim3(static_cast<unsigned>((nthreads + kThreads - 1) / kThreads)), dim3(kThreads), st, E(12),
           reinterpret_cast<const float*>(ws + L.dBh), reinterpret_cast<const float*>(ws + L.dCh),
           static_cast<const float2*>(nullptr), a.dB, a.dC, rows, a.H, a.G, N);
  return hipGetLastError();
}

hipError_t run_chunk_bwd_f32(const BwdArgs& a, hipStream_t st) {
  if (a.P == 64 && a.N == 128) return launch_bwd_f32<64, 128>(a, st);
  if (a.P == 64 && a.N == 64) return launch_bwd_f32<64, 64>(a, st);
  if (a.P == 64 && a.N == 32) return launch_bwd_f32<64, 32>(a, st);
  if (a.P == 32 && a.N == 128) return launch_bwd_f32<32, 128>(a, st);
  if (a.P == 32 && a.N == 64) return launch_bwd_f32<32, 64>(a, st);
  if (a.P == 32 && a.N == 32) return launch_bwd_f32<32, 32>(a, st);
  return hipErrorInvalidValue;
}

template <int P, int N>
static hipError_t launch_cplx_bwd(const CplxBwdArgs& a, hipStream_t st) {
  constexpr int NE = 2 * N;
  const int nc = (a.T + kQ - 1) / kQ;
  const hipEvent_t* ev = a.events;
  auto E = [&](int k) { return ev ? ev + 2 * k : nullptr; };
  const F32BwdLayout L = f32_layout(a.Bsz, a.T, a.H, P, N, true);
  char* ws = static_cast<char*>(a.workspace);
  float* S = reinterpret_cast<float*>(ws + L.S);
  float* dec = reinterpret_cast<float*>(ws + L.dec);
  float* adj = reinterpret_cast<float*>(ws + L.adj);
  double* u = reinterpret_cast<double*>(ws + L.u);
  float* alpha = reinterpret_cast<float*>(ws + L.alpha);
  float* h0e = reinterpret_cast<float*>(ws + L.h0e);
  float* dhfe = reinterpret_cast<float*>(ws + L.dhfe);
  float* hfe = reinterpret_cast<float*>(ws + L.hfe);
  float* dh0e = reinterpret_cast<float*>(ws + L.dh0e);
  float2* rot = reinterpret_cast<float2*>(ws + L.rot);
  // the sequence frame (event slot 0)
  launch_k(true, ssd_cplx_frame_kernel, dim3(a.H, a.Bsz), dim3(kFrameThreads), st, E(0), a.dt, a.dt_bias, a.dt_min,
           a.dt_max, a.A, a.h0, a.dh_final, u, rot, alpha, h0e, dhfe, a.T, a.H, P, N);
  // the rotated-frame real problem: 2N features (B and C rotated as they are
  // staged), decay alpha, input scale 1
  const float2* rotc = rot;
  hipError_t e = run_states_f32(a.x, a.dt, alpha, a.B, a.dt_bias, a.dt_min, a.dt_max, S, dec, a.Bsz, a.T,
                                a.H, P, a.G, NE, kQ, 3, rotc, st, E(1));
  if (e == hipSuccess) e = run_pass_f32(S, dec, h0e, hfe, a.Bsz, a.H, P, NE, nc, st, E(2));
  if (e == hipSuccess)
    e = run_states_f32(a.dy, a.dt, alpha, a.C, a.dt_bias, a.dt_min, a.dt_max, adj, nullptr, a.Bsz, a.T,
                       a.H, P, a.G, NE, kQ, 4, rotc, st, E(3));
  if (e != hipSuccess) return e;
  launch_k(true, ssd_f32_adj_pass_kernel, dim3((P * NE / 4 + kThreads - 1) / kThreads, a.H, a.Bsz),
           dim3(kThreads), st, E(4), adj, static_cast<const float*>(dec), static_cast<const float*>(dhfe),
           dh0e, static_cast<const float*>(S), reinterpret_cast<double*>(ws + L.cst), a.H, P * NE, nc);
  // each head its own group: dB, dC rotated back and written by the block kernels
  const bool direct = a.G == a.H;
  e = launch_f32_core<P, NE, true>(a.x, a.dt, alpha, a.A, a.dt_bias, a.dt_min, a.dt_max, a.B, a.C, a.G,
                                   a.dy, nullptr, a.dx, a.ddt, a.dA, nullptr, a.ddt_bias,
                                   reinterpret_cast<float*>(ws + L.dBh), reinterpret_cast<float*>(ws + L.dCh),
                                   rot, direct ? a.dB : nullptr, direct ? a.dC : nullptr, ws, L, a.Bsz, a.T,
                                   a.H, st, ev);
  if (e != hipSuccess) return e;
  const size_t rows = static_cast<size_t>(a.Bsz) * a.T;
  const size_t nthreads = direct ? 0 : rows * a.G * N;
  launch_k(nthreads > 0, ssd_f32_group_sum_kernel<true>,
           dim3(static_cast<unsigned>((nthreads + kThreads - 1) / kThreads)), dim3(kThreads), st, E(12),
           reinterpret_cast<const float*>(ws + L.dBh), reinterpret_cast<const float*>(ws + L.dCh),
           static_cast<const float2*>(rot), a.dB, a.dC, rows, a.H, a.G, N);
  const size_t total = static_cast<size_t>(a.Bsz) * a.H * P * N;
  launch_k(a.dh0 != nullptr, ssd_cplx_dh0_kernel,
           dim3(static_cast<unsigned>((total + kThreads - 1) / kThreads)), dim3(kThreads), st, E(13),
           static_cast<const float*>(dh0e), a.dh0, total, N);
  return hipGetLastError();
}

hipError_t run_complex_bwd(const CplxBwdArgs& a, hipStream_t st) {
  if (a.P == 64 && a.N == 64) return launch_cplx_bwd<64, 64>(a, st);
  if (a.P == 64 && a.N == 32) return launch_cplx_bwd<64, 32>(a, st);
  if (a.P == 64 && a.N == 16) return launch_cplx_bwd<64, 16>(a, st);
  if (a.P == 32 && a.N == 64) return launch_cplx_bwd<32, 64>(a, st);
  if (a.P == 32 && a.N == 32) return launch_cplx_bwd<32, 32>(a, st);
  if (a.P == 32 && a.N == 16) return launch_cplx_bwd<32, 16>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ssd
