// Bias-free linear layers of the Mamba-3-Lite block on gfx950: z = x W^T
// row by row (out[m][n] = sum_k x[m][k] W[n][k], W stored (out, in) as the
// block's Linear layers store it).  The MIMO head mixer is this map on the
// scan output flattened per token to H*P features, head-major, with W of
// (H*P, H*P); out_proj is the same map with W of (d_model, H*P) (Block
// Anatomy, section 6, rows 9-10; Numerical Stability in Mamba-3-Lite, section
// 3.1: these projections run in bf16 under autocast, fp32 accumulation).
//
// One workgroup per 128 x 128 output tile (4 waves, 2 x 2, each 64 x 64), K in
// steps of 64 staged through two LDS sets (rows K-contiguous for both
// operands, so the matrix-core fragments are plain 16-byte row reads): step s
// is multiplied from one set while step s + 1, loaded into registers a step
// earlier, is written into the other, one barrier per step.  x may be fp32
// (rounded to bf16, nearest even, as it is staged) or bf16; W is bf16.
//
// The product is formed transposed, Z^T[n][m] = W[n][.] x[m][.]: a lane's
// accumulator holds one m and four n of a 16 x 16 tile, and the two n tiles of
// a pair are permuted (tile t covers n = 32 pair + 4 t + 8 (r / 4) + r % 4 for
// its row r), so that a lane holds 8 consecutive n: one 16-byte store of bf16
// z (two of fp32).  Workgroup order: the Nout / 128 tiles of one block of 128
// rows run on one XCD, one after another, so x's rows are fetched from HBM once
// and then served from that XCD's L2; W (at most a few MB) stays in every L2.

#include "ssd_chunk_common.h"

namespace ssd {

namespace {

constexpr int kLinBM = 128, kLinBN = 128, kLinBK = 64;
constexpr int kLinPitch = kLinBK + 16;  // bf16 elements: 160-byte rows

}  // namespace

template <bool XF32, bool ZF32>
__global__ __launch_bounds__(kThreads, 2) void ssd_linear_kernel(
    const void* __restrict__ xv, const uint16_t* __restrict__ W, void* __restrict__ zv, int M,
    int K, int Nout, int mblocks, int nblocks) {
  // two LDS sets: step s is multiplied from one while step s + 1 is staged
  // into the other (one barrier per step; 80 KB: two workgroups per CU)
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][kLinBM * kLinPitch];
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][kLinBN * kLinPitch];

  // tile of this workgroup: the row blocks are spread over the XCDs, and the
  // output blocks of one row block follow each other on its XCD
  const int id = blockIdx.x;
  const int slot = id / kXCD;
  const int mb = id % kXCD + kXCD * (slot / nblocks);
  const int nb = slot % nblocks;
  if (mb >= mblocks) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane >> 4, r16 = lane & 15;
  const int wid = wave_id();
  const int wm = wid & 1, wn = wid >> 1;  // this wave's 64 x 64 block

  constexpr int XES = XF32 ? 4 : 2;  // bytes per x element
  const size_t m0 = static_cast<size_t>(mb) * kLinBM;
  const int rows = min(kLinBM, M - static_cast<int>(m0));
  const uint32_t xrow = static_cast<uint32_t>(K) * XES;
  const buf_t xbuf = make_buf(static_cast<const char*>(xv) + m0 * xrow,
                              static_cast<uint32_t>(rows) * xrow);
  const uint32_t wrow = static_cast<uint32_t>(K) * 2;
  const buf_t wbuf = make_buf(W + static_cast<size_t>(nb) * kLinBN * K, kLinBN * wrow);

  // one K step of both tiles, in registers: x as XVPT 16-byte pieces per thread
  // (fp32: 16 per row, bf16: 8 per row), W as 4
  constexpr int XVPR = kLinBK * XES / 16;        // 16-byte pieces per row
  constexpr int XVPT = kLinBM * XVPR / kThreads;  // per thread
  constexpr int WVPR = kLinBK * 2 / 16;
  constexpr int WVPT = kLinBN * WVPR / kThreads;
  uint4 xr[XVPT], wr[WVPT];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XVPT; ++i) {
      const int it = tid + i * kThreads;
      xr[i] = buf_load16(xbuf, static_cast<uint32_t>(it / XVPR) * xrow + (k0 * XES) + (it % XVPR) * 16);
    }
#pragma unroll
    for (int i = 0; i < WVPT; ++i) {
      const int it = tid + i * kThreads;
      wr[i] = buf_load16(wbuf, static_cast<uint32_t>(it / WVPR) * wrow + k0 * 2 + (it % WVPR) * 16);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XVPT; ++i) {
      const int it = tid + i * kThreads;
      const int row = it / XVPR, v = it % XVPR;
      if constexpr (XF32) {
        const uint4 u = xr[i];
        *reinterpret_cast<uint2*>(xl[buf] + row * kLinPitch + v * 4) =
            make_uint2(pack_bf16x2(__uint_as_float(u.x), __uint_as_float(u.y)),
                       pack_bf16x2(__uint_as_float(u.z), __uint_as_float(u.w)));
      } else {
        *reinterpret_cast<uint4*>(xl[buf] + row * kLinPitch + v * 8) = xr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < WVPT; ++i) {
      const int it = tid + i * kThreads;
      *reinterpret_cast<uint4*>(wl[buf] + (it / WVPR) * kLinPitch + (it % WVPR) * 8) = wr[i];
    }
  };

  f32x4 acc[4][4];  // [n tile][m tile]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / kLinBK;
  load(0);
  stage(0);
  if (nsteps > 1) load(kLinBK);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    // step s + 1 into the other set (its last reads were step s - 1's, before
    // the previous barrier), then the loads of step s + 2
    if (s + 1 < nsteps) {
      stage(cur ^ 1);
      if (s + 2 < nsteps) load((s + 2) * kLinBK);
    }
#pragma unroll
    for (int ks = 0; ks < kLinBK; ks += 32) {
      uint4 af[4], bf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // n tile t of the wave: pair t / 2, half t % 2, permuted rows
        const int nl = wn * 64 + 32 * (t >> 1) + 4 * (t & 1) + 8 * (r16 >> 2) + (r16 & 3);
        af[t] = *reinterpret_cast<const uint4*>(wl[cur] + nl * kLinPitch + ks + 8 * q);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        bf[mt] = *reinterpret_cast<const uint4*>(xl[cur] + (wm * 64 + mt * 16 + r16) * kLinPitch + ks + 8 * q);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[t][mt] = mfma_bf16(as_bf16x8(af[t]), as_bf16x8(bf[mt]), acc[t][mt]);
    }
    __syncthreads();  // step s + 1's set complete; step s's set free
  }

  // z rows out: lane holds row m = mb*128 + wm*64 + mt*16 + r16 and, per pair of
  // n tiles, n = nb*128 + wn*64 + 32 pair + 8q .. +7 (rows past M are dropped)
  constexpr int ZES = ZF32 ? 4 : 2;
  const uint32_t zrow = static_cast<uint32_t>(Nout) * ZES;
  const buf_t zbuf = make_buf(static_cast<char*>(zv) + m0 * zrow, static_cast<uint32_t>(rows) * zrow);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint32_t roff = static_cast<uint32_t>(wm * 64 + mt * 16 + r16) * zrow;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const f32x4 a = acc[2 * pr][mt], c = acc[2 * pr + 1][mt];
      const int n0 = nb * kLinBN + wn * 64 + 32 * pr + 8 * q;
      if constexpr (ZF32) {
        buf_store16(zbuf, roff + n0 * 4, __builtin_bit_cast(uint4, a));
        buf_store16(zbuf, roff + (n0 + 4) * 4, __builtin_bit_cast(uint4, c));
      } else {
        buf_store16(zbuf, roff + n0 * 2,
                    make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(c[0], c[1]),
                               pack_bf16x2(c[2], c[3])));
      }
    }
  }
}

hipError_t run_linear(const LinearArgs& a, hipStream_t st) {
  if (a.M == 0) {
    if (a.events) {
      (void)hipEventRecord(a.events[0], st);
      (void)hipEventRecord(a.events[1], st);
    }
    return hipSuccess;
  }
  const int mblocks = (a.M + kLinBM - 1) / kLinBM;
  const int nblocks = a.Nout / kLinBN;
  const unsigned grid = static_cast<unsigned>((mblocks + kXCD - 1) / kXCD) * kXCD * nblocks;
  const bool xf = a.x_dtype == 0, zf = a.z_dtype == 0;
  if (xf && zf)
    launch_k(true, ssd_linear_kernel<true, true>, dim3(grid), dim3(kThreads), st, a.events, a.x, a.W,
             a.z, a.M, a.K, a.Nout, mblocks, nblocks);
  else if (xf)
    launch_k(true, ssd_linear_kernel<true, false>, dim3(grid), dim3(kThreads), st, a.events, a.x, a.W,
             a.z, a.M, a.K, a.Nout, mblocks, nblocks);
  else if (zf)
    launch_k(true, ssd_linear_kernel<false, true>, dim3(grid), dim3(kThreads), st, a.events, a.x, a.W,
             a.z, a.M, a.K, a.Nout, mblocks, nblocks);
  else
    launch_k(true, ssd_linear_kernel<false, false>, dim3(grid), dim3(kThreads), st, a.events, a.x, a.W,
             a.z, a.M, a.K, a.Nout, mblocks, nblocks);
  return hipGetLastError();
}

}  // namespace ssd
