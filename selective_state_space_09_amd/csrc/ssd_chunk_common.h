// Shared device code of the chunked SSD kernels (gfx950): workgroup order,
// the per-chunk prologue (step sizes and cumulative decay exponents), register
// staging of token slabs, and the inter-chunk state-passing kernel.
#pragma once

#include <hip/hip_ext.h>

#include <type_traits>

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {

constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU
constexpr int kXCD = 8;    // XCDs of an MI355X

template <typename E>
struct Pad;
template <>
struct Pad<float> {
  static constexpr int row = 4;  // fp32 elements of padding per LDS row
};

// (b, c, h) of work unit `id` under the XCD-grouped order: consecutive ids go
// to consecutive XCDs, and the H heads of one (b, c) pair share an XCD (and
// its L2, which then serves their common B and C rows).  False for the
// padding units of the last, partial group of 8 (b, c) pairs.
__device__ __forceinline__ bool unit_coords(int id, int H, int nc, int npairs, int& b, int& c,
                                            int& h) {
  const int k = id / kXCD;
  const int j = (id % kXCD) + kXCD * (k / H);
  h = k % H;
  if (j >= npairs) return false;
  b = j / nc;
  c = j % nc;
  return true;
}
__device__ __forceinline__ bool unit_of_block(int H, int nc, int npairs, int& b, int& c, int& h) {
  return unit_coords(blockIdx.x, H, nc, npairs, b, c, h);
}

// Variable-length batches of the bf16 real forward: sequence b holds the token
// rows cu[b] .. cu[b+1]-1 of the packed inputs; its segments (of K chunks,
// the last one possibly shorter) are the global segments segstart[b] ..
// segstart[b+1]-1, and seg[j] = (b, segment of b) of global segment j, or
// (-1, -1) for the padding past the last one.  With cu == nullptr every
// sequence has T tokens and global segment j is (j / nseg, j % nseg).
struct VarLen {
  const int* cu;
  const int2* seg;
  const int* segstart;
};

// The segment a workgroup works on: sequence b, segment sg of it, head (or
// head group) h under the XCD-grouped order of unit_coords; gs its global
// segment index (states, h_in); row0 the sequence's first token row, T its
// length.  False for padding units.
struct SegView {
  int b, sg, h, gs, T;
  size_t row0;
};
__device__ __forceinline__ bool seg_of_block(const VarLen& v, int Hu, int T, int nseg, int npairs,
                                             SegView& s) {
  const int id = blockIdx.x;
  const int k = id / kXCD;
  const int j = (id % kXCD) + kXCD * (k / Hu);
  s.h = k % Hu;
  if (j >= npairs) return false;
  s.gs = j;
  if (v.cu) {
    const int2 e = v.seg[j];
    if (e.x < 0) return false;
    s.b = e.x;
    s.sg = e.y;
    const int r = v.cu[e.x];
    s.row0 = static_cast<size_t>(r);
    s.T = v.cu[e.x + 1] - r;
  } else {
    s.b = j / nseg;
    s.sg = j % nseg;
    s.row0 = static_cast<size_t>(s.b) * T;
    s.T = T;
  }
  return true;
}


// Launch of one kernel of a forward call.  With a start/stop event pair
// (ev != NULL) the events are bound to the kernel's own dispatch
// (hipExtLaunchKernelGGL), so that they time the kernel alone; a kernel that
// is not run (run == false) records its pair back to back.
template <typename F, typename... Args>
inline void launch_k(bool run, F kernel, dim3 grid, dim3 block, hipStream_t st,
                     const hipEvent_t* ev, Args... args) {
  if (!run) {
    if (ev) {
      (void)hipEventRecord(ev[0], st);
      (void)hipEventRecord(ev[1], st);
    }
    return;
  }
  if (ev)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev[0], ev[1], 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// ---------------------------------------------------------------------------
// Per-chunk prologue of the fp32 kernels: step sizes and cumulative decay
// exponents.
//
// Thread l < Q handles token l of the chunk (l >= Lc is padding: step 0); d is
// its raw dt (loaded by the caller, ignored for l >= Lc).  Writes dl[l] (step
// size) and cs_hi/cs_lo[l] (double-float of the inclusive cumulative exponent
// A*sum(delta)).  Returns this thread's cumulative exponent (double) and
// stores the chunk total in *tot.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double chunk_prologue(float dt_raw, int Lc, float a_re, float bias,
                                                 float lo, float hi, float* dl, float* cs_hi,
                                                 float* cs_lo, double* wsum, double* tot, int Q) {
  const int l = threadIdx.x;
  // (computed in every lane, then selected: a use under a branch would pull
  // the caller's dt load into that branch, behind every load issued before it)
  const float dv = step_size(dt_raw, bias, lo, hi);
  const float d = l < Lc ? dv : 0.0f;
  const double cum = block_inclusive_scan(static_cast<double>(a_re) * static_cast<double>(d), wsum);
  if (l < Q) {
    dl[l] = d;
    const float ehi = static_cast<float>(cum);
    cs_hi[l] = ehi;
    cs_lo[l] = static_cast<float>(cum - static_cast<double>(ehi));
    if (l == Q - 1) *tot = cum;
  }
  __syncthreads();
  return cum;
}

// exp(cs_l - cs_s) from double-float exponents.
__device__ __forceinline__ float decay_between(float hl, float ll, float hs, float ls) {
  return __expf((hl - hs) + (ll - ls));
}

// ---------------------------------------------------------------------------
// An ST-token slab of one row-major array, fetched into registers as 16-byte
// vectors: item it -> rows (RPI of them) and vector v = it % VPR of those rows.
// Rows at or past Lc read as zero.  All loads of a slab are issued together.
// ---------------------------------------------------------------------------
template <int ST, int VPR, int RPI>
struct Slab {
  static constexpr int ITEMS = (ST / RPI) * VPR;
  static constexpr int PER = (ITEMS + kThreads - 1) / kThreads;
  uint4 v[PER][RPI];

  // base: first element of token s0 = 0 of the chunk slice, in bytes;
  // row_bytes: stride between tokens in bytes.
  __device__ __forceinline__ void load(const char* __restrict__ base, size_t row_bytes, int s0,
                                       int Lc) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      const int vv = it % VPR, rg = it / VPR;
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        const int s = s0 + rg * RPI + r;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (it < ITEMS && s < Lc)
          val = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(s) * row_bytes + vv * 16);
        v[i][r] = val;
      }
    }
  }

  // the same with rows at or past Lc (>= 1) read as row Lc - 1 instead of
  // zero: no load under a branch (which ends in a wait for it where the
  // branch joins), for callers whose products weight those rows by zero
  __device__ __forceinline__ void load_clamped(const char* __restrict__ base, size_t row_bytes, int s0,
                                               int Lc) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      const int vv = it % VPR, rg = it / VPR;
#pragma unroll
      for (int r = 0; r < RPI; ++r) {
        const int s = min(s0 + rg * RPI + r, Lc - 1);
        if (ITEMS % kThreads == 0 || it < ITEMS)
          v[i][r] = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(s) * row_bytes + vv * 16);
      }
    }
  }
};

// The same slab fetched through a buffer descriptor: rows at or past the
// described range read as zero (no per-row test).  voff: byte offset of token
// s0 = 0 of the slab's rows in the descriptor.
template <int ST, int VPR, int NTHR = kThreads>
struct BufSlab {
  static constexpr int ITEMS = ST * VPR;
  static constexpr int PER = (ITEMS + NTHR - 1) / NTHR;
  uint4 v[PER];

  __device__ __forceinline__ void load(buf_t r, uint32_t row_bytes, int s0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = threadIdx.x + i * NTHR;
      const int vv = it % VPR, rg = it / VPR;
      if (ITEMS % NTHR == 0 || it < ITEMS)
        v[i] = buf_load16(r, static_cast<uint32_t>(s0 + rg) * row_bytes + vv * 16);
    }
  }
};

// x slab -> xT[p][s - s0]  (transposed, s contiguous).
template <int ST, int P>
struct XSlabF32 : Slab<ST, P / 4, 1> {
  __device__ __forceinline__ void store(float* xT) const {
    constexpr int XP = ST + Pad<float>::row;
#pragma unroll
    for (int i = 0; i < this->PER; ++i) {
      const int it = threadIdx.x + i * kThreads;
      if (it >= this->ITEMS) break;
      const int pg = it % (P / 4), sl = it / (P / 4);
      const uint4 u = this->v[i][0];
      xT[(pg * 4 + 0) * XP + sl] = __uint_as_float(u.x);
      xT[(pg * 4 + 1) * XP + sl] = __uint_as_float(u.y);
      xT[(pg * 4 + 2) * XP + sl] = __uint_as_float(u.z);
      xT[(pg * 4 + 3) * XP + sl] = __uint_as_float(u.w);
    }
  }
};

// ---------------------------------------------------------------------------
// Kernel 2: inter-chunk scan of states, in place.
//   states[b][c][h] : S_c on entry, h_in(c) on exit.
// Real: one thread per 4 consecutive (p, n).  Complex: one thread per 4
// consecutive n of one p, re and im together (planar re | im in the
// workspace; h0/h_final interleaved (re, im) as complex64).
// ---------------------------------------------------------------------------
template <bool CPLX, int N>
__global__ __launch_bounds__(kThreads) void ssd_pass_kernel(
    float* __restrict__ states, const float* __restrict__ decay, const float* __restrict__ h0,
    float* __restrict__ h_final, int H, int P, int nc) {
  constexpr int KC = CPLX ? 2 * N : N;
  constexpr int PF = 4;  // chunks in flight per thread
  const int h = blockIdx.y, b = blockIdx.z;
  const int e4 = blockIdx.x * kThreads + threadIdx.x;  // group of 4 elements
  const int groups = P * N / 4;
  if (e4 >= groups) return;
  const int p = (e4 * 4) / N, n = (e4 * 4) % N;
  const size_t chunk_stride = static_cast<size_t>(H) * P * KC;
  float* base = states + (static_cast<size_t>(b) * nc * H + h) * (static_cast<size_t>(P) * KC) +
                static_cast<size_t>(p) * KC + n;
  const float* dc = decay + (static_cast<size_t>(b) * H + h) * nc * 2;
  const size_t pub = ((static_cast<size_t>(b) * H + h) * P + p) * N + n;  // public (p, n) index

  float4 hr = make_float4(0.f, 0.f, 0.f, 0.f), hi = hr;
  if (h0) {
    if (CPLX) {
      const float4* src = reinterpret_cast<const float4*>(h0 + pub * 2);
      const float4 u = src[0], v = src[1];
      hr = make_float4(u.x, u.z, v.x, v.z);
      hi = make_float4(u.y, u.w, v.y, v.w);
    } else {
      hr = *reinterpret_cast<const float4*>(h0 + pub);
    }
  }

  float4 cur_r[PF], cur_i[PF];
  float2 cur_d[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    if (j < nc) {
      cur_r[j] = *reinterpret_cast<const float4*>(base + j * chunk_stride);
      if (CPLX) cur_i[j] = *reinterpret_cast<const float4*>(base + j * chunk_stride + N);
      cur_d[j] = *reinterpret_cast<const float2*>(dc + 2 * j);
    }
  }
  for (int c0 = 0; c0 < nc; c0 += PF) {
    float4 nxt_r[PF], nxt_i[PF];
    float2 nxt_d[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cn = c0 + PF + j;
      if (cn < nc) {
        nxt_r[j] = *reinterpret_cast<const float4*>(base + cn * chunk_stride);
        if (CPLX) nxt_i[j] = *reinterpret_cast<const float4*>(base + cn * chunk_stride + N);
        nxt_d[j] = *reinterpret_cast<const float2*>(dc + 2 * cn);
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int cc = c0 + j;
      if (cc < nc) {
        float* slot = base + cc * chunk_stride;
        *reinterpret_cast<float4*>(slot) = hr;
        if (CPLX) {
          *reinterpret_cast<float4*>(slot + N) = hi;
          const float dr = cur_d[j].x, di = cur_d[j].y;
          const float4 sr = cur_r[j], si = cur_i[j];
          float4 nr, ni;
          nr.x = dr * hr.x - di * hi.x + sr.x;
          nr.y = dr * hr.y - di * hi.y + sr.y;
          nr.z = dr * hr.z - di * hi.z + sr.z;
          nr.w = dr * hr.w - di * hi.w + sr.w;
          ni.x = dr * hi.x + di * hr.x + si.x;
          ni.y = dr * hi.y + di * hr.y + si.y;
          ni.z = dr * hi.z + di * hr.z + si.z;
          ni.w = dr * hi.w + di * hr.w + si.w;
          hr = nr;
          hi = ni;
        } else {
          const float d = cur_d[j].x;
          const float4 s = cur_r[j];
          hr = make_float4(d * hr.x + s.x, d * hr.y + s.y, d * hr.z + s.z, d * hr.w + s.w);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      cur_r[j] = nxt_r[j];
      if (CPLX) cur_i[j] = nxt_i[j];
      cur_d[j] = nxt_d[j];
    }
  }
  if (h_final) {
    if (CPLX) {
      float4* dst = reinterpret_cast<float4*>(h_final + pub * 2);
      dst[0] = make_float4(hr.x, hi.x, hr.y, hi.y);
      dst[1] = make_float4(hr.z, hi.z, hr.w, hi.w);
    } else {
      *reinterpret_cast<float4*>(h_final + pub) = hr;
    }
  }
}

// launch of the inter-chunk scan for one shape
template <bool CPLX, int N>
inline void launch_pass(float* states, const float* decay, const float* h0, float* h_final,
                        int Bsz, int H, int P, int nc, hipStream_t st, const hipEvent_t* ev) {
  const int groups = P * N / 4;
  dim3 grid((groups + kThreads - 1) / kThreads, H, Bsz);
  launch_k(true, ssd_pass_kernel<CPLX, N>, grid, dim3(kThreads), st, ev, states, decay, h0,
           h_final, H, P, nc);
}

}  // namespace ssd
