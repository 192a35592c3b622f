// Device-side helpers shared by the gfx950 SSD kernels: element conversion,
// MFMA operand types, the step-size gate and the per-chunk prefix scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;
constexpr int kThreads = 256;  // 4 waves per workgroup in every chunk kernel

// bfloat16 values travel as uint16 bit patterns (the top half of a float32).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two float32 -> bfloat16 by the hardware conversion (v_cvt_pk_bf16_f32:
// round to nearest, ties to even, in the default rounding mode)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}


// Step size of one token: softplus(dt + bias) = ln(1 + e^z), evaluated as
// max(z, 0) + ln(1 + e^-|z|), then clamped to [lo, hi] (Numerical Stability
// in Mamba-3-Lite, section 4: the gate is softplus, always positive).
__device__ __forceinline__ float step_size(float dt, float bias, float lo, float hi) {
  const float z = dt + bias;
  const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
  return fminf(fmaxf(sp, lo), hi);
}

// Index of this wave in the workgroup, as a wave-uniform (scalar) value, so
// that branches on it compile to scalar branches with every lane active.
// (The gfx950 LDS transpose read exchanges data across lanes and must not run
// under a partial or empty EXEC mask.)
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

// Inclusive prefix sum of one double per thread over a 256-thread block.
// wsum must be a __shared__ array of 4 doubles.  Contains __syncthreads().
__device__ __forceinline__ double block_inclusive_scan(double v, double* wsum) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double n = __shfl_up(v, o, kWave);
    if (lane >= o) v += n;
  }
  if (lane == kWave - 1) wsum[wid] = v;
  __syncthreads();
  double add = 0.0;
  for (int k = 0; k < wid; ++k) add += wsum[k];
  return v + add;
}

// Inclusive prefix sum of one float per lane over a wave, by DPP lane moves
// (the gfx9 pattern: row shifts by 1, 2, 4, 8 inside rows of 16 lanes, then
// the broadcasts of lane 15 and lane 31 into the upper rows).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  float t;
  t = dpp_mov<0x111>(v); if (r >= 1) v += t;   // row_shr:1
  t = dpp_mov<0x112>(v); if (r >= 2) v += t;   // row_shr:2
  t = dpp_mov<0x114>(v); if (r >= 4) v += t;   // row_shr:4
  t = dpp_mov<0x118>(v); if (r >= 8) v += t;   // row_shr:8
  t = dpp_mov<0x142>(v); if ((lane & 31) >= 16) v += t;  // row_bcast:15
  t = dpp_mov<0x143>(v); if (lane >= 32) v += t;         // row_bcast:31
  return v;
}

// The same in double: each DPP lane move carries the two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp_mov_d(double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u & 0xFFFFFFFFull), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                        static_cast<unsigned>(lo));
}
__device__ __forceinline__ double wave_inclusive_sum_d(double v) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15;
  double t;
  t = dpp_mov_d<0x111>(v); if (r >= 1) v += t;
  t = dpp_mov_d<0x112>(v); if (r >= 2) v += t;
  t = dpp_mov_d<0x114>(v); if (r >= 4) v += t;
  t = dpp_mov_d<0x118>(v); if (r >= 8) v += t;
  t = dpp_mov_d<0x142>(v); if ((lane & 31) >= 16) v += t;
  t = dpp_mov_d<0x143>(v); if (lane >= 32) v += t;
  return v;
}

// fp32 -> bf16 hi + bf16 lo with hi + lo = v to ~2^-17 |v| (the operand split
// of fp32 products computed as three bf16 products, hi*hi + hi*lo + lo*hi)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = static_cast<__bf16>(v);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v - static_cast<float>(h)));
}
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  uint16_t ah, al, bh, bl;
  split_bf16(a, ah, al);
  split_bf16(b, bh, bl);
  hi = static_cast<uint32_t>(ah) | (static_cast<uint32_t>(bh) << 16);
  lo = static_cast<uint32_t>(al) | (static_cast<uint32_t>(bl) << 16);
}

// cos/sin of an angle given in double: reduced to [-pi, pi] in double, then
// evaluated in float.  Angles of a 256-token chunk reach ~80 rad; reducing in
// float would cost ~1e-5 rad of phase.
__device__ __forceinline__ void rot_cs(double ang, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  const double r = ang - two_pi * rint(ang * (1.0 / two_pi));
  sincosf(static_cast<float>(r), &s, &c);
}

// Raw buffer access (gfx9 buffer descriptor, dword3 0x00020000): offsets are
// bytes from `base`; loads at or past `bytes` return zero and stores there are
// dropped, which bounds every access to the described range.
// The descriptor lives in scalar registers: base and bytes must be the same in
// every lane of the wave.  They are taken from the first lane explicitly, so
// that values the compiler computes in vector registers (64-bit address
// arithmetic) do not turn each access into a per-lane loop.
typedef __amdgpu_buffer_rsrc_t buf_t;
__device__ __forceinline__ buf_t make_buf(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* pu = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, static_cast<short>(0),
                                           static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(buf_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(buf_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store8(buf_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v),
                                        r, off, 0, 0);
}
// Nontemporal store (cache policy bit nt): for data no later access of the
// same kernel or the next one reads.
__device__ __forceinline__ void buf_store8_nt(buf_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v),
                                        r, off, 0, 2);
}
__device__ __forceinline__ void buf_store16_nt(buf_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                         r, off, 0, 2);
}
__device__ __forceinline__ void buf_store16(buf_t r, uint32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v),
                                         r, off, 0, 0);
}

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

// The same read with the four 4-column pieces of each row CS columns apart:
// lane i receives column col0 + CS (i / 4) + i % 4 of rows row0 .. row0+3
// (CS = 4 is lds_tr4).
template <int CS>
__device__ __forceinline__ uint2 lds_tr4s(const uint16_t* tile, int pitch, int row0, int col0) {
  const int m = threadIdx.x & 15;
  const uint16_t* a = tile + (row0 + (m >> 2)) * pitch + col0 + CS * (m & 3);
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(const_cast<uint16_t*>(a)));
  return __builtin_bit_cast(uint2, r);
}

// MFMA wrappers (gfx950).  Operand layouts for the 16x16 forms, lane i,
// q = i / 16:  A holds row i % 16, B holds column i % 16, and the k values
// of a lane are k-group q; the accumulator holds column i % 16, rows
// 4q .. 4q+3.  The kernels only rely on A and B sharing one k assignment.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace ssd
