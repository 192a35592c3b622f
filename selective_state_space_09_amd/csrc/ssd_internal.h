// Internal interface between the C ABI (ssd_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ssd {

struct ChunkArgs {
  const void* x;
  const float* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* dt_bias;
  float dt_min, dt_max;
  const float* h0;
  void* y;
  float* h_final;
  int Bsz, T, H, P, G, N, chunk, dtype;
  void* workspace;
  hipEvent_t* events;  // NULL, or 6: start/stop of each of the 3 kernels
};

struct DecodeArgs {
  float* h;
  const float* x;
  const float* dt;
  const float* A;
  const float* B;
  const float* C;
  const float* D;
  const float* dt_bias;
  float dt_min, dt_max;
  float* y;
  int Bsz, H, P, G, N;
  hipEvent_t* events;  // NULL, or start/stop of the decode kernel
};

struct ConvArgs {
  const void* xbc;         // (Bsz, T, ld) rows; the step: (Bsz, ld) float32
  int ld;                  // elements between consecutive token rows
  const float* w;          // (Ch, 4)
  const float* bias;       // (Ch) or NULL
  const float* state_in;   // (Bsz, 3, Ch) or NULL (prefill only)
  float* state_out;        // (Bsz, 3, Ch) or NULL; the step's state, in place
  int act;                 // 1 = SiLU
  void* x;                 // (Bsz, T, HP)
  void* B;                 // (Bsz, T, GN)
  void* C;                 // (Bsz, T, GN)
  int Bsz, T, HP, GN, dtype;
  hipEvent_t* events;      // NULL, or start/stop of the kernel
};

struct BwdArgs {
  const void* x;
  const float* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const float* dt_bias;
  float dt_min, dt_max;
  const float* h0;
  const void* dy;
  const float* dh_final;
  void* dx;
  float* ddt;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* ddt_bias;
  float* dh0;
  int Bsz, T, H, P, G, N, chunk;
  void* workspace;
  hipEvent_t* events;  // NULL, or 22: start/stop of each of the 11 kernels
};

// floats of chunk-boundary states: (Bsz, nc, H, P, KC), KC = N or 2N
inline size_t workspace_state_floats(int Bsz, int nc, int H, int P, int KC) {
  return static_cast<size_t>(Bsz) * nc * H * P * KC;
}

// floats of per-chunk decay factors: (Bsz, H, nc, 2)
inline size_t workspace_decay_floats(int Bsz, int nc, int H) {
  return static_cast<size_t>(Bsz) * H * nc * 2;
}

// floats of per-token (exponent, step size) pairs of the real form:
// (Bsz, nc, H, chunk, 2)
inline size_t workspace_token_floats(int Bsz, int nc, int H, int chunk) {
  return static_cast<size_t>(Bsz) * nc * H * chunk * 2;
}

// floats of the complex form's per-token table (alpha u, cos theta, sin theta, 0):
// (Bsz, nc, H, chunk, 4)
inline size_t workspace_cplx_token_floats(int Bsz, int nc, int H, int chunk) {
  return static_cast<size_t>(Bsz) * nc * H * chunk * 4;
}

hipError_t run_chunk_real(const ChunkArgs& a, hipStream_t st);
hipError_t run_chunk_real_bf16(const ChunkArgs& a, hipStream_t st);
hipError_t run_chunk_complex(const ChunkArgs& a, hipStream_t st);
// a.x = the in_proj rows (Bsz, T, ld): [x | B_re | B_im | C_re | C_im | dt], G = H
hipError_t run_chunk_complex_packed(const ChunkArgs& a, int ld, hipStream_t st);
hipError_t run_decode(const DecodeArgs& a, hipStream_t st);
hipError_t run_complex_decode(const DecodeArgs& a, hipStream_t st);  // D unused
hipError_t run_chunk_states_bf16(const ChunkArgs& a, hipStream_t st);  // state + pass kernels only
hipError_t run_chunk_bwd_bf16(const BwdArgs& a, hipStream_t st);
size_t bwd_workspace_bytes(int Bsz, int T, int H, int P, int G, int N, int chunk);
int bwd_heads_per_group(int H, int G);
hipError_t run_conv1d(const ConvArgs& a, hipStream_t st);
hipError_t run_conv1d_step(const ConvArgs& a, hipStream_t st);  // float32, T = 1
int conv_tokens_per_thread();

}  // namespace ssd
