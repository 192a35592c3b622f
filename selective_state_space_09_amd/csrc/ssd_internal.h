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

struct LinearArgs {
  const void* x;        // (M, K), fp32 (x_dtype 0) or bf16 (1)
  int x_dtype;
  const uint16_t* W;    // (Nout, K) bf16
  void* z;              // (M, Nout), fp32 (z_dtype 0) or bf16 (1)
  int z_dtype;
  int M, K, Nout;
  hipEvent_t* events;   // NULL, or start/stop of the kernel
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

// ---------------------------------------------------------------------------
// Workspace of the bfloat16 real forward.  A workgroup of its chunk-state and
// output kernels walks a segment of K consecutive chunks of one (batch, head)
// and carries the state across them, so states are kept at segment ends only:
//   S     fp32 (Bsz, nseg, H, P, N)  each segment's own end state from zero
//   Hin   bf16 (Bsz, nseg, H, P, N)  the state entering each segment (the
//                                    output kernel's matrix-core operand)
//   decay fp32 (Bsz, H, nseg)        each segment's decay factor
//   tok   float2 (Bsz, nc, H, chunk) per token: A u_l (cumulative step from
//                                    the chunk start times A) and delta_l
// nseg = ceil(nc / K).  K is the largest power of two (<= 16, <= nc) that
// leaves at least `target` (batch, segment, head) workgroups; chunks below 64
// tokens always use K = 1.  Uniform batches: 512, one round of the
// multi-chunk output kernel at two workgroups per CU (at the BitMamba shape
// K = 2: 63.7 -> 60.3 us per step, against 1024 single-chunk workgroups in
// 1.33 rounds at three per CU; at T65536 K = 16: 606 -> 586 us).
// Variable-length batches: 2048 over all their chunks (sequences of uneven
// length leave segments of uneven length; the six-prompt batch runs 92 us at
// K = 1 against 102 us at K = 2).
// ---------------------------------------------------------------------------
constexpr long long kSegTargetUnits = 512;
constexpr long long kSegTargetUnitsVarlen = 2048;

inline int bf16_segment_chunks(int Bsz, int nc, int H, int chunk, long long target = kSegTargetUnits) {
  if (chunk < 64) return 1;
  const long long units = static_cast<long long>(Bsz) * nc * H;
  int K = 1;
  while (K < 16 && 2 * K <= nc && units / (2LL * K) >= target) K *= 2;
  return K;
}

struct Bf16FwdLayout {
  size_t S, Hin, decay, tok, total;  // byte offsets, total bytes
  size_t table;                      // variable lengths: seg, segstart, cu (host-built)
};

inline Bf16FwdLayout bf16_fwd_layout(int Bsz, int nc, int H, int P, int N, int chunk, int K) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int nseg = (nc + K - 1) / K;
  const size_t st = static_cast<size_t>(Bsz) * nseg * H * P * N;
  Bf16FwdLayout L{};
  size_t o = 0;
  L.S = o;
  o += up(st * 4);
  L.Hin = o;
  o += up(st * 2);
  L.decay = o;
  o += up(static_cast<size_t>(Bsz) * H * nseg * 4);
  L.tok = o;
  o += up(static_cast<size_t>(Bsz) * nc * H * chunk * 8);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------
// Variable-length batch of the bf16 real forward.  cu: the (nseq + 1) host
// offsets of the sequences' token rows in the packed inputs (cu[0] = 0,
// non-decreasing, cu[nseq] = Ttot).  Each sequence is cut into chunks (a last,
// shorter one) and segments of K chunks (a last, shorter one) on its own; the
// segments of all sequences are numbered in sequence order (global segment
// index), and the workspace holds per global segment what the uniform layout
// holds per (batch, segment): S, Hin (npairs, H, P, N), decay (npairs, H) --
// segment-major --, tok (npairs * K chunks, H, chunk); then the table the
// kernels read: seg (npairs int2: sequence, segment of it), segstart
// (nseq + 1), cu (nseq + 1).
// ---------------------------------------------------------------------------
struct VarlenPlan {
  int nseq, Ttot, K, npairs, max_nc;
  long long nc_tot;
};
// false (and *why) for an invalid cu or sizes beyond the kernels' limits
bool varlen_plan(const int* cu, int nseq, int H, int chunk, VarlenPlan& p, const char** why);
Bf16FwdLayout bf16_varlen_layout(const VarlenPlan& p, int H, int P, int N, int chunk);
// a.Bsz = nseq, a.T = Ttot; the table is copied into the workspace from cu
hipError_t run_chunk_varlen_bf16(const ChunkArgs& a, const VarlenPlan& p, const int* cu, hipStream_t st);

hipError_t run_chunk_real(const ChunkArgs& a, hipStream_t st);
// the convolution over a variable-length batch: a.Bsz = nseq sequences, a.T
// the longest; cu the host offsets, copied to `workspace` ((nseq+1) ints)
hipError_t run_conv1d_varlen(const ConvArgs& a, const int* cu, void* workspace, hipStream_t st);
hipError_t run_chunk_real_bf16(const ChunkArgs& a, hipStream_t st);
hipError_t run_chunk_complex(const ChunkArgs& a, hipStream_t st);
// a.x = the in_proj rows (Bsz, T, ld): [x | B_re | B_im | C_re | C_im | dt], G = H
hipError_t run_chunk_complex_packed(const ChunkArgs& a, int ld, hipStream_t st);
hipError_t run_decode(const DecodeArgs& a, hipStream_t st);
hipError_t run_complex_decode(const DecodeArgs& a, hipStream_t st);  // D unused
// state + pass kernels only, one chunk per segment (K = 1: per-chunk boundary
// states, decays and the token table in bf16_fwd_layout(..., 1); the S region
// then holds the fp32 boundary states h_in(c))
hipError_t run_chunk_states_bf16(const ChunkArgs& a, hipStream_t st);
hipError_t run_chunk_bwd_bf16(const BwdArgs& a, hipStream_t st);
// fp32 chunk-state kernel for the backward (chunk <= 64): mode 0 forward
// chunk states S_c and decays (input scale delta), 1 the same with input
// scale 1, 2 adjoint chunk states G_c = sum_l e^{cs_l} x_l (x) B_l (x = dy,
// B = C; decay unused); 3 and 4 are 1 and 2 on complex rows (B or C as N/2
// (re, im) pairs per group row, N the real feature count) rotated per token by
// rot (Bsz, T, H) = (cos, sin) theta into [Re B e^{-i theta} | Im ..] (3) or
// [Re C e^{i theta} | -Im ..] (4).  states (Bsz, nc, H, P, N) fp32; decay
// (Bsz, H, nc, 2).  P in {32, 64}, N in {32, 64, 128}.
hipError_t run_states_f32(const float* x, const float* dt, const float* A, const float* B,
                          const float* dt_bias, float dt_min, float dt_max, float* states,
                          float* decay, int Bsz, int T, int H, int P, int G, int N, int chunk,
                          int mode, const float2* rot, hipStream_t st, const hipEvent_t* ev);
// fp32 state passing in place (h_in over S; h0, h_final may be null)
hipError_t run_pass_f32(float* states, const float* decay, const float* h0, float* h_final, int Bsz,
                        int H, int P, int N, int nc, hipStream_t st, const hipEvent_t* ev);
// the fp32 backward (real form, dtype 0) and the complex backward; chunk 64
hipError_t run_chunk_bwd_f32(const BwdArgs& a, hipStream_t st);
size_t bwd_f32_workspace_bytes(int Bsz, int T, int H, int P, int G, int N, bool cplx);
struct CplxBwdArgs {
  const float* x;
  const float* dt;
  const float* A;  // (H, 2)
  const float* B;  // (Bsz, T, G, N, 2)
  const float* C;
  const float* dt_bias;
  float dt_min, dt_max;
  const float* h0;        // (Bsz, H, P, N, 2) or null
  const float* dy;        // (Bsz, T, H, P)
  const float* dh_final;  // (Bsz, H, P, N, 2) or null
  float* dx;
  float* ddt;
  float* dA;  // (H, 2)
  float* dB;  // (Bsz, T, G, N, 2)
  float* dC;
  float* ddt_bias;
  float* dh0;  // (Bsz, H, P, N, 2) or null
  int Bsz, T, H, P, G, N;
  void* workspace;
  hipEvent_t* events;  // NULL, or 28: start/stop of each of the 14 kernel slots
};
hipError_t run_complex_bwd(const CplxBwdArgs& a, hipStream_t st);
size_t bwd_workspace_bytes(int Bsz, int T, int H, int P, int G, int N, int chunk);
int bwd_heads_per_group(int H, int G);
hipError_t run_conv1d(const ConvArgs& a, hipStream_t st);
hipError_t run_linear(const LinearArgs& a, hipStream_t st);  // K % 64 == 0, Nout % 128 == 0
hipError_t run_conv1d_step(const ConvArgs& a, hipStream_t st);  // float32, T = 1
int conv_tokens_per_thread();

}  // namespace ssd
