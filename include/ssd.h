/*
 * ssd.h -- C ABI of the MI355X (gfx950) selective state-space (SSD) scan.
 *
 * What is computed (page titles and sections of the sources):
 *
 *  Real (Mamba-2) form, one scalar A_h < 0 per head (Mamba-3-Lite README,
 *  its statement of the Mamba-2 recurrence; Block Anatomy page, section 4.4 for
 *  exp(softplus(dt) * A); step size also on the input term, the usual
 *  Mamba-2 discretisation):
 *      delta_t = clamp(softplus(dt_t + dt_bias_h), dt_min, dt_max)
 *      h_t     = exp(A_h delta_t) h_{t-1} + delta_t x_t B_t^T      (P x N)
 *      y_t     = h_t C_t + D_h x_t
 *
 *  Complex (Mamba-3-Lite) form (README, the complex recurrence; Block
 *  Anatomy section 6, the real part is returned):
 *      h_t = exp((alpha_h + i beta_h) delta_t) h_{t-1} + x_t B_t^T  (complex)
 *      y_t = Re(h_t C_t)          -- C is not conjugated; no D term
 *
 *  Both are evaluated chunkwise (chunk length Q): within a chunk through the
 *  decay matrix L[l,s] = exp(cs_l - cs_s) 1[l >= s] and across chunks by a
 *  linear scan of chunk-end states (Numerical Stability in Mamba-3-Lite,
 *  section 4).  The result equals the sequential recurrence up to rounding.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers (memory of the current HIP
 *    device), row-major and contiguous, last index fastest.  The caller owns
 *    every buffer; the library never allocates, frees or keeps a pointer
 *    after the call returns.
 *  - x, B, C, y, h0, h_final, h and workspace must be 16-byte aligned; dt, A,
 *    D and dt_bias 4-byte aligned.
 *  - Head h reads B/C group g = h / (H / G)  (H % G == 0).
 *  - dt is the raw (pre-softplus) step; dt_bias may be NULL (zero bias);
 *    dt_min/dt_max clamp the step after softplus (0 and +INFINITY disable).
 *  - stream is a hipStream_t passed as void* (NULL = the null stream).  The
 *    call only enqueues work and returns; buffers must stay valid until the
 *    stream has passed it.  Faults inside kernels surface at the caller's
 *    next synchronisation.
 *  - Every argument is validated before any HIP call, so a rejected call has
 *    no effect on the device.  There is no fallback path: unsupported shapes
 *    are errors.
 *  - Return value: SSD_OK or one of the error codes below; ssd_last_error()
 *    then describes the problem (thread-local, valid until the next call on
 *    the same thread).
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 1

/* status codes */
#define SSD_OK 0
#define SSD_EINVAL 1          /* null pointer, bad size, misaligned pointer  */
#define SSD_EUNSUPPORTED 2    /* valid but not built: P, N, chunk or dtype   */
#define SSD_EWORKSPACE 3      /* workspace missing or smaller than required  */
#define SSD_EHIP 4            /* a HIP launch reported an error              */

/* element types of x, B, C and y in ssd_chunk_fwd */
#define SSD_F32 0
#define SSD_BF16 1

/* Supported sizes of the chunked forwards:
 *   P (head dim) in {16, 32, 64, 128}; N (state) in {16, 32, 64, 128} for the
 *   real form and {16, 32, 64} for the complex form; chunk in
 *   {16, 32, 64, 128, 256}; any T >= 0 (a last, shorter chunk is handled as if
 *   padded with identity steps).  The decode step takes N in
 *   {16, 32, 64, 128, 256} and any P >= 1. */

/* Version of this ABI (SSD_ABI_VERSION of the built library). */
int ssd_abi_version(void);

/* Description of the last error on this thread ("" when none). */
const char *ssd_last_error(void);

/*
 * Bytes of device workspace ssd_chunk_fwd (is_complex = 0) or
 * ssd_complex_chunk_fwd (is_complex = 1) needs for these sizes: room for the
 * chunk-boundary states as fp32, (Bsz, nc, H, P, N) real or (Bsz, nc, H, P, 2N)
 * complex with nc = ceil(T / chunk), plus one decay factor per (b, h, chunk),
 * plus for the real form one (exponent, step size) float pair per token and
 * head.  (The bf16 real path keeps its chunk states in fp32 too, and beside
 * them the bf16 copy of each boundary state that its output kernel reads.)
 * Returns 0 for sizes the library rejects, among them any whose 1-D grid
 * would exceed 2^31 - 1 workgroups (ceil(Bsz * nc / 8) * 8 * H) or whose
 * chunk of token rows exceeds 4 GiB (chunk * H * P * 4 or chunk * G * N * 8).
 */
size_t ssd_workspace_size(int Bsz, int T, int H, int P, int G, int N, int chunk,
                          int is_complex);

/*
 * Real chunked forward (Mamba-2 form above).
 *   x        (Bsz, T, H, P)  dtype (SSD_F32 or SSD_BF16 bit patterns)
 *   dt       (Bsz, T, H)     float32, raw step
 *   A        (H)             float32, A_h (negative for a decaying scan)
 *   B, C     (Bsz, T, G, N)  dtype
 *   D        (H)             float32 or NULL (no skip term)
 *   dt_bias  (H)             float32 or NULL
 *   h0       (Bsz, H, P, N)  float32 initial state, or NULL for zeros
 *   y        (Bsz, T, H, P)  dtype, written (bf16 rounded to nearest even
 *                            from the fp32 accumulator)
 *   h_final  (Bsz, H, P, N)  float32 state after token T-1, or NULL
 *   workspace of at least ssd_workspace_size(..., 0) bytes, device memory
 * The state and all accumulation are fp32 for both dtypes.
 */
int ssd_chunk_fwd(const void *x, const float *dt, const float *A, const void *B,
                  const void *C, const float *D, const float *dt_bias,
                  float dt_min, float dt_max, const float *h0, void *y,
                  float *h_final, int Bsz, int T, int H, int P, int G, int N,
                  int chunk, int dtype, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * Complex chunked forward (Mamba-3-Lite form above).
 *   x        (Bsz, T, H, P)     float32 (real token content)
 *   dt       (Bsz, T, H)        float32, raw step
 *   A        (H, 2)             float32 (alpha_h, beta_h) = complex64
 *   B, C     (Bsz, T, G, N, 2)  float32 (re, im) pairs = complex64
 *   dt_bias  (H)                float32 or NULL
 *   h0       (Bsz, H, P, N, 2)  complex64 initial state, or NULL for zeros
 *   y        (Bsz, T, H, P)     float32, Re(h_t C_t)
 *   h_final  (Bsz, H, P, N, 2)  complex64 final state, or NULL
 *   workspace of at least ssd_workspace_size(..., 1) bytes
 */
int ssd_complex_chunk_fwd(const float *x, const float *dt, const float *A,
                          const float *B, const float *C, const float *dt_bias,
                          float dt_min, float dt_max, const float *h0, float *y,
                          float *h_final, int Bsz, int T, int H, int P, int G,
                          int N, int chunk, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Allocation-free variant of ssd_chunk_fwd, for callers that cannot call
 * hipMalloc or take a workspace argument: code under HIP graph capture,
 * tight serving loops, harnesses that forbid device allocation.  Same
 * arguments, kernels and results as ssd_chunk_fwd without the workspace:
 * the chunk states, decays and per-token tables live in a scratch array of
 * SSD_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call there).  The call allocates nothing.
 *   - A shape whose workspace (ssd_workspace_size(..., 0)) exceeds
 *     SSD_NOALLOC_SCRATCH_BYTES is rejected with SSD_EWORKSPACE before any
 *     HIP call.
 *   - Every call on one GPU shares that GPU's scratch array; calls whose
 *     work overlaps on one GPU (two streams, two host threads) race on it.
 *     Calls on one stream are ordered and safe.
 *   - The scratch contents left by an earlier call do not matter (nothing
 *     in it must start at zero).
 */
#define SSD_NOALLOC_SCRATCH_BYTES (64ull << 20)
int ssd_chunk_fwd_noalloc(const void *x, const float *dt, const float *A,
                          const void *B, const void *C, const float *D,
                          const float *dt_bias, float dt_min, float dt_max,
                          const float *h0, void *y, float *h_final, int Bsz,
                          int T, int H, int P, int G, int N, int chunk,
                          int dtype, void *stream);

/*
 * Measurement variants of the two chunked forwards: identical arguments,
 * kernels and results, plus `events`, an array of 6 hipEvent_t (passed as
 * void*): the start and stop of the chunk-state kernel, of the inter-chunk
 * state-passing kernel and of the output kernel, in that order, each pair
 * bound to its kernel's dispatch on `stream` (so that it times the kernel
 * alone); a kernel that a call does not run (T = 0) has its pair recorded
 * back to back.  NULL: the plain calls.  The caller creates and owns the
 * events.
 */
int ssd_chunk_fwd_ev(const void *x, const float *dt, const float *A,
                     const void *B, const void *C, const float *D,
                     const float *dt_bias, float dt_min, float dt_max,
                     const float *h0, void *y, float *h_final, int Bsz, int T,
                     int H, int P, int G, int N, int chunk, int dtype,
                     void *workspace, size_t workspace_bytes, void *stream,
                     void *const *events);

/*
 * Variable-length batch of the real chunked forward: nseq independent
 * sequences of different lengths packed along the token axis, each one the
 * recurrence above from its own h0 (the batched prefill of a Mamba-2 layer
 * whose states then continue in ssd_step_decode).
 *   cu_seqlens (nseq + 1)   int32, HOST memory (the one host array of this
 *                           ABI): sequence b holds the token rows
 *                           cu_seqlens[b] .. cu_seqlens[b+1]-1;
 *                           cu_seqlens[0] = 0, non-decreasing, Ttot =
 *                           cu_seqlens[nseq]; empty sequences are allowed
 *                           (their h_final is their h0).  1 <= nseq <= 65535.
 *   x, y     (Ttot, H, P)    bfloat16 (dtype must be SSD_BF16)
 *   dt       (Ttot, H)       float32, raw step
 *   B, C     (Ttot, G, N)    bfloat16
 *   A, D, dt_bias (H)        as in ssd_chunk_fwd
 *   h0, h_final (nseq, H, P, N) float32 or NULL
 *   workspace of at least ssd_varlen_workspace_size(cu_seqlens, ...) bytes
 * Chunks and segments never span two sequences: every sequence is cut into
 * chunks from its own first token, so sequence b's outputs equal those of
 * ssd_chunk_fwd on it alone (bit for bit when both calls pick the same
 * segment length).  The library checks cu_seqlens, builds its segment table
 * on the host and copies it into the workspace on `stream` (a small
 * host-to-device copy from pageable memory; cu_seqlens may be reused once the
 * call returns).  Invalid cu_seqlens: SSD_EINVAL before any HIP call.
 * ssd_varlen_workspace_size returns 0 for arguments the call would reject.
 */
size_t ssd_varlen_workspace_size(const int *cu_seqlens, int nseq, int H, int P,
                                 int G, int N, int chunk);
int ssd_chunk_fwd_varlen(const void *x, const float *dt, const float *A,
                         const void *B, const void *C, const float *D,
                         const float *dt_bias, float dt_min, float dt_max,
                         const float *h0, void *y, float *h_final,
                         const int *cu_seqlens, int nseq, int H, int P, int G,
                         int N, int chunk, int dtype, void *workspace,
                         size_t workspace_bytes, void *stream);
/* the same with the 6 measurement events of ssd_chunk_fwd_ev */
int ssd_chunk_fwd_varlen_ev(const void *x, const float *dt, const float *A,
                            const void *B, const void *C, const float *D,
                            const float *dt_bias, float dt_min, float dt_max,
                            const float *h0, void *y, float *h_final,
                            const int *cu_seqlens, int nseq, int H, int P,
                            int G, int N, int chunk, int dtype, void *workspace,
                            size_t workspace_bytes, void *stream,
                            void *const *events);

int ssd_complex_chunk_fwd_ev(const float *x, const float *dt, const float *A,
                             const float *B, const float *C,
                             const float *dt_bias, float dt_min, float dt_max,
                             const float *h0, float *y, float *h_final, int Bsz,
                             int T, int H, int P, int G, int N, int chunk,
                             void *workspace, size_t workspace_bytes,
                             void *stream, void *const *events);

/*
 * One recurrent step of the real form for a single new token per sequence
 * (the recurrence of the Mamba-3-Lite README applied once), in place:
 *   h        (Bsz, H, P, N)  float32 state, read and overwritten
 *   x        (Bsz, H, P)     float32
 *   dt       (Bsz, H)        float32, raw step
 *   A, D, dt_bias (H)        as in ssd_chunk_fwd (D, dt_bias may be NULL)
 *   B, C     (Bsz, G, N)     float32
 *   y        (Bsz, H, P)     float32, computed from the updated state
 * Needs no workspace.
 */
int ssd_step_decode(float *h, const float *x, const float *dt, const float *A,
                    const float *B, const float *C, const float *D,
                    const float *dt_bias, float dt_min, float dt_max, float *y,
                    int Bsz, int H, int P, int G, int N, void *stream);

/*
 * Measurement variant of ssd_step_decode: identical arguments, kernel and
 * result, plus `events`, 2 hipEvent_t (passed as void*) bound to the decode
 * kernel's dispatch on `stream` (start, stop), or NULL.
 */
int ssd_step_decode_ev(float *h, const float *x, const float *dt, const float *A,
                       const float *B, const float *C, const float *D,
                       const float *dt_bias, float dt_min, float dt_max, float *y,
                       int Bsz, int H, int P, int G, int N, void *stream,
                       void *const *events);

/*
 * One recurrent step of the complex form for a single new token per sequence
 * (the complex promotion of the recurrence in the Mamba-3-Lite README applied
 * once), in place:
 *   h[b,h,p,n] <- exp((A_re + i A_im) delta) h[b,h,p,n] + B[b,g,n] x[b,h,p]
 *   y[b,h,p]    = Re(sum_n C[b,g,n] h[b,h,p,n])     (after the update)
 * with delta = clamp(softplus(dt + dt_bias)) as in ssd_chunk_fwd, no step
 * factor on the input and no D (the conventions of ssd_complex_chunk_fwd).
 *   h        (Bsz, H, P, N, 2)  complex64 state as float32 (re, im) pairs,
 *                               read and overwritten; 16-byte aligned
 *   x        (Bsz, H, P)        float32
 *   dt       (Bsz, H)           float32, raw step
 *   A        (H, 2)             float32 (re, im)
 *   B, C     (Bsz, G, N, 2)     float32 (re, im); 16-byte aligned
 *   dt_bias  (H) or NULL
 *   y        (Bsz, H, P)        float32
 * N must be one of 16, 32, 64, 128; any P >= 1; H a multiple of G.  Needs no
 * workspace.  Errors as for ssd_step_decode; nothing is launched on error.
 */
int ssd_complex_step_decode(float *h, const float *x, const float *dt, const float *A,
                            const float *B, const float *C, const float *dt_bias,
                            float dt_min, float dt_max, float *y,
                            int Bsz, int H, int P, int G, int N, void *stream);

/*
 * Measurement variant of ssd_complex_step_decode: identical arguments, kernel
 * and result, plus `events`, 2 hipEvent_t (passed as void*) bound to the
 * kernel's dispatch on `stream` (start, stop), or NULL.
 */
int ssd_complex_step_decode_ev(float *h, const float *x, const float *dt, const float *A,
                               const float *B, const float *C, const float *dt_bias,
                               float dt_min, float dt_max, float *y,
                               int Bsz, int H, int P, int G, int N, void *stream,
                               void *const *events);

/*
 * Depthwise causal convolution of the Mamba-2 layer (Mamba-3-Lite block page,
 * section 5.1 "Zero causal convolution": before the scan, Mamba-1/2 replace
 * each channel's value at position t by a learned combination of that
 * channel's values at positions t-3 .. t).  Over the Ch = HP + 2*GN channels
 * x|B|C of each token row:
 *   v[b,t,c]   = bias[c] + sum_{j=0..3} w[c,j] * in[b, t-3+j, c]
 *   out[b,t,c] = act ? v / (1 + exp(-v)) : v          (act 1 = SiLU)
 * where in[b,p,c] for p < 0 is state_in[b, 3+p, c].  out is split into the
 * three contiguous inputs of ssd_chunk_fwd: channels [0, HP) to x, [HP,
 * HP+GN) to B, [HP+GN, Ch) to C.
 *   xbc        (Bsz, T, ld) elements of `dtype` (SSD_F32 or SSD_BF16);
 *              channels 0..Ch-1 of each row are read, the rest never (the
 *              in_proj output row can be passed at the offset of its x slice)
 *   w          (Ch, 4) float32 taps, oldest position first
 *   bias       (Ch) float32, or NULL (zero)
 *   state_in   (Bsz, 3, Ch) float32: raw inputs at positions -3, -2, -1, or
 *              NULL (zeros: a fresh sequence)
 *   x          (Bsz, T, HP) `dtype`        = (Bsz, T, H, P) of the scan
 *   B, C       (Bsz, T, GN) `dtype`        = (Bsz, T, G, N); NULL if GN = 0
 *   state_out  (Bsz, 3, Ch) float32: raw inputs at positions T-3 .. T-1 (from
 *              state_in where negative), the state_in of the next segment or
 *              of ssd_conv1d_step; or NULL.  Must not overlap state_in.
 * K (kernel size) must be 4.  HP, GN and ld must be multiples of 8 (bf16) or
 * 4 (fp32), ld >= Ch; xbc, x, B, C, w, bias and both states 16-byte aligned.
 * T = 0 is allowed (only state_out is written).  Arithmetic in float32, one
 * rounding to `dtype` on output.  Outputs must not overlap inputs.  Needs no
 * workspace.  Errors: SSD_EINVAL (bad pointer, size, alignment, overlapping
 * states), SSD_EUNSUPPORTED (K, dtype, channel counts, sizes past the 32-bit
 * addressing of one batch entry's rows), SSD_EHIP; nothing runs on error.
 */
int ssd_conv1d_fwd(const void *xbc, long long ld, const float *w, const float *bias,
                   const float *state_in, int act, void *x, void *B, void *C,
                   float *state_out, int Bsz, int T, int HP, int GN, int K, int dtype,
                   void *stream);

/*
 * The convolution over a variable-length batch (the prefill of nseq sequences
 * of different lengths, packed along the token axis, as for
 * ssd_chunk_fwd_varlen): each sequence is convolved on its own, from its own
 * state_in row, and leaves its own state_out row.
 *   cu_seqlens (nseq + 1)  int32, HOST memory: sequence b holds the token rows
 *                          cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens[0] =
 *                          0, non-decreasing; empty sequences allowed: their
 *                          state_out is their state_in); 1 <= nseq <= 65535
 *   xbc        (Ttot, ld)  as in ssd_conv1d_fwd, Ttot = cu_seqlens[nseq]
 *   x, B, C    (Ttot, HP), (Ttot, GN), (Ttot, GN)
 *   state_in, state_out (nseq, 3, Ch) float32 or NULL
 *   workspace  of ssd_conv1d_varlen_workspace_size(nseq) bytes (the device
 *              copy of cu_seqlens, written on `stream` from pageable memory;
 *              cu_seqlens may be reused once the call returns)
 * Each sequence's result equals ssd_conv1d_fwd on it alone, bit for bit.
 * Other arguments and errors as in ssd_conv1d_fwd (the 32-bit addressing
 * limit applies to the longest sequence); invalid cu_seqlens: SSD_EINVAL.
 */
size_t ssd_conv1d_varlen_workspace_size(int nseq);
int ssd_conv1d_fwd_varlen(const void *xbc, long long ld, const float *w, const float *bias,
                          const float *state_in, int act, void *x, void *B, void *C,
                          float *state_out, const int *cu_seqlens, int nseq, int HP, int GN,
                          int K, int dtype, void *workspace, size_t workspace_bytes,
                          void *stream);
/* the same with the 2 measurement events of ssd_conv1d_fwd_ev */
int ssd_conv1d_fwd_varlen_ev(const void *xbc, long long ld, const float *w, const float *bias,
                             const float *state_in, int act, void *x, void *B, void *C,
                             float *state_out, const int *cu_seqlens, int nseq, int HP, int GN,
                             int K, int dtype, void *workspace, size_t workspace_bytes,
                             void *stream, void *const *events);

/*
 * Measurement variant of ssd_conv1d_fwd: identical arguments, kernel and
 * result, plus `events`, 2 hipEvent_t (passed as void*) bound to the kernel's
 * dispatch on `stream` (start, stop), or NULL.
 */
int ssd_conv1d_fwd_ev(const void *xbc, long long ld, const float *w, const float *bias,
                      const float *state_in, int act, void *x, void *B, void *C,
                      float *state_out, int Bsz, int T, int HP, int GN, int K, int dtype,
                      void *stream, void *const *events);

/*
 * One decode step of the convolution (the segment of one token), in place:
 *   state  (Bsz, 3, Ch) float32, read as positions t-3 .. t-1 and overwritten
 *          with t-2 .. t (the state_out layout of ssd_conv1d_fwd)
 *   xt     (Bsz, ld) float32 token rows (channels 0..Ch-1 read)
 *   w, bias, act as in ssd_conv1d_fwd
 *   x      (Bsz, HP), B, C (Bsz, GN) float32: the inputs of ssd_step_decode
 * HP, GN and ld must be multiples of 4; pointers 16-byte aligned; K = 4.
 * Errors as for ssd_conv1d_fwd.
 */
int ssd_conv1d_step(float *state, const float *xt, long long ld, const float *w,
                    const float *bias, int act, float *x, float *B, float *C,
                    int Bsz, int HP, int GN, int K, void *stream);

/*
 * Measurement variant of ssd_conv1d_step, with 2 hipEvent_t (start, stop)
 * bound to the kernel's dispatch, or NULL.
 */
int ssd_conv1d_step_ev(float *state, const float *xt, long long ld, const float *w,
                       const float *bias, int act, float *x, float *B, float *C,
                       int Bsz, int HP, int GN, int K, void *stream, void *const *events);

/*
 * Backward of ssd_chunk_fwd for the real form: the gradient of
 *   loss = sum_{b,t,h,p} dy[b,t,h,p] y[b,t,h,p] + <dh_final, h_final>
 * with respect to every input (reverse-mode derivative of the recurrence of
 * the Mamba-3-Lite README's classical Mamba-2 form, evaluated chunkwise as in
 * Numerical Stability in Mamba-3-Lite, section 4).  The forward's chunk
 * states are recomputed inside the call; y is not needed.
 *   inputs      x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0 exactly as given
 *               to ssd_chunk_fwd; dy (Bsz,T,H,P) in x's dtype; dh_final
 *               (Bsz,H,P,N) float32 or NULL (zero)
 *   dx          (Bsz,T,H,P) x's dtype
 *   ddt         (Bsz,T,H) float32, gradient of the raw dt (zero where the
 *               step is clamped: the clamp passes the derivative on its closed
 *               interval only)
 *   dB, dC      (Bsz,T,G,N) float32, summed over the heads of each group
 *   dA, dD, ddt_bias  (H) float32, summed over batch and tokens (written even
 *               when D or dt_bias is NULL)
 *   dh0         (Bsz,H,P,N) float32, or NULL (not written)
 *   workspace   ssd_bwd_workspace_size(...) bytes, 256-byte aligned
 * Built for dtype SSD_BF16 with P in {32, 64}, N in {64, 128}, chunk in
 * {64, 128, 256}, and for dtype SSD_F32 (x, B, C, dy and dx float32; fp32
 * matrix products) with P in {32, 64}, N in {32, 64, 128} and chunk 64
 * (SSD_EUNSUPPORTED otherwise).
 * dB, dC, dh0, h0 and dh_final 16-byte aligned.  Outputs are overwritten, not
 * accumulated, and must not overlap inputs.  Errors as for ssd_chunk_fwd.
 * Workspace: ssd_bwd_workspace_size (SSD_BF16) or ssd_bwd_workspace_size_f32.
 */
size_t ssd_bwd_workspace_size(int Bsz, int T, int H, int P, int G, int N, int chunk);
size_t ssd_bwd_workspace_size_f32(int Bsz, int T, int H, int P, int G, int N);

int ssd_chunk_bwd(const void *x, const float *dt, const float *A, const void *B,
                  const void *C, const float *D, const float *dt_bias, float dt_min,
                  float dt_max, const float *h0, const void *dy, const float *dh_final,
                  void *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                  float *ddt_bias, float *dh0, int Bsz, int T, int H, int P, int G, int N,
                  int chunk, int dtype, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * Measurement variant of ssd_chunk_bwd: identical arguments, kernels and
 * result, plus `events` (hipEvent_t passed as void*), or NULL.  SSD_BF16: 22
 * events, a start/stop pair bound to each of 11 kernel slots in order (chunk
 * states, state passing, adjoint chunk states, adjoint passing (which also
 * forms the chunk constants of da), dx/dB blocks, dC blocks, chunk constants
 * (an empty pair, recorded back to back), step-size gradients per chunk,
 * their sums per head (an empty pair: they run in the next slot's launch),
 * the sums of dB and dC and the per-head sums (one launch), an empty pair).
 * SSD_F32: 28 events, the 14
 * slots of ssd_complex_chunk_bwd_ev (the complex-only slots record their pair
 * back to back).
 */
int ssd_chunk_bwd_ev(const void *x, const float *dt, const float *A, const void *B,
                     const void *C, const float *D, const float *dt_bias, float dt_min,
                     float dt_max, const float *h0, const void *dy, const float *dh_final,
                     void *dx, float *ddt, float *dA, float *dB, float *dC, float *dD,
                     float *ddt_bias, float *dh0, int Bsz, int T, int H, int P, int G, int N,
                     int chunk, int dtype, void *workspace, size_t workspace_bytes,
                     void *stream, void *const *events);

/*
 * Backward of ssd_complex_chunk_fwd (Mamba-3-Lite README, the complex
 * recurrence; Block Anatomy, section 7, pitfall 7: the gradient of the complex
 * A is complex): the gradient of
 *   loss = sum_t dy_t . y_t + sum Re(conj(dh_final) h_final)
 * with respect to every input.  Complex arrays as ssd_complex_chunk_fwd,
 * (re, im) float32 pairs; every complex gradient is returned as
 * (dL/d re, dL/d im).
 *   dy          (Bsz,T,H,P) float32;  dh_final (Bsz,H,P,N,2), or NULL (zero)
 *   dx          (Bsz,T,H,P)   ddt (Bsz,T,H)   dA (H,2)   ddt_bias (H)
 *   dB, dC      (Bsz,T,G,N,2), summed over the heads of each group
 *   dh0         (Bsz,H,P,N,2), or NULL (not written)
 * Computed in the sequence-wide rotated frame, where the complex recurrence is
 * two real ones with one real decay, with fp32 matrix products and fp64
 * angles and scans.  P in {32, 64}, N in {16, 32, 64}, chunk 64
 * (SSD_EUNSUPPORTED otherwise).  x, B, C, dy, dx, dB, dC, h0, dh_final, dh0
 * 16-byte aligned, A and dA 8-byte aligned.  Outputs are overwritten and
 * must not overlap inputs.  Workspace: ssd_complex_bwd_workspace_size bytes,
 * 256-byte aligned.  Errors as for ssd_complex_chunk_fwd.
 */
size_t ssd_complex_bwd_workspace_size(int Bsz, int T, int H, int P, int G, int N);

/* Measurement variant of ssd_complex_chunk_bwd: identical arguments, kernels
 * and result, plus `events`, 28 hipEvent_t (passed as void*) or NULL: a
 * start/stop pair bound to each of 14 kernel slots in order (rotation into
 * the sequence frame, chunk states, state passing, adjoint chunk states,
 * adjoint passing (which also forms the chunk constants), column-side blocks,
 * row-side blocks, chunk constants (an empty pair), the
 * last token's rotation term, rho sums per chunk, step-size gradients per
 * chunk, their sums per head, dB/dC group sums, dh0). */
int ssd_complex_chunk_bwd_ev(const float *x, const float *dt, const float *A, const float *B,
                             const float *C, const float *dt_bias, float dt_min, float dt_max,
                             const float *h0, const float *dy, const float *dh_final, float *dx,
                             float *ddt, float *dA, float *dB, float *dC, float *ddt_bias,
                             float *dh0, int Bsz, int T, int H, int P, int G, int N, int chunk,
                             void *workspace, size_t workspace_bytes, void *stream,
                             void *const *events);

int ssd_complex_chunk_bwd(const float *x, const float *dt, const float *A, const float *B,
                          const float *C, const float *dt_bias, float dt_min, float dt_max,
                          const float *h0, const float *dy, const float *dh_final, float *dx,
                          float *ddt, float *dA, float *dB, float *dC, float *ddt_bias,
                          float *dh0, int Bsz, int T, int H, int P, int G, int N, int chunk,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * ssd_complex_chunk_fwd reading its inputs in place from the rows of the
 * Mamba-3-Lite in_proj output (block page, sections 4.1-4.2: one row of
 * width H(D + 4N + 1) per token, head-major slices, float32 after the casts):
 *   proj[b,t, 0 .. HP)             x      (head h at h*P, P = D)
 *   proj[b,t, HP + h*N + n]        Re B   proj[b,t, HP + HN + h*N + n]   Im B
 *   proj[b,t, HP + 2HN + h*N + n]  Re C   proj[b,t, HP + 3HN + h*N + n]  Im C
 *   proj[b,t, HP + 4HN + h]        dt
 * with HP = H*P, HN = H*N; per-head B and C (G = H).  Rows are `ld` floats
 * apart (ld >= H(P + 4N + 1), a multiple of 4; any columns past the slices
 * are not read); proj 16-byte aligned.  Nothing is copied: the kernels read
 * the planar real and imaginary slices directly.  Everything else (A,
 * dt_bias, clamp, h0, y, h_final, the workspace of
 * ssd_workspace_size(..., is_complex = 1), errors) as ssd_complex_chunk_fwd.
 */
int ssd_complex_chunk_fwd_packed(const float *proj, long long ld, const float *A,
                                 const float *dt_bias, float dt_min, float dt_max,
                                 const float *h0, float *y, float *h_final, int Bsz, int T,
                                 int H, int P, int N, int chunk, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Measurement variant of ssd_complex_chunk_fwd_packed (6 events, as
 * ssd_complex_chunk_fwd_ev). */
int ssd_complex_chunk_fwd_packed_ev(const float *proj, long long ld, const float *A,
                                    const float *dt_bias, float dt_min, float dt_max,
                                    const float *h0, float *y, float *h_final, int Bsz, int T,
                                    int H, int P, int N, int chunk, void *workspace,
                                    size_t workspace_bytes, void *stream, void *const *events);

/*
 * Bias-free linear layer z = x W^T row by row (z[m][n] = sum_k x[m][k] W[n][k],
 * W stored (out_features, in_features)) on the matrix cores: bf16 operands,
 * fp32 accumulation.  These are the MIMO head mixer and out_proj of the
 * Mamba-3-Lite block (Block Anatomy, Numerical Stability & Scaling, section
 * 6, rows 9-10: single bias-free Linear layers; Numerical Stability in
 * Mamba-3-Lite, section 3.1: projection GEMMs run in bf16 under autocast).
 *   x  (M, K)     x_dtype SSD_F32 (rounded to bf16, nearest even, as it is
 *                 read) or SSD_BF16
 *   W  (Nout, K)  bf16
 *   z  (M, Nout)  z_dtype SSD_F32, or SSD_BF16 (rounded to nearest even from
 *                 the fp32 sum)
 * K a multiple of 64 (>= 64), Nout a multiple of 128 (>= 128), M >= 0.  x, W
 * and z are caller-owned device memory, 16-byte aligned; no workspace.
 * Errors: SSD_EINVAL for null/misaligned pointers or negative sizes,
 * SSD_EUNSUPPORTED for K, Nout off those multiples, a bad dtype or a grid
 * beyond 32 bits; validated before any HIP call.
 */
int ssd_linear_fwd(const void *x, int x_dtype, const void *W, void *z,
                   int z_dtype, int M, int K, int Nout, void *stream);

/* The same with a start/stop hipEvent_t pair (events[0], events[1]) bound to
 * the kernel's dispatch, for measurement. */
int ssd_linear_fwd_ev(const void *x, int x_dtype, const void *W, void *z,
                      int z_dtype, int M, int K, int Nout, void *stream,
                      void *const *events);

/*
 * The MIMO head mixer (Block Anatomy, section 6, row 9): y (Bsz, T, H, P), the
 * scan output, read per token as H*P features head-major (feature h*P + p:
 * the plain flatten of (H, P)), mixed by W (H*P, H*P): z (Bsz, T, H, P) =
 * ssd_linear_fwd(y as (Bsz*T, H*P), W).  H*P must be a multiple of 128.
 */
int ssd_mimo_fwd(const void *y, int y_dtype, const void *W, void *z,
                 int z_dtype, int Bsz, int T, int H, int P, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */
