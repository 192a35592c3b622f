// C ABI of the SSD library (declared in include/ssd.h): argument validation,
// workspace sizing and kernel dispatch.  Validation runs before any HIP call,
// so rejected calls never touch the device.

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/ssd.h"
#include "ssd_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SSD_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool in_set(int v, const int* set, int n) {
  for (int i = 0; i < n; ++i)
    if (set[i] == v) return true;
  return false;
}

const int kPs[] = {16, 32, 64, 128};
const int kNsReal[] = {16, 32, 64, 128};
const int kNsCplx[] = {16, 32, 64};
const int kChunks[] = {16, 32, 64, 128, 256};
const int kNsDecode[] = {16, 32, 64, 128, 256};
const int kNsCplxDecode[] = {16, 32, 64, 128};

// Shape checks shared by both chunked forwards.  Returns SSD_OK or an error.
int check_chunk_shape(int Bsz, int T, int H, int P, int G, int N, int chunk, int is_complex) {
  if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk <= 0)
    return fail(SSD_EINVAL, "sizes must be positive (T >= 0): Bsz=%d T=%d H=%d P=%d G=%d N=%d chunk=%d",
                Bsz, T, H, P, G, N, chunk);
  if (H % G != 0) return fail(SSD_EINVAL, "H=%d is not a multiple of G=%d", H, G);
  if (!in_set(P, kPs, 4)) return fail(SSD_EUNSUPPORTED, "P=%d not in {16,32,64,128}", P);
  if (is_complex ? !in_set(N, kNsCplx, 3) : !in_set(N, kNsReal, 4))
    return fail(SSD_EUNSUPPORTED, "N=%d not supported (%s)", N,
                is_complex ? "complex: {16,32,64}" : "real: {16,32,64,128}");
  if (!in_set(chunk, kChunks, 5)) return fail(SSD_EUNSUPPORTED, "chunk=%d not in {16,32,64,128,256}", chunk);
  // 32-bit grid limits and index headroom
  const long long nc = (static_cast<long long>(T) + chunk - 1) / chunk;
  if (nc > 2147483647LL || static_cast<long long>(H) > 65535 || Bsz > 65535)
    return fail(SSD_EUNSUPPORTED, "grid too large: nc=%lld H=%d Bsz=%d", nc, H, Bsz);
  // 1-D grids: (b, chunk) pairs rounded to whole XCD groups, times H
  const long long pairs = (Bsz * nc + 7) / 8 * 8;
  if (pairs * H > 2147483647LL)
    return fail(SSD_EUNSUPPORTED, "grid too large: Bsz*nc*H = %lld workgroups", pairs * H);
  // one chunk's token rows are addressed by 32-bit byte offsets
  if (static_cast<long long>(chunk) * H * P * 4 > 4294967295LL ||
      static_cast<long long>(chunk) * G * N * 8 > 4294967295LL)
    return fail(SSD_EUNSUPPORTED, "one chunk's rows exceed 4 GiB: chunk=%d H=%d P=%d G=%d N=%d",
                chunk, H, P, G, N);
  return SSD_OK;
}

int check_clamp(float lo, float hi) {
  if (!(lo >= 0.0f) || !(hi >= lo))
    return fail(SSD_EINVAL, "need 0 <= dt_min <= dt_max (got %g, %g)", lo, hi);
  return SSD_OK;
}

// Workspace of a chunked forward.  The real form covers both of its paths
// (float32: per-chunk fp32 states, decays and token table; bfloat16: the
// segment layout of ssd_internal.h), since the size query takes no dtype.
size_t workspace_bytes_for(int Bsz, int T, int H, int P, int N, int chunk, int is_complex) {
  const int nc = (T + chunk - 1) / chunk;
  const int KC = is_complex ? 2 * N : N;
  const size_t floats = ssd::workspace_state_floats(Bsz, nc, H, P, KC) +
                        ssd::workspace_decay_floats(Bsz, nc, H) +
                        (is_complex ? ssd::workspace_cplx_token_floats(Bsz, nc, H, chunk)
                                    : ssd::workspace_token_floats(Bsz, nc, H, chunk));
  size_t bytes = floats * sizeof(float);
  if (!is_complex) {
    const size_t b16 =
        ssd::bf16_fwd_layout(Bsz, nc, H, P, N, chunk, ssd::bf16_segment_chunks(Bsz, nc, H, chunk)).total;
    if (b16 > bytes) bytes = b16;
  }
  return (bytes + 255) / 256 * 256 + 256;
}

int check_ptr(const void* p, const char* name, uintptr_t align, bool required) {
  if (!p) {
    if (required) return fail(SSD_EINVAL, "%s is NULL", name);
    return SSD_OK;
  }
  if (!aligned(p, align)) return fail(SSD_EINVAL, "%s is not %u-byte aligned", name, (unsigned)align);
  return SSD_OK;
}

#define SSD_TRY(expr)          \
  do {                         \
    const int rc_ = (expr);    \
    if (rc_ != SSD_OK) return rc_; \
  } while (0)

int launch_status(hipError_t e) {
  if (e != hipSuccess) return fail(SSD_EHIP, "HIP error: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_last_error(void) { return g_err; }

size_t ssd_workspace_size(int Bsz, int T, int H, int P, int G, int N, int chunk, int is_complex) {
  if (check_chunk_shape(Bsz, T, H, P, G, N, chunk, is_complex) != SSD_OK) return 0;
  return workspace_bytes_for(Bsz, T, H, P, N, chunk, is_complex);
}

}  // extern "C"

namespace {

// Arguments of the real chunked forward other than the workspace.
int check_real_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                   const float* D, const float* dt_bias, float dt_min, float dt_max,
                   const float* h0, const void* y, const float* h_final, int Bsz, int T, int H,
                   int P, int G, int N, int chunk, int dtype) {
  SSD_TRY(check_chunk_shape(Bsz, T, H, P, G, N, chunk, 0));
  if (dtype != SSD_F32 && dtype != SSD_BF16)
    return fail(SSD_EUNSUPPORTED, "dtype=%d is neither SSD_F32 nor SSD_BF16", dtype);
  const bool has_tokens = T > 0;
  SSD_TRY(check_ptr(x, "x", 16, has_tokens));
  SSD_TRY(check_ptr(dt, "dt", 4, has_tokens));
  SSD_TRY(check_ptr(A, "A", 4, has_tokens));
  SSD_TRY(check_ptr(B, "B", 16, has_tokens));
  SSD_TRY(check_ptr(C, "C", 16, has_tokens));
  SSD_TRY(check_ptr(y, "y", 16, has_tokens));
  SSD_TRY(check_ptr(D, "D", 4, false));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_ptr(h0, "h0", 16, false));
  SSD_TRY(check_ptr(h_final, "h_final", 16, false));
  return check_clamp(dt_min, dt_max);
}

}  // namespace

extern "C" {

int ssd_chunk_fwd_ev(const void* x, const float* dt, const float* A, const void* B,
                     const void* C, const float* D, const float* dt_bias, float dt_min,
                     float dt_max, const float* h0, void* y, float* h_final, int Bsz, int T,
                     int H, int P, int G, int N, int chunk, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream, void* const* events) {
  SSD_TRY(check_real_fwd(x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final, Bsz, T, H,
                         P, G, N, chunk, dtype));
  const size_t need = workspace_bytes_for(Bsz, T, H, P, N, chunk, 0);
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  if (workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  ssd::ChunkArgs a{x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final,
                   Bsz, T, H, P, G, N, chunk, dtype, workspace,
                   reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_chunk_real(a, static_cast<hipStream_t>(stream)));
}

int ssd_chunk_fwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                  const float* D, const float* dt_bias, float dt_min, float dt_max,
                  const float* h0, void* y, float* h_final, int Bsz, int T, int H, int P, int G,
                  int N, int chunk, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return ssd_chunk_fwd_ev(x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final, Bsz, T,
                          H, P, G, N, chunk, dtype, workspace, workspace_bytes, stream, nullptr);
}

// ---- variable-length batches (bf16 real forward) ----

size_t ssd_varlen_workspace_size(const int* cu_seqlens, int nseq, int H, int P, int G, int N, int chunk) {
  if (!cu_seqlens) return 0;
  ssd::VarlenPlan p{};
  const char* why = nullptr;
  if (!ssd::varlen_plan(cu_seqlens, nseq, H, chunk, p, &why)) return 0;
  if (check_chunk_shape(1, p.Ttot, H, P, G, N, chunk, 0) != SSD_OK) return 0;
  return ssd::bf16_varlen_layout(p, H, P, N, chunk).total + 256;
}

int ssd_chunk_fwd_varlen_ev(const void* x, const float* dt, const float* A, const void* B,
                            const void* C, const float* D, const float* dt_bias, float dt_min,
                            float dt_max, const float* h0, void* y, float* h_final,
                            const int* cu_seqlens, int nseq, int H, int P, int G, int N, int chunk,
                            int dtype, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events) {
  if (!cu_seqlens) return fail(SSD_EINVAL, "cu_seqlens is NULL");
  ssd::VarlenPlan p{};
  const char* why = nullptr;
  if (!ssd::varlen_plan(cu_seqlens, nseq, H, chunk > 0 ? chunk : 1, p, &why))
    return fail(SSD_EINVAL, "cu_seqlens: %s", why);
  if (dtype != SSD_BF16)
    return fail(SSD_EUNSUPPORTED, "variable-length batches take bfloat16 x, B, C, y (dtype=%d)", dtype);
  SSD_TRY(check_real_fwd(x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final, 1, p.Ttot, H, P,
                         G, N, chunk, dtype));
  const size_t need = ssd::bf16_varlen_layout(p, H, P, N, chunk).total + 256;
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  if (workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  ssd::ChunkArgs a{x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final,
                   nseq, p.Ttot, H, P, G, N, chunk, dtype, workspace,
                   reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_chunk_varlen_bf16(a, p, cu_seqlens, static_cast<hipStream_t>(stream)));
}

int ssd_chunk_fwd_varlen(const void* x, const float* dt, const float* A, const void* B, const void* C,
                         const float* D, const float* dt_bias, float dt_min, float dt_max,
                         const float* h0, void* y, float* h_final, const int* cu_seqlens, int nseq,
                         int H, int P, int G, int N, int chunk, int dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return ssd_chunk_fwd_varlen_ev(x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final,
                                 cu_seqlens, nseq, H, P, G, N, chunk, dtype, workspace, workspace_bytes,
                                 stream, nullptr);
}

}  // extern "C"

// ---- the allocation-free forward ----

// Scratch memory of ssd_chunk_fwd_noalloc.  Each GPU the library runs on
// holds its own copy of this array (at its own address) until the process
// ends.  Host code never uses the array's name as a device address: the
// address is looked up per device (hipGetSymbolAddress) and kept below.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, looked up on the
// first call there.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSD_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSD_EUNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SSD_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_chunk_fwd_noalloc(const void* x, const float* dt, const float* A, const void* B,
                          const void* C, const float* D, const float* dt_bias, float dt_min,
                          float dt_max, const float* h0, void* y, float* h_final, int Bsz,
                          int T, int H, int P, int G, int N, int chunk, int dtype,
                          void* stream) {
  SSD_TRY(check_real_fwd(x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final, Bsz, T, H,
                         P, G, N, chunk, dtype));
  const size_t need = workspace_bytes_for(Bsz, T, H, P, N, chunk, 0);
  if (need > SSD_NOALLOC_SCRATCH_BYTES)
    return fail(SSD_EWORKSPACE,
                "this shape needs %zu bytes of scratch; the allocation-free forward holds %llu "
                "(use ssd_chunk_fwd with a workspace)",
                need, static_cast<unsigned long long>(SSD_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  SSD_TRY(scratch_of_current_device(&ws));
  ssd::ChunkArgs a{x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, y, h_final,
                   Bsz, T, H, P, G, N, chunk, dtype, ws, nullptr};
  return launch_status(ssd::run_chunk_real(a, static_cast<hipStream_t>(stream)));
}

int ssd_complex_chunk_fwd_ev(const float* x, const float* dt, const float* A, const float* B,
                             const float* C, const float* dt_bias, float dt_min, float dt_max,
                             const float* h0, float* y, float* h_final, int Bsz, int T, int H,
                             int P, int G, int N, int chunk, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events) {
  SSD_TRY(check_chunk_shape(Bsz, T, H, P, G, N, chunk, 1));
  const bool has_tokens = T > 0;
  SSD_TRY(check_ptr(x, "x", 16, has_tokens));
  SSD_TRY(check_ptr(dt, "dt", 4, has_tokens));
  SSD_TRY(check_ptr(A, "A", 8, has_tokens));
  SSD_TRY(check_ptr(B, "B", 16, has_tokens));
  SSD_TRY(check_ptr(C, "C", 16, has_tokens));
  SSD_TRY(check_ptr(y, "y", 16, has_tokens));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_ptr(h0, "h0", 16, false));
  SSD_TRY(check_ptr(h_final, "h_final", 16, false));
  SSD_TRY(check_clamp(dt_min, dt_max));
  const size_t need = workspace_bytes_for(Bsz, T, H, P, N, chunk, 1);
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  if (workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  ssd::ChunkArgs a{x, dt, A, B, C, nullptr, dt_bias, dt_min, dt_max, h0, y, h_final,
                   Bsz, T, H, P, G, N, chunk, SSD_F32, workspace,
                   reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_chunk_complex(a, static_cast<hipStream_t>(stream)));
}

int ssd_complex_chunk_fwd(const float* x, const float* dt, const float* A, const float* B,
                          const float* C, const float* dt_bias, float dt_min, float dt_max,
                          const float* h0, float* y, float* h_final, int Bsz, int T, int H, int P,
                          int G, int N, int chunk, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return ssd_complex_chunk_fwd_ev(x, dt, A, B, C, dt_bias, dt_min, dt_max, h0, y, h_final, Bsz,
                                  T, H, P, G, N, chunk, workspace, workspace_bytes, stream,
                                  nullptr);
}

int ssd_complex_chunk_fwd_packed_ev(const float* proj, long long ld, const float* A,
                                    const float* dt_bias, float dt_min, float dt_max,
                                    const float* h0, float* y, float* h_final, int Bsz, int T,
                                    int H, int P, int N, int chunk, void* workspace,
                                    size_t workspace_bytes, void* stream, void* const* events) {
  SSD_TRY(check_chunk_shape(Bsz, T, H, P, H, N, chunk, 1));
  const long long width = static_cast<long long>(H) * (P + 4LL * N + 1);
  if (ld < width)
    return fail(SSD_EINVAL, "ld=%lld is smaller than H*(P+4N+1) = %lld", ld, width);
  if (ld % 4 != 0) return fail(SSD_EINVAL, "ld=%lld is not a multiple of 4 floats", ld);
  if (static_cast<long long>(chunk) * ld * 4 > 4294967295LL - 16)
    return fail(SSD_EUNSUPPORTED, "one chunk's rows exceed 4 GiB: chunk=%d ld=%lld", chunk, ld);
  const bool has_tokens = T > 0;
  SSD_TRY(check_ptr(proj, "proj", 16, has_tokens));
  SSD_TRY(check_ptr(A, "A", 8, has_tokens));
  SSD_TRY(check_ptr(y, "y", 16, has_tokens));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_ptr(h0, "h0", 16, false));
  SSD_TRY(check_ptr(h_final, "h_final", 16, false));
  SSD_TRY(check_clamp(dt_min, dt_max));
  const size_t need = workspace_bytes_for(Bsz, T, H, P, N, chunk, 1);
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  if (workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  ssd::ChunkArgs a{proj, nullptr, A, nullptr, nullptr, nullptr, dt_bias, dt_min, dt_max, h0, y,
                   h_final, Bsz, T, H, P, H, N, chunk, SSD_F32, workspace,
                   reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_chunk_complex_packed(a, static_cast<int>(ld),
                                                     static_cast<hipStream_t>(stream)));
}

int ssd_complex_chunk_fwd_packed(const float* proj, long long ld, const float* A,
                                 const float* dt_bias, float dt_min, float dt_max, const float* h0,
                                 float* y, float* h_final, int Bsz, int T, int H, int P, int N,
                                 int chunk, void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_complex_chunk_fwd_packed_ev(proj, ld, A, dt_bias, dt_min, dt_max, h0, y, h_final, Bsz,
                                         T, H, P, N, chunk, workspace, workspace_bytes, stream,
                                         nullptr);
}

int ssd_step_decode(float* h, const float* x, const float* dt, const float* A, const float* B,
                    const float* C, const float* D, const float* dt_bias, float dt_min,
                    float dt_max, float* y, int Bsz, int H, int P, int G, int N, void* stream) {
  return ssd_step_decode_ev(h, x, dt, A, B, C, D, dt_bias, dt_min, dt_max, y, Bsz, H, P, G, N,
                            stream, nullptr);
}

int ssd_step_decode_ev(float* h, const float* x, const float* dt, const float* A, const float* B,
                       const float* C, const float* D, const float* dt_bias, float dt_min,
                       float dt_max, float* y, int Bsz, int H, int P, int G, int N, void* stream,
                       void* const* events) {
  if (Bsz <= 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0)
    return fail(SSD_EINVAL, "sizes must be positive: Bsz=%d H=%d P=%d G=%d N=%d", Bsz, H, P, G, N);
  if (H % G != 0) return fail(SSD_EINVAL, "H=%d is not a multiple of G=%d", H, G);
  if (!in_set(N, kNsDecode, 5)) return fail(SSD_EUNSUPPORTED, "N=%d not in {16,32,64,128,256}", N);
  if (static_cast<long long>(Bsz) * H > 2147483647LL)
    return fail(SSD_EUNSUPPORTED, "Bsz*H too large");
  SSD_TRY(check_ptr(h, "h", 16, true));
  SSD_TRY(check_ptr(x, "x", 4, true));
  SSD_TRY(check_ptr(dt, "dt", 4, true));
  SSD_TRY(check_ptr(A, "A", 4, true));
  SSD_TRY(check_ptr(B, "B", 16, true));
  SSD_TRY(check_ptr(C, "C", 16, true));
  SSD_TRY(check_ptr(y, "y", 4, true));
  SSD_TRY(check_ptr(D, "D", 4, false));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_clamp(dt_min, dt_max));
  ssd::DecodeArgs a{h, x, dt, A, B, C, D, dt_bias, dt_min, dt_max, y, Bsz, H, P, G, N,
                    reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_decode(a, static_cast<hipStream_t>(stream)));
}

int ssd_complex_step_decode(float* h, const float* x, const float* dt, const float* A,
                            const float* B, const float* C, const float* dt_bias, float dt_min,
                            float dt_max, float* y, int Bsz, int H, int P, int G, int N,
                            void* stream) {
  return ssd_complex_step_decode_ev(h, x, dt, A, B, C, dt_bias, dt_min, dt_max, y, Bsz, H, P, G,
                                    N, stream, nullptr);
}

int ssd_complex_step_decode_ev(float* h, const float* x, const float* dt, const float* A,
                               const float* B, const float* C, const float* dt_bias,
                               float dt_min, float dt_max, float* y, int Bsz, int H, int P,
                               int G, int N, void* stream, void* const* events) {
  if (Bsz <= 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0)
    return fail(SSD_EINVAL, "sizes must be positive: Bsz=%d H=%d P=%d G=%d N=%d", Bsz, H, P, G, N);
  if (H % G != 0) return fail(SSD_EINVAL, "H=%d is not a multiple of G=%d", H, G);
  if (!in_set(N, kNsCplxDecode, 4)) return fail(SSD_EUNSUPPORTED, "N=%d not in {16,32,64,128}", N);
  if (static_cast<long long>(Bsz) * H > 2147483647LL)
    return fail(SSD_EUNSUPPORTED, "Bsz*H too large");
  SSD_TRY(check_ptr(h, "h", 16, true));
  SSD_TRY(check_ptr(x, "x", 4, true));
  SSD_TRY(check_ptr(dt, "dt", 4, true));
  SSD_TRY(check_ptr(A, "A", 4, true));
  SSD_TRY(check_ptr(B, "B", 16, true));
  SSD_TRY(check_ptr(C, "C", 16, true));
  SSD_TRY(check_ptr(y, "y", 4, true));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_clamp(dt_min, dt_max));
  ssd::DecodeArgs a{h, x, dt, A, B, C, nullptr, dt_bias, dt_min, dt_max, y, Bsz, H, P, G, N,
                    reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_complex_decode(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- depthwise causal convolution ----

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return a && b && x < y + nb && y < x + na;
}

// Checks shared by the prefill and the step.  V = channels per 16-byte vector.
int check_conv_common(int Bsz, int HP, int GN, long long ld, int K, int act, int V) {
  if (Bsz <= 0 || HP <= 0 || GN < 0)
    return fail(SSD_EINVAL, "sizes must be positive (GN >= 0): Bsz=%d HP=%d GN=%d", Bsz, HP, GN);
  if (K != 4) return fail(SSD_EUNSUPPORTED, "K=%d: only kernel size 4 is built", K);
  if (act != 0 && act != 1) return fail(SSD_EINVAL, "act=%d not in {0, 1}", act);
  if (HP % V != 0 || GN % V != 0)
    return fail(SSD_EUNSUPPORTED, "HP=%d and GN=%d must be multiples of %d", HP, GN, V);
  const long long Ch = static_cast<long long>(HP) + 2LL * GN;
  if (Ch > 2147483647LL / 4) return fail(SSD_EUNSUPPORTED, "too many channels: %lld", Ch);
  if (ld < Ch) return fail(SSD_EINVAL, "ld=%lld is smaller than HP + 2*GN = %lld", ld, Ch);
  if (ld % V != 0) return fail(SSD_EINVAL, "ld=%lld is not a multiple of %d", ld, V);
  if (ld > 2147483647LL) return fail(SSD_EUNSUPPORTED, "ld=%lld too large", ld);
  if (Bsz > 65535) return fail(SSD_EUNSUPPORTED, "Bsz=%d above 65535", Bsz);
  return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_conv1d_fwd(const void* xbc, long long ld, const float* w, const float* bias,
                   const float* state_in, int act, void* x, void* B, void* C, float* state_out,
                   int Bsz, int T, int HP, int GN, int K, int dtype, void* stream) {
  return ssd_conv1d_fwd_ev(xbc, ld, w, bias, state_in, act, x, B, C, state_out, Bsz, T, HP, GN,
                           K, dtype, stream, nullptr);
}

int ssd_conv1d_fwd_ev(const void* xbc, long long ld, const float* w, const float* bias,
                      const float* state_in, int act, void* x, void* B, void* C, float* state_out,
                      int Bsz, int T, int HP, int GN, int K, int dtype, void* stream,
                      void* const* events) {
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_EUNSUPPORTED, "dtype=%d", dtype);
  const int V = dtype == SSD_BF16 ? 8 : 4;
  const long long es = dtype == SSD_BF16 ? 2 : 4;
  if (T < 0) return fail(SSD_EINVAL, "T=%d is negative", T);
  SSD_TRY(check_conv_common(Bsz, HP, GN, ld, K, act, V));
  // one batch entry's rows (and a run of tokens past T) are addressed by
  // 32-bit byte offsets; blocks of 4 runs of tokens fill grid.y
  const int tt = ssd::conv_tokens_per_thread();
  if ((static_cast<long long>(T) + tt) * ld * es > 4294967295LL - 16)
    return fail(SSD_EUNSUPPORTED, "one batch entry's rows exceed 4 GiB: T=%d ld=%lld", T, ld);
  if ((static_cast<long long>(T) + 4LL * tt - 1) / (4LL * tt) > 65535)
    return fail(SSD_EUNSUPPORTED, "T=%d too long", T);
  const bool has_tokens = T > 0;
  SSD_TRY(check_ptr(xbc, "xbc", 16, has_tokens));
  SSD_TRY(check_ptr(w, "w", 16, true));
  SSD_TRY(check_ptr(bias, "bias", 16, false));
  SSD_TRY(check_ptr(state_in, "state_in", 16, false));
  SSD_TRY(check_ptr(state_out, "state_out", 16, false));
  SSD_TRY(check_ptr(x, "x", 16, has_tokens));
  SSD_TRY(check_ptr(B, "B", 16, has_tokens && GN > 0));
  SSD_TRY(check_ptr(C, "C", 16, has_tokens && GN > 0));
  const size_t Ch = static_cast<size_t>(HP) + 2 * static_cast<size_t>(GN);
  const size_t sbytes = static_cast<size_t>(Bsz) * 3 * Ch * 4;
  if (overlaps(state_in, sbytes, state_out, sbytes))
    return fail(SSD_EINVAL, "state_in and state_out overlap");
  ssd::ConvArgs a{xbc, static_cast<int>(ld), w, bias, state_in, state_out, act, x, B, C,
                  Bsz, T, HP, GN, dtype,
                  reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_conv1d(a, static_cast<hipStream_t>(stream)));
}

size_t ssd_conv1d_varlen_workspace_size(int nseq) {
  if (nseq <= 0 || nseq > 65535) return 0;
  return (static_cast<size_t>(nseq) + 1) * 4 / 256 * 256 + 256;
}

int ssd_conv1d_fwd_varlen_ev(const void* xbc, long long ld, const float* w, const float* bias,
                             const float* state_in, int act, void* x, void* B, void* C,
                             float* state_out, const int* cu_seqlens, int nseq, int HP, int GN, int K,
                             int dtype, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events) {
  if (!cu_seqlens) return fail(SSD_EINVAL, "cu_seqlens is NULL");
  if (nseq <= 0 || nseq > 65535) return fail(SSD_EINVAL, "nseq=%d not in [1, 65535]", nseq);
  if (cu_seqlens[0] != 0) return fail(SSD_EINVAL, "cu_seqlens: cu_seqlens[0] must be 0");
  int Tmax = 0;
  for (int b = 0; b < nseq; ++b) {
    if (cu_seqlens[b + 1] < cu_seqlens[b]) return fail(SSD_EINVAL, "cu_seqlens: must be non-decreasing");
    const int t = cu_seqlens[b + 1] - cu_seqlens[b];
    Tmax = t > Tmax ? t : Tmax;
  }
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_EUNSUPPORTED, "dtype=%d", dtype);
  const int V = dtype == SSD_BF16 ? 8 : 4;
  const long long es = dtype == SSD_BF16 ? 2 : 4;
  SSD_TRY(check_conv_common(nseq, HP, GN, ld, K, act, V));
  const int tt = ssd::conv_tokens_per_thread();
  if ((static_cast<long long>(Tmax) + tt) * ld * es > 4294967295LL - 16)
    return fail(SSD_EUNSUPPORTED, "one sequence's rows exceed 4 GiB: T=%d ld=%lld", Tmax, ld);
  if ((static_cast<long long>(Tmax) + 4LL * tt - 1) / (4LL * tt) > 65535)
    return fail(SSD_EUNSUPPORTED, "a sequence of T=%d is too long", Tmax);
  const bool has_tokens = cu_seqlens[nseq] > 0;
  SSD_TRY(check_ptr(xbc, "xbc", 16, has_tokens));
  SSD_TRY(check_ptr(w, "w", 16, true));
  SSD_TRY(check_ptr(bias, "bias", 16, false));
  SSD_TRY(check_ptr(state_in, "state_in", 16, false));
  SSD_TRY(check_ptr(state_out, "state_out", 16, false));
  SSD_TRY(check_ptr(x, "x", 16, has_tokens));
  SSD_TRY(check_ptr(B, "B", 16, has_tokens && GN > 0));
  SSD_TRY(check_ptr(C, "C", 16, has_tokens && GN > 0));
  const size_t Ch = static_cast<size_t>(HP) + 2 * static_cast<size_t>(GN);
  const size_t sbytes = static_cast<size_t>(nseq) * 3 * Ch * 4;
  if (overlaps(state_in, sbytes, state_out, sbytes))
    return fail(SSD_EINVAL, "state_in and state_out overlap");
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  const size_t need = ssd_conv1d_varlen_workspace_size(nseq);
  if (workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  ssd::ConvArgs a{xbc, static_cast<int>(ld), w, bias, state_in, state_out, act, x, B, C,
                  nseq, Tmax, HP, GN, dtype,
                  reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_conv1d_varlen(a, cu_seqlens, workspace, static_cast<hipStream_t>(stream)));
}

int ssd_conv1d_fwd_varlen(const void* xbc, long long ld, const float* w, const float* bias,
                          const float* state_in, int act, void* x, void* B, void* C, float* state_out,
                          const int* cu_seqlens, int nseq, int HP, int GN, int K, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_conv1d_fwd_varlen_ev(xbc, ld, w, bias, state_in, act, x, B, C, state_out, cu_seqlens, nseq,
                                  HP, GN, K, dtype, workspace, workspace_bytes, stream, nullptr);
}

int ssd_conv1d_step(float* state, const float* xt, long long ld, const float* w,
                    const float* bias, int act, float* x, float* B, float* C, int Bsz, int HP,
                    int GN, int K, void* stream) {
  return ssd_conv1d_step_ev(state, xt, ld, w, bias, act, x, B, C, Bsz, HP, GN, K, stream,
                            nullptr);
}

int ssd_conv1d_step_ev(float* state, const float* xt, long long ld, const float* w,
                       const float* bias, int act, float* x, float* B, float* C, int Bsz, int HP,
                       int GN, int K, void* stream, void* const* events) {
  SSD_TRY(check_conv_common(Bsz, HP, GN, ld, K, act, 4));
  SSD_TRY(check_ptr(state, "state", 16, true));
  SSD_TRY(check_ptr(xt, "xt", 16, true));
  SSD_TRY(check_ptr(w, "w", 16, true));
  SSD_TRY(check_ptr(bias, "bias", 16, false));
  SSD_TRY(check_ptr(x, "x", 16, true));
  SSD_TRY(check_ptr(B, "B", 16, GN > 0));
  SSD_TRY(check_ptr(C, "C", 16, GN > 0));
  ssd::ConvArgs a{xt, static_cast<int>(ld), w, bias, nullptr, state, act, x, B, C,
                  Bsz, 1, HP, GN, SSD_F32,
                  reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_conv1d_step(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- backward of the chunked real form ----

extern "C" {

size_t ssd_bwd_workspace_size(int Bsz, int T, int H, int P, int G, int N, int chunk) {
  if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || chunk <= 0 || H % G != 0)
    return 0;
  return ssd::bwd_workspace_bytes(Bsz, T, H, P, G, N, chunk);
}

int ssd_chunk_bwd(const void* x, const float* dt, const float* A, const void* B, const void* C,
                  const float* D, const float* dt_bias, float dt_min, float dt_max,
                  const float* h0, const void* dy, const float* dh_final, void* dx, float* ddt,
                  float* dA, float* dB, float* dC, float* dD, float* ddt_bias, float* dh0,
                  int Bsz, int T, int H, int P, int G, int N, int chunk, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_chunk_bwd_ev(x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, dy, dh_final, dx, ddt,
                          dA, dB, dC, dD, ddt_bias, dh0, Bsz, T, H, P, G, N, chunk, dtype,
                          workspace, workspace_bytes, stream, nullptr);
}

int ssd_chunk_bwd_ev(const void* x, const float* dt, const float* A, const void* B, const void* C,
                     const float* D, const float* dt_bias, float dt_min, float dt_max,
                     const float* h0, const void* dy, const float* dh_final, void* dx, float* ddt,
                     float* dA, float* dB, float* dC, float* dD, float* ddt_bias, float* dh0,
                     int Bsz, int T, int H, int P, int G, int N, int chunk, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream,
                     void* const* events) {
  SSD_TRY(check_chunk_shape(Bsz, T, H, P, G, N, chunk, 0));
  const bool f32 = dtype == SSD_F32;
  if (dtype != SSD_BF16 && !f32) return fail(SSD_EUNSUPPORTED, "dtype=%d", dtype);
  if (f32) {
    if (!((P == 64 || P == 32) && (N == 32 || N == 64 || N == 128)))
      return fail(SSD_EUNSUPPORTED, "fp32 backward: (P, N) = (%d, %d) not in {32, 64} x {32, 64, 128}", P,
                  N);
    if (chunk != 64) return fail(SSD_EUNSUPPORTED, "fp32 backward: chunk=%d, must be 64", chunk);
  } else {
    if (!((P == 64 || P == 32) && (N == 64 || N == 128)))
      return fail(SSD_EUNSUPPORTED, "backward: (P, N) = (%d, %d) not in {32, 64} x {64, 128}", P, N);
    if (chunk < 64) return fail(SSD_EUNSUPPORTED, "backward: chunk=%d not in {64, 128, 256}", chunk);
  }
  const bool has_tokens = T > 0;
  SSD_TRY(check_ptr(x, "x", 16, has_tokens));
  SSD_TRY(check_ptr(dt, "dt", 4, has_tokens));
  SSD_TRY(check_ptr(A, "A", 4, true));
  SSD_TRY(check_ptr(B, "B", 16, has_tokens));
  SSD_TRY(check_ptr(C, "C", 16, has_tokens));
  SSD_TRY(check_ptr(D, "D", 4, false));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_ptr(h0, "h0", 16, false));
  SSD_TRY(check_ptr(dy, "dy", 16, has_tokens));
  SSD_TRY(check_ptr(dh_final, "dh_final", 16, false));
  SSD_TRY(check_ptr(dx, "dx", 16, has_tokens));
  SSD_TRY(check_ptr(ddt, "ddt", 4, has_tokens));
  SSD_TRY(check_ptr(dA, "dA", 4, true));
  SSD_TRY(check_ptr(dB, "dB", 16, has_tokens));
  SSD_TRY(check_ptr(dC, "dC", 16, has_tokens));
  SSD_TRY(check_ptr(dD, "dD", 4, true));
  SSD_TRY(check_ptr(ddt_bias, "ddt_bias", 4, true));
  SSD_TRY(check_ptr(dh0, "dh0", 16, false));
  SSD_TRY(check_clamp(dt_min, dt_max));
  const int hpg = ssd::bwd_heads_per_group(H, G);
  const long long nc = (static_cast<long long>(T) + chunk - 1) / chunk;
  const long long bpairs = (static_cast<long long>(Bsz) * nc * (chunk / 64) + 7) / 8 * 8;
  if (bpairs * (H / hpg) > 2147483647LL)
    return fail(SSD_EUNSUPPORTED, "grid too large for the backward");
  const size_t need = f32 ? ssd::bwd_f32_workspace_bytes(Bsz, T, H, P, G, N, false)
                          : ssd::bwd_workspace_bytes(Bsz, T, H, P, G, N, chunk);
  if (!workspace || workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  ssd::BwdArgs a{x, dt, A, B, C, D, dt_bias, dt_min, dt_max, h0, dy, dh_final, dx, ddt, dA, dB,
                 dC, dD, ddt_bias, dh0, Bsz, T, H, P, G, N, chunk, workspace,
                 reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  if (f32) return launch_status(ssd::run_chunk_bwd_f32(a, static_cast<hipStream_t>(stream)));
  return launch_status(ssd::run_chunk_bwd_bf16(a, static_cast<hipStream_t>(stream)));
}

size_t ssd_bwd_workspace_size_f32(int Bsz, int T, int H, int P, int G, int N) {
  if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0) return 0;
  return ssd::bwd_f32_workspace_bytes(Bsz, T, H, P, G, N, false);
}

size_t ssd_complex_bwd_workspace_size(int Bsz, int T, int H, int P, int G, int N) {
  if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0) return 0;
  return ssd::bwd_f32_workspace_bytes(Bsz, T, H, P, G, N, true);
}

int ssd_complex_chunk_bwd(const float* x, const float* dt, const float* A, const float* B,
                          const float* C, const float* dt_bias, float dt_min, float dt_max,
                          const float* h0, const float* dy, const float* dh_final, float* dx,
                          float* ddt, float* dA, float* dB, float* dC, float* ddt_bias, float* dh0,
                          int Bsz, int T, int H, int P, int G, int N, int chunk, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return ssd_complex_chunk_bwd_ev(x, dt, A, B, C, dt_bias, dt_min, dt_max, h0, dy, dh_final, dx, ddt,
                                  dA, dB, dC, ddt_bias, dh0, Bsz, T, H, P, G, N, chunk, workspace,
                                  workspace_bytes, stream, nullptr);
}

int ssd_complex_chunk_bwd_ev(const float* x, const float* dt, const float* A, const float* B,
                             const float* C, const float* dt_bias, float dt_min, float dt_max,
                             const float* h0, const float* dy, const float* dh_final, float* dx,
                             float* ddt, float* dA, float* dB, float* dC, float* ddt_bias,
                             float* dh0, int Bsz, int T, int H, int P, int G, int N, int chunk,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events) {
  SSD_TRY(check_chunk_shape(Bsz, T, H, P, G, N, chunk, 1));
  if (!((P == 64 || P == 32) && (N == 16 || N == 32 || N == 64)))
    return fail(SSD_EUNSUPPORTED, "complex backward: (P, N) = (%d, %d) not in {32, 64} x {16, 32, 64}", P,
                N);
  if (chunk != 64) return fail(SSD_EUNSUPPORTED, "complex backward: chunk=%d, must be 64", chunk);
  const bool has_tokens = T > 0;
  SSD_TRY(check_ptr(x, "x", 16, has_tokens));
  SSD_TRY(check_ptr(dt, "dt", 4, has_tokens));
  SSD_TRY(check_ptr(A, "A", 8, true));
  SSD_TRY(check_ptr(B, "B", 16, has_tokens));
  SSD_TRY(check_ptr(C, "C", 16, has_tokens));
  SSD_TRY(check_ptr(dt_bias, "dt_bias", 4, false));
  SSD_TRY(check_ptr(h0, "h0", 16, false));
  SSD_TRY(check_ptr(dy, "dy", 16, has_tokens));
  SSD_TRY(check_ptr(dh_final, "dh_final", 16, false));
  SSD_TRY(check_ptr(dx, "dx", 16, has_tokens));
  SSD_TRY(check_ptr(ddt, "ddt", 4, has_tokens));
  SSD_TRY(check_ptr(dA, "dA", 8, true));
  SSD_TRY(check_ptr(dB, "dB", 16, has_tokens));
  SSD_TRY(check_ptr(dC, "dC", 16, has_tokens));
  SSD_TRY(check_ptr(ddt_bias, "ddt_bias", 4, true));
  SSD_TRY(check_ptr(dh0, "dh0", 16, false));
  SSD_TRY(check_clamp(dt_min, dt_max));
  const size_t need = ssd::bwd_f32_workspace_bytes(Bsz, T, H, P, G, N, true);
  if (!workspace || workspace_bytes < need)
    return fail(SSD_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  SSD_TRY(check_ptr(workspace, "workspace", 256, true));
  ssd::CplxBwdArgs a{x, dt, A, B, C, dt_bias, dt_min, dt_max, h0, dy, dh_final, dx, ddt, dA, dB, dC,
                     ddt_bias, dh0, Bsz, T, H, P, G, N, workspace,
                     reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_complex_bwd(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- bias-free linear layers (MIMO, out_proj) ----

extern "C" {

int ssd_linear_fwd_ev(const void* x, int x_dtype, const void* W, void* z, int z_dtype, int M,
                      int K, int Nout, void* stream, void* const* events) {
  if (M < 0 || K <= 0 || Nout <= 0)
    return fail(SSD_EINVAL, "sizes must be positive (M >= 0): M=%d K=%d Nout=%d", M, K, Nout);
  if (K % 64 != 0) return fail(SSD_EUNSUPPORTED, "K=%d is not a multiple of 64", K);
  if (Nout % 128 != 0) return fail(SSD_EUNSUPPORTED, "Nout=%d is not a multiple of 128", Nout);
  if ((x_dtype != SSD_F32 && x_dtype != SSD_BF16) || (z_dtype != SSD_F32 && z_dtype != SSD_BF16))
    return fail(SSD_EUNSUPPORTED, "x_dtype=%d z_dtype=%d: each must be SSD_F32 or SSD_BF16",
                x_dtype, z_dtype);
  // one block of 128 rows (x and z) and W are addressed by 32-bit byte offsets
  if (128LL * K * 4 > 4294967295LL || 128LL * Nout * 4 > 4294967295LL ||
      static_cast<long long>(Nout) * K * 2 > 4294967295LL)
    return fail(SSD_EUNSUPPORTED, "K=%d Nout=%d too large", K, Nout);
  const long long mblocks = (static_cast<long long>(M) + 127) / 128;
  if ((mblocks + 7) / 8 * 8 * (Nout / 128) > 2147483647LL)
    return fail(SSD_EUNSUPPORTED, "grid too large: M=%d Nout=%d", M, Nout);
  SSD_TRY(check_ptr(x, "x", 16, M > 0));
  SSD_TRY(check_ptr(W, "W", 16, true));
  SSD_TRY(check_ptr(z, "z", 16, M > 0));
  ssd::LinearArgs a{x, x_dtype, static_cast<const uint16_t*>(W), z, z_dtype, M, K, Nout,
                    reinterpret_cast<hipEvent_t*>(const_cast<void**>(events))};
  return launch_status(ssd::run_linear(a, static_cast<hipStream_t>(stream)));
}

int ssd_linear_fwd(const void* x, int x_dtype, const void* W, void* z, int z_dtype, int M, int K,
                   int Nout, void* stream) {
  return ssd_linear_fwd_ev(x, x_dtype, W, z, z_dtype, M, K, Nout, stream, nullptr);
}

int ssd_mimo_fwd(const void* y, int y_dtype, const void* W, void* z, int z_dtype, int Bsz, int T,
                 int H, int P, void* stream) {
  if (Bsz <= 0 || T < 0 || H <= 0 || P <= 0)
    return fail(SSD_EINVAL, "sizes must be positive (T >= 0): Bsz=%d T=%d H=%d P=%d", Bsz, T, H, P);
  const long long M = static_cast<long long>(Bsz) * T, HP = static_cast<long long>(H) * P;
  if (M > 2147483647LL || HP > 2147483647LL)
    return fail(SSD_EUNSUPPORTED, "Bsz*T=%lld or H*P=%lld too large", M, HP);
  return ssd_linear_fwd_ev(y, y_dtype, W, z, z_dtype, static_cast<int>(M), static_cast<int>(HP),
                           static_cast<int>(HP), stream, nullptr);
}

}  // extern "C"
