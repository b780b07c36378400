// C ABI of libdmel_bench (dmel_bench.h): host validation before any HIP call,
// then the launches.
#include "dmel_bench.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "bench_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) { return fail(DMEL_EHIP, "%s: %s", what, hipGetErrorString(e)); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

const char* dmel_bench_last_error(void) { return g_last_error.c_str(); }

size_t dmel_bench_dft_matrix_bytes(void) { return dmel::dft_matrix_bytes(); }

int dmel_bench_dft_matrix(void* matrix, void* stream) {
  if (matrix == nullptr) return fail(DMEL_EINVAL, "matrix is NULL");
  if (!aligned(matrix, 256)) return fail(DMEL_EALIGN, "matrix is not 256-byte aligned");
  hipError_t e = dmel::launch_dft_matrix(static_cast<uint16_t*>(matrix), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "dft matrix launch");
}

size_t dmel_bench_dft_gemm_workspace_bytes(int64_t n_frames_total) {
  return n_frames_total < 0 ? 0 : dmel::dft_gemm_workspace_bytes(n_frames_total);
}

int dmel_bench_frames_dft_gemm(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                               const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                               int64_t n_frames_total, const float* carry, const void* matrix, float* logmel,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (n_samples_total < 0 || n_clips < 0 || n_frames_total < 0) return fail(DMEL_EINVAL, "negative count");
  if (n_frames_total > n_samples_total / dmel::kHop)
    return fail(DMEL_ESHAPE, "n_frames_total %lld exceeds n_samples_total / 800", (long long)n_frames_total);
  if (n_frames_total > 0 && n_clips == 0) return fail(DMEL_ESHAPE, "frames requested but n_clips is 0");
  if (ctx == nullptr) return fail(DMEL_EINVAL, "ctx is NULL");
  if (ctx->dev_mem == nullptr) return fail(DMEL_ESTATE, "ctx has no device tables");
  const size_t need = dmel::dft_gemm_workspace_bytes(n_frames_total);
  if (workspace_bytes < need)
    return fail(DMEL_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (n_frames_total == 0) return DMEL_OK;
  if (audio == nullptr || sample_off == nullptr || frame_off == nullptr || matrix == nullptr || logmel == nullptr ||
      workspace == nullptr)
    return fail(DMEL_EINVAL, "NULL pointer argument");
  if (!aligned(audio, 4) || !aligned(sample_off, 8) || !aligned(frame_off, 8) || !aligned(matrix, 256) ||
      !aligned(workspace, 256) || (carry != nullptr && !aligned(carry, 4)))
    return fail(DMEL_EALIGN, "misaligned pointer argument");
  hipError_t e = dmel::launch_dft_gemm_frames(ctx->tabs, audio, n_samples_total, sample_off, frame_off, n_clips,
                                              n_frames_total, carry, static_cast<const uint16_t*>(matrix), logmel,
                                              workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "dft gemm launch");
}

int dmel_bench_rounding_probe(const float* c, const uint16_t* e, int64_t n, float* out, void* stream) {
  if (n < 0 || n % 1024 != 0) return fail(DMEL_ESHAPE, "n must be a non-negative multiple of 1024 (got %lld)", (long long)n);
  if (n == 0) return DMEL_OK;
  if (c == nullptr || e == nullptr || out == nullptr) return fail(DMEL_EINVAL, "NULL pointer argument");
  if (!aligned(c, 16) || !aligned(e, 16) || !aligned(out, 16)) return fail(DMEL_EALIGN, "arrays must be 16-byte aligned");
  hipError_t err = dmel::launch_rounding_probe(c, e, n, out, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? DMEL_OK : hip_fail(err, "rounding probe launch");
}

int dmel_bench_valu_rate(int32_t kind, int32_t blocks, int32_t iters, float* out, void* stream) {
  if (kind < 0 || kind > 16) return fail(DMEL_EINVAL, "kind must be in [0, 16] (got %d)", kind);
  if (blocks < 1 || iters < 1) return fail(DMEL_EINVAL, "blocks and iters must be positive");
  if (out == nullptr) return fail(DMEL_EINVAL, "NULL pointer argument");
  if (!aligned(out, 4)) return fail(DMEL_EALIGN, "out must be 4-byte aligned");
  hipError_t err = dmel::launch_valu_rate(kind, blocks, iters, out, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? DMEL_OK : hip_fail(err, "valu rate launch");
}

int dmel_bench_lds_rate(int32_t mode, int32_t blocks, int32_t iters, float* out, void* stream) {
  if (mode < 0 || mode > 3) return fail(DMEL_EINVAL, "mode must be in [0, 3] (got %d)", mode);
  if (blocks < 1 || iters < 1) return fail(DMEL_EINVAL, "blocks and iters must be positive");
  if (out == nullptr) return fail(DMEL_EINVAL, "NULL pointer argument");
  if (!aligned(out, 4)) return fail(DMEL_EALIGN, "out must be 4-byte aligned");
  hipError_t err = dmel::launch_lds_rate(mode, blocks, iters, out, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? DMEL_OK : hip_fail(err, "lds rate launch");
}

}  // extern "C"
