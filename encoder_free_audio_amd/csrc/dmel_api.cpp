// C ABI of libdmel: argument validation (host only, before any HIP call),
// context management and kernel launches.  See include/dmel.h.
#include "dmel.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"

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

int hip_fail(hipError_t e, const char* what) {
  return fail(DMEL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validation of the audio arguments shared by dmel_frames/levels/forward.
int check_audio(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total, const int64_t* sample_off,
                const int64_t* frame_off, int32_t n_clips, int64_t n_frames_total, const void* out,
                const char* out_name) {
  if (n_samples_total < 0) return fail(DMEL_EINVAL, "n_samples_total is negative (%lld)", (long long)n_samples_total);
  if (n_clips < 0) return fail(DMEL_EINVAL, "n_clips is negative (%d)", n_clips);
  if (n_frames_total < 0) return fail(DMEL_EINVAL, "n_frames_total is negative (%lld)", (long long)n_frames_total);
  if (n_frames_total > n_samples_total / dmel::kHop)
    return fail(DMEL_ESHAPE, "n_frames_total %lld exceeds n_samples_total / 800 = %lld", (long long)n_frames_total,
                (long long)(n_samples_total / dmel::kHop));
  if (n_frames_total > 0 && n_clips == 0) return fail(DMEL_ESHAPE, "frames requested but n_clips is 0");
  if (n_frames_total > 0) {
    if (audio == nullptr) return fail(DMEL_EINVAL, "audio is NULL");
    if (sample_off == nullptr || frame_off == nullptr) return fail(DMEL_EINVAL, "sample_off / frame_off is NULL");
    if (out == nullptr) return fail(DMEL_EINVAL, "%s is NULL", out_name);
    if (!aligned(audio, 4)) return fail(DMEL_EALIGN, "audio is not 4-byte aligned");
    if (!aligned(sample_off, 8) || !aligned(frame_off, 8)) return fail(DMEL_EALIGN, "offset arrays are not 8-byte aligned");
  }
  if (ctx == nullptr) return fail(DMEL_EINVAL, "ctx is NULL");
  if (ctx->dev_mem == nullptr) return fail(DMEL_ESTATE, "ctx has no device tables");
  return DMEL_OK;
}

int check_table(const uint16_t* table, int32_t d_model) {
  if (d_model < 16 || d_model > 65536 || d_model % 16 != 0)
    return fail(DMEL_ESHAPE, "d_model must be a multiple of 16 in [16, 65536] (got %d)", d_model);
  if (table == nullptr) return fail(DMEL_EINVAL, "table is NULL");
  if (!aligned(table, 16)) return fail(DMEL_EALIGN, "table is not 16-byte aligned");
  return DMEL_OK;
}

int check_out(void* out, int32_t out_dtype, int64_t out_row_stride, int32_t width, const int64_t* out_rows) {
  if (out_dtype != DMEL_BF16 && out_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported out_dtype %d", out_dtype);
  if (out == nullptr) return fail(DMEL_EINVAL, "out is NULL");
  const int64_t esize = out_dtype == DMEL_BF16 ? 2 : 4;
  if (out_row_stride < width) return fail(DMEL_ESHAPE, "out_row_stride %lld < d_model %d", (long long)out_row_stride, width);
  if (!aligned(out, 16)) return fail(DMEL_EALIGN, "out is not 16-byte aligned");
  if ((out_row_stride * esize) % 16 != 0) return fail(DMEL_EALIGN, "out_row_stride * element size is not a multiple of 16 bytes");
  if (out_rows != nullptr && !aligned(out_rows, 8)) return fail(DMEL_EALIGN, "out_rows is not 8-byte aligned");
  return DMEL_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Table layout accepted by the embedding kernels.
int check_layout(int32_t n_bins, int32_t n_levels) {
  if (n_bins < 1 || n_bins > dmel::kEmbMaxBins)
    return fail(DMEL_ESHAPE, "n_bins must be in [1, %d] (got %d)", dmel::kEmbMaxBins, n_bins);
  if (n_levels < 1 || n_levels > dmel::kEmbMaxLevels)
    return fail(DMEL_ESHAPE, "n_levels must be in [1, %d] (got %d)", dmel::kEmbMaxLevels, n_levels);
  return DMEL_OK;
}

bool released_layout(int32_t n_bins, int32_t n_levels) {
  return n_bins == dmel::kMels && n_levels == dmel::kLevels;
}

// [a, a + na) and [b, b + nb) share a byte (empty ranges never do).
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

int check_config(const dmel_config* c) {
  if (c->n_mel_bins < 1 || c->n_mel_bins > dmel::kMaxMels)
    return fail(DMEL_EINVAL, "n_mel_bins must be in [1, %d] (got %d)", dmel::kMaxMels, c->n_mel_bins);
  if (c->mel_vocab_size < 1 || c->mel_vocab_size > dmel::kMaxLevels)
    return fail(DMEL_EINVAL, "mel_vocab_size must be in [1, %d] (got %d)", dmel::kMaxLevels, c->mel_vocab_size);
  if (!std::isfinite(c->min_value) || !std::isfinite(c->max_value) || !(c->min_value < c->max_value))
    return fail(DMEL_EINVAL, "need finite min_value < max_value (got %g, %g)", c->min_value, c->max_value);
  const double width = static_cast<double>(c->max_value) - static_cast<double>(c->min_value);
  if (!(width >= 1e-6) || !(width <= 1e30))
    return fail(DMEL_EINVAL, "max_value - min_value must be in [1e-6, 1e30] (got %g)", width);
  return DMEL_OK;
}

}  // namespace

extern "C" {

int dmel_get_params(dmel_params* out) {
  if (out == nullptr) return fail(DMEL_EINVAL, "out is NULL");
  out->sample_rate = dmel::kSampleRate;
  out->hop = dmel::kHop;
  out->window = dmel::kWindow;
  out->n_fft = dmel::kNfft;
  out->n_bins = dmel::kBins;
  out->n_mels = dmel::kMels;
  out->n_levels = dmel::kLevels;
  out->n_rows = dmel::kRows;
  out->clamp_min = dmel::kClampMin;
  out->clamp_max = dmel::kClampMax;
  out->log_floor = dmel::kLogFloor;
  out->f_min_hz = 0.0f;
  out->f_max_hz = dmel::kSampleRate / 2.0f;
  return DMEL_OK;
}

int64_t dmel_num_frames(int64_t n_samples) { return n_samples < 0 ? -1 : n_samples / dmel::kHop; }

int dmel_default_config(dmel_config* out) {
  if (out == nullptr) return fail(DMEL_EINVAL, "out is NULL");
  out->n_mel_bins = dmel::kMels;
  out->mel_vocab_size = dmel::kLevels;
  out->min_value = dmel::kClampMin;
  out->max_value = dmel::kClampMax;
  return DMEL_OK;
}

int dmel_get_config(const dmel_ctx* ctx, dmel_config* out) {
  if (ctx == nullptr || out == nullptr) return fail(DMEL_EINVAL, "ctx / out is NULL");
  *out = ctx->cfg;
  return DMEL_OK;
}

const char* dmel_last_error(void) { return g_last_error.c_str(); }

int dmel_create(dmel_ctx** out, int device) { return dmel_create_config(out, device, nullptr); }

int dmel_create_config(dmel_ctx** out, int device, const dmel_config* config) {
  if (out == nullptr) return fail(DMEL_EINVAL, "out is NULL");
  *out = nullptr;
  dmel_config cfg;
  dmel_default_config(&cfg);
  if (config != nullptr) {
    int rc = check_config(config);
    if (rc != DMEL_OK) return rc;
    cfg = *config;
  }
  int n_dev = 0;
  hipError_t e = hipGetDeviceCount(&n_dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device < 0 || device >= n_dev) return fail(DMEL_EINVAL, "device %d out of range (%d devices)", device, n_dev);
  int prev = 0;
  e = hipGetDevice(&prev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipSetDevice(device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  // the device address of the allocation-free forward's scratch (once per device)
  e = dmel::noalloc_init(device);
  if (e != hipSuccess) {
    (void)hipSetDevice(prev);
    return hip_fail(e, "scratch symbol lookup");
  }

  dmel::HostTables* h = new (std::nothrow) dmel::HostTables;
  dmel_ctx* ctx = new (std::nothrow) dmel_ctx;
  if (h == nullptr || ctx == nullptr) {
    delete h;
    delete ctx;
    (void)hipSetDevice(prev);
    return fail(DMEL_ENOMEM, "host allocation failed");
  }
  if (!dmel::build_host_tables(h, cfg.n_mel_bins, cfg.mel_vocab_size, cfg.min_value, cfg.max_value)) {
    delete h;
    delete ctx;
    (void)hipSetDevice(prev);
    return fail(DMEL_EINVAL, "filter schedule for %d filters exceeds its table", cfg.n_mel_bins);
  }
  // layout: window | tw800 | tw1600 | twa | seg_start | seg_lo | seg_hi | seg_inv | q_edge |
  //         lds_image | mel_w | mel_first | mel_filt | mel_round
  size_t off_window = 0;
  size_t off_tw800 = round_up(off_window + sizeof(h->window), 256);
  size_t off_tw1600 = round_up(off_tw800 + sizeof(h->tw800), 256);
  size_t off_twa = round_up(off_tw1600 + sizeof(h->tw1600), 256);
  size_t off_seg = round_up(off_twa + sizeof(h->twa), 256);
  size_t off_lo = round_up(off_seg + sizeof(h->seg_start), 256);
  size_t off_hi = round_up(off_lo + sizeof(h->seg_lo), 256);
  size_t off_inv = round_up(off_hi + sizeof(h->seg_hi), 256);
  size_t off_qe = round_up(off_inv + sizeof(h->seg_inv), 256);
  size_t off_img = round_up(off_qe + sizeof(h->q_edge), 256);
  size_t off_mw = round_up(off_img + sizeof(h->lds_image), 256);
  size_t off_mb = round_up(off_mw + sizeof(h->mel_w), 256);
  size_t off_mf = round_up(off_mb + sizeof(h->mel_first), 256);
  size_t off_mr = round_up(off_mf + sizeof(h->mel_filt), 256);
  size_t total = round_up(off_mr + sizeof(h->mel_round), 256);
  char* staging = new (std::nothrow) char[total];
  if (staging == nullptr) {
    delete h;
    delete ctx;
    (void)hipSetDevice(prev);
    return fail(DMEL_ENOMEM, "host allocation failed");
  }
  std::memset(staging, 0, total);
  std::memcpy(staging + off_window, h->window, sizeof(h->window));
  std::memcpy(staging + off_tw800, h->tw800, sizeof(h->tw800));
  std::memcpy(staging + off_tw1600, h->tw1600, sizeof(h->tw1600));
  std::memcpy(staging + off_twa, h->twa, sizeof(h->twa));
  std::memcpy(staging + off_seg, h->seg_start, sizeof(h->seg_start));
  std::memcpy(staging + off_lo, h->seg_lo, sizeof(h->seg_lo));
  std::memcpy(staging + off_hi, h->seg_hi, sizeof(h->seg_hi));
  std::memcpy(staging + off_inv, h->seg_inv, sizeof(h->seg_inv));
  std::memcpy(staging + off_qe, h->q_edge, sizeof(h->q_edge));
  std::memcpy(staging + off_img, h->lds_image, sizeof(h->lds_image));
  std::memcpy(staging + off_mw, h->mel_w, sizeof(h->mel_w));
  std::memcpy(staging + off_mb, h->mel_first, sizeof(h->mel_first));
  std::memcpy(staging + off_mf, h->mel_filt, sizeof(h->mel_filt));
  std::memcpy(staging + off_mr, h->mel_round, sizeof(h->mel_round));
  int rc = DMEL_OK;
  char* dev = nullptr;
  e = hipMalloc(reinterpret_cast<void**>(&dev), total);
  if (e != hipSuccess) {
    rc = fail(DMEL_ENOMEM, "hipMalloc of %zu bytes failed: %s", total, hipGetErrorString(e));
  } else {
    e = hipMemcpy(dev, staging, total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      rc = hip_fail(e, "hipMemcpy of constant tables");
      (void)hipFree(dev);
      dev = nullptr;
    }
  }
  if (rc == DMEL_OK) {
    ctx->device = device;
    ctx->dev_mem = dev;
    ctx->tabs.window = reinterpret_cast<const float*>(dev + off_window);
    ctx->tabs.tw800 = reinterpret_cast<const float2*>(dev + off_tw800);
    ctx->tabs.tw1600 = reinterpret_cast<const float2*>(dev + off_tw1600);
    ctx->tabs.twa = reinterpret_cast<const float2*>(dev + off_twa);
    ctx->tabs.seg_start = reinterpret_cast<const int*>(dev + off_seg);
    ctx->tabs.seg_lo = reinterpret_cast<const float*>(dev + off_lo);
    ctx->tabs.seg_hi = reinterpret_cast<const float*>(dev + off_hi);
    ctx->tabs.seg_inv = reinterpret_cast<const float*>(dev + off_inv);
    ctx->tabs.q_edge = reinterpret_cast<const float*>(dev + off_qe);
    ctx->tabs.lds_image = reinterpret_cast<const float*>(dev + off_img);
    ctx->tabs.mel_in_lds = h->mel_in_lds;
    ctx->tabs.mel_w = reinterpret_cast<const float4*>(dev + off_mw);
    ctx->tabs.mel_first = reinterpret_cast<const int*>(dev + off_mb);
    ctx->tabs.mel_filt = reinterpret_cast<const int*>(dev + off_mf);
    ctx->tabs.mel_round = reinterpret_cast<const int*>(dev + off_mr);
    ctx->tabs.n_mels = cfg.n_mel_bins;
    ctx->tabs.n_levels = cfg.mel_vocab_size;
    ctx->tabs.q_lo = cfg.min_value;
    ctx->tabs.q_hi = cfg.max_value;
    ctx->tabs.q_scale = static_cast<float>(cfg.mel_vocab_size / (static_cast<double>(cfg.max_value) - cfg.min_value));
    ctx->cfg = cfg;
    *out = ctx;
  } else {
    delete ctx;
  }
  delete[] staging;
  delete h;
  (void)hipSetDevice(prev);
  return rc;
}

int dmel_destroy(dmel_ctx* ctx) {
  if (ctx == nullptr) return DMEL_OK;
  int rc = DMEL_OK;
  if (ctx->dev_mem != nullptr) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(ctx->device);
    hipError_t e = hipFree(ctx->dev_mem);
    if (e != hipSuccess) rc = hip_fail(e, "hipFree");
    (void)hipSetDevice(prev);
  }
  ctx->dev_mem = nullptr;
  delete ctx;
  return rc;
}

int dmel_frames(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total, const int64_t* sample_off,
                const int64_t* frame_off, int32_t n_clips, int64_t n_frames_total, const float* carry,
                float* logmel, void* stream) {
  int rc = check_audio(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, logmel, "logmel");
  if (rc != DMEL_OK) return rc;
  if (carry != nullptr && !aligned(carry, 4)) return fail(DMEL_EALIGN, "carry is not 4-byte aligned");
  if (n_frames_total == 0) return DMEL_OK;
  hipError_t e = dmel::launch_frontend(ctx->tabs, audio, n_samples_total, sample_off, frame_off, n_clips,
                                       n_frames_total, carry, logmel, nullptr, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "frontend launch");
}

int dmel_levels(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total, const int64_t* sample_off,
                const int64_t* frame_off, int32_t n_clips, int64_t n_frames_total, const float* carry,
                uint8_t* levels, void* stream) {
  int rc = check_audio(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, levels, "levels");
  if (rc != DMEL_OK) return rc;
  if (carry != nullptr && !aligned(carry, 4)) return fail(DMEL_EALIGN, "carry is not 4-byte aligned");
  if (n_frames_total == 0) return DMEL_OK;
  hipError_t e = dmel::launch_frontend(ctx->tabs, audio, n_samples_total, sample_off, frame_off, n_clips,
                                       n_frames_total, carry, nullptr, levels, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "frontend launch");
}

int dmel_rms_gram(const uint16_t* table, int32_t n_bins, int32_t n_levels, int32_t d_model, double* gram,
                  void* stream) {
  int rc = check_layout(n_bins, n_levels);
  if (rc != DMEL_OK) return rc;
  rc = check_table(table, d_model);
  if (rc != DMEL_OK) return rc;
  if (gram == nullptr) return fail(DMEL_EINVAL, "gram is NULL");
  if (!aligned(gram, 16)) return fail(DMEL_EALIGN, "gram is not 16-byte aligned");
  hipError_t e = dmel::launch_gram(table, n_bins, n_levels, d_model, gram, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "gram launch");
}

int dmel_rms_scale(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels, const double* gram,
                   int32_t d_model, float eps, float* scale, void* stream) {
  if (n_tokens < 0) return fail(DMEL_EINVAL, "n_tokens is negative");
  int rc = check_layout(n_bins, n_levels);
  if (rc != DMEL_OK) return rc;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(DMEL_EINVAL, "eps must be finite and >= 0");
  if (d_model <= 0) return fail(DMEL_ESHAPE, "d_model must be positive");
  if (n_tokens == 0) return DMEL_OK;
  if (levels == nullptr || gram == nullptr || scale == nullptr) return fail(DMEL_EINVAL, "NULL pointer argument");
  if (released_layout(n_bins, n_levels) && !aligned(levels, 16))
    return fail(DMEL_EALIGN, "levels is not 16-byte aligned");
  if (!aligned(gram, 16)) return fail(DMEL_EALIGN, "gram is not 16-byte aligned");
  if (!aligned(scale, 4)) return fail(DMEL_EALIGN, "scale is not 4-byte aligned");
  hipError_t e = dmel::launch_rms_scale(levels, n_tokens, n_bins, n_levels, gram, d_model, eps, scale, nullptr,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "rms_scale launch");
}

int dmel_embed(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels, const uint16_t* table,
               int32_t d_model, const float* rms_weight, const float* rms_scale, void* out, int32_t out_dtype,
               int64_t out_row_stride, const int64_t* out_rows, void* stream) {
  if (n_tokens < 0) return fail(DMEL_EINVAL, "n_tokens is negative");
  int rc = check_layout(n_bins, n_levels);
  if (rc != DMEL_OK) return rc;
  rc = check_table(table, d_model);
  if (rc != DMEL_OK) return rc;
  rc = check_out(out, out_dtype, out_row_stride, d_model, out_rows);
  if (rc != DMEL_OK) return rc;
  if (rms_weight != nullptr && rms_scale == nullptr) return fail(DMEL_EINVAL, "rms_weight given without rms_scale");
  if (rms_weight != nullptr && (!aligned(rms_weight, 4) || !aligned(rms_scale, 4)))
    return fail(DMEL_EALIGN, "rms_weight / rms_scale not 4-byte aligned");
  if (n_tokens == 0) return DMEL_OK;
  if (levels == nullptr) return fail(DMEL_EINVAL, "levels is NULL");
  if (released_layout(n_bins, n_levels) && !aligned(levels, 16))
    return fail(DMEL_EALIGN, "levels is not 16-byte aligned");
  hipError_t e = dmel::launch_embed(levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, out,
                                    out_dtype == DMEL_F32, out_row_stride, out_rows, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "embed launch");
}

int dmel_embed_train(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels, const uint16_t* table,
                     int32_t d_model, const float* rms_weight, const float* rms_scale, void* out, int32_t out_dtype,
                     int64_t out_row_stride, const int64_t* out_rows, float* sums, void* stream) {
  if (n_tokens < 0) return fail(DMEL_EINVAL, "n_tokens is negative");
  int rc = check_layout(n_bins, n_levels);
  if (rc != DMEL_OK) return rc;
  rc = check_table(table, d_model);
  if (rc != DMEL_OK) return rc;
  rc = check_out(out, out_dtype, out_row_stride, d_model, out_rows);
  if (rc != DMEL_OK) return rc;
  if (rms_weight != nullptr && rms_scale == nullptr) return fail(DMEL_EINVAL, "rms_weight given without rms_scale");
  if (rms_weight != nullptr && (!aligned(rms_weight, 4) || !aligned(rms_scale, 4)))
    return fail(DMEL_EALIGN, "rms_weight / rms_scale not 4-byte aligned");
  if (n_tokens == 0) return DMEL_OK;
  if (levels == nullptr) return fail(DMEL_EINVAL, "levels is NULL");
  if (sums == nullptr) return fail(DMEL_EINVAL, "sums is NULL");
  if (released_layout(n_bins, n_levels) && !aligned(levels, 16))
    return fail(DMEL_EALIGN, "levels is not 16-byte aligned");
  if (!aligned(sums, 16)) return fail(DMEL_EALIGN, "sums is not 16-byte aligned");
  const size_t T = static_cast<size_t>(n_tokens), D = static_cast<size_t>(d_model);
  const size_t b_sums = T * D * 4;
  // the output's extent: rows up to the largest index a token may use
  const size_t esz = out_dtype == DMEL_F32 ? 4 : 2;
  const size_t b_out = out_rows == nullptr ? ((T - 1) * static_cast<size_t>(out_row_stride) + D) * esz : 0;
  if (overlaps(sums, b_sums, levels, T * n_bins) ||
      overlaps(sums, b_sums, table, static_cast<size_t>(n_bins) * n_levels * D * 2) ||
      (out_rows == nullptr && overlaps(sums, b_sums, out, b_out)) || (out_rows != nullptr && sums == out))
    return fail(DMEL_EINVAL, "sums overlaps another argument");
  hipError_t e = dmel::launch_embed(levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, out,
                                    out_dtype == DMEL_F32, out_row_stride, out_rows, static_cast<hipStream_t>(stream),
                                    sums);
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "embed launch");
}

size_t dmel_forward_workspace_bytes(int64_t n_frames_total) {
  if (n_frames_total < 0) return 0;
  const size_t n = static_cast<size_t>(n_frames_total);
  return round_up(n * dmel::kMels, 256) + round_up(n * sizeof(float), 256) +
         round_up(dmel::rms_partials_bytes(n_frames_total), 256);
}

}  // extern "C"

namespace {

// Validation shared by dmel_forward and dmel_forward_noalloc (everything but
// the intermediates' memory).
int check_forward(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total, const int64_t* sample_off,
                  const int64_t* frame_off, int32_t n_clips, int64_t n_frames_total, const float* carry,
                  const uint16_t* table, int32_t d_model, const float* rms_weight, const double* gram, float eps,
                  void* out, int32_t out_dtype, int64_t out_row_stride, const int64_t* out_rows) {
  int rc = check_audio(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, out, "out");
  if (rc != DMEL_OK) return rc;
  if (carry != nullptr && !aligned(carry, 4)) return fail(DMEL_EALIGN, "carry is not 4-byte aligned");
  rc = check_layout(ctx->cfg.n_mel_bins, ctx->cfg.mel_vocab_size);
  if (rc != DMEL_OK) return rc;
  rc = check_table(table, d_model);
  if (rc != DMEL_OK) return rc;
  rc = check_out(out, out_dtype, out_row_stride, d_model, out_rows);
  if (rc != DMEL_OK) return rc;
  if (rms_weight != nullptr) {
    if (gram == nullptr) return fail(DMEL_EINVAL, "rms_weight given without gram");
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(DMEL_EINVAL, "eps must be finite and >= 0");
    if (!aligned(rms_weight, 4)) return fail(DMEL_EALIGN, "rms_weight is not 4-byte aligned");
    if (!aligned(gram, 16)) return fail(DMEL_EALIGN, "gram is not 16-byte aligned");
  }
  return DMEL_OK;
}

// The forward's launches: levels -> (scales) -> tokens, with the
// intermediates at `levels` / `scale` / `partials` (partials may be NULL).
int forward_launch(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total, const int64_t* sample_off,
                   const int64_t* frame_off, int32_t n_clips, int64_t n_frames_total, const float* carry,
                   const uint16_t* table, int32_t d_model, const float* rms_weight, const double* gram, float eps,
                   void* out, int32_t out_dtype, int64_t out_row_stride, const int64_t* out_rows, uint8_t* levels,
                   float* scale, void* partials, hipStream_t s) {
  const int32_t n_bins = ctx->cfg.n_mel_bins, n_levels = ctx->cfg.mel_vocab_size;
  hipError_t e = dmel::launch_frontend(ctx->tabs, audio, n_samples_total, sample_off, frame_off, n_clips,
                                       n_frames_total, carry, nullptr, levels, s);
  if (e != hipSuccess) return hip_fail(e, "frontend launch");
  if (rms_weight != nullptr) {
    e = dmel::launch_rms_scale(levels, n_frames_total, n_bins, n_levels, gram, d_model, eps, scale, partials, s);
    if (e != hipSuccess) return hip_fail(e, "rms_scale launch");
  }
  e = dmel::launch_embed(levels, n_frames_total, n_bins, n_levels, table, d_model, rms_weight,
                         rms_weight ? scale : nullptr, out, out_dtype == DMEL_F32, out_row_stride, out_rows, s);
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "embed launch");
}

}  // namespace

extern "C" {

int dmel_forward(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total, const int64_t* sample_off,
                 const int64_t* frame_off, int32_t n_clips, int64_t n_frames_total, const float* carry,
                 const uint16_t* table, int32_t d_model, const float* rms_weight, const double* gram, float eps,
                 void* out, int32_t out_dtype, int64_t out_row_stride, const int64_t* out_rows, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int rc = check_forward(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, table,
                         d_model, rms_weight, gram, eps, out, out_dtype, out_row_stride, out_rows);
  if (rc != DMEL_OK) return rc;
  const size_t need = dmel_forward_workspace_bytes(n_frames_total);
  if (workspace_bytes < need)
    return fail(DMEL_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (n_frames_total == 0) return DMEL_OK;
  if (workspace == nullptr) return fail(DMEL_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(DMEL_EALIGN, "workspace is not 256-byte aligned");
  // levels [n, n_bins] (n_bins <= 80), then the scales, then the partials
  auto* base = static_cast<char*>(workspace);
  const size_t off_scale = round_up(static_cast<size_t>(n_frames_total) * dmel::kMels, 256);
  const size_t off_part = off_scale + round_up(static_cast<size_t>(n_frames_total) * sizeof(float), 256);
  void* partials = dmel::rms_partials_bytes(n_frames_total) > 0 ? base + off_part : nullptr;
  return forward_launch(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, table,
                        d_model, rms_weight, gram, eps, out, out_dtype, out_row_stride, out_rows,
                        reinterpret_cast<uint8_t*>(base), reinterpret_cast<float*>(base + off_scale), partials,
                        static_cast<hipStream_t>(stream));
}

int dmel_forward_noalloc(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                         const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                         int64_t n_frames_total, const float* carry, const uint16_t* table, int32_t d_model,
                         const float* rms_weight, const double* gram, float eps, void* out, int32_t out_dtype,
                         int64_t out_row_stride, const int64_t* out_rows, void* stream) {
  int rc = check_forward(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, table,
                         d_model, rms_weight, gram, eps, out, out_dtype, out_row_stride, out_rows);
  if (rc != DMEL_OK) return rc;
  if (n_frames_total > dmel::kNoAllocMaxFrames)
    return fail(DMEL_ENOMEM, "%lld frames exceed the %lld frames the fixed scratch holds (call dmel_forward with a "
                "workspace, or split the batch)", (long long)n_frames_total, (long long)dmel::kNoAllocMaxFrames);
  if (n_frames_total == 0) return DMEL_OK;
  auto* base = static_cast<char*>(dmel::noalloc_scratch(ctx->device));
  if (base == nullptr) return fail(DMEL_ESTATE, "no scratch address for device %d", ctx->device);
  // the scratch address belongs to ctx's device: the work must run there
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev != ctx->device) return fail(DMEL_ESTATE, "ctx belongs to device %d, the work would run on device %d", ctx->device, dev);
  void* partials = n_frames_total <= dmel::kNoAllocPartialFrames ? base + dmel::kNoAllocPartOff : nullptr;
  return forward_launch(ctx, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames_total, carry, table,
                        d_model, rms_weight, gram, eps, out, out_dtype, out_row_stride, out_rows,
                        reinterpret_cast<uint8_t*>(base), reinterpret_cast<float*>(base + dmel::kNoAllocScaleOff),
                        partials, static_cast<hipStream_t>(stream));
}

int dmel_gather_rows(const uint16_t* table, int64_t n_table_rows, int32_t d_model, const int32_t* ids, int64_t n,
                     uint16_t* out, int64_t out_row_stride, const int64_t* out_rows, void* stream) {
  if (n < 0 || n_table_rows < 0) return fail(DMEL_EINVAL, "negative count");
  if (d_model <= 0 || d_model % 8 != 0) return fail(DMEL_ESHAPE, "d_model must be a positive multiple of 8");
  int rc = check_out(out, DMEL_BF16, out_row_stride, d_model, out_rows);
  if (rc != DMEL_OK) return rc;
  if (n == 0) return DMEL_OK;
  if (table == nullptr || ids == nullptr) return fail(DMEL_EINVAL, "table / ids is NULL");
  if (!aligned(table, 16)) return fail(DMEL_EALIGN, "table is not 16-byte aligned");
  if (!aligned(ids, 4)) return fail(DMEL_EALIGN, "ids is not 4-byte aligned");
  hipError_t e = dmel::launch_gather_rows(table, n_table_rows, d_model, ids, n, out, out_row_stride, out_rows,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "gather_rows launch");
}

int dmel_shortconv(const uint16_t* x, int64_t n_tokens, int32_t channels, const int64_t* seq_off, int32_t n_seqs,
                   const float* weight, const uint16_t* state_in, uint16_t* state_out, void* y, int32_t y_dtype,
                   void* stream) {
  if (n_tokens < 0 || n_seqs < 0) return fail(DMEL_EINVAL, "negative count");
  if (channels < 8 || channels > (1 << 20) || channels % 8 != 0)
    return fail(DMEL_ESHAPE, "channels must be a multiple of 8 in [8, 1048576] (got %d)", channels);
  if (n_tokens > 0 && n_seqs == 0) return fail(DMEL_ESHAPE, "tokens given but n_seqs is 0");
  if (y_dtype != DMEL_BF16 && y_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported y_dtype %d", y_dtype);
  if (n_tokens == 0 && (state_out == nullptr || n_seqs == 0)) return DMEL_OK;
  if (seq_off == nullptr) return fail(DMEL_EINVAL, "seq_off is NULL");
  if (n_tokens > 0 && (x == nullptr || y == nullptr || weight == nullptr))
    return fail(DMEL_EINVAL, "x / y / weight is NULL");
  if (!aligned(seq_off, 8)) return fail(DMEL_EALIGN, "seq_off is not 8-byte aligned");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(weight, 16) || !aligned(state_in, 16) ||
      !aligned(state_out, 16))
    return fail(DMEL_EALIGN, "x, y, weight and the state arrays must be 16-byte aligned");
  const size_t C = static_cast<size_t>(channels), T = static_cast<size_t>(n_tokens), S = static_cast<size_t>(n_seqs);
  const size_t bx = T * C * 2, by = T * C * (y_dtype == DMEL_F32 ? 4 : 2), bs = S * 3 * C * 2, bw = C * 16,
               bo = (S + 1) * 8;
  // written buffers must not share memory with anything the kernel reads or writes
  if (overlaps(y, by, x, bx) || overlaps(y, by, state_in, bs) || overlaps(y, by, state_out, bs) ||
      overlaps(y, by, weight, bw) || overlaps(y, by, seq_off, bo))
    return fail(DMEL_EINVAL, "y overlaps another argument");
  if (overlaps(state_out, bs, x, bx) || overlaps(state_out, bs, state_in, bs) || overlaps(state_out, bs, weight, bw) ||
      overlaps(state_out, bs, seq_off, bo))
    return fail(DMEL_EINVAL, "state_out overlaps another argument (use two state buffers in turn)");
  hipError_t e = dmel::launch_shortconv(x, n_tokens, channels, seq_off, n_seqs, weight, state_in, state_out, y,
                                        y_dtype == DMEL_F32, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "shortconv launch");
}

size_t dmel_embed_backward_workspace_bytes(int64_t n_tokens, int32_t n_bins, int32_t n_levels, int32_t d_model) {
  if (n_tokens < 0 || n_bins < 1 || n_bins > dmel::kEmbMaxBins || n_levels < 1 || n_levels > dmel::kEmbMaxLevels ||
      d_model < 16)
    return 0;
  return dmel::bwd_layout(n_tokens, n_bins, d_model, nullptr);
}

int dmel_embed_backward(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels, const void* dsum,
                        int32_t dsum_dtype, int32_t d_model, float* dtable, int32_t accumulate, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (n_tokens < 0) return fail(DMEL_EINVAL, "n_tokens is negative");
  int rc = check_layout(n_bins, n_levels);
  if (rc != DMEL_OK) return rc;
  if (d_model < 16 || d_model > 65536 || d_model % 16 != 0)
    return fail(DMEL_ESHAPE, "d_model must be a multiple of 16 in [16, 65536] (got %d)", d_model);
  if (dsum_dtype != DMEL_BF16 && dsum_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported dsum_dtype %d", dsum_dtype);
  if (dtable == nullptr) return fail(DMEL_EINVAL, "dtable is NULL");
  if (!aligned(dtable, 16)) return fail(DMEL_EALIGN, "dtable is not 16-byte aligned");
  const size_t need = dmel_embed_backward_workspace_bytes(n_tokens, n_bins, n_levels, d_model);
  if (workspace_bytes < need)
    return fail(DMEL_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (n_tokens > 0) {
    if (levels == nullptr || dsum == nullptr || workspace == nullptr)
      return fail(DMEL_EINVAL, "levels / dsum / workspace is NULL");
    if (!aligned(dsum, 16)) return fail(DMEL_EALIGN, "dsum is not 16-byte aligned");
    if (!aligned(workspace, 256)) return fail(DMEL_EALIGN, "workspace is not 256-byte aligned");
    const size_t T = static_cast<size_t>(n_tokens), D = static_cast<size_t>(d_model);
    const size_t b_tab = static_cast<size_t>(n_bins) * n_levels * D * 4;
    const size_t b_ds = T * D * (dsum_dtype == DMEL_F32 ? 4 : 2);
    if (overlaps(dtable, b_tab, dsum, b_ds) || overlaps(dtable, b_tab, levels, T * n_bins) ||
        overlaps(dtable, b_tab, workspace, need) || overlaps(workspace, need, dsum, b_ds) ||
        overlaps(workspace, need, levels, T * n_bins))
      return fail(DMEL_EINVAL, "dtable / workspace overlap another argument");
  }
  hipError_t e = dmel::launch_embed_backward(levels, n_tokens, n_bins, n_levels, dsum, dsum_dtype == DMEL_BF16, d_model,
                                             dtable, accumulate != 0, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "embed backward launch");
}

size_t dmel_rms_backward_workspace_bytes(int64_t n_tokens, int32_t d_model) {
  if (n_tokens < 0 || d_model < 16 || d_model % 16 != 0) return 0;
  return dmel::rms_bwd_layout(n_tokens, d_model, nullptr);
}

size_t dmel_rms_backward_stored_workspace_bytes(int64_t n_tokens, int32_t d_model) {
  if (n_tokens < 0 || d_model < 16 || d_model % 16 != 0) return 0;
  return dmel::rms_bwd_stored_bytes(n_tokens, d_model);
}

int dmel_rms_backward(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels, const uint16_t* table,
                      int32_t d_model, const float* rms_weight, const float* rms_scale, const void* dy, int32_t dy_dtype,
                      float* dsum, float* dweight, int32_t accumulate_dweight, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (n_tokens < 0) return fail(DMEL_EINVAL, "n_tokens is negative");
  int rc = check_layout(n_bins, n_levels);
  if (rc != DMEL_OK) return rc;
  rc = check_table(table, d_model);
  if (rc != DMEL_OK) return rc;
  if (dy_dtype != DMEL_BF16 && dy_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported dy_dtype %d", dy_dtype);
  if (rms_weight == nullptr) return fail(DMEL_EINVAL, "rms_weight is NULL");
  if (!aligned(rms_weight, 4)) return fail(DMEL_EALIGN, "rms_weight is not 4-byte aligned");
  if (dweight != nullptr && !aligned(dweight, 4)) return fail(DMEL_EALIGN, "dweight is not 4-byte aligned");
  const size_t need_min = dmel_rms_backward_workspace_bytes(n_tokens, d_model);
  if (workspace_bytes < need_min)
    return fail(DMEL_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need_min);
  // a workspace that can hold the sums selects the stored-sum second pass
  const size_t need_stored = dmel_rms_backward_stored_workspace_bytes(n_tokens, d_model);
  const bool stored = n_tokens > 0 && workspace_bytes >= need_stored;
  const size_t need = stored ? need_stored : need_min;
  if (n_tokens > 0) {
    if (levels == nullptr || rms_scale == nullptr || dy == nullptr || dsum == nullptr || workspace == nullptr)
      return fail(DMEL_EINVAL, "levels / rms_scale / dy / dsum / workspace is NULL");
    if (released_layout(n_bins, n_levels) && !aligned(levels, 16))
      return fail(DMEL_EALIGN, "levels is not 16-byte aligned");
    if (!aligned(dy, 16) || !aligned(dsum, 16) || !aligned(rms_scale, 4))
      return fail(DMEL_EALIGN, "dy / dsum must be 16-byte aligned, rms_scale 4-byte aligned");
    if (!aligned(workspace, 256)) return fail(DMEL_EALIGN, "workspace is not 256-byte aligned");
    const size_t T = static_cast<size_t>(n_tokens), D = static_cast<size_t>(d_model);
    const size_t b_ds = T * D * 4, b_dy = T * D * (dy_dtype == DMEL_F32 ? 4 : 2);
    if (overlaps(dsum, b_ds, dy, b_dy) || overlaps(dsum, b_ds, workspace, need) || overlaps(dsum, b_ds, levels, T * n_bins) ||
        overlaps(dsum, b_ds, rms_scale, T * 4) || overlaps(dsum, b_ds, dweight, D * 4) ||
        overlaps(workspace, need, dy, b_dy) || overlaps(dweight, D * 4, workspace, need))
      return fail(DMEL_EINVAL, "dsum / dweight / workspace overlap another argument");
  }
  hipError_t e = dmel::launch_rms_backward(levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, dy,
                                           dy_dtype == DMEL_BF16, dsum, dweight, accumulate_dweight != 0, workspace,
                                           stored, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "rms backward launch");
}

size_t dmel_rms_backward_sums_workspace_bytes(int64_t n_tokens, int32_t d_model) {
  if (n_tokens < 0 || d_model < 16 || d_model % 16 != 0) return 0;
  return dmel::rms_bwd_sums_bytes(n_tokens, d_model);
}

int dmel_rms_backward_sums(const float* sums, int64_t n_tokens, int32_t d_model, const float* rms_weight,
                           const float* rms_scale, const void* dy, int32_t dy_dtype, float* dsum, float* dweight,
                           int32_t accumulate_dweight, void* workspace, size_t workspace_bytes, void* stream) {
  if (n_tokens < 0) return fail(DMEL_EINVAL, "n_tokens is negative");
  if (d_model < 16 || d_model > 65536 || d_model % 16 != 0)
    return fail(DMEL_ESHAPE, "d_model must be a multiple of 16 in [16, 65536] (got %d)", d_model);
  if (dy_dtype != DMEL_BF16 && dy_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported dy_dtype %d", dy_dtype);
  if (rms_weight == nullptr) return fail(DMEL_EINVAL, "rms_weight is NULL");
  if (!aligned(rms_weight, 4)) return fail(DMEL_EALIGN, "rms_weight is not 4-byte aligned");
  if (dweight != nullptr && !aligned(dweight, 4)) return fail(DMEL_EALIGN, "dweight is not 4-byte aligned");
  const size_t need = dmel_rms_backward_sums_workspace_bytes(n_tokens, d_model);
  if (workspace_bytes < need)
    return fail(DMEL_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (n_tokens > 0) {
    if (sums == nullptr || rms_scale == nullptr || dy == nullptr || dsum == nullptr || workspace == nullptr)
      return fail(DMEL_EINVAL, "sums / rms_scale / dy / dsum / workspace is NULL");
    if (!aligned(sums, 16) || !aligned(dy, 16) || !aligned(dsum, 16) || !aligned(rms_scale, 4))
      return fail(DMEL_EALIGN, "sums / dy / dsum must be 16-byte aligned, rms_scale 4-byte aligned");
    if (!aligned(workspace, 256)) return fail(DMEL_EALIGN, "workspace is not 256-byte aligned");
    const size_t T = static_cast<size_t>(n_tokens), D = static_cast<size_t>(d_model);
    const size_t b_ds = T * D * 4, b_dy = T * D * (dy_dtype == DMEL_F32 ? 4 : 2);
    if (overlaps(dsum, b_ds, dy, b_dy) || overlaps(dsum, b_ds, workspace, need) || overlaps(dsum, b_ds, sums, b_ds) ||
        overlaps(dsum, b_ds, rms_scale, T * 4) || overlaps(dsum, b_ds, dweight, D * 4) ||
        overlaps(workspace, need, dy, b_dy) || overlaps(workspace, need, sums, b_ds) ||
        overlaps(dweight, D * 4, workspace, need) || overlaps(dweight, D * 4, sums, b_ds))
      return fail(DMEL_EINVAL, "dsum / dweight / workspace overlap another argument");
  }
  hipError_t e = dmel::launch_rms_backward_sums(sums, n_tokens, d_model, rms_weight, rms_scale, dy,
                                                dy_dtype == DMEL_BF16, dsum, dweight, accumulate_dweight != 0,
                                                workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "rms backward launch");
}

size_t dmel_hmlp_workspace_bytes(int32_t n_images, int32_t height, int32_t width, int32_t hidden) {
  if (n_images < 0 || height < 0 || width < 0 || height % 40 || width % 40 || hidden < 128 || hidden % 128) return 0;
  const int64_t P = static_cast<int64_t>(n_images) * (height / 40) * (width / 40);
  return dmel::hmlp_layout(P, hidden, nullptr);
}

int dmel_hmlp_stage(const uint16_t* x, int64_t n_rows, int32_t k, const uint16_t* weight, const float* bias, int32_t n,
                    int32_t gelu, void* y, int32_t y_dtype, void* stream) {
  if (n_rows < 0) return fail(DMEL_EINVAL, "n_rows is negative");
  if (k < 32 || k % 32 != 0 || k > (1 << 20)) return fail(DMEL_ESHAPE, "k must be a positive multiple of 32 (got %d)", k);
  if (n < 128 || n % 128 != 0 || n > (1 << 20)) return fail(DMEL_ESHAPE, "n must be a positive multiple of 128 (got %d)", n);
  if (y_dtype != DMEL_BF16 && y_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported y_dtype %d", y_dtype);
  if (n_rows == 0) return DMEL_OK;
  if (x == nullptr || weight == nullptr || bias == nullptr || y == nullptr) return fail(DMEL_EINVAL, "NULL argument");
  if (!aligned(x, 16) || !aligned(weight, 16) || !aligned(bias, 4) || !aligned(y, 4))
    return fail(DMEL_EALIGN, "x and weight must be 16-byte aligned, bias and y 4-byte aligned");
  const size_t by = static_cast<size_t>(n_rows) * n * (y_dtype == DMEL_F32 ? 4 : 2);
  if (overlaps(y, by, x, static_cast<size_t>(n_rows) * k * 2) || overlaps(y, by, weight, static_cast<size_t>(n) * k * 2) ||
      overlaps(y, by, bias, static_cast<size_t>(n) * 4))
    return fail(DMEL_EINVAL, "y overlaps another argument");
  hipError_t e = dmel::launch_gemm_bf16(x, weight, bias, y, n_rows, n, k, gelu != 0, y_dtype == DMEL_F32,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "hmlp stage launch");
}

int dmel_hmlp_forward(const uint16_t* images, int32_t n_images, int32_t height, int32_t width, const uint16_t* w1,
                      const float* b1, const uint16_t* w2, const float* b2, const uint16_t* w3, const float* b3,
                      const uint16_t* w4, const float* b4, int32_t hidden, int32_t d_model, void* out, int32_t out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (n_images < 0 || height < 0 || width < 0) return fail(DMEL_EINVAL, "negative size");
  if (height % 40 || width % 40) return fail(DMEL_ESHAPE, "height and width must be multiples of 40 (got %d x %d)", height, width);
  if (hidden < 128 || hidden % 128 || hidden > 16384) return fail(DMEL_ESHAPE, "hidden must be a multiple of 128 in [128, 16384]");
  if (d_model < 128 || d_model % 128 || d_model > 65536) return fail(DMEL_ESHAPE, "d_model must be a multiple of 128 in [128, 65536]");
  if (out_dtype != DMEL_BF16 && out_dtype != DMEL_F32) return fail(DMEL_EDTYPE, "unsupported out_dtype %d", out_dtype);
  const int64_t P = static_cast<int64_t>(n_images) * (height / 40) * (width / 40);
  if (P == 0) return DMEL_OK;
  const uint16_t* w[4] = {w1, w2, w3, w4};
  const float* b[4] = {b1, b2, b3, b4};
  for (int i = 0; i < 4; ++i) {
    if (w[i] == nullptr || b[i] == nullptr) return fail(DMEL_EINVAL, "stage %d weight or bias is NULL", i + 1);
    if (!aligned(w[i], 16) || !aligned(b[i], 4)) return fail(DMEL_EALIGN, "stage %d weight must be 16-byte aligned", i + 1);
  }
  if (images == nullptr || out == nullptr || workspace == nullptr) return fail(DMEL_EINVAL, "images / out / workspace is NULL");
  if (!aligned(images, 2) || !aligned(out, 4) || !aligned(workspace, 256))
    return fail(DMEL_EALIGN, "images 2-byte, out 4-byte, workspace 256-byte aligned");
  const size_t need = dmel::hmlp_layout(P, hidden, nullptr);
  if (workspace_bytes < need)
    return fail(DMEL_ENOMEM, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  const size_t bo = static_cast<size_t>(P) * d_model * (out_dtype == DMEL_F32 ? 4 : 2);
  const size_t bi = static_cast<size_t>(n_images) * height * width * 3 * 2;
  if (overlaps(out, bo, images, bi) || overlaps(out, bo, workspace, need) || overlaps(workspace, need, images, bi))
    return fail(DMEL_EINVAL, "out / workspace overlap another argument");
  hipError_t e = dmel::launch_hmlp(images, n_images, height, width, w, b, hidden, d_model, out, out_dtype == DMEL_F32,
                                   workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DMEL_OK : hip_fail(e, "hmlp launch");
}

}  // extern "C"
