// Host-side checks of libdmel built with AddressSanitizer and
// UndefinedBehaviorSanitizer on its host code: every argument-validation path
// the CPU tests reach, the workspace-size functions and the host tables of
// many front-end configurations.  No call here reaches the GPU (validation
// fails first, or the call is a pure host computation), so the driver runs on
// a machine without one.  Exits 0 and prints "ok" when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "dmel.h"
#include "internal.h"

static int g_failures = 0;

#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
      ++g_failures;                                                         \
    }                                                                       \
  } while (0)

// an aligned address that validation rejects before it is ever dereferenced
static void* const FAKE = reinterpret_cast<void*>(uintptr_t{1} << 20);

int main() {
  dmel_params p;
  EXPECT(dmel_get_params(&p) == DMEL_OK && p.n_rows == 1280 && p.hop == 800);
  EXPECT(dmel_get_params(nullptr) == DMEL_EINVAL);
  EXPECT(dmel_num_frames(-1) == -1 && dmel_num_frames(799) == 0 && dmel_num_frames(16000) == 20);
  dmel_config cfg;
  EXPECT(dmel_default_config(&cfg) == DMEL_OK && cfg.n_mel_bins == 80 && cfg.mel_vocab_size == 16);
  dmel_ctx* ctx = nullptr;
  EXPECT(dmel_create(nullptr, 0) == DMEL_EINVAL);
  dmel_config bad = cfg;
  bad.mel_vocab_size = 0;
  EXPECT(dmel_create_config(&ctx, 0, &bad) == DMEL_EINVAL && std::strlen(dmel_last_error()) > 0);
  bad = cfg;
  bad.min_value = NAN;
  EXPECT(dmel_create_config(&ctx, 0, &bad) == DMEL_EINVAL);
  EXPECT(dmel_destroy(nullptr) == DMEL_OK);

  // audio entry points: counts, shapes, NULLs, alignment, missing context
  const float* a = static_cast<const float*>(FAKE);
  const int64_t* off = static_cast<const int64_t*>(FAKE);
  EXPECT(dmel_frames(nullptr, a, -1, off, off, 1, 0, nullptr, static_cast<float*>(FAKE), nullptr) == DMEL_EINVAL);
  EXPECT(dmel_frames(nullptr, a, 1600, off, off, 1, 3, nullptr, static_cast<float*>(FAKE), nullptr) == DMEL_ESHAPE);
  EXPECT(dmel_frames(nullptr, nullptr, 1600, off, off, 1, 2, nullptr, static_cast<float*>(FAKE), nullptr) ==
         DMEL_EINVAL);
  EXPECT(dmel_frames(nullptr, a + 1, 1600, off, off, 1, 2, nullptr, static_cast<float*>(FAKE), nullptr) ==
         DMEL_EINVAL);  // (the NULL context is reported first)
  EXPECT(dmel_levels(nullptr, a, 1600, off, off, 1, 2, nullptr, static_cast<uint8_t*>(FAKE), nullptr) ==
         DMEL_EINVAL);
  EXPECT(dmel_frames(nullptr, a, 1600, off, off, 0, 2, nullptr, static_cast<float*>(FAKE), nullptr) == DMEL_ESHAPE);

  // embedding, Gram and scale
  const uint8_t* lv = static_cast<const uint8_t*>(FAKE);
  const uint16_t* tb = static_cast<const uint16_t*>(FAKE);
  EXPECT(dmel_embed(lv, 4, 80, 16, tb, 6008, nullptr, nullptr, FAKE, DMEL_BF16, 6144, nullptr, nullptr) ==
         DMEL_ESHAPE);
  EXPECT(dmel_embed(lv, 4, 81, 16, tb, 6144, nullptr, nullptr, FAKE, DMEL_BF16, 6144, nullptr, nullptr) ==
         DMEL_ESHAPE);
  EXPECT(dmel_embed(lv, 4, 80, 16, tb, 6144, nullptr, nullptr, FAKE, 7, 6144, nullptr, nullptr) == DMEL_EDTYPE);
  EXPECT(dmel_embed(lv, -1, 80, 16, tb, 6144, nullptr, nullptr, FAKE, DMEL_BF16, 6144, nullptr, nullptr) ==
         DMEL_EINVAL);
  EXPECT(dmel_embed(lv, 4, 80, 16, tb + 1, 6144, nullptr, nullptr, FAKE, DMEL_BF16, 6144, nullptr, nullptr) ==
         DMEL_EALIGN);
  EXPECT(dmel_rms_gram(nullptr, 80, 16, 6144, static_cast<double*>(FAKE), nullptr) == DMEL_EINVAL);
  EXPECT(dmel_rms_gram(tb, 80, 16, 6144, reinterpret_cast<double*>(static_cast<char*>(FAKE) + 8), nullptr) ==
         DMEL_EALIGN);
  EXPECT(dmel_rms_scale(lv, 5, 80, 16, static_cast<const double*>(FAKE), 6144, -1.0f, static_cast<float*>(FAKE),
                        nullptr) == DMEL_EINVAL);
  EXPECT(dmel_rms_scale(lv, 5, 80, 32, static_cast<const double*>(FAKE), 6144, 1e-6f, static_cast<float*>(FAKE),
                        nullptr) == DMEL_ESHAPE);
  EXPECT(dmel_gather_rows(tb, 10, 12, static_cast<const int32_t*>(FAKE), 5, static_cast<uint16_t*>(FAKE), 16,
                          nullptr, nullptr) == DMEL_ESHAPE);

  // forward entry points without a context
  EXPECT(dmel_forward(nullptr, a, 1600, off, off, 1, 2, nullptr, tb, 6144, nullptr, nullptr, 1e-6f, FAKE, DMEL_BF16,
                      6144, nullptr, FAKE, dmel_forward_workspace_bytes(2), nullptr) == DMEL_EINVAL);
  EXPECT(dmel_forward_noalloc(nullptr, a, 1600, off, off, 1, 2, nullptr, tb, 6144, nullptr, nullptr, 1e-6f, FAKE,
                              DMEL_BF16, 6144, nullptr, nullptr) == DMEL_EINVAL);

  // workspace sizes (pure host arithmetic)
  EXPECT(dmel_forward_workspace_bytes(-1) == 0);
  EXPECT(dmel_forward_workspace_bytes(1536000) >= size_t{1536000} * 84);
  EXPECT(dmel_embed_backward_workspace_bytes(0, 80, 16, 6144) == 0);
  EXPECT(dmel_embed_backward_workspace_bytes(1536000, 80, 16, 6144) >= size_t{1536000} * 80);
  EXPECT(dmel_embed_backward_workspace_bytes(100, 81, 16, 6144) == 0);
  EXPECT(dmel_rms_backward_workspace_bytes(1000, 6144) > 0 && dmel_rms_backward_workspace_bytes(-1, 6144) == 0);
  EXPECT(dmel_rms_backward_stored_workspace_bytes(1000, 6144) >= size_t{1000} * 6144 * 4);
  EXPECT(dmel_hmlp_workspace_bytes(2, 80, 120, 256) > 0 && dmel_hmlp_workspace_bytes(2, 81, 120, 256) == 0);

  // shortconv and backward validation
  EXPECT(dmel_shortconv(tb, 4, 12, off, 1, a, nullptr, nullptr, FAKE, DMEL_BF16, nullptr) == DMEL_ESHAPE);
  EXPECT(dmel_embed_backward(lv, 4, 80, 16, FAKE, 9, 6144, static_cast<float*>(FAKE), 0, FAKE, size_t{1} << 30,
                             nullptr) == DMEL_EDTYPE);
  EXPECT(dmel_rms_backward(lv, 4, 80, 16, tb, 6144, a, a, FAKE, DMEL_BF16, static_cast<float*>(FAKE), nullptr, 0,
                           FAKE, 0, nullptr) == DMEL_ENOMEM);
  float* const fs = static_cast<float*>(FAKE);
  EXPECT(dmel_rms_backward_sums_workspace_bytes(1000, 6144) >= dmel_rms_backward_workspace_bytes(1000, 6144) + 4000);
  EXPECT(dmel_rms_backward_sums_workspace_bytes(-1, 6144) == 0 && dmel_rms_backward_sums_workspace_bytes(9, 100) == 0);
  EXPECT(dmel_rms_backward_sums(fs, 4, 6144, a, a, FAKE, DMEL_BF16, fs, nullptr, 0, FAKE, 0, nullptr) == DMEL_ENOMEM);
  EXPECT(dmel_rms_backward_sums(fs, 4, 6008, a, a, FAKE, DMEL_BF16, fs, nullptr, 0, FAKE, size_t{1} << 30,
                                nullptr) == DMEL_ESHAPE);
  EXPECT(dmel_rms_backward_sums(nullptr, 4, 6144, a, a, FAKE, DMEL_F32, fs + (1 << 20), nullptr, 0, FAKE,
                                size_t{1} << 30, nullptr) == DMEL_EINVAL);
  EXPECT(dmel_embed_train(lv, 4, 80, 16, tb, 6144, nullptr, nullptr, FAKE, DMEL_BF16, 6144, nullptr, nullptr,
                          nullptr) == DMEL_EINVAL);
  EXPECT(dmel_embed_train(lv, 4, 80, 16, tb, 6144, nullptr, nullptr, FAKE, DMEL_BF16, 6144, nullptr, fs + 1,
                          nullptr) == DMEL_EALIGN);

  // host tables of many configurations
  auto* t = new dmel::HostTables;
  const int mels[] = {1, 2, 40, 64, 80, 100, 128};
  const int levels[] = {1, 2, 8, 16, 100, 256};
  const float ranges[][2] = {{-7.0f, 2.0f}, {-1.5f, 2.0f}, {-5.0f, 1.0f}, {0.0f, 1e-6f}, {-1e29f, 1e29f}};
  for (int m : mels) {
    for (int l : levels) {
      for (const auto& r : ranges) {
        dmel::build_host_tables(t, m, l, r[0], r[1]);
        EXPECT(t->seg_start[0] == 0 && t->seg_start[m + 1] <= dmel::kBins);
        for (int s = 0; s < m + 1; ++s) EXPECT(t->seg_start[s] <= t->seg_start[s + 1]);
        for (int k = 1; k < l; ++k) EXPECT(t->q_edge[k] <= t->q_edge[k + 1] || k + 1 >= l);
      }
    }
  }
  delete t;
  if (g_failures == 0) std::printf("ok\n");
  return g_failures == 0 ? 0 : 1;
}
