// Internal declarations shared by the host API and the HIP kernels of libdmel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "dmel.h"

namespace dmel {

// Front-end constants ("Inside Inkling: Audio Design", Part 1 and "Why this is
// a reasonable bet": 16 kHz, hop 800, window 1600, 80 mel bins, 16 levels).
constexpr int kSampleRate = 16000;
constexpr int kHop = 800;
constexpr int kWindow = 1600;
constexpr int kNfft = 1600;
constexpr int kBins = 801;    // one-sided bins of the 1600-point FFT
constexpr int kHalf = 800;    // the real FFT runs as an 800-point complex FFT
constexpr int kMels = 80;
constexpr int kLevels = 16;
constexpr int kRows = kMels * kLevels;  // 1280
constexpr float kClampMin = -7.0f;
constexpr float kClampMax = 2.0f;
constexpr float kLogFloor = 1e-10f;

// Configurable front end (the config keys n_mel_bins, mel_vocab_size,
// dmel_min_value, dmel_max_value): limits of what the kernels support.
constexpr int kMaxMels = 128;        // filters of the front end
constexpr int kMaxLevels = 256;      // quantizer levels (levels are bytes)
constexpr int kEmbMaxBins = kMels;   // the embedding's LDS slice holds 80 bins
constexpr int kEmbMaxLevels = kLevels;  // ... of up to 16 rows each

// Device-resident constant tables of a context.
struct FrontTables {
  const float* window;   // [1600] periodic Hann
  const float2* tw800;   // [800] exp(-2 pi i m / 800)
  const float2* tw1600;  // [401] exp(-2 pi i k / 1600)
  const float2* twa;     // [24][32]: exp(-2 pi i n1 k2 / 800) at [k2 - 1][n1]
  // Mel filterbank by segment: bins [seg_start[s], seg_start[s+1]) lie
  // between triangle edges s and s+1 (lo = seg_lo[s], hi = seg_hi[s]); such a
  // bin at frequency f feeds filter s (its rising side) with weight
  // (f - lo) / (hi - lo) and filter s-1 (its falling side) with (hi - f) / (hi - lo).
  const int* seg_start;   // [n_mels + 2] (82 for the released 80 filters)
  const float* seg_lo;    // [n_mels + 1] lower edge (Hz)
  const float* seg_hi;    // [n_mels + 1] upper edge (Hz)
  const float* seg_inv;   // [n_mels + 1] 1 / (hi - lo)
  // Quantizer: level = number of edges k = 1 .. n_levels - 1 that the clamped
  // value c reaches.  q_edge[k] is the smallest fp32 value >= the fp64 edge
  // lo + ((hi - lo) * k) / n_levels, so the fp32 test c >= q_edge[k] is the
  // exact comparison with the fp64 edge.
  const float* q_edge;    // [n_levels + 1]
  // The tables the front end reads per lane, packed as the kernel stages them
  // in LDS (kImg* float offsets): window, twa, tw1600, q_edge and, when the
  // filter schedule has at most kMelLdsChunks chunks (mel_in_lds), its
  // weights, first bins and filters.
  const float* lds_image;  // [kImgFull]
  int mel_in_lds;
  // Filter step as a fixed schedule (tables.cpp).  Filter j is one weighted
  // sum over its contiguous bins [seg_start[j], seg_start[j + 2]), taken in
  // chunks of 8 bins.  Four wavefronts of a workgroup run one round each for
  // 8 of its frames (lane = 8 * slot + frame).  Round r is the
  // chunk list [base, base + chunks) with base, chunks, sides = mel_round[8r],
  // [8r + 1], [8r + 2]; side h < sides is the chunk range [start_h,
  // start_{h+1}) of the round (start_h = mel_round[8r + 3 + h], relative to
  // base).  With i = 8 (kMelMaxSides r + h) + slot, side h gives the slot the
  // filter mel_filt[i] (-1: none) and its first chunk starts at bin
  // mel_first[i] (>= -8, = slot mod 8, so that the 8 slots' reads fall in
  // distinct LDS banks; the bins before the filter's range have weight 0).
  // Chunk c, slot s: weights mel_w[16c + s] (bins 0..3 of the chunk) and
  // mel_w[16c + 8 + s] (bins 4..7), 0 outside the filter's range.  Weights are
  // the triangle values times 1/4: the kernel's power spectrum is 4 |X|^2.
  const float4* mel_w;
  const int* mel_first;
  const int* mel_filt;
  const int* mel_round;
  int n_mels;             // filters, 1 .. 128
  int n_levels;           // 1 .. 256
  float q_lo, q_hi;       // clamp range
  float q_scale;          // n_levels / (hi - lo), for the first estimate
};

// Limits of the filter schedule: kMelMaxSides sides per round, kMelChunks
// chunks in all (every filter count 1 .. 128 needs at most 101), and the
// powers read, which lie in bins [-8, kMelReadEnd) (below 808 for every filter
// count); the kernel keeps the powers outside [0, 801) there at zero.
constexpr int kMelMaxSides = (kMaxMels + 31) / 32;
constexpr int kMelChunks = 128;
constexpr int kMelReadEnd = 808;

// Float offsets of the front end's LDS table image (16-byte aligned parts).
// The window is stored as w[0..800]: the periodic Hann window is symmetric,
// w[n] = w[1600 - n].
constexpr int kImgWindow = 0;                                // [801]
constexpr int kImgTwa = 804;                                 // [24 * 32 * 2]
constexpr int kImgTw1600 = kImgTwa + 2 * 24 * 32;            // [401 * 2]
constexpr int kImgEdge = kImgTw1600 + 2 * (kHalf / 2 + 1) + 2;  // [kMaxLevels + 1]
constexpr int kImgFloats = (kImgEdge + kMaxLevels + 1 + 3) / 4 * 4;  // without the schedule
constexpr int kMelLdsChunks = 40;
constexpr int kImgMelW = kImgFloats;                          // [kMelLdsChunks][16] float4
constexpr int kImgMelFirst = kImgMelW + kMelLdsChunks * 64;    // [4 * kMelMaxSides * 8] int
constexpr int kImgMelFilt = kImgMelFirst + 4 * kMelMaxSides * 8;  // [4 * kMelMaxSides * 8] int
constexpr int kImgFull = kImgMelFilt + 4 * kMelMaxSides * 8;

// Host-built tables, in the layout FrontTables points to (see tables.cpp).
struct HostTables {
  float window[kWindow];
  float tw800[2 * kHalf];
  float tw1600[2 * (kHalf / 2 + 1)];
  float twa[2 * 24 * 32];
  int seg_start[kMaxMels + 2];
  float seg_lo[kMaxMels + 1];
  float seg_hi[kMaxMels + 1];
  float seg_inv[kMaxMels + 1];
  float q_edge[kMaxLevels + 1];
  alignas(16) float lds_image[kImgFull];
  int mel_in_lds;
  alignas(16) float mel_w[kMelChunks * 16 * 4];
  int mel_first[4 * kMelMaxSides * 8];
  int mel_filt[4 * kMelMaxSides * 8];
  int mel_round[4 * 8];
};
// n_mels in [1, 128], n_levels in [1, 256], lo < hi (validated by the caller).
// Returns false only if the filter schedule exceeds kMelChunks or kMelReadEnd
// (no filter count in range does).
bool build_host_tables(HostTables* t, int n_mels, int n_levels, float lo, float hi);

// Kernel launchers (all enqueue on `stream` and return the launch status).
hipError_t launch_frontend(const FrontTables& tabs, const float* audio, int64_t n_samples_total,
                           const int64_t* sample_off, const int64_t* frame_off, int n_clips,
                           int64_t n_frames, const float* carry, float* logmel, uint8_t* levels,
                           hipStream_t stream);

// Embedding-side layout: levels [n, n_bins] (1 <= n_bins <= 80), table rows
// n_levels * bin + level (1 <= n_levels <= 16).  Internally every kernel works
// in the released 80 x 16 row space (row 16 * bin + level): missing bins read
// a row of -0.0 (an exact no-op in the fp32 sum, and 0 in the Gram matrix).
// sums_out (may be NULL): each token's fp32 sum before the RMSNorm, [n, d].
hipError_t launch_embed(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                        const uint16_t* table, int d_model, const float* rms_weight, const float* rms_scale,
                        void* out, bool out_f32, int64_t out_row_stride, const int64_t* out_rows,
                        hipStream_t stream, float* sums_out = nullptr);

hipError_t launch_gram(const uint16_t* table, int n_bins, int n_levels, int d_model, double* gram,
                       hipStream_t stream);

// Batches up to this many tokens take a small-batch RMSNorm-scale path: with
// a partials buffer (rms_partials_bytes), a bin-parallel kernel that stages G
// in LDS plus an in-order total; without one, a kernel that reads the Gram
// matrix directly.  Larger batches stage G in LDS per token block.  All three
// give bit-identical scales.
constexpr int64_t kRmsDirectMax = 131072;

size_t rms_partials_bytes(int64_t n_tokens);  // 0 above kRmsDirectMax
hipError_t launch_rms_scale(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                            const double* gram, int d_model, float eps, float* scale, void* partials,
                            hipStream_t stream);

// Short convolution (width 4, residual) over ragged requests with per-request
// state; channels % 8 == 0.
hipError_t launch_shortconv(const uint16_t* x, int64_t n_tokens, int channels, const int64_t* seq_off, int n_seqs,
                            const float* weight, const uint16_t* state_in, uint16_t* state_out, void* y,
                            bool y_f32, hipStream_t stream);

// Backward of the embedding (table gradient: every row sums its tokens'
// gradients in token order from +0, exactly) and of its RMSNorm.
size_t bwd_layout(int64_t n_tokens, int n_bins, int d_model, size_t* offs);
hipError_t launch_embed_backward(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels, const void* dsum,
                                 bool dsum_bf16, int d_model, float* dtable, bool accumulate, void* workspace,
                                 hipStream_t stream);
size_t rms_bwd_layout(int64_t n_tokens, int d_model, size_t* off_dw);
size_t rms_bwd_stored_bytes(int64_t n_tokens, int d_model);
// stored: the workspace holds rms_bwd_stored_bytes (the first pass keeps the
// sums, the second streams them) instead of recomputing the sums twice.
hipError_t launch_rms_backward(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                               const uint16_t* table, int d_model, const float* rms_weight, const float* rms_scale,
                               const void* dy, bool dy_bf16, float* ds, float* dweight, bool accumulate_dweight,
                               void* workspace, bool stored, hipStream_t stream);
// The same from sums the forward kept (launch_embed's sums_out): both passes
// stream them, with the first pass's arithmetic and order unchanged, so the
// results equal launch_rms_backward's bit for bit.  Workspace:
// rms_bwd_sums_bytes.
size_t rms_bwd_sums_bytes(int64_t n_tokens, int d_model);
hipError_t launch_rms_backward_sums(const float* sums, int64_t n_tokens, int d_model, const float* rms_weight,
                                    const float* rms_scale, const void* dy, bool dy_bf16, float* ds, float* dweight,
                                    bool accumulate_dweight, void* workspace, hipStream_t stream);

// hMLP image front end (four stages over 40 x 40 patches) and its stage GEMM.
size_t hmlp_layout(int64_t n_patches, int hidden, size_t* off);
hipError_t launch_hmlp(const uint16_t* images, int n_images, int height, int width, const uint16_t* const w[4],
                       const float* const b[4], int hidden, int d_model, void* out, bool out_f32, void* workspace,
                       hipStream_t stream);
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, const float* bias, void* C, int64_t M, int N, int K,
                            bool gelu, bool out_f32, hipStream_t stream);

// Scratch of the allocation-free forward (noalloc.hip): a static device array
// of kNoAllocScratchBytes per GPU holding, for at most kNoAllocMaxFrames
// frames, the levels [n, 80] at 0, the RMSNorm scales [n] at kNoAllocScaleOff
// and, for at most kNoAllocPartialFrames frames, the RMSNorm partial sums at
// kNoAllocPartOff.  noalloc_init looks its address up on `device` (which must
// be current); noalloc_scratch returns it (nullptr before noalloc_init).
constexpr int64_t kNoAllocMaxFrames = 262144;
constexpr int64_t kNoAllocPartialFrames = 4096;
constexpr size_t kNoAllocScaleOff = static_cast<size_t>(kNoAllocMaxFrames) * kMels;
constexpr size_t kNoAllocPartOff = kNoAllocScaleOff + static_cast<size_t>(kNoAllocMaxFrames) * 4;
constexpr size_t kNoAllocScratchBytes = kNoAllocPartOff + static_cast<size_t>(kNoAllocPartialFrames) * kMels * 16;
hipError_t noalloc_init(int device);
void* noalloc_scratch(int device);

hipError_t launch_gather_rows(const uint16_t* table, int64_t n_table_rows, int d_model,
                              const int32_t* ids, int64_t n, uint16_t* out, int64_t out_row_stride,
                              const int64_t* out_rows, hipStream_t stream);

}  // namespace dmel

// A context (include/dmel.h): its device and the constant tables of its
// front-end configuration in one device allocation.
struct dmel_ctx {
  int device = -1;
  void* dev_mem = nullptr;  // one allocation holding every constant table
  dmel_config cfg{};
  dmel::FrontTables tabs{};
};
