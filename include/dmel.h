/*
 * dmel.h - C ABI of libdmel, the gfx950 (MI355X) implementation of the dMel
 * audio front end: 16 kHz mono audio -> 80-bin log-mel -> 16 levels per bin ->
 * one d_model-wide token per frame (the sum of 80 rows of a 1280-row table).
 *
 * The method is described in "Inside Inkling: Audio Design", Part 1 -
 * Modeling (pipeline, nn.Embedding(80 x 16 = 1280 -> 6144), optional RMSNorm)
 * and its subsection "Why this is a reasonable bet" (hop 800, window 1600,
 * 20 frames per second, n_mel_bins 80, mel_vocab_size 16, clamp [-7, 2], each
 * bin owning a block of 16 rows).  Steps the page leaves open are fixed as:
 * periodic Hann window, 1600-point FFT (801 bins), power spectrum, 80 HTK
 * triangles over 0..8000 Hz (unit peak, edges equally spaced in mel),
 * ln(max(M, 1e-10)), level = min(15, floor((clamp(x, -7, 2) + 7) * 16 / 9))
 * evaluated exactly, causal framing (frame t of a clip covers samples
 * [800 t - 800, 800 t + 800), with the clip's 800-sample carry or zeros before
 * sample 0, so a clip of N samples gives floor(N / 800) frames), table row
 * 16 * bin + level, sum in fp32 in bin order 0..79, and
 * RMSNorm y = s * w / sqrt(mean(s^2) + eps).
 *
 * Conventions shared by every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller, unless a
 *    comment says otherwise.  The library allocates nothing after
 *    dmel_create and never synchronises inside a call: every compute call
 *    validates its arguments on the host, enqueues work on `stream`
 *    (a hipStream_t; NULL = the legacy default stream) and returns.
 *  - Argument validation is host code that runs before any HIP call.  On an
 *    error the call returns a negative dmel_status, enqueues nothing, and
 *    dmel_last_error() describes the failure (thread-local).  A failed launch
 *    returns DMEL_EHIP with the HIP error string.
 *  - Ragged clips: clip c is audio[sample_off[c] .. sample_off[c+1]) and its
 *    frames are token rows frame_off[c] .. frame_off[c+1), where
 *    frame_off[0] = 0 and frame_off[c+1] - frame_off[c] =
 *    (sample_off[c+1] - sample_off[c]) / 800.  Both arrays are device int64
 *    [n_clips + 1] and must be non-decreasing.  Offsets that break these rules
 *    never cause an out-of-bounds access: a frame that does not lie inside
 *    [0, n_samples_total) has every sample bounds-checked, and samples outside
 *    the audio read as zeros (a clip reaching past either end gives the
 *    log-mel of its zero-extended copy).
 *  - bf16 values travel as their uint16 bit patterns.  bf16 outputs are
 *    rounded to nearest-even.
 */
#ifndef DMEL_H
#define DMEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dmel_status {
  DMEL_OK = 0,
  DMEL_EINVAL = -1,  /* null pointer, negative count, bad enum value */
  DMEL_ESHAPE = -2,  /* inconsistent sizes (d_model, strides, frame counts) */
  DMEL_EDTYPE = -3,  /* unsupported output dtype */
  DMEL_EALIGN = -4,  /* pointer or stride not aligned as required */
  DMEL_EHIP = -5,    /* a HIP runtime call or kernel launch failed */
  DMEL_ENOMEM = -6,  /* device allocation failed (dmel_create only) or workspace too small */
  DMEL_ESTATE = -7   /* context not usable (wrong device, destroyed) */
} dmel_status;

typedef enum dmel_dtype { DMEL_BF16 = 0, DMEL_F32 = 1 } dmel_dtype;

/* Fixed constants of the front end (read-only). */
typedef struct dmel_params {
  int32_t sample_rate;  /* 16000 */
  int32_t hop;          /* 800 */
  int32_t window;       /* 1600 */
  int32_t n_fft;        /* 1600 */
  int32_t n_bins;       /* 801 */
  int32_t n_mels;       /* 80 */
  int32_t n_levels;     /* 16 */
  int32_t n_rows;       /* 1280 = n_mels * n_levels */
  float clamp_min;      /* -7.0 */
  float clamp_max;      /* 2.0 */
  float log_floor;      /* 1e-10 */
  float f_min_hz;       /* 0 */
  float f_max_hz;       /* 8000 */
} dmel_params;

/* Front-end configuration, the released config's keys ("Why this is a
 * reasonable bet": n_mel_bins 80, mel_vocab_size 16, dmel_min_value -7.0,
 * dmel_max_value 2.0; the Coda "What I don't know yet" gives -1.5 as the
 * serving code's default minimum).  The quantizer is the same uniform floor
 * for every configuration: with c = clamp(x, min_value, max_value) and V =
 * mel_vocab_size, level = number of edges e_k = min + ((max - min) * k) / V
 * (k = 1 .. V-1, evaluated in fp64) with c >= e_k, i.e.
 * min(V - 1, floor((c - min) * V / (max - min))) decided exactly.  The
 * filterbank has n_mel_bins HTK triangles over 0..8000 Hz (n_mel_bins + 2
 * edges equally spaced in mel). */
typedef struct dmel_config {
  int32_t n_mel_bins;      /* filters, 1..128 (the embedding accepts up to 80) */
  int32_t mel_vocab_size;  /* levels per bin, 1..256 (the embedding accepts up to 16) */
  float min_value;         /* clamp range: finite, min_value < max_value, */
  float max_value;         /* 1e-6 <= max_value - min_value <= 1e30 */
} dmel_config;

/* Opaque per-device context: holds the window, FFT twiddles, the sparse
 * mel filterbank and the quantizer edges of its configuration, uploaded once
 * to the device it was created on. */
typedef struct dmel_ctx dmel_ctx;

/* Fills *out with the constants above.  DMEL_EINVAL if out is NULL. */
int dmel_get_params(dmel_params* out);

/* Frames produced by a clip of n_samples samples: floor(n_samples / 800)
 * (the "audio_tokens" count a server reports for that clip; "Inside Inkling:
 * Audio Design", Part 3, "Where audio touches the serving path").
 * Returns -1 for a negative count. */
int64_t dmel_num_frames(int64_t n_samples);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* dmel_last_error(void);

/* Fills *out with the released configuration (80, 16, -7.0, 2.0).
 * DMEL_EINVAL if out is NULL. */
int dmel_default_config(dmel_config* out);

/* Creates a context on HIP device `device`: allocates and uploads the constant
 * tables (about 30 KB), synchronously.  The only call that allocates device
 * memory.  The caller's current device is left unchanged.
 * Errors: DMEL_EINVAL (out NULL, bad device), DMEL_ENOMEM, DMEL_EHIP. */
int dmel_create(dmel_ctx** out, int device);

/* As dmel_create, with the front end configured by *config (NULL: the
 * released configuration).  Errors: as dmel_create, and DMEL_EINVAL for a
 * configuration outside the ranges of dmel_config. */
int dmel_create_config(dmel_ctx** out, int device, const dmel_config* config);

/* The configuration a context was created with.  DMEL_EINVAL on NULL. */
int dmel_get_config(const dmel_ctx* ctx, dmel_config* out);

/* Frees a context (NULL is a no-op).  Work already enqueued with it must have
 * completed. */
int dmel_destroy(dmel_ctx* ctx);

/* Log-mel of every frame ("an 80-channel log-mel spectrogram", Part 1).
 *  audio      fp32 [n_samples_total], 4-byte aligned
 *  carry      fp32 [n_clips, 800] or NULL: the samples that precede each clip
 *             (the previous hop of a stream); NULL means zeros
 *  logmel     fp32 [n_frames_total, n_mel_bins] out, row-major (n_mel_bins of
 *             the context's configuration: 80 by default)
 * Frames are independent; the result depends only on each frame's 1600
 * samples.  Arithmetic is fp32.
 * Errors: DMEL_EINVAL, DMEL_ESHAPE (n_frames_total > n_samples_total / 800),
 * DMEL_EALIGN, DMEL_EHIP. */
int dmel_frames(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                int64_t n_frames_total, const float* carry, float* logmel, void* stream);

/* Levels of every frame ("each of the 80 mel energies in a frame is quantized
 * to one of 16 levels", Part 1; clamp range [-7, 2], "Why this is a reasonable
 * bet"; the quantizer of the context's configuration, see dmel_config).  Same
 * audio arguments as dmel_frames.
 *  levels     uint8 [n_frames_total, n_mel_bins] out, values 0..mel_vocab_size-1.
 * The level is decided exactly from the fp32 log-mel value that dmel_frames
 * returns for the same input. */
int dmel_levels(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                int64_t n_frames_total, const float* carry, uint8_t* levels, void* stream);

/* Table layout of the embedding calls: n_bins bins (1..80) of n_levels rows
 * each (1..16), table row n_levels * bin + level; the released layout is
 * n_bins = 80, n_levels = 16 (row 16 * bin + level, 1280 rows).  Other values
 * give DMEL_ESHAPE. */

/* Gram matrix of the table, G[r][r'] = sum_c E[r][c] * E[r'][c], accumulated
 * and stored in fp64, for the RMSNorm of dmel_embed / dmel_forward.
 *  table      bf16 [n_bins * n_levels, d_model], 16-byte aligned, row-major
 *  gram       fp64 [1280, 1280] out, 16-byte aligned (both triangles are
 *             written), indexed by 16 * bin + level whatever the layout;
 *             entries of (bin, level) pairs outside the layout are 0
 * Recompute whenever the table's contents change.  d_model % 16 == 0. */
int dmel_rms_gram(const uint16_t* table, int32_t n_bins, int32_t n_levels, int32_t d_model, double* gram,
                  void* stream);

/* Per-token RMSNorm scale r_t = 1 / sqrt(|s_t|^2 / d_model + eps), where
 * |s_t|^2 = sum_{j,j'} G[16 j + L_tj][16 j' + L_tj'] is the squared norm of
 * the exact sum of the token's n_bins rows (the "optional RMSNorm" of Part 1),
 * evaluated in fp64 in a fixed order (every batch size gives a token the same
 * bits).  It differs from the norm of the fp32-rounded sum by the rounding of
 * that sum (about 1e-7 relative for tables whose selected rows do not cancel
 * almost completely) plus about 1e-16 times the sum of the absolute Gram terms
 * over |s|^2.
 *  levels     uint8 [n_tokens, n_bins] (16-byte aligned for the released
 *             layout); values >= n_levels read as n_levels - 1
 *  gram       fp64 [1280, 1280] from dmel_rms_gram with the same layout
 *  scale      fp32 [n_tokens] out
 * Errors: DMEL_EINVAL (eps < 0 or not finite), DMEL_EALIGN, DMEL_ESHAPE. */
int dmel_rms_scale(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels,
                   const double* gram, int32_t d_model, float eps, float* scale, void* stream);

/* Bag-of-bins embedding ("A frame's 80 rows are summed into one 6144-dimensional
 * vector, with an optional RMSNorm", Part 1; "each mel bin owns its own block of
 * 16 rows", "Why this is a reasonable bet").
 *  levels     uint8 [n_tokens, n_bins] (16-byte aligned for the released
 *             layout); values >= n_levels read as n_levels - 1, so no table
 *             read is out of bounds
 *  table      bf16 [n_bins * n_levels, d_model], 16-byte aligned; row
 *             n_levels * bin + level (16 * bin + level when released)
 *  d_model    multiple of 16, 16 <= d_model <= 65536
 *  rms_weight fp32 [d_model] or NULL (NULL: no RMSNorm)
 *  rms_scale  fp32 [n_tokens] from dmel_rms_scale; required iff rms_weight
 *  out        out_dtype (DMEL_BF16 / DMEL_F32) rows of d_model values; token i
 *             goes to row out_rows ? out_rows[i] : i, i.e. at
 *             out + row * out_row_stride elements; 16-byte aligned, and
 *             out_row_stride * element size must be a multiple of 16 bytes
 *  out_rows   int64 [n_tokens] or NULL; rows must be distinct and in range
 * Token value: s = E[r_0], then s = fl32(s + E[r_j]) for j = 1..n_bins-1,
 * exactly (bit-identical to that sequential fp32 sum); with RMSNorm,
 * y = s * r * w in fp32. */
int dmel_embed(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels,
               const uint16_t* table, int32_t d_model, const float* rms_weight, const float* rms_scale,
               void* out, int32_t out_dtype, int64_t out_row_stride, const int64_t* out_rows,
               void* stream);

/* dmel_embed for training: the same output, and each token's fp32 sum s
 * (before the RMSNorm) kept for the backward (the sums the derivative of the
 * RMSNorm needs, see dmel_rms_backward_sums; training the front end is the
 * Coda's experimental case, "Inside Inkling: Audio Design").
 *  sums       fp32 [n_tokens, d_model] out, 16-byte aligned, token i at row i
 *             (not out_rows[i]); bit-identical to dmel_embed's fp32 output
 *             without RMSNorm; must not overlap out, levels or table
 * Other arguments and errors as dmel_embed. */
int dmel_embed_train(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels,
                     const uint16_t* table, int32_t d_model, const float* rms_weight, const float* rms_scale,
                     void* out, int32_t out_dtype, int64_t out_row_stride, const int64_t* out_rows,
                     float* sums, void* stream);

/* Bytes of device workspace dmel_forward needs for n_frames_total frames
 * (levels plus per-token scales, and for batches of at most 131,072 frames
 * 1280 bytes per frame of RMSNorm partial sums; each part 256-byte aligned).
 * 0 for a negative count. */
size_t dmel_forward_workspace_bytes(int64_t n_frames_total);

/* End to end: audio -> levels -> tokens, i.e. dmel_levels, then (when
 * rms_weight is non-NULL) dmel_rms_scale with `gram`, then dmel_embed, on one
 * stream, with the table layout of the context's configuration (n_bins =
 * n_mel_bins, n_levels = mel_vocab_size; DMEL_ESHAPE when that is not an
 * embedding layout).  Audio arguments as dmel_frames, table/output arguments
 * as dmel_embed.  `workspace` is device memory of at least
 * dmel_forward_workspace_bytes(n_frames_total) bytes, 256-byte aligned; it
 * holds intermediates only and may be reused once the call's work is done.
 * gram is required iff rms_weight is non-NULL. */
int dmel_forward(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                 const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                 int64_t n_frames_total, const float* carry, const uint16_t* table,
                 int32_t d_model, const float* rms_weight, const double* gram, float eps,
                 void* out, int32_t out_dtype, int64_t out_row_stride, const int64_t* out_rows,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Largest batch dmel_forward_noalloc accepts, in frames (about 3.6 hours of
 * audio). */
#define DMEL_NOALLOC_MAX_FRAMES 262144

/* dmel_forward without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The intermediates (levels, RMSNorm scales, and for
 * batches of at most 4096 frames the RMSNorm partial sums) live in a fixed
 * array of the library, 26 MiB on each GPU, whose address dmel_create looks
 * up on its device.  Arguments and results as dmel_forward, minus the
 * workspace; the same kernels run, so the results are the same bits.
 * Allocates nothing.  At most DMEL_NOALLOC_MAX_FRAMES frames per call
 * (DMEL_ENOMEM beyond).  Every call on a GPU shares that GPU's array and
 * leaves its last contents there: calls that overlap on one GPU (other
 * streams, other threads) race, so the caller serialises them.  ctx must
 * belong to the device the work runs on (the stream's device, or the current
 * device for the NULL stream): DMEL_ESTATE otherwise. */
int dmel_forward_noalloc(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                         const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                         int64_t n_frames_total, const float* carry, const uint16_t* table, int32_t d_model,
                         const float* rms_weight, const double* gram, float eps, void* out, int32_t out_dtype,
                         int64_t out_row_stride, const int64_t* out_rows, void* stream);

/* Row copy for the text positions of an interleaved sequence (one audio item
 * expands into its frame positions among text tokens; "Inside Inkling: Audio
 * Design", Part 3, "Where audio touches the serving path").
 *  table      bf16 [n_table_rows, d_model], 16-byte aligned
 *  ids        int32 [n]; an id outside [0, n_table_rows) writes a zero row
 *  out        bf16; row i goes to out + (out_rows ? out_rows[i] : i) * out_row_stride,
 *             16-byte aligned rows as in dmel_embed
 * d_model % 8 == 0. */
int dmel_gather_rows(const uint16_t* table, int64_t n_table_rows, int32_t d_model,
                     const int32_t* ids, int64_t n, uint16_t* out, int64_t out_row_stride,
                     const int64_t* out_rows, void* stream);

/* Short convolution of the decoder over a batch of requests ("Inside Inkling:
 * Audio Design", Part 3 - Inference, "Short convolutions": per-channel causal
 * convolution of width 4 with a residual,
 *     y[t][c] = x[t][c] + sum_{d=0}^{3} w[c][d] * x[t-d][c];
 * "Where audio touches the serving path": each request keeps a small
 * convolution state).
 *  x          bf16 [n_tokens, channels]; request s is rows
 *             seq_off[s] .. seq_off[s+1] (seq_off: int64 [n_seqs + 1],
 *             seq_off[0] = 0, non-decreasing, seq_off[n_seqs] = n_tokens;
 *             requests may be empty)
 *  weight     fp32 [channels, 4]: weight[c][d] multiplies x[t-d][c]
 *  state_in   bf16 [n_seqs, 3, channels] or NULL (zeros): the three inputs
 *             before each request's first token, oldest first
 *  state_out  bf16 [n_seqs, 3, channels] or NULL: receives the last three
 *             inputs of [state_in, request tokens] (an empty request keeps
 *             its state); must not overlap any other argument - callers that
 *             carry the state alternate two buffers
 *  y          y_dtype (DMEL_BF16 / DMEL_F32) [n_tokens, channels]; must not
 *             overlap any other argument
 * channels % 8 == 0; x, y, weight and the states 16-byte aligned.
 * Arithmetic is fp32: a = w0 x[t]; a = fma(w1, x[t-1], a); a = fma(w2,
 * x[t-2], a); a = fma(w3, x[t-3], a); y = x[t] + a, rounded to nearest-even
 * for bf16 output.  Offsets that break the rules above give unspecified
 * values but no out-of-bounds access.
 * Errors: DMEL_EINVAL (NULL where data is needed, overlapping buffers),
 * DMEL_ESHAPE, DMEL_EDTYPE, DMEL_EALIGN, DMEL_EHIP. */
int dmel_shortconv(const uint16_t* x, int64_t n_tokens, int32_t channels, const int64_t* seq_off,
                   int32_t n_seqs, const float* weight, const uint16_t* state_in, uint16_t* state_out,
                   void* y, int32_t y_dtype, void* stream);

/* Backward of the front end's trainable parts, for training it jointly with
 * the model (the pages give no backward; "Inside Inkling: Audio Design",
 * Coda, says the front ends are frozen in post-training and training them is
 * experimental).  It is the derivative of dmel_embed:
 *   with RMSNorm, y = s * r * w, r = 1 / sqrt(mean(s^2) + eps):
 *     ds = r * (w * dy) - (r^3 / D) * (sum_c w_c dy_c s_c) * s
 *     dw = sum_t dy_t * s_t * r_t
 *   without it, ds = dy;
 *   the table gradient: dtable[row] = sum of ds_t over the (t, bin) whose
 *   selected row is row. */

/* Bytes of workspace dmel_embed_backward needs (0 for invalid sizes). */
size_t dmel_embed_backward_workspace_bytes(int64_t n_tokens, int32_t n_bins, int32_t n_levels, int32_t d_model);

/* Table gradient of the bag-of-bins embedding.
 *  levels     uint8 [n_tokens, n_bins]; values >= n_levels read as n_levels - 1
 *  dsum       dsum_dtype (DMEL_F32, or DMEL_BF16 for an upstream bf16
 *             gradient without RMSNorm) [n_tokens, d_model], 16-byte aligned:
 *             the gradient with respect to each token's fp32 sum
 *  dtable     fp32 [n_bins * n_levels, d_model] out (row n_levels * bin + level),
 *             16-byte aligned; overwritten, or added to when accumulate != 0
 *  workspace  device memory, 256-byte aligned, >= the size above
 * Summation order: the plain definition - each row adds the gradients of the
 * tokens that selected it in increasing token order, one fp32 add per token,
 * starting from +0 (so an unselected row is +0); with accumulate != 0 the row
 * becomes fl32(dtable + that sum).  Results are bit-identical to that
 * sequential definition and repeat bit for bit.  d_model % 16 == 0;
 * n_bins <= 80, n_levels <= 16.  dtable and workspace must not overlap other
 * arguments. */
int dmel_embed_backward(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels,
                        const void* dsum, int32_t dsum_dtype, int32_t d_model, float* dtable,
                        int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace dmel_rms_backward needs (0 for invalid sizes). */
size_t dmel_rms_backward_workspace_bytes(int64_t n_tokens, int32_t d_model);

/* Bytes of workspace with which dmel_rms_backward keeps the fp32 sums between
 * its passes (the above + n_tokens * d_model * 4 + n_tokens * 4, each part
 * 256-byte aligned; 0 for invalid sizes).  With at least this much, the second
 * pass streams the stored sums instead of recomputing them; the results are
 * the same bits either way. */
size_t dmel_rms_backward_stored_workspace_bytes(int64_t n_tokens, int32_t d_model);

/* Backward of the RMSNorm of dmel_embed: the gradient with respect to each
 * token's fp32 sum and to the RMSNorm weight.  The sums are recomputed from
 * the levels and the table exactly as dmel_embed computes them.
 *  levels, table, rms_weight, rms_scale   as given to dmel_embed (rms_scale from
 *             dmel_rms_scale)
 *  dy         dy_dtype [n_tokens, d_model], 16-byte aligned: upstream gradient
 *  dsum       fp32 [n_tokens, d_model] out, 16-byte aligned
 *  dweight    fp32 [d_model] out or NULL; overwritten, or added to when
 *             accumulate_dweight != 0
 *  workspace  device memory, 256-byte aligned, >= dmel_rms_backward_workspace_bytes
 *             (>= dmel_rms_backward_stored_workspace_bytes: the sums are kept,
 *             not recomputed, for the second pass)
 * fp32 arithmetic in a fixed order (results repeat bit for bit). */
int dmel_rms_backward(const uint8_t* levels, int64_t n_tokens, int32_t n_bins, int32_t n_levels,
                      const uint16_t* table, int32_t d_model, const float* rms_weight,
                      const float* rms_scale, const void* dy, int32_t dy_dtype, float* dsum,
                      float* dweight, int32_t accumulate_dweight, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Bytes of workspace dmel_rms_backward_sums needs (dmel_rms_backward_workspace_bytes
 * + n_tokens * 4, 256-byte aligned; 0 for invalid sizes). */
size_t dmel_rms_backward_sums_workspace_bytes(int64_t n_tokens, int32_t d_model);

/* dmel_rms_backward from the sums dmel_embed_train kept, instead of the
 * levels and the table: both passes stream the sums (no recomputation), with
 * the same arithmetic in the same order, so dsum and dweight are the same bits
 * as dmel_rms_backward's.
 *  sums       fp32 [n_tokens, d_model], 16-byte aligned, from dmel_embed_train
 *  rms_weight, rms_scale, dy, dsum, dweight, accumulate_dweight   as
 *             dmel_rms_backward
 *  workspace  device memory, 256-byte aligned, >= the size above
 * Errors: DMEL_EINVAL (NULL where data is needed, overlapping buffers),
 * DMEL_ESHAPE (d_model), DMEL_EDTYPE, DMEL_EALIGN, DMEL_ENOMEM (workspace too
 * small), DMEL_EHIP. */
int dmel_rms_backward_sums(const float* sums, int64_t n_tokens, int32_t d_model, const float* rms_weight,
                           const float* rms_scale, const void* dy, int32_t dy_dtype, float* dsum,
                           float* dweight, int32_t accumulate_dweight, void* workspace,
                           size_t workspace_bytes, void* stream);

/* hMLP image front end: one d_model-wide embedding per 40 x 40 pixel patch
 * ("Inside Inkling: Audio Design", Part 1, "Why this is a reasonable bet": a
 * 4-layer hMLP over 40x40 patches; "Why Thinking Machines Built Inkling
 * Without a Vision Encoder": a four-stage hMLP stem per 40 x 40 tile).  The
 * pages give no widths or merge pattern; read as: stage 1 maps each 5 x 5 x 3
 * sub-patch, flattened (row, column, channel), to `hidden` channels; stages
 * 2-4 map the 2 x 2 neighbouring outputs of the previous stage, concatenated
 * in (row, column) order, to hidden, hidden and d_model channels; each stage
 * adds its bias, stages 1-3 apply the exact GELU x * Phi(x), and the hidden
 * activations are rounded to bf16 (nearest even).  Matrix-core bf16 products
 * with fp32 accumulation. */

/* Bytes of workspace dmel_hmlp_forward needs (0 for invalid sizes). */
size_t dmel_hmlp_workspace_bytes(int32_t n_images, int32_t height, int32_t width, int32_t hidden);

/* Patch embeddings of a batch of images.
 *  images   bf16 [n_images, height, width, 3] (height-width-channel), sides
 *           multiples of 40
 *  w1, b1   bf16 [hidden, 75], fp32 [hidden]
 *  w2, b2   bf16 [hidden, 4 * hidden], fp32 [hidden]
 *  w3, b3   bf16 [hidden, 4 * hidden], fp32 [hidden]
 *  w4, b4   bf16 [d_model, 4 * hidden], fp32 [d_model]; weights 16-byte aligned
 *  out      out_dtype [n_images * height/40 * width/40, d_model]: patches
 *           image by image, row-major over the patch grid
 *  workspace  device memory, 256-byte aligned, >= dmel_hmlp_workspace_bytes
 * hidden and d_model are multiples of 128.  Errors: DMEL_EINVAL, DMEL_ESHAPE,
 * DMEL_EDTYPE, DMEL_EALIGN, DMEL_ENOMEM (workspace too small), DMEL_EHIP. */
int dmel_hmlp_forward(const uint16_t* images, int32_t n_images, int32_t height, int32_t width,
                      const uint16_t* w1, const float* b1, const uint16_t* w2, const float* b2,
                      const uint16_t* w3, const float* b3, const uint16_t* w4, const float* b4,
                      int32_t hidden, int32_t d_model, void* out, int32_t out_dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* One hMLP stage on its own: y = x weight^T + bias, then GELU when gelu != 0.
 *  x       bf16 [n_rows, k], 16-byte aligned (k % 32 == 0)
 *  weight  bf16 [n, k], 16-byte aligned (n % 128 == 0); bias fp32 [n]
 *  y       y_dtype [n_rows, n] (bf16 rounded to nearest even, or fp32) */
int dmel_hmlp_stage(const uint16_t* x, int64_t n_rows, int32_t k, const uint16_t* weight,
                    const float* bias, int32_t n, int32_t gelu, void* y, int32_t y_dtype,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DMEL_H */
