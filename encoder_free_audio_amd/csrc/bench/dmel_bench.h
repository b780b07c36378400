/*
 * dmel_bench.h - C ABI of libdmel_bench, the benchmark-only companion of
 * libdmel.  It holds what the product library does not ship: the measured
 * alternative to the front end's FFT (the DFT as a matrix-core product), and
 * an in-bounds probe of how the vector and matrix instructions round one fp32
 * add, the evidence behind the choice of plain adds for the embedding sum.
 * Only the benchmark and its tests load it.  Conventions as include/dmel.h:
 * device pointers owned by the caller, host validation before any HIP call,
 * work enqueued on `stream`, negative dmel_status on error with the message
 * in dmel_bench_last_error().
 */
#ifndef DMEL_BENCH_H
#define DMEL_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "dmel.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Thread-local description of the last failure in this thread ("" if none). */
const char* dmel_bench_last_error(void);

/* The log-mel of dmel_frames ("an 80-channel log-mel spectrogram", "Inside
 * Inkling: Audio Design", Part 1) with the 1600-point DFT of each windowed
 * frame computed as one bf16 matrix-core product instead of the LDS FFT:
 * frame and DFT matrix are split into bf16 high and low parts and
 * X = Fh Dh + Fh Dl + Fl Dh is accumulated in fp32 (K = 4800, 1792 output
 * columns: 801 real, 801 imaginary, zero padding), then power, mel filters
 * and log as in dmel_frames.  About 400 times the FFT's arithmetic. */

/* Bytes of the split DFT matrix buffer (bf16 [1792, 4800] + 1792 fp32 zeros). */
size_t dmel_bench_dft_matrix_bytes(void);

/* Fills `matrix` (device, 256-byte aligned, dmel_bench_dft_matrix_bytes()
 * bytes) with the split DFT matrix.  Errors: DMEL_EINVAL (NULL), DMEL_EALIGN,
 * DMEL_EHIP. */
int dmel_bench_dft_matrix(void* matrix, void* stream);

/* Workspace: 9,600 bytes of split frames and 7,168 bytes of spectrum per
 * frame (0 for a negative count). */
size_t dmel_bench_dft_gemm_workspace_bytes(int64_t n_frames_total);

/* dmel_frames through the matrix product.  Arguments as dmel_frames (ctx from
 * dmel_create), plus the matrix dmel_bench_dft_matrix filled and a workspace
 * of at least dmel_bench_dft_gemm_workspace_bytes(n_frames_total) bytes,
 * 256-byte aligned.  Errors: as dmel_frames, DMEL_ENOMEM (workspace too
 * small). */
int dmel_bench_frames_dft_gemm(const dmel_ctx* ctx, const float* audio, int64_t n_samples_total,
                               const int64_t* sample_off, const int64_t* frame_off, int32_t n_clips,
                               int64_t n_frames_total, const float* carry, const void* matrix, float* logmel,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Rounding probe: for every case i, c[i] (fp32) + e[i] (bf16 bits) computed
 *  out[0 * n + i]  by v_add_f32,
 *  out[1 * n + i]  by v_mfma_f32_32x32x16_bf16 with c as the accumulator and
 *                  a one-hot row selecting e (D = C + A B),
 *  out[2 * n + i]  by the same product with a zero accumulator: the selected
 *                  value alone (e itself when the matrix core passes one
 *                  product through unchanged),
 *  out[3 * n + i]  by v_dot2_f32_bf16 with (e, 0) . (1, 0) + c.
 * Cases come in tiles of 1024 (32 x 32 products); in the one-hot products
 * the other 15 values of e's column are the e of other cases of the tile,
 * multiplied by 0.  n % 1024 == 0; all arrays device, 16-byte aligned; out
 * fp32 [4, n]. */
int dmel_bench_rounding_probe(const float* c, const uint16_t* e, int64_t n, float* out, void* stream);

/* Vector-ALU issue rate: `blocks` workgroups of 256 threads, each lane
 * running 16 independent chains of one instruction form for `iters` rounds
 * (16 * iters instructions per lane): kind 0 v_add_f32 (VOP2, VGPR operands),
 * 1 v_add_f32 (VOP3), 2 v_add_f32 with an SGPR operand, 3 v_fmac_f32 (VOP2),
 * 4 v_fma_f32 (VOP3), 5 v_mul_f32 (VOP2), 6 v_lshlrev_b32 by 16, 7 v_and_b32
 * with a VGPR mask, 8 v_and_b32 with a literal mask, 9 v_cvt_f32_bf16 (SDWA,
 * high half), 10 v_cvt_f32_bf16 (VOP1), 11 v_mov_b32 SDWA (low word to high
 * word), 12 v_perm_b32, 13 v_alignbit_b32 by 16, 14 v_mul_u32_u24 by 65536,
 * 15 one v_mfma_f32_32x32x16_bf16 per round and no adds, 16 that MFMA and
 * the 16 adds of kind 0 per round.  out: fp32 [blocks * 256], one value per
 * lane (keeps the chains live).  The caller times the launch. */
int dmel_bench_valu_rate(int32_t kind, int32_t blocks, int32_t iters, float* out, void* stream);

/* LDS read rate: `blocks` workgroups of 256 threads with 36 KB of LDS each;
 * every lane issues four ds_read_b128 per round (64 B) for `iters` rounds:
 * mode 0 linear pieces, 1 one address for all lanes, 2 and 3 the embedding's
 * gather (the 16-float row a random level selects in a 16-row block, row
 * pitch 80 B or 64 B).  out: fp32 [blocks * 256].  The caller times it. */
int dmel_bench_lds_rate(int32_t mode, int32_t blocks, int32_t iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DMEL_BENCH_H */
