// Internal declarations of libdmel_bench.
#pragma once

#include "internal.h"

namespace dmel {

// Log-mel through the DFT as a matrix-core product (dft_gemm.hip).
size_t dft_matrix_bytes();
size_t dft_gemm_workspace_bytes(int64_t n_frames);
hipError_t launch_dft_matrix(uint16_t* B, hipStream_t stream);
hipError_t launch_dft_gemm_frames(const FrontTables& tabs, const float* audio, int64_t n_samples_total,
                                  const int64_t* sample_off, const int64_t* frame_off, int n_clips, int64_t n_frames,
                                  const float* carry, const uint16_t* B, float* logmel, void* workspace,
                                  hipStream_t stream);

// Rounding probe (rounding_probe.hip); n % 1024 == 0.
hipError_t launch_rounding_probe(const float* c, const uint16_t* e, int64_t n, float* out, hipStream_t stream);

// Vector-ALU issue-rate calibration (valu_rate.hip): kind 0..16.
hipError_t launch_valu_rate(int kind, int blocks, int iters, float* out, hipStream_t stream);
// LDS ds_read_b128 rate (valu_rate.hip): mode 0..3.
hipError_t launch_lds_rate(int mode, int blocks, int iters, float* out, hipStream_t stream);

}  // namespace dmel
