// Rounding probe: one fp32 add c + e (e a bf16 value) done by the vector
// unit, by a matrix-core product with c as its accumulator, by a product
// with a zero accumulator, and by the bf16 dot instruction.  The bag-of-bins
// embedding needs every such add rounded to nearest-even in a fixed order;
// this measures which instructions deliver exactly that.
//
// A wave takes a tile of 1024 cases, (row m, column n) of a 32 x 32 product:
// case base + 32 m + n.  v_mfma_f32_32x32x16_bf16 lane layout (as in the GEMM
// of hmlp.hip): A lane = row (lane & 31), K = 8 (lane >> 5) .. + 7; B lane =
// column (lane & 31), same K; D lane = column (lane & 31), rows
// 8 (r >> 2) + 4 (lane >> 5) + (r & 3), r = 0 .. 15.  Row m's one-hot A row
// selects K = m % 16, and B[k][n] = e of case (16 h + k, n), so two products
// (h = 0, 1) give every case its own e; each keeps the rows of its half.
#include "bench_internal.h"

namespace dmel {
namespace {

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 pbf16x2_t __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(256)
rounding_probe_kernel(const float* __restrict__ c, const uint16_t* __restrict__ e, int64_t n_tiles,
                      float* __restrict__ out, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (tile >= n_tiles) return;  // the whole wave: no barriers here
  const int64_t base = tile * 1024;
  const int col = lane & 31, kh = lane >> 5;
  // case index of D element r of this lane
  auto case_of = [&](int r) { return base + 32 * (8 * (r >> 2) + 4 * kh + (r & 3)) + col; };
  pf32x16_t acc_c, zero;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc_c[r] = c[case_of(r)];
    zero[r] = 0.0f;
  }
  pbf16x8_t a;
  const int row = lane & 31;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int k = 8 * kh + kk;
    a[kk] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(k == (row & 15) ? 0x3F80u : 0u));
  }
  pf32x16_t d_acc[2], d_zero[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pbf16x8_t b;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = 8 * kh + kk;
      b[kk] = __builtin_bit_cast(__bf16, e[base + 32 * (16 * h + k) + col]);
    }
    d_acc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc_c, 0, 0, 0);
    d_zero[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, zero, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * kh + (r & 3);
    const int h = m >> 4;
    const int64_t i = case_of(r);
    const uint16_t eb = e[i];
    const float ef = __uint_as_float(static_cast<uint32_t>(eb) << 16);
    out[i] = acc_c[r] + ef;
    out[n + i] = h == 0 ? d_acc[0][r] : d_acc[1][r];
    out[2 * n + i] = h == 0 ? d_zero[0][r] : d_zero[1][r];
    pbf16x2_t x, y;
    x[0] = __builtin_bit_cast(__bf16, eb);
    x[1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0));
    y[0] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0x3F80u));
    y[1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(0));
    out[3 * n + i] = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc_c[r], false);
  }
}

}  // namespace

hipError_t launch_rounding_probe(const float* c, const uint16_t* e, int64_t n, float* out, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t tiles = n / 1024;
  const int64_t blocks = (tiles + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rounding_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, c, e, tiles,
                     out, n);
  return hipGetLastError();
}

}  // namespace dmel
