// Vector-ALU issue rates on this GPU: the ceiling the bag-of-bins sum's adds
// are measured against.  Each lane runs 16 independent chains of one
// instruction form for `iters` rounds (registers only, no memory inside the
// loop), so the rate is the instruction's issue rate, not a latency:
//   kind 0  v_add_f32, VOP2 encoding, VGPR operands (the embedding's adds)
//   kind 1  v_add_f32, VOP3 encoding (_e64), VGPR operands
//   kind 2  v_add_f32 with an SGPR operand
//   kind 3  v_fmac_f32 (VOP2 fused multiply-add)
//   kind 4  v_fma_f32 (VOP3 fused multiply-add)
//   kind 5  v_mul_f32 (VOP2)
// The instruction forms are written in inline asm so that the compiler can
// neither merge nor re-encode them (packed fp32 instructions stay disabled).
#include "bench_internal.h"

namespace dmel {
namespace {

template <int KIND>
__global__ void __launch_bounds__(256) valu_rate_kernel(float* __restrict__ out, int iters, float s) {
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = static_cast<float>(threadIdx.x) * 1e-3f + static_cast<float>(i);
  const float v = static_cast<float>(threadIdx.x) * 1e-7f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (KIND == 0) asm volatile("v_add_f32_e32 %0, %0, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 1) asm volatile("v_add_f32_e64 %0, %0, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 2) asm volatile("v_add_f32_e32 %0, %1, %0" : "+v"(acc[i]) : "s"(s));
      if (KIND == 3) asm volatile("v_fmac_f32_e32 %0, %1, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 4) asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 5) asm volatile("v_mul_f32_e32 %0, %0, %1" : "+v"(acc[i]) : "v"(v));
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += acc[i];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = t;
}

}  // namespace

hipError_t launch_valu_rate(int kind, int blocks, int iters, float* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (kind) {
    case 0: hipLaunchKernelGGL(valu_rate_kernel<0>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 1: hipLaunchKernelGGL(valu_rate_kernel<1>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 2: hipLaunchKernelGGL(valu_rate_kernel<2>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 3: hipLaunchKernelGGL(valu_rate_kernel<3>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 4: hipLaunchKernelGGL(valu_rate_kernel<4>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 5: hipLaunchKernelGGL(valu_rate_kernel<5>, grid, block, 0, stream, out, iters, 1e-7f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dmel
