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
//   kind 6  v_lshlrev_b32 by 16 (widens the low bf16 of a word to fp32)
//   kind 7  v_and_b32 with a VGPR mask (widens the high bf16 of a word)
//   kind 8  v_and_b32 with the literal 0xffff0000
//   kind 9  v_cvt_f32_bf16, SDWA form reading the high half
//   kind 10 v_cvt_f32_bf16, VOP1 (the low half)
//   kind 11 v_mov_b32 SDWA, low word to the high word, low word zeroed
//   kind 12 v_perm_b32 (the low 16 bits to the high half)
//   kind 13 v_alignbit_b32 with a zero low source, shift 16
//   kind 14 v_mul_u32_u24 by 65536
//   kind 15 one v_mfma_f32_32x32x16_bf16 per round (a chain on its own
//           accumulators), no adds
//   kind 16 the same MFMA plus the 16 v_add_f32 (VOP2) of kind 0 per round,
//           independent of each other: whether the matrix core and the adds
//           overlap
// The instruction forms are written in inline asm so that the compiler can
// neither merge nor re-encode them (packed fp32 instructions stay disabled).
//
// LDS read rate (lds_rate_kernel): each lane issues four ds_read_b128 per
// round and waits for them; mode 0 reads 1 KB-apart linear pieces (lane l at
// 16 l), mode 1 makes every lane read the same address, modes 2 and 3 read the
// four 16-byte chunks of a 16-float row chosen by a per-lane random level out
// of a 16-row block (row pitch 80 B or 64 B), moving to the next block each
// round - the access pattern of the embedding's gathers.
#include "bench_internal.h"

namespace dmel {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ void __launch_bounds__(256) valu_rate_kernel(float* __restrict__ out, int iters, float s) {
  f32x16_t d = {};
  bf16x8_t fa, fb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fa[i] = static_cast<__bf16>(1e-3f * static_cast<float>(i + threadIdx.x));
    fb[i] = static_cast<__bf16>(2e-3f * static_cast<float>(i));
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = static_cast<float>(threadIdx.x) * 1e-3f + static_cast<float>(i);
  const float v = static_cast<float>(threadIdx.x) * 1e-7f;
  const uint32_t mask = 0xFFFF0000u ^ (threadIdx.x >> 9);  // 0xffff0000 (threadIdx.x < 256)
  const uint32_t zero = threadIdx.x >> 9;                    // 0
  const uint32_t psel = 0x05040C0Cu ^ zero;                  // result bytes: 0, 0, bytes 0 and 1 of src0
  for (int it = 0; it < iters; ++it) {
    if (KIND == 15 || KIND == 16) d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, d, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (KIND == 0 || KIND == 16) asm volatile("v_add_f32_e32 %0, %0, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 1) asm volatile("v_add_f32_e64 %0, %0, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 2) asm volatile("v_add_f32_e32 %0, %1, %0" : "+v"(acc[i]) : "s"(s));
      if (KIND == 3) asm volatile("v_fmac_f32_e32 %0, %1, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 4) asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 5) asm volatile("v_mul_f32_e32 %0, %0, %1" : "+v"(acc[i]) : "v"(v));
      if (KIND == 6) asm volatile("v_lshlrev_b32_e32 %0, 16, %0" : "+v"(acc[i]));
      if (KIND == 7) asm volatile("v_and_b32_e32 %0, %1, %0" : "+v"(acc[i]) : "v"(mask));
      if (KIND == 8) asm volatile("v_and_b32_e32 %0, 0xffff0000, %0" : "+v"(acc[i]));
      if (KIND == 9)
        asm volatile("v_cvt_f32_bf16_sdwa %0, %0 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1" : "+v"(acc[i]));
      if (KIND == 10) asm volatile("v_cvt_f32_bf16_e32 %0, %0" : "+v"(acc[i]));
      if (KIND == 11)
        asm volatile("v_mov_b32_sdwa %0, %0 dst_sel:WORD_1 dst_unused:UNUSED_PAD src0_sel:WORD_0" : "+v"(acc[i]));
      if (KIND == 12) asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(acc[i]) : "v"(zero), "v"(psel));
      if (KIND == 13) asm volatile("v_alignbit_b32 %0, %0, %1, 16" : "+v"(acc[i]) : "v"(zero));
      if (KIND == 14) asm volatile("v_mul_u32_u24_e32 %0, 0x10000, %0" : "+v"(acc[i]));
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) t += acc[i] + d[i];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = t;
}

constexpr int kLdsProbeBytes = 36 * 1024;  // four workgroups per CU

__global__ void __launch_bounds__(256) lds_rate_kernel(float* __restrict__ out, int mode, int iters) {
  __shared__ __attribute__((aligned(16))) float s[kLdsProbeBytes / 4];
  for (int i = threadIdx.x; i < kLdsProbeBytes / 4; i += 256) s[i] = static_cast<float>(i & 1023);
  __syncthreads();
  const int l = threadIdx.x & 63;
  uint32_t h = (threadIdx.x + 977u * blockIdx.x) * 2654435761u;
  h ^= h >> 15;
  const int level = static_cast<int>(h & 15u);
  // byte offsets: linear at most 16 * 63 + 3072 + 16 = 4096; rows at most
  // 32767 + 48 + 16 < 36 KB (blocks of 1280 B wrap inside 32 KB)
  uint32_t base = mode == 0 ? 16u * l : mode == 1 ? 0u : mode == 2 ? 80u * level : 64u * level;
  typedef __attribute__((address_space(3))) float lds_float_t;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_float_t*)s));  // LDS byte offset
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int it = 0; it < iters; ++it) {
    float4 v0, v1, v2, v3;
    const uint32_t a = lds0 + base;
    if (mode == 0) {
      asm volatile(
          "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:1024\n ds_read_b128 %2, %4 offset:2048\n"
          " ds_read_b128 %3, %4 offset:3072\n s_waitcnt lgkmcnt(0)"
          : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3)
          : "v"(a));
    } else {
      asm volatile(
          "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:16\n ds_read_b128 %2, %4 offset:32\n"
          " ds_read_b128 %3, %4 offset:48\n s_waitcnt lgkmcnt(0)"
          : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3)
          : "v"(a));
    }
    acc.x += v0.x + v1.y;
    acc.y += v2.z + v3.w;
    acc.z += v0.w + v1.x;
    acc.w += v2.y + v3.z;
    if (mode >= 2) base = (base + 1280u) & 0x7FFFu;
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

}  // namespace

hipError_t launch_lds_rate(int mode, int blocks, int iters, float* out, hipStream_t stream) {
  if (mode < 0 || mode > 3) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lds_rate_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, out, mode, iters);
  return hipGetLastError();
}

hipError_t launch_valu_rate(int kind, int blocks, int iters, float* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (kind) {
    case 0: hipLaunchKernelGGL(valu_rate_kernel<0>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 1: hipLaunchKernelGGL(valu_rate_kernel<1>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 2: hipLaunchKernelGGL(valu_rate_kernel<2>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 3: hipLaunchKernelGGL(valu_rate_kernel<3>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 4: hipLaunchKernelGGL(valu_rate_kernel<4>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 5: hipLaunchKernelGGL(valu_rate_kernel<5>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 6: hipLaunchKernelGGL(valu_rate_kernel<6>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 7: hipLaunchKernelGGL(valu_rate_kernel<7>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 8: hipLaunchKernelGGL(valu_rate_kernel<8>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 9: hipLaunchKernelGGL(valu_rate_kernel<9>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 10: hipLaunchKernelGGL(valu_rate_kernel<10>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 11: hipLaunchKernelGGL(valu_rate_kernel<11>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 12: hipLaunchKernelGGL(valu_rate_kernel<12>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 13: hipLaunchKernelGGL(valu_rate_kernel<13>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 14: hipLaunchKernelGGL(valu_rate_kernel<14>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 15: hipLaunchKernelGGL(valu_rate_kernel<15>, grid, block, 0, stream, out, iters, 1e-7f); break;
    case 16: hipLaunchKernelGGL(valu_rate_kernel<16>, grid, block, 0, stream, out, iters, 1e-7f); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dmel
