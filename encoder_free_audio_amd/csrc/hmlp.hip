// hMLP image front end: four stages over 40 x 40 pixel patches.
//
// "Inside Inkling: Audio Design", Part 1, "Why this is a reasonable bet":
// vision uses a 4-layer hMLP over 40x40 patches; "Why Thinking Machines Built
// Inkling Without a Vision Encoder": every 40 x 40 tile goes through a
// four-stage hMLP stem.  Readings (the pages give no widths or merge
// pattern): stage 1 maps each 5 x 5 x 3 sub-patch (row, column, channel)
// linearly to w channels, stages 2-4 map the 2 x 2 neighbouring outputs of
// the previous stage, concatenated in (row, column) order, to w, w and d
// channels; every stage adds a bias and stages 1-3 apply the exact GELU;
// hidden activations are bf16.
//
// Every stage is a dense contraction, so it runs on the matrix cores: one
// bf16 GEMM kernel (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with the
// bias and GELU fused into its epilogue.  No data moves between stages: the
// 64 sub-patches of a patch are numbered in Morton (Z) order, so the four
// children of a stage-2 position are four consecutive stage-1 rows, and the
// stage-1 output [P * 64, w] read as [P * 16, 4 w] is already the stage-2
// input (likewise for stages 3 and 4).
#include "internal.h"

namespace dmel {
namespace {

constexpr int kK1 = 75;     // 5 x 5 x 3
constexpr int kK1Pad = 96;  // stage-1 K padded to the GEMM's K step
constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kPitch = 40;  // bf16 per LDS row (80 bytes: 16-byte reads of 16 rows hit distinct bank groups)
constexpr int kGemmThreads = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 hb16x2_t __attribute__((ext_vector_type(2)));
typedef float hf32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t to_bf16(float v) {
  hf32x2_t x;
  x[0] = v;
  x[1] = 0.0f;
  return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, __builtin_convertvector(x, hb16x2_t)) & 0xFFFFu);
}

// Morton index m (0..63) of an 8 x 8 grid -> (y, x): bits y2 x2 y1 x1 y0 x0.
__device__ __forceinline__ void demorton8(int m, int& y, int& x) {
  y = ((m >> 5) & 1) << 2 | ((m >> 3) & 1) << 1 | ((m >> 1) & 1);
  x = ((m >> 4) & 1) << 2 | ((m >> 2) & 1) << 1 | (m & 1);
}

// A1[p * 64 + m][k]: sub-patch m (Morton order) of patch p, k = (dy * 5 + dx) * 3 + c
// for k < 75, zeros up to 96.  One thread per (row, k).
__global__ void __launch_bounds__(256)
im2col_kernel(const uint16_t* __restrict__ img, int n_images, int height, int width, uint16_t* __restrict__ a1,
              int64_t n_rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_rows * kK1Pad) return;
  const int64_t row = i / kK1Pad;
  const int k = static_cast<int>(i - row * kK1Pad);
  uint16_t v = 0;
  if (k < kK1) {
    const int pw = width / 40, ph = height / 40;
    const int64_t p = row >> 6;
    const int m = static_cast<int>(row & 63);
    const int64_t im = p / (static_cast<int64_t>(ph) * pw);
    const int pr = static_cast<int>((p / pw) % ph), pc = static_cast<int>(p % pw);
    int y, x;
    demorton8(m, y, x);
    const int dy = k / 15, dx = (k / 3) % 5, c = k % 3;
    const int64_t py = pr * 40 + y * 5 + dy, px = pc * 40 + x * 5 + dx;
    v = img[((im * height + py) * width + px) * 3 + c];
  }
  a1[i] = v;
}

// W1 [n, 75] -> [n, 96] with zeros.
__global__ void __launch_bounds__(256)
pad_w1_kernel(const uint16_t* __restrict__ w, int n, uint16_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n * kK1Pad) return;
  const int r = i / kK1Pad, k = i - r * kK1Pad;
  out[i] = k < kK1 ? w[r * kK1 + k] : static_cast<uint16_t>(0);
}

// C[M, N] = A[M, K] B[N, K]^T + bias (then GELU), bf16 or fp32 out.
// Workgroup tile 128 x 128, K step 32; four waves as 2 x 2, each 64 x 64 =
// 2 x 2 MFMA tiles of 32 x 32.  Operands are staged in LDS (80-byte rows)
// through registers one K step ahead.  N % 128 == 0, K % 32 == 0; rows past M
// read zeros and are not written.
__global__ void __launch_bounds__(kGemmThreads)
gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, const float* __restrict__ bias,
            void* __restrict__ C, int64_t M, int N, int K, int gelu, int out_f32) {
  __shared__ uint4 As4[kBM * kPitch / 8];
  __shared__ uint4 Bs4[kBN * kPitch / 8];
  const uint16_t* As = reinterpret_cast<const uint16_t*>(As4);
  const uint16_t* Bs = reinterpret_cast<const uint16_t*>(Bs4);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int nbn = N / kBN;
  const int64_t bm = blockIdx.x / nbn;
  const int bn = static_cast<int>(blockIdx.x % nbn);
  const int64_t row0 = bm * kBM;
  const int col0 = bn * kBN;

  uint4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kGemmThreads;
      const int r = c >> 2, kq = c & 3;
      ra[i] = make_uint4(0u, 0u, 0u, 0u);
      if (row0 + r < M) ra[i] = *reinterpret_cast<const uint4*>(A + (row0 + r) * K + k0 + kq * 8);
      rb[i] = *reinterpret_cast<const uint4*>(B + static_cast<int64_t>(col0 + r) * K + k0 + kq * 8);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kGemmThreads;
      const int r = c >> 2, kq = c & 3;
      As4[(r * kPitch + kq * 8) / 8] = ra[i];
      Bs4[(r * kPitch + kq * 8) / 8] = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  gload(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    sstore();
    __syncthreads();
    if (k0 + kBK < K) gload(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t fa[2], fb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra_row = wm * 64 + t * 32 + (lane & 31);
        const int rb_row = wn * 64 + t * 32 + (lane & 31);
        const int kofs = kk * 16 + (lane >> 5) * 8;
        fa[t] = *reinterpret_cast<const bf16x8_t*>(As + ra_row * kPitch + kofs);
        fb[t] = *reinterpret_cast<const bf16x8_t*>(Bs + rb_row * kPitch + kofs);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) of each 32 x 32 tile and rows
  // 8 (i / 4) + 4 (lane / 32) + i % 4
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int col = col0 + wn * 64 + b * 32 + (lane & 31);
    const float bb = bias[col];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t row = row0 + wm * 64 + a * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row >= M) continue;
        float v = acc[a][b][i] + bb;
        if (gelu) v = 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
        if (out_f32) {
          static_cast<float*>(C)[row * N + col] = v;
        } else {
          static_cast<uint16_t*>(C)[row * N + col] = to_bf16(v);
        }
      }
    }
  }
}

hipError_t gemm(const uint16_t* A, const uint16_t* B, const float* bias, void* C, int64_t M, int N, int K, bool gelu,
                bool out_f32, hipStream_t stream) {
  const int64_t blocks = ((M + kBM - 1) / kBM) * (N / kBN);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kGemmThreads), 0, stream, A, B, bias, C, M,
                     N, K, gelu ? 1 : 0, out_f32 ? 1 : 0);
  return hipGetLastError();
}

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t hmlp_layout(int64_t n_patches, int hidden, size_t* off) {
  const size_t P = static_cast<size_t>(n_patches), w = static_cast<size_t>(hidden);
  const size_t b_a1 = up256(P * 64 * kK1Pad * 2), b_h1 = up256(P * 64 * w * 2), b_h2 = up256(P * 16 * w * 2),
               b_h3 = up256(P * 4 * w * 2), b_w1 = up256(w * kK1Pad * 2);
  if (off != nullptr) {
    off[0] = 0;
    off[1] = b_a1;
    off[2] = b_a1 + b_h1;
    off[3] = b_a1 + b_h1 + b_h2;
    off[4] = b_a1 + b_h1 + b_h2 + b_h3;
  }
  return b_a1 + b_h1 + b_h2 + b_h3 + b_w1;
}

hipError_t launch_hmlp(const uint16_t* images, int n_images, int height, int width, const uint16_t* const w[4],
                       const float* const b[4], int hidden, int d_model, void* out, bool out_f32, void* workspace,
                       hipStream_t stream) {
  const int64_t P = static_cast<int64_t>(n_images) * (height / 40) * (width / 40);
  if (P == 0) return hipSuccess;
  size_t off[5];
  hmlp_layout(P, hidden, off);
  char* ws = static_cast<char*>(workspace);
  auto* a1 = reinterpret_cast<uint16_t*>(ws + off[0]);
  auto* h1 = reinterpret_cast<uint16_t*>(ws + off[1]);
  auto* h2 = reinterpret_cast<uint16_t*>(ws + off[2]);
  auto* h3 = reinterpret_cast<uint16_t*>(ws + off[3]);
  auto* w1p = reinterpret_cast<uint16_t*>(ws + off[4]);
  const int64_t rows1 = P * 64;
  const int64_t n_a1 = rows1 * kK1Pad;
  if ((n_a1 + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(im2col_kernel, dim3(static_cast<unsigned>((n_a1 + 255) / 256)), dim3(256), 0, stream, images,
                     n_images, height, width, a1, rows1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pad_w1_kernel, dim3((hidden * kK1Pad + 255) / 256), dim3(256), 0, stream, w[0], hidden, w1p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = gemm(a1, w1p, b[0], h1, rows1, hidden, kK1Pad, true, false, stream)) != hipSuccess) return e;
  if ((e = gemm(h1, w[1], b[1], h2, P * 16, hidden, 4 * hidden, true, false, stream)) != hipSuccess) return e;
  if ((e = gemm(h2, w[2], b[2], h3, P * 4, hidden, 4 * hidden, true, false, stream)) != hipSuccess) return e;
  return gemm(h3, w[3], b[3], out, P, d_model, 4 * hidden, false, out_f32, stream);
}

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, const float* bias, void* C, int64_t M, int N, int K,
                            bool gelu, bool out_f32, hipStream_t stream) {
  return gemm(A, B, bias, C, M, N, K, gelu, out_f32, stream);
}

}  // namespace dmel
