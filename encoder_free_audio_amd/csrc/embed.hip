// Bag-of-bins embedding: token = sum of the 80 table rows 16 * bin + level,
// accumulated in fp32 in bin order 0..79, optional RMSNorm, bf16/fp32 output.
//
// "Inside Inkling: Audio Design", Part 1: the audio "encoder" is one
// nn.Embedding(80 x 16 = 1280 -> 6144); a frame's 80 selected rows are summed
// into one 6144-d vector, with an optional RMSNorm.  "Why this is a reasonable
// bet": each mel bin owns a block of 16 rows (row = 16 * bin + level here).
//
// The sum is defined as s = E[r_0], s = fl32(s + E[r_j]) for j = 1..79.  That
// needs one IEEE fp32 add per (token, column, bin).  Matrix-core accumulation
// and the packed dot instructions do not round every such add to nearest-even
// on gfx950, so the adds run as plain VALU v_add_f32 and the kernel is built
// around feeding them:
//  * a workgroup owns 1024 tokens (one per thread) and a group of column
//    strips 16 columns wide;
//  * for each strip the whole 1280 x 16 slice of the table is converted to
//    fp32 once and staged in LDS with an 80-byte row pitch: the 16 rows of a
//    bin then start in 16 distinct 4-bank groups, so the per-lane gathers
//    (each lane reads the row its own level selects) are free of bank
//    conflicts;
//  * per bin a lane issues four 16-byte LDS reads and 16 adds; accumulators
//    stay in registers; the epilogue applies the RMSNorm scale and weight and
//    rounds to bf16.
#include "internal.h"

namespace dmel {
namespace {

constexpr int kEmbThreads = 1024;   // tokens per workgroup
constexpr int kStrip = 16;          // fp32 columns per strip
constexpr int kPitch = 20;          // floats per LDS row (80 bytes)
constexpr int kStripsPerGroup = 4;  // strips a workgroup walks through

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Clamp each byte of x to at most 15.
__device__ __forceinline__ uint32_t clamp_levels(uint32_t x) {
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;              // nonzero nibble where byte >= 16
  const uint32_t big = ((hi + 0x0F0F0F0Fu) & 0x10101010u);  // bit 4 of each byte >= 16
  const uint32_t mask = (big >> 4) * 0xFFu;                 // 0xFF in those bytes
  return (x & ~mask) | (0x0F0F0F0Fu & mask);
}

// LDS address of the staged row that bin j selects for this lane's token.
__device__ __forceinline__ const float4* row_ptr(const float* tab, const uint32_t (&lv)[20], int j) {
  const uint32_t L = (lv[j >> 2] >> (8 * (j & 3))) & 0xFFu;
  return reinterpret_cast<const float4*>(tab + (kLevels * j + L) * kPitch);
}

__global__ void __launch_bounds__(kEmbThreads)
embed_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, const uint16_t* __restrict__ table,
             int d_model, const float* __restrict__ rms_weight, const float* __restrict__ rms_scale,
             void* __restrict__ out, int out_f32, int64_t out_row_stride,
             const int64_t* __restrict__ out_rows, int n_groups, int n_strips) {
  __shared__ float4 tab4[kRows * kPitch / 4];
  float* tab = reinterpret_cast<float*>(tab4);

  const int tid = threadIdx.x;
  const int grp = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_groups));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(n_groups);
  const int64_t t = tb * kEmbThreads + tid;
  const bool active = t < n_tokens;

  uint32_t lv[20];
  if (active) {
    const uint4* p = reinterpret_cast<const uint4*>(levels + t * kMels);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint4 q = p[i];
      lv[4 * i + 0] = clamp_levels(q.x);
      lv[4 * i + 1] = clamp_levels(q.y);
      lv[4 * i + 2] = clamp_levels(q.z);
      lv[4 * i + 3] = clamp_levels(q.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 20; ++i) lv[i] = 0;
  }
  float scale = 1.0f;
  int64_t orow = t;
  if (active) {
    if (rms_weight != nullptr) scale = rms_scale[t];
    if (out_rows != nullptr) orow = out_rows[t];
  }

  for (int s = 0; s < kStripsPerGroup; ++s) {
    const int strip = grp * kStripsPerGroup + s;
    if (strip >= n_strips) break;
    const int col0 = strip * kStrip;
    // make the levels look modified here so that the 80 row offsets are not
    // hoisted out of the strip loop (keeping them live would spill)
#pragma unroll
    for (int i = 0; i < 20; ++i) asm volatile("" : "+v"(lv[i]));
    __syncthreads();
    // stage the 1280 x 16 slice as fp32, 80-byte rows
    for (int i = tid; i < kRows * 2; i += kEmbThreads) {
      const int row = i >> 1;
      const int h = i & 1;
      const uint4 v = *reinterpret_cast<const uint4*>(table + static_cast<int64_t>(row) * d_model + col0 + 8 * h);
      float4* d = reinterpret_cast<float4*>(tab + row * kPitch + 8 * h);
      d[0] = make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                         bf16_to_f32(v.y >> 16));
      d[1] = make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                         bf16_to_f32(v.w >> 16));
    }
    __syncthreads();

    // Software pipeline over the 80 bins: the four 16-byte reads of bin j + 1
    // are issued, then an empty asm that "modifies" the accumulators and
    // clobbers memory pins them ahead of the adds of bin j, so a wave always
    // has the next bin's reads in flight while it adds the current one.
    float acc[kStrip];
#pragma unroll
    for (int c = 0; c < kStrip; ++c) acc[c] = 0.0f;
    float4 cur[4];
    {
      const float4* r = row_ptr(tab, lv, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) cur[q] = r[q];
    }
#pragma unroll
    for (int j = 0; j < kMels; ++j) {
      float4 nxt[4];
      if (j + 1 < kMels) {
        const float4* r = row_ptr(tab, lv, j + 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) nxt[q] = r[q];
      }
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                   "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]), "+v"(acc[9]), "+v"(acc[10]), "+v"(acc[11]),
                   "+v"(acc[12]), "+v"(acc[13]), "+v"(acc[14]), "+v"(acc[15])::"memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j == 0) {
          // the sum starts from the first row itself (not from +0)
          acc[4 * q + 0] = cur[q].x;
          acc[4 * q + 1] = cur[q].y;
          acc[4 * q + 2] = cur[q].z;
          acc[4 * q + 3] = cur[q].w;
        } else {
          acc[4 * q + 0] += cur[q].x;
          acc[4 * q + 1] += cur[q].y;
          acc[4 * q + 2] += cur[q].z;
          acc[4 * q + 3] += cur[q].w;
        }
      }
      if (j + 1 < kMels) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
      }
    }

    if (active) {
      if (rms_weight != nullptr) {
#pragma unroll
        for (int c = 0; c < kStrip; ++c) acc[c] = (acc[c] * scale) * rms_weight[col0 + c];
      }
      if (out_f32) {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + orow * out_row_stride + col0);
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        o[2] = make_float4(acc[8], acc[9], acc[10], acc[11]);
        o[3] = make_float4(acc[12], acc[13], acc[14], acc[15]);
      } else {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = f32_to_bf16_rne(acc[2 * i]) | (f32_to_bf16_rne(acc[2 * i + 1]) << 16);
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + orow * out_row_stride + col0);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gram matrix G = E E^T (fp64 accumulation of exact bf16 products, stored
// fp32).  One workgroup per 16 x 16 block (bin j rows x bin j' rows), j <= j'.
// ---------------------------------------------------------------------------
constexpr int kGramChunk = 256;

__global__ void __launch_bounds__(256)
gram_kernel(const uint16_t* __restrict__ table, int d_model, float* __restrict__ gram) {
  __shared__ float a_s[16][kGramChunk + 1];
  __shared__ float b_s[16][kGramChunk + 1];
  // blockIdx.x enumerates the upper-triangle pairs (j, j')
  int idx = blockIdx.x;
  int j = 0;
  while (idx >= kMels - j) {
    idx -= kMels - j;
    ++j;
  }
  const int jp = j + idx;
  const int tid = threadIdx.x;
  const int ri = tid >> 4, rj = tid & 15;
  double acc = 0.0;
  for (int c0 = 0; c0 < d_model; c0 += kGramChunk) {
    const int width = min(kGramChunk, d_model - c0);
    __syncthreads();
    for (int i = tid; i < 16 * kGramChunk; i += 256) {
      const int r = i / kGramChunk, c = i - r * kGramChunk;
      float va = 0.0f, vb = 0.0f;
      if (c < width) {
        va = bf16_to_f32(table[static_cast<int64_t>(kLevels * j + r) * d_model + c0 + c]);
        vb = bf16_to_f32(table[static_cast<int64_t>(kLevels * jp + r) * d_model + c0 + c]);
      }
      a_s[r][c] = va;
      b_s[r][c] = vb;
    }
    __syncthreads();
    for (int c = 0; c < width; ++c) acc = fma(static_cast<double>(a_s[ri][c]), static_cast<double>(b_s[rj][c]), acc);
  }
  const int r = kLevels * j + ri, rp = kLevels * jp + rj;
  gram[static_cast<int64_t>(r) * kRows + rp] = static_cast<float>(acc);
  gram[static_cast<int64_t>(rp) * kRows + r] = static_cast<float>(acc);
}

// ---------------------------------------------------------------------------
// RMSNorm scale from the Gram matrix: |s|^2 = sum_j G[r_j][r_j]
// + 2 sum_{j < j'} G[r_j][r_j'].  For each bin j the rows 16j..16j+15 of the
// upper triangle (columns 16j..1279) are staged in LDS; every thread adds the
// terms of its tokens.  Partial sums per bin are fp32, the total fp64.
// ---------------------------------------------------------------------------
constexpr int kScaleThreads = 256;
constexpr int kScaleTokPerThread = 2;
constexpr int kScaleTokens = kScaleThreads * kScaleTokPerThread;
constexpr int kLvPitch = 21;  // dwords per staged level row: an odd pitch spreads lanes over all banks

__global__ void __launch_bounds__(kScaleThreads)
rms_scale_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, const float* __restrict__ gram,
                 int d_model, float eps, float* __restrict__ scale) {
  __shared__ float g_s[16 * kRows];                         // 80 KB
  __shared__ uint32_t lv_s[kScaleTokens * kLvPitch];        // 42 KB, 84-byte rows
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kScaleTokens;
  // stage this block's levels (clamped to 15)
  for (int i = tid; i < kScaleTokens * (kMels / 16); i += kScaleThreads) {
    const int tok = i / (kMels / 16), q = i - tok * (kMels / 16);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t0 + tok < n_tokens) v = reinterpret_cast<const uint4*>(levels + (t0 + tok) * kMels)[q];
    uint32_t* d = lv_s + tok * kLvPitch + 4 * q;
    d[0] = clamp_levels(v.x);
    d[1] = clamp_levels(v.y);
    d[2] = clamp_levels(v.z);
    d[3] = clamp_levels(v.w);
  }
  double total[kScaleTokPerThread];
#pragma unroll
  for (int k = 0; k < kScaleTokPerThread; ++k) total[k] = 0.0;

  for (int j = 0; j < kMels; ++j) {
    const int row_len = kRows - kLevels * j;
    __syncthreads();
    for (int i = tid; i < 16 * row_len; i += kScaleThreads) {
      const int r = i / row_len, c = i - r * row_len;
      g_s[i] = gram[static_cast<int64_t>(kLevels * j + r) * kRows + kLevels * j + c];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScaleTokPerThread; ++k) {
      const uint8_t* L = reinterpret_cast<const uint8_t*>(lv_s + (tid + kScaleThreads * k) * kLvPitch);
      const float* grow = g_s + L[j] * row_len;
      float diag = grow[L[j]];
      float off = 0.0f;
      for (int jp = j + 1; jp < kMels; ++jp) off += grow[kLevels * (jp - j) + L[jp]];
      total[k] += static_cast<double>(diag) + 2.0 * static_cast<double>(off);
    }
  }
#pragma unroll
  for (int k = 0; k < kScaleTokPerThread; ++k) {
    const int64_t t = t0 + tid + kScaleThreads * k;
    if (t < n_tokens) {
      const double ms = total[k] / static_cast<double>(d_model);
      scale[t] = static_cast<float>(1.0 / sqrt(ms + static_cast<double>(eps)));
    }
  }
}

// ---------------------------------------------------------------------------
// Row gather for text positions: out[row(i)] = table[ids[i]] (zeros for an id
// out of range).  One 16-byte chunk per thread per iteration.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
gather_rows_kernel(const uint16_t* __restrict__ table, int64_t n_table_rows, int d_model,
                   const int32_t* __restrict__ ids, int64_t n, uint16_t* __restrict__ out,
                   int64_t out_row_stride, const int64_t* __restrict__ out_rows) {
  const int chunks = d_model / 8;
  const int64_t total = n * chunks;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = i / chunks;
    const int c = static_cast<int>(i - r * chunks);
    const int64_t id = ids[r];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (id >= 0 && id < n_table_rows) v = reinterpret_cast<const uint4*>(table + id * d_model)[c];
    const int64_t orow = out_rows != nullptr ? out_rows[r] : r;
    reinterpret_cast<uint4*>(out + orow * out_row_stride)[c] = v;
  }
}

}  // namespace

hipError_t launch_embed(const uint8_t* levels, int64_t n_tokens, const uint16_t* table, int d_model,
                        const float* rms_weight, const float* rms_scale, void* out, bool out_f32,
                        int64_t out_row_stride, const int64_t* out_rows, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int n_strips = d_model / kStrip;
  const int n_groups = (n_strips + kStripsPerGroup - 1) / kStripsPerGroup;
  const int64_t tblocks = (n_tokens + kEmbThreads - 1) / kEmbThreads;
  const int64_t blocks = tblocks * n_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(embed_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kEmbThreads), 0, stream, levels,
                     n_tokens, table, d_model, rms_weight, rms_scale, out, out_f32 ? 1 : 0, out_row_stride,
                     out_rows, n_groups, n_strips);
  return hipGetLastError();
}

hipError_t launch_gram(const uint16_t* table, int d_model, float* gram, hipStream_t stream) {
  const int pairs = kMels * (kMels + 1) / 2;
  hipLaunchKernelGGL(gram_kernel, dim3(pairs), dim3(256), 0, stream, table, d_model, gram);
  return hipGetLastError();
}

hipError_t launch_rms_scale(const uint8_t* levels, int64_t n_tokens, const float* gram, int d_model,
                            float eps, float* scale, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t blocks = (n_tokens + kScaleTokens - 1) / kScaleTokens;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rms_scale_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kScaleThreads), 0, stream,
                     levels, n_tokens, gram, d_model, eps, scale);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* table, int64_t n_table_rows, int d_model, const int32_t* ids,
                              int64_t n, uint16_t* out, int64_t out_row_stride, const int64_t* out_rows,
                              hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t total = n * (d_model / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, table,
                     n_table_rows, d_model, ids, n, out, out_row_stride, out_rows);
  return hipGetLastError();
}

}  // namespace dmel
