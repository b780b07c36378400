// Backward of the bag-of-bins embedding and of its RMSNorm.
//
// The pages give no backward ("Inside Inkling: Audio Design", Coda: the
// front ends are frozen in post-training, training them is experimental); it
// is the derivative of the forward in embed.hip:
//   y = s * r * w,  r = 1 / sqrt(mean(s^2) + eps)   (r from dmel_rms_scale)
//   ds = r * (w * dy) - (r^3 / D) * (sum_c w_c dy_c s_c) * s
//   dw = sum_t dy_t * s_t * r_t
//   dE[row] = sum of ds_t over the (t, j) whose selected row r_tj is row.
//
// Table gradient order: the plain definition - every row adds the gradients
// of the tokens that selected it in increasing token order, one fp32 add per
// token, starting from +0; accumulating gives dtable + that sum.  The kernels
// reproduce this order exactly, so results repeat bit for bit and equal the
// sequential definition.
//
// Kernels:
//  * levels_t_kernel - the levels by bin ([bin][token], clamped), so that a
//    chunk's 64 levels of one bin are 64 contiguous bytes.
//  * scatter_kernel (bf16 gradients) / scatter16_kernel (fp32 gradients) - a
//    workgroup owns 8 bins (one wave each) and 256 columns (4 per lane), or
//    16 bins and 128 columns (2 per lane), and walks every 64-token chunk of
//    the batch in order; the chunk's 64 x 256 gradient tile and its levels are copied
//    straight into LDS (double-buffered), and each wave takes the 64 tokens
//    in order: one ds_read_b128 of the token's row (static offset) and four
//    v_add_f32 into the accumulators of the token's level, which the wave
//    selects with the GPR index mode (the level is the same in every lane,
//    and the 16 x 4 accumulators sit in 64 consecutive registers).  Every
//    row's sum is thus one chain in token order across the whole batch.  The
//    workgroups that share a tile (the bin groups of one strip) run on the
//    same XCD and start together, so its L2 serves most of their re-reads.
//  * rms_dot_kernel / rms_ds_kernel - the RMSNorm backward: the forward sum
//    is recomputed exactly as embed_kernel computes it (embed_core.h); the
//    first pass forms sum_c w_c dy_c s_c per token and per-workgroup partial
//    sums of dy * s * r per column, the second pass writes ds.
#include <algorithm>

#include "embed_core.h"

namespace dmel {
namespace {

constexpr int kChunk = 64;                   // tokens per staged tile
constexpr int kBwdCols = 256;                // columns per workgroup (4 per lane)
constexpr int kBwdBins = 8;                  // bins per workgroup (one per wave)
constexpr int kBwdThreads = 64 * kBwdBins;   // 512
constexpr int kRowBytes = kBwdCols * 4;      // one token's 256 fp32 gradients
constexpr int kTileBytes = kChunk * kRowBytes;           // 64 KB
constexpr int kLvBytes = kBwdBins * kChunk;              // the chunk's levels of the 8 bins
static_assert(kChunk / kBwdBins * kBwdBins == kChunk, "tile copy: whole rows per wave");
static_assert(kLvBytes == 32 * 16, "level copy: one 16-byte piece per lane of half a wave");

// ---------------------------------------------------------------------------
// Levels by bin: lvt[j][t] = min(levels[t][j], n_levels - 1) for t < n_tokens
// and 0 up to the end of the last chunk (those tokens add a row of -0.0, see
// tile_dma).  A workgroup transposes 64 tokens through LDS.  Also fills the
// row of -0.0 that stands in for tokens past the batch.
__global__ void __launch_bounds__(256)
levels_t_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels, int64_t t_pad,
                uint8_t* __restrict__ lvt, float* __restrict__ neg_zero) {
  __shared__ uint8_t tile[kChunk * kEmbMaxBins];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kChunk;
  const uint32_t vmax = static_cast<uint32_t>(n_levels - 1);
  for (int i = tid; i < kChunk * n_bins; i += 256) {
    const int64_t t = t0 + i / n_bins;
    uint32_t v = 0;
    if (t < n_tokens) {
      v = levels[t0 * n_bins + i];
      v = v < vmax ? v : vmax;
    }
    tile[i] = static_cast<uint8_t>(v);
  }
  __syncthreads();
  for (int i = tid; i < kChunk * n_bins; i += 256) {
    const int j = i / kChunk, q = i - j * kChunk;
    lvt[static_cast<int64_t>(j) * t_pad + t0 + q] = tile[q * n_bins + j];
  }
  if (blockIdx.x == 0) {
    for (int i = tid; i < kBwdCols; i += 256) neg_zero[i] = -0.0f;
  }
}

// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

// bf16 gradients: read through registers (converted to fp32 on the way), so
// a tile is loaded into registers during the previous chunk and stored at the
// top of its own; rows past the batch hold -0.0.
constexpr int kBf16Items = kChunk * kBwdCols / 8 / kBwdThreads;   // 8 bf16 per item: 4
__device__ __forceinline__ void tile_load_bf16(uint4 (&r)[kBf16Items], const uint16_t* g, int64_t n_tokens,
                                               int d_model, int64_t t0, int c_strip, int tid) {
#pragma unroll
  for (int k = 0; k < kBf16Items; ++k) {
    const int i = tid + k * kBwdThreads;   // row i / 32, 8-column group i % 32
    const int64_t t = t0 + (i >> 5);
    const int c = min(c_strip + 8 * (i & 31), d_model - 8);
    r[k] = t < n_tokens ? *reinterpret_cast<const uint4*>(g + t * d_model + c)
                        : make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u);
  }
}
__device__ __forceinline__ void tile_store_bf16(char* tb, const uint4 (&r)[kBf16Items], int tid) {
#pragma unroll
  for (int k = 0; k < kBf16Items; ++k) {
    const int i = tid + k * kBwdThreads;
    float4* d = reinterpret_cast<float4*>(tb + (i >> 5) * kRowBytes + (i & 31) * 32);
    const uint4 v = r[k];
    d[0] = make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                       bf16_to_f32(v.y >> 16));
    d[1] = make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                       bf16_to_f32(v.w >> 16));
  }
}

// The chunk's levels of the workgroup's 8 bins (64 bytes each, from the
// by-bin copy) into level buffer `lb`: lanes 0..31 of wave 0 copy 16 bytes
// each.  Bins past n_bins read the last bin's levels (unused).
__device__ __forceinline__ void levels_dma(char* lb, const uint8_t* lvt, int64_t t_pad, int bin0, int n_bins,
                                           int64_t t0, int wave, int lane) {
  if (wave == 0 && lane < 32) {
    const int j = min(bin0 + (lane >> 2), n_bins - 1);
    __builtin_amdgcn_global_load_lds(lvt + j * t_pad + t0 + 16 * (lane & 3), (lds_void_t*)lb, 16, 0, 0);
  }
}

__device__ __forceinline__ void add4(float4& a, const float4& v) {
  a.x += v.x;
  a.y += v.y;
  a.z += v.z;
  a.w += v.w;
}

// The 16 level accumulators of a lane's 4 columns, one 16-wide vector per
// column, pinned to v64..v127 so that a wave-uniform level can select the
// accumulator through the GPR index mode.
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// acc[L] += row, with L = the token's level: in the GPR index mode (index L,
// relative source 0 and destination) one v_add_f32 per column adds the row
// into register 64 + L (+ 16, 32, 48 for the other columns).  The mode keeps
// its index in M0, which the asm declares as an output, so the compiler sets
// M0 again wherever it needs it.
#define DMEL_ADD_LEVEL(L, R)                                                                         \
  do {                                                                                               \
    uint32_t m0_out_;                                                                                \
    asm volatile(                                                                                    \
        "s_set_gpr_idx_on %5, gpr_idx(SRC0,DST)\n\t"                                                 \
        "v_add_f32 v64, v64, %6\n\t"                                                                 \
        "v_add_f32 v80, v80, %7\n\t"                                                                 \
        "v_add_f32 v96, v96, %8\n\t"                                                                 \
        "v_add_f32 v112, v112, %9\n\t"                                                               \
        "s_set_gpr_idx_off"                                                                          \
        : "+{v[64:79]}"(ax), "+{v[80:95]}"(ay), "+{v[96:111]}"(az), "+{v[112:127]}"(aw), "={m0}"(m0_out_) \
        : "s"(L), "v"((R).x), "v"((R).y), "v"((R).z), "v"((R).w));                                  \
  } while (0)

// One chunk of the scatter: `cur` holds chunk ch (tile + levels), the copy of
// chunk ch + 1 goes to `nxt`.  The two buffers are distinct LDS arrays so
// that the compiler can see that the reads of one do not wait for the copies
// into the other.
__device__ __forceinline__ void scatter_chunk(char* cur_tile, char* cur_lv, char* nxt_tile, char* nxt_lv,
                                              int64_t ch, const uint16_t* g, int64_t n_tokens, int n_bins,
                                              int d_model, const uint8_t* lvt, int64_t t_pad, int64_t n_chunks,
                                              int c_strip, int bin0, bool bin_ok, int wave, int lane, int tid,
                                              uint4 (&rb)[kBf16Items], f32x16_t& ax, f32x16_t& ay, f32x16_t& az,
                                              f32x16_t& aw) {
  (void)nxt_tile;  // the next tile waits in registers (rb) until its chunk starts
  tile_store_bf16(cur_tile, rb, tid);
  // this wave's copies of chunk ch have landed; after the barrier every
  // wave's have, and every wave is done with chunk ch - 1
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (ch + 1 < n_chunks) {
    tile_load_bf16(rb, g, n_tokens, d_model, (ch + 1) * kChunk, c_strip, tid);
    levels_dma(nxt_lv, lvt, t_pad, bin0, n_bins, (ch + 1) * kChunk, wave, lane);
  }
  if (bin_ok) {
    // the wave's 64 levels (the same in every lane) into scalar registers
    const auto* lw = reinterpret_cast<const uint32_t*>(cur_lv + wave * kChunk);
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) w[q] = __builtin_amdgcn_readfirstlane(lw[q]);
    const float4* row = reinterpret_cast<const float4*>(cur_tile) + lane;   // token t at row[64 t]
    float4 r[kChunk];
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = row[t * (kRowBytes / 16)];
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      if (t + 8 < kChunk) r[t + 8] = row[(t + 8) * (kRowBytes / 16)];
      const uint32_t L = (w[t >> 2] >> (8 * (t & 3))) & 15u;
      DMEL_ADD_LEVEL(L, r[t]);
    }
  }
}

// bf16 gradients.  Workgroup (bin group, strip): 8 bins (one wave each) and 256 columns (4
// per lane), walking every chunk of the batch in order.  Per chunk each wave
// takes the 64 tokens in order: the token's row from the LDS tile (static
// offsets, read 8 tokens ahead) is added into the accumulator of the token's
// level, so every row's gradient is one chain in token order across the
// whole batch.  Writes out = acc (or fl32(out + acc) when accumulating).
// Chunk ch is staged in buffer ch % 2: its copy is issued right after the
// barrier that starts chunk ch - 1 (all waves have then finished chunk ch - 2,
// the buffer's previous contents), so it lands while chunk ch - 1 is added;
// one barrier per chunk.
__global__ void __launch_bounds__(kBwdThreads)
scatter_kernel(const uint16_t* __restrict__ g, int64_t n_tokens, int n_bins, int n_levels, int d_model,
               const uint8_t* __restrict__ lvt, int64_t t_pad, int64_t n_chunks, int n_groups, int n_strips,
               int per_xcd, float* __restrict__ out, int accumulate) {
  __shared__ __attribute__((aligned(1024))) char tile_a[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char tile_b[kTileBytes];
  __shared__ __attribute__((aligned(16))) char lv_a[kLvBytes];
  __shared__ __attribute__((aligned(16))) char lv_b[kLvBytes];
  // blockIdx -> (strip, bin group): workgroup b runs on XCD b % 8; XCD x
  // takes strips x * per_xcd .. x * per_xcd + per_xcd - 1 with all their bin
  // groups, so the bin groups of a strip share its tiles in that XCD's L2
  const int bid = static_cast<int>(blockIdx.x);
  const int local = bid >> 3;
  const int grp = local % n_groups;
  const int strip = (bid & 7) * per_xcd + local / n_groups;
  if (local / n_groups >= per_xcd || strip >= n_strips) return;  // before any barrier: the whole workgroup leaves

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bin0 = grp * kBwdBins;
  const int j = bin0 + wave;
  const bool bin_ok = j < n_bins;
  const int c_strip = strip * kBwdCols;
  const int c0 = c_strip + 4 * lane;

  f32x16_t ax = 0.0f, ay = 0.0f, az = 0.0f, aw = 0.0f;

  uint4 rb[kBf16Items];
  tile_load_bf16(rb, g, n_tokens, d_model, 0, c_strip, tid);
  levels_dma(lv_a, lvt, t_pad, bin0, n_bins, 0, wave, lane);
  for (int64_t ch = 0; ch < n_chunks; ch += 2) {
    scatter_chunk(tile_a, lv_a, tile_b, lv_b, ch, g, n_tokens, n_bins, d_model, lvt, t_pad, n_chunks, c_strip, bin0,
                  bin_ok, wave, lane, tid, rb, ax, ay, az, aw);
    if (ch + 1 < n_chunks) {
      scatter_chunk(tile_b, lv_b, tile_a, lv_a, ch + 1, g, n_tokens, n_bins, d_model, lvt, t_pad, n_chunks, c_strip,
                    bin0, bin_ok, wave, lane, tid, rb, ax, ay, az, aw);
    }
  }

  if (!bin_ok || c0 >= d_model) return;
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    if (l < n_levels) {
      const int64_t rw = static_cast<int64_t>(j) * n_levels + l;
      float4* o = reinterpret_cast<float4*>(out + rw * d_model + c0);
      const float4 a = make_float4(ax[l], ay[l], az[l], aw[l]);
      float4 v = a;
      if (accumulate) {
        v = *o;
        add4(v, a);
      }
      *o = v;
    }
  }
}
#undef DMEL_ADD_LEVEL

// fp32 gradients: 16 bins x 128 columns per workgroup (two columns per lane),
// so that each copied tile serves twice the bins of scatter_kernel while the
// launch still has 240 workgroups (5 bin groups x 48 strips).  The same chunk
// walk, buffers and token order; per token a wave reads 512 bytes of the row
// (ds_read_b64) and adds two columns into the accumulators of the token's
// level (16 levels x 2 columns pinned to v64..v95).
constexpr int kS16Bins = 16;
constexpr int kS16Cols = 128;
constexpr int kS16Threads = 64 * kS16Bins;             // 1024
constexpr int kS16RowBytes = kS16Cols * 4;             // 512
constexpr int kS16TileBytes = kChunk * kS16RowBytes;   // 32 KB
static_assert(kChunk / kS16Bins == 4, "tile copy: four rows per wave, two per load");
static_assert(kS16Bins * kChunk == 64 * 16, "level copy: one 16-byte piece per lane of a wave");
static_assert(kS16Cols <= kBwdCols, "rows past the batch read the row of -0.0");

// Chunk rows into tile buffer `tb`: wave w copies rows 4w .. 4w + 3, two per
// load (lanes 0..31 the first row, 32..63 the second; lane i takes columns
// 4 (i & 31) .. + 3).  Rows past the batch copy the row of -0.0.
__device__ __forceinline__ void tile_dma16(char* tb, const float* g, const float* neg_zero, int64_t n_tokens,
                                           int d_model, int64_t t0, int c_strip, int wave, int lane) {
  const int c = min(c_strip + 4 * (lane & 31), d_model - 4);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r0 = wave * 4 + 2 * i;
    const int64_t t = t0 + r0 + (lane >> 5);
    const float* src = t < n_tokens ? g + t * d_model + c : neg_zero + 4 * (lane & 31);
    __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(tb + r0 * kS16RowBytes), 16, 0, 0);
  }
}

// The chunk's levels of the workgroup's 16 bins: the 64 lanes of wave 0 copy
// 16 bytes each.  Bins past n_bins read the last bin's levels (unused).
__device__ __forceinline__ void levels_dma16(char* lb, const uint8_t* lvt, int64_t t_pad, int bin0, int n_bins,
                                             int64_t t0, int wave, int lane) {
  if (wave == 0) {
    const int j = min(bin0 + (lane >> 2), n_bins - 1);
    __builtin_amdgcn_global_load_lds(lvt + j * t_pad + t0 + 16 * (lane & 3), (lds_void_t*)lb, 16, 0, 0);
  }
}

#define DMEL_ADD_LEVEL2(L, R)                                                                        \
  do {                                                                                               \
    uint32_t m0_out_;                                                                                \
    asm volatile(                                                                                    \
        "s_set_gpr_idx_on %3, gpr_idx(SRC0,DST)\n\t"                                                 \
        "v_add_f32 v64, v64, %4\n\t"                                                                 \
        "v_add_f32 v80, v80, %5\n\t"                                                                 \
        "s_set_gpr_idx_off"                                                                          \
        : "+{v[64:79]}"(ax), "+{v[80:95]}"(ay), "={m0}"(m0_out_)                                       \
        : "s"(L), "v"((R).x), "v"((R).y));                                                           \
  } while (0)

__device__ __forceinline__ void scatter16_chunk(char* cur_tile, char* cur_lv, char* nxt_tile, char* nxt_lv,
                                                int64_t ch, const float* g, int64_t n_tokens, int n_bins,
                                                int d_model, const uint8_t* lvt, int64_t t_pad,
                                                const float* neg_zero, int64_t n_chunks, int c_strip, int bin0,
                                                bool bin_ok, int wave, int lane, f32x16_t& ax, f32x16_t& ay) {
  // this wave's copies of chunk ch have landed; after the barrier every
  // wave's have, and every wave is done with chunk ch - 1
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (ch + 1 < n_chunks) {
    tile_dma16(nxt_tile, g, neg_zero, n_tokens, d_model, (ch + 1) * kChunk, c_strip, wave, lane);
    levels_dma16(nxt_lv, lvt, t_pad, bin0, n_bins, (ch + 1) * kChunk, wave, lane);
  }
  if (bin_ok) {
    const auto* lw = reinterpret_cast<const uint32_t*>(cur_lv + wave * kChunk);
    uint32_t w[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) w[q] = __builtin_amdgcn_readfirstlane(lw[q]);
    const float2* row = reinterpret_cast<const float2*>(cur_tile) + lane;   // token t at row[64 t]
    float2 r[kChunk];
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = row[t * (kS16RowBytes / 8)];
#pragma unroll
    for (int t = 0; t < kChunk; ++t) {
      if (t + 8 < kChunk) r[t + 8] = row[(t + 8) * (kS16RowBytes / 8)];
      const uint32_t L = (w[t >> 2] >> (8 * (t & 3))) & 15u;
      DMEL_ADD_LEVEL2(L, r[t]);
    }
  }
}

__global__ void __launch_bounds__(kS16Threads)
scatter16_kernel(const float* __restrict__ g, int64_t n_tokens, int n_bins, int n_levels, int d_model,
                 const uint8_t* __restrict__ lvt, int64_t t_pad, const float* __restrict__ neg_zero,
                 int64_t n_chunks, int n_groups, int n_strips, int per_xcd, float* __restrict__ out, int accumulate) {
  __shared__ __attribute__((aligned(1024))) char tile_a[kS16TileBytes];
  __shared__ __attribute__((aligned(1024))) char tile_b[kS16TileBytes];
  __shared__ __attribute__((aligned(16))) char lv_a[kS16Bins * kChunk];
  __shared__ __attribute__((aligned(16))) char lv_b[kS16Bins * kChunk];
  // blockIdx -> (strip, bin group) as in scatter_kernel
  const int bid = static_cast<int>(blockIdx.x);
  const int local = bid >> 3;
  const int grp = local % n_groups;
  const int strip = (bid & 7) * per_xcd + local / n_groups;
  if (local / n_groups >= per_xcd || strip >= n_strips) return;  // before any barrier: the whole workgroup leaves

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bin0 = grp * kS16Bins;
  const int j = bin0 + wave;
  const bool bin_ok = j < n_bins;
  const int c_strip = strip * kS16Cols;
  const int c0 = c_strip + 2 * lane;

  f32x16_t ax = 0.0f, ay = 0.0f;
  tile_dma16(tile_a, g, neg_zero, n_tokens, d_model, 0, c_strip, wave, lane);
  levels_dma16(lv_a, lvt, t_pad, bin0, n_bins, 0, wave, lane);
  for (int64_t ch = 0; ch < n_chunks; ch += 2) {
    scatter16_chunk(tile_a, lv_a, tile_b, lv_b, ch, g, n_tokens, n_bins, d_model, lvt, t_pad, neg_zero, n_chunks,
                    c_strip, bin0, bin_ok, wave, lane, ax, ay);
    if (ch + 1 < n_chunks) {
      scatter16_chunk(tile_b, lv_b, tile_a, lv_a, ch + 1, g, n_tokens, n_bins, d_model, lvt, t_pad, neg_zero,
                      n_chunks, c_strip, bin0, bin_ok, wave, lane, ax, ay);
    }
  }

  if (!bin_ok || c0 >= d_model) return;
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    if (l < n_levels) {
      const int64_t rw = static_cast<int64_t>(j) * n_levels + l;
      float2* o = reinterpret_cast<float2*>(out + rw * d_model + c0);
      float2 v = make_float2(ax[l], ay[l]);
      if (accumulate) {
        const float2 p = *o;
        v = make_float2(p.x + v.x, p.y + v.y);
      }
      *o = v;
    }
  }
}
#undef DMEL_ADD_LEVEL2

// Zero fill (kept out of hipMemsetAsync so that a caller may capture the
// calls in a graph).
__global__ void __launch_bounds__(256) zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

hipError_t zero_fill(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm backward.  Workgroups as embed_kernel: 1024 tokens (one per lane)
// and a group of 16-column strips.
// ---------------------------------------------------------------------------
// A strip's 16 upstream gradients of token t, read raw at the start of the
// strip (bf16: two 16-byte pieces, fp32: four) and widened in its epilogue,
// so the read is in flight during the strip's adds.
template <bool kDyBf16>
using DyRaw = uint4[kDyBf16 ? 2 : 4];
template <bool kDyBf16>
__device__ __forceinline__ void load_dy_raw(DyRaw<kDyBf16>& raw, const void* dy, int64_t t, int d_model, int col0,
                                            bool active) {
  constexpr int n = kDyBf16 ? 2 : 4;
  if (!active) {
#pragma unroll
    for (int i = 0; i < n; ++i) raw[i] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const uint4* p = kDyBf16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dy) + t * d_model + col0)
                           : reinterpret_cast<const uint4*>(static_cast<const float*>(dy) + t * d_model + col0);
#pragma unroll
  for (int i = 0; i < n; ++i) raw[i] = p[i];
}
template <bool kDyBf16>
__device__ __forceinline__ void unpack_dy(float (&gr)[kStrip], const DyRaw<kDyBf16>& raw) {
  if (kDyBf16) {
    const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gr[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      gr[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      gr[4 * q] = __uint_as_float(raw[q].x);
      gr[4 * q + 1] = __uint_as_float(raw[q].y);
      gr[4 * q + 2] = __uint_as_float(raw[q].z);
      gr[4 * q + 3] = __uint_as_float(raw[q].w);
    }
  }
}

// Sums each of 16 values over the wavefront's 64 lanes with a transposing
// butterfly: every exchange halves the number of values a lane carries, so 17
// exchanges do the work of 96.  Afterwards lane L holds the total of value
// (L >> 2) & 15 (and so do L ^ 1, L ^ 2, L ^ 3).
__device__ __forceinline__ float wave_sum16(const float (&q)[16], int lane) {
  float a[8], b[4], c[2];
  const bool h5 = (lane & 32) != 0, h4 = (lane & 16) != 0, h3 = (lane & 8) != 0, h2 = (lane & 4) != 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float send = h5 ? q[i] : q[8 + i];
    a[i] = (h5 ? q[8 + i] : q[i]) + __shfl_xor(send, 32, 64);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float send = h4 ? a[i] : a[4 + i];
    b[i] = (h4 ? a[4 + i] : a[i]) + __shfl_xor(send, 16, 64);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = h3 ? b[i] : b[2 + i];
    c[i] = (h3 ? b[2 + i] : b[i]) + __shfl_xor(send, 8, 64);
  }
  float d = (h2 ? c[1] : c[0]) + __shfl_xor(h2 ? c[0] : c[1], 4, 64);
  d += __shfl_xor(d, 2, 64);
  d += __shfl_xor(d, 1, 64);
  return d;
}

// The first pass's work on one strip, given the exact fp32 sums acc of
// columns col0 .. col0 + 15 of this thread's token: the token's dot chain
// (one fma per column, in column order), and the strip's 16 column sums of
// dy * s * r over the workgroup's tokens (a transposing butterfly per
// wavefront, then the 16 wavefronts in order) into dw_part.  Contains a
// barrier; the caller keeps `red` unwritten until the first 16 threads have
// read it (another barrier).
// (dot_strip_q: the dot chain and the wavefront's butterfly, whose result
// lane L holds for column (L >> 2) & 15; red_sum: the sum over the 16
// wavefronts in order.)
template <bool kDyBf16>
__device__ __forceinline__ float dot_strip_q(int col0, const float (&acc)[kStrip], const DyRaw<kDyBf16>& dyr,
                                             const float* __restrict__ rms_weight, float r, float& dot, int tid) {
  float gr[kStrip];
  unpack_dy<kDyBf16>(gr, dyr);
  float q[kStrip];
#pragma unroll
  for (int c = 0; c < kStrip; ++c) {
    dot = fmaf(rms_weight[col0 + c] * gr[c], acc[c], dot);
    q[c] = (gr[c] * acc[c]) * r;
  }
  return wave_sum16(q, tid & 63);
}
__device__ __forceinline__ float red_sum(const float (*red)[kStrip], int c) {
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kEmbThreads / 64; ++w) v += red[w][c];
  return v;
}
template <bool kDyBf16>
__device__ __forceinline__ void dot_strip(int col0, const float (&acc)[kStrip], const DyRaw<kDyBf16>& dyr,
                                          const float* __restrict__ rms_weight, float r, float& dot,
                                          float (*red)[kStrip], int tid, float* __restrict__ dw_part, int64_t tb,
                                          int d_model) {
  const float qs = dot_strip_q<kDyBf16>(col0, acc, dyr, rms_weight, r, dot, tid);
  if ((tid & 3) == 0) red[tid >> 6][(tid >> 2) & 15] = qs;
  __syncthreads();
  if (tid < kStrip) dw_part[tb * d_model + col0 + tid] = red_sum(red, tid);
}

// Pass 1: per token, sum_c w_c dy_c s_c over the workgroup's strips (dot_part
// [n_tokens, n_groups]); per column, sum over the workgroup's tokens of
// dy * s * r (dw_part [token blocks, d_model]); with s_out, the sums s
// themselves (fp32 [n_tokens, d_model]) for the streaming second pass.
template <bool kAny, bool kDyBf16>
__global__ void __launch_bounds__(kEmbThreads)
rms_dot_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
               const uint16_t* __restrict__ table, int d_model, const float* __restrict__ rms_weight,
               const float* __restrict__ rms_scale, const void* __restrict__ dy, float* __restrict__ dot_part,
               float* __restrict__ dw_part, float* __restrict__ s_out, int n_groups, int n_strips,
               int strips_per_group) {
  __shared__ float4 tab4[kRows * kPitch / 4];
  __shared__ float red[kEmbThreads / 64][kStrip];
  float* tab = reinterpret_cast<float*>(tab4);
  const int tid = threadIdx.x;
  const int grp = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_groups));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(n_groups);
  const int64_t t = tb * kEmbThreads + tid;
  const bool active = t < n_tokens;
  const int s_first = grp * strips_per_group;
  const int s_end = min(n_strips, s_first + strips_per_group);
  uint32_t offs[40];
  token_offsets<kAny>(offs, levels, t, active, n_bins, n_levels);
  const float r = active ? rms_scale[t] : 0.0f;
  float dot = 0.0f;
  DyRaw<kDyBf16> dyr;
  sum_strips<kAny>(tab, table, d_model, s_first, s_end, tid, n_bins, n_levels, offs,
                   [&](int col0) { load_dy_raw<kDyBf16>(dyr, dy, t, d_model, col0, active); },
                   [&](int col0, float (&acc)[kStrip]) {
                     if (s_out != nullptr && active) {
                       float4* so = reinterpret_cast<float4*>(s_out + t * d_model + col0);
                       so[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
                       so[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
                       so[2] = make_float4(acc[8], acc[9], acc[10], acc[11]);
                       so[3] = make_float4(acc[12], acc[13], acc[14], acc[15]);
                     }
                     dot_strip<kDyBf16>(col0, acc, dyr, rms_weight, r, dot, red, tid, dw_part, tb, d_model);
                   });
  if (active) dot_part[t * n_groups + grp] = dot;
}

// Pass 1 from sums the forward kept (sums [n_tokens, d_model] fp32): the same
// workgroups, strips and per-strip arithmetic as rms_dot_kernel, with the
// sums read instead of recomputed.  Strips go in pairs: a lane reads a whole
// 128-byte line of its token's sums (and of dy: four strips of bf16 at a
// time), the two strips' butterflies are independent, and one pair of
// barriers serves both.  (A thread past the batch adds +0 where
// rms_dot_kernel adds a zero of either sign; the column sums are then equal,
// and dw_reduce_kernel starts from +0, so the results are the same bits.)
template <bool kDyBf16>
__global__ void __launch_bounds__(kEmbThreads)
rms_dot_sums_kernel(const float* __restrict__ sums, int64_t n_tokens, int d_model, const float* __restrict__ rms_weight,
                    const float* __restrict__ rms_scale, const void* __restrict__ dy, float* __restrict__ dot_part,
                    float* __restrict__ dw_part, int n_groups, int n_strips, int strips_per_group) {
  __shared__ float red[2][kEmbThreads / 64][kStrip];
  const int tid = threadIdx.x;
  const int grp = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_groups));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(n_groups);
  const int64_t t = tb * kEmbThreads + tid;
  const bool active = t < n_tokens;
  const int s_first = grp * strips_per_group;
  const int s_end = min(n_strips, s_first + strips_per_group);
  const float r = active ? rms_scale[t] : 0.0f;
  float dot = 0.0f;
  auto load_sums = [&](int col0, float (&acc)[kStrip]) {
    if (active) {
      const float4* sp = reinterpret_cast<const float4*>(sums + t * d_model + col0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = sp[q];
        acc[4 * q] = v.x;
        acc[4 * q + 1] = v.y;
        acc[4 * q + 2] = v.z;
        acc[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < kStrip; ++c) acc[c] = 0.0f;
    }
  };
  // dy is read a whole 128-byte line per lane at a time: 4 strips of bf16, 2 of fp32
  constexpr int kDyStrips = kDyBf16 ? 4 : 2;
  for (int s0 = s_first; s0 < s_end; s0 += kDyStrips) {
    DyRaw<kDyBf16> dyq[kDyStrips];
#pragma unroll
    for (int i = 0; i < kDyStrips; ++i) {
      if (s0 + i < s_end) load_dy_raw<kDyBf16>(dyq[i], dy, t, d_model, (s0 + i) * kStrip, active);
    }
#pragma unroll
    for (int p = 0; p < kDyStrips; p += 2) {
      const int strip = s0 + p;
      if (strip >= s_end) break;  // the same in every thread
      const int col0 = strip * kStrip;
      const bool two = strip + 1 < s_end;
      float acc0[kStrip], acc1[kStrip];
      load_sums(col0, acc0);
      if (two) load_sums(col0 + kStrip, acc1);
      const float qs0 = dot_strip_q<kDyBf16>(col0, acc0, dyq[p], rms_weight, r, dot, tid);
      float qs1 = 0.0f;
      if (two) qs1 = dot_strip_q<kDyBf16>(col0 + kStrip, acc1, dyq[p + 1], rms_weight, r, dot, tid);
      if ((tid & 3) == 0) {
        red[0][tid >> 6][(tid >> 2) & 15] = qs0;
        red[1][tid >> 6][(tid >> 2) & 15] = qs1;
      }
      __syncthreads();
      if (tid < kStrip) dw_part[tb * d_model + col0 + tid] = red_sum(red[0], tid);
      else if (two && tid < 2 * kStrip) dw_part[tb * d_model + col0 + tid] = red_sum(red[1], tid - kStrip);
      __syncthreads();  // red is read before the next pair writes it
    }
  }
  if (active) dot_part[t * n_groups + grp] = dot;
}

// Pass 2: ds = r (w dy) - (r^3 / D) dot s, written fp32.
template <bool kAny, bool kDyBf16>
__global__ void __launch_bounds__(kEmbThreads)
rms_ds_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
              const uint16_t* __restrict__ table, int d_model, const float* __restrict__ rms_weight,
              const float* __restrict__ rms_scale, const void* __restrict__ dy, const float* __restrict__ dot_part,
              float* __restrict__ ds, int n_groups, int n_strips, int strips_per_group) {
  __shared__ float4 tab4[kRows * kPitch / 4];
  float* tab = reinterpret_cast<float*>(tab4);
  const int tid = threadIdx.x;
  const int grp = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_groups));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(n_groups);
  const int64_t t = tb * kEmbThreads + tid;
  const bool active = t < n_tokens;
  const int s_first = grp * strips_per_group;
  const int s_end = min(n_strips, s_first + strips_per_group);
  uint32_t offs[40];
  token_offsets<kAny>(offs, levels, t, active, n_bins, n_levels);
  float r = 0.0f, coef = 0.0f;
  if (active) {
    r = rms_scale[t];
    float dot = 0.0f;
    for (int g = 0; g < n_groups; ++g) dot += dot_part[t * n_groups + g];
    coef = ((r * r) * r) / static_cast<float>(d_model) * dot;
  }
  DyRaw<kDyBf16> dyr;
  sum_strips<kAny>(tab, table, d_model, s_first, s_end, tid, n_bins, n_levels, offs,
                   [&](int col0) { load_dy_raw<kDyBf16>(dyr, dy, t, d_model, col0, active); },
                   [&](int col0, float (&acc)[kStrip]) {
                     if (!active) return;
                     float gr[kStrip];
                     unpack_dy<kDyBf16>(gr, dyr);
                     float o[kStrip];
#pragma unroll
                     for (int c = 0; c < kStrip; ++c) o[c] = fmaf(-coef, acc[c], r * (rms_weight[col0 + c] * gr[c]));
                     float4* p = reinterpret_cast<float4*>(ds + t * d_model + col0);
                     p[0] = make_float4(o[0], o[1], o[2], o[3]);
                     p[1] = make_float4(o[4], o[5], o[6], o[7]);
                     p[2] = make_float4(o[8], o[9], o[10], o[11]);
                     p[3] = make_float4(o[12], o[13], o[14], o[15]);
                   });
}

// Second pass from stored sums (when the workspace holds them): the per-token
// factor (r^3 / D) dot, then ds = r (w dy) - factor s as a stream over the
// stored sums: the same expressions, in the same order, as rms_ds_kernel.
__global__ void __launch_bounds__(256)
rms_coef_kernel(const float* __restrict__ dot_part, const float* __restrict__ rms_scale, int64_t n_tokens,
                int n_groups, int d_model, float* __restrict__ coef) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_tokens) return;
  const float r = rms_scale[t];
  float dot = 0.0f;
  for (int g = 0; g < n_groups; ++g) dot += dot_part[t * n_groups + g];
  coef[t] = ((r * r) * r) / static_cast<float>(d_model) * dot;
}

template <bool kDyBf16>
__global__ void __launch_bounds__(256)
rms_ds_stream_kernel(const float* __restrict__ s, const void* __restrict__ dy, const float* __restrict__ rms_weight,
                     const float* __restrict__ rms_scale, const float* __restrict__ coef, int64_t n_tokens,
                     int d_model, float* __restrict__ ds) {
  // a workgroup takes whole tokens (their scale and coefficient are uniform
  // loads), its threads 4 columns each
  const int q4 = d_model / 4;
  for (int64_t t = blockIdx.x; t < n_tokens; t += gridDim.x) {
    const float r = rms_scale[t], cf = coef[t];
    const int64_t row = t * q4;
    for (int c4 = threadIdx.x; c4 < q4; c4 += 256) {
      const int64_t i = row + c4;
      const float4 sv = reinterpret_cast<const float4*>(s)[i];
      float gr[4];
      if (kDyBf16) {
        const uint2 h = reinterpret_cast<const uint2*>(dy)[i];
        gr[0] = bf16_to_f32(h.x & 0xFFFFu);
        gr[1] = bf16_to_f32(h.x >> 16);
        gr[2] = bf16_to_f32(h.y & 0xFFFFu);
        gr[3] = bf16_to_f32(h.y >> 16);
      } else {
        const float4 g = reinterpret_cast<const float4*>(dy)[i];
        gr[0] = g.x;
        gr[1] = g.y;
        gr[2] = g.z;
        gr[3] = g.w;
      }
      const float4 w = reinterpret_cast<const float4*>(rms_weight)[c4];
      reinterpret_cast<float4*>(ds)[i] =
          make_float4(fmaf(-cf, sv.x, r * (w.x * gr[0])), fmaf(-cf, sv.y, r * (w.y * gr[1])),
                      fmaf(-cf, sv.z, r * (w.z * gr[2])), fmaf(-cf, sv.w, r * (w.w * gr[3])));
    }
  }
}

// dw[c] = (accumulate ? dw[c] : 0) + sum over token blocks, in order.
__global__ void __launch_bounds__(256)
dw_reduce_kernel(const float* __restrict__ dw_part, int64_t n_blocks, int d_model, float* __restrict__ dw,
                 int accumulate) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d_model) return;
  float v = 0.0f;
  for (int64_t b = 0; b < n_blocks; ++b) v += dw_part[b * d_model + c];
  dw[c] = accumulate ? dw[c] + v : v;
}

// strips per workgroup for the recompute passes (as launch_embed chooses)
int strips_per_group(int64_t tblocks, int n_strips) {
  static const int kCounts[] = {16, 8, 4, 3, 2, 1};
  int64_t cost[6];
  int64_t min_cost = -1;
  for (int i = 0; i < 6; ++i) {
    const int g = kCounts[i];
    const int64_t wgs = tblocks * ((n_strips + g - 1) / g);
    cost[i] = ((wgs + 255) / 256) * g;
    if (min_cost < 0 || cost[i] < min_cost) min_cost = cost[i];
  }
  for (int i = 0; i < 6; ++i)
    if (cost[i] * 100 <= min_cost * 105) return kCounts[i];
  return 1;
}

}  // namespace

size_t bwd_layout(int64_t n_tokens, int n_bins, int d_model, size_t* offs) {
  // levels by bin [n_bins][t_pad] (t_pad = whole chunks), then the row of
  // -0.0; nothing for an empty batch
  (void)d_model;
  if (offs) offs[0] = 0;
  if (n_tokens <= 0) return 0;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t t_pad = static_cast<size_t>((n_tokens + kChunk - 1) / kChunk) * kChunk;
  const size_t b_lvt = up(static_cast<size_t>(n_bins) * t_pad);
  const size_t b_nz = up(kBwdCols * sizeof(float));
  if (offs) offs[0] = b_lvt;
  return b_lvt + b_nz;
}

hipError_t launch_embed_backward(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels, const void* dsum,
                                 bool dsum_bf16, int d_model, float* dtable, bool accumulate, void* workspace,
                                 hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(n_bins) * n_levels;
  if (n_tokens <= 0) {
    if (accumulate) return hipSuccess;
    return zero_fill(dtable, rows * d_model, stream);
  }
  size_t offs[1];
  bwd_layout(n_tokens, n_bins, d_model, offs);
  auto* lvt = static_cast<uint8_t*>(workspace);
  auto* neg_zero = reinterpret_cast<float*>(static_cast<char*>(workspace) + offs[0]);
  const int64_t n_chunks = (n_tokens + kChunk - 1) / kChunk;
  const int64_t t_pad = n_chunks * kChunk;
  if (n_chunks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(levels_t_kernel, dim3(static_cast<unsigned>(n_chunks)), dim3(256), 0, stream, levels, n_tokens,
                     n_bins, n_levels, t_pad, lvt, neg_zero);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_groups = (n_bins + kBwdBins - 1) / kBwdBins;
  const int n_strips = (d_model + kBwdCols - 1) / kBwdCols;
  const int per_xcd = (n_strips + 7) / 8;
  const int64_t blocks = static_cast<int64_t>(per_xcd) * 8 * n_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (dsum_bf16) {
    hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBwdThreads), 0, stream,
                       static_cast<const uint16_t*>(dsum), n_tokens, n_bins, n_levels, d_model, lvt, t_pad, n_chunks,
                       n_groups, n_strips, per_xcd, dtable, accumulate ? 1 : 0);
  } else {
    const int groups16 = (n_bins + kS16Bins - 1) / kS16Bins;
    const int strips16 = (d_model + kS16Cols - 1) / kS16Cols;
    const int per_xcd16 = (strips16 + 7) / 8;
    const int64_t blocks16 = static_cast<int64_t>(per_xcd16) * 8 * groups16;
    hipLaunchKernelGGL(scatter16_kernel, dim3(static_cast<unsigned>(blocks16)), dim3(kS16Threads), 0, stream,
                       static_cast<const float*>(dsum), n_tokens, n_bins, n_levels, d_model, lvt, t_pad, neg_zero,
                       n_chunks, groups16, strips16, per_xcd16, dtable, accumulate ? 1 : 0);
  }
  return hipGetLastError();
}

size_t rms_bwd_layout(int64_t n_tokens, int d_model, size_t* off_dw) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const int n_strips = d_model / kStrip;
  const int64_t tblocks = (n_tokens + kEmbThreads - 1) / kEmbThreads;
  const int g = strips_per_group(tblocks, n_strips);
  const int n_groups = (n_strips + g - 1) / g;
  const size_t b_dot = up(static_cast<size_t>(n_tokens) * n_groups * sizeof(float));
  const size_t b_dw = up(static_cast<size_t>(tblocks) * d_model * sizeof(float));
  if (off_dw) *off_dw = b_dot;
  return b_dot + b_dw;
}

// The larger workspace of the stored-sum second pass: the layout above, then
// the sums fp32 [n_tokens, d_model], then the per-token factors.
size_t rms_bwd_stored_bytes(int64_t n_tokens, int d_model) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t n = static_cast<size_t>(n_tokens);
  return rms_bwd_layout(n_tokens, d_model, nullptr) + up(n * d_model * sizeof(float)) + up(n * sizeof(float));
}

hipError_t launch_rms_backward(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                               const uint16_t* table, int d_model, const float* rms_weight, const float* rms_scale,
                               const void* dy, bool dy_bf16, float* ds, float* dweight, bool accumulate_dweight,
                               void* workspace, bool stored, hipStream_t stream) {
  if (n_tokens <= 0) {
    if (dweight == nullptr || accumulate_dweight) return hipSuccess;
    return zero_fill(dweight, d_model, stream);
  }
  size_t off_dw = 0;
  rms_bwd_layout(n_tokens, d_model, &off_dw);
  auto* dot_part = static_cast<float*>(workspace);
  auto* dw_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + off_dw);
  const int n_strips = d_model / kStrip;
  const int64_t tblocks = (n_tokens + kEmbThreads - 1) / kEmbThreads;
  const int g = strips_per_group(tblocks, n_strips);
  const int n_groups = (n_strips + g - 1) / g;
  const int64_t blocks = tblocks * n_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool any = !(n_bins == kMels && n_levels == kLevels);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kEmbThreads);
#define DMEL_RMS_PASS(KERNEL, ...)                                                                           \
  do {                                                                                                       \
    if (any && dy_bf16) hipLaunchKernelGGL((KERNEL<true, true>), grid, block, 0, stream, __VA_ARGS__);       \
    else if (any) hipLaunchKernelGGL((KERNEL<true, false>), grid, block, 0, stream, __VA_ARGS__);            \
    else if (dy_bf16) hipLaunchKernelGGL((KERNEL<false, true>), grid, block, 0, stream, __VA_ARGS__);        \
    else hipLaunchKernelGGL((KERNEL<false, false>), grid, block, 0, stream, __VA_ARGS__);                    \
  } while (0)
  const size_t base = rms_bwd_layout(n_tokens, d_model, nullptr);
  float* s_store = stored ? reinterpret_cast<float*>(static_cast<char*>(workspace) + base) : nullptr;
  DMEL_RMS_PASS(rms_dot_kernel, levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, dy,
                dot_part, dw_part, s_store, n_groups, n_strips, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (stored) {
    const size_t b_s = (static_cast<size_t>(n_tokens) * d_model * sizeof(float) + 255) / 256 * 256;
    auto* coef = reinterpret_cast<float*>(static_cast<char*>(workspace) + base + b_s);
    hipLaunchKernelGGL(rms_coef_kernel, dim3(static_cast<unsigned>((n_tokens + 255) / 256)), dim3(256), 0, stream,
                       dot_part, rms_scale, n_tokens, n_groups, d_model, coef);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned sb = static_cast<unsigned>(std::min<int64_t>(n_tokens, 256 * 64));
    if (dy_bf16) {
      hipLaunchKernelGGL(rms_ds_stream_kernel<true>, dim3(sb), dim3(256), 0, stream, s_store, dy, rms_weight,
                         rms_scale, coef, n_tokens, d_model, ds);
    } else {
      hipLaunchKernelGGL(rms_ds_stream_kernel<false>, dim3(sb), dim3(256), 0, stream, s_store, dy, rms_weight,
                         rms_scale, coef, n_tokens, d_model, ds);
    }
  } else {
    DMEL_RMS_PASS(rms_ds_kernel, levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, dy,
                  dot_part, ds, n_groups, n_strips, g);
  }
#undef DMEL_RMS_PASS
  e = hipGetLastError();
  if (e != hipSuccess || dweight == nullptr) return e;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((d_model + 255) / 256), dim3(256), 0, stream, dw_part, tblocks, d_model,
                     dweight, accumulate_dweight ? 1 : 0);
  return hipGetLastError();
}

size_t rms_bwd_sums_bytes(int64_t n_tokens, int d_model) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  return rms_bwd_layout(n_tokens, d_model, nullptr) + up(static_cast<size_t>(n_tokens) * sizeof(float));
}

hipError_t launch_rms_backward_sums(const float* sums, int64_t n_tokens, int d_model, const float* rms_weight,
                                    const float* rms_scale, const void* dy, bool dy_bf16, float* ds, float* dweight,
                                    bool accumulate_dweight, void* workspace, hipStream_t stream) {
  if (n_tokens <= 0) {
    if (dweight == nullptr || accumulate_dweight) return hipSuccess;
    return zero_fill(dweight, d_model, stream);
  }
  size_t off_dw = 0;
  const size_t base = rms_bwd_layout(n_tokens, d_model, &off_dw);
  auto* dot_part = static_cast<float*>(workspace);
  auto* dw_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + off_dw);
  auto* coef = reinterpret_cast<float*>(static_cast<char*>(workspace) + base);
  const int n_strips = d_model / kStrip;
  const int64_t tblocks = (n_tokens + kEmbThreads - 1) / kEmbThreads;
  const int g = strips_per_group(tblocks, n_strips);
  const int n_groups = (n_strips + g - 1) / g;
  const int64_t blocks = tblocks * n_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kEmbThreads);
  if (dy_bf16) {
    hipLaunchKernelGGL(rms_dot_sums_kernel<true>, grid, block, 0, stream, sums, n_tokens, d_model, rms_weight,
                       rms_scale, dy, dot_part, dw_part, n_groups, n_strips, g);
  } else {
    hipLaunchKernelGGL(rms_dot_sums_kernel<false>, grid, block, 0, stream, sums, n_tokens, d_model, rms_weight,
                       rms_scale, dy, dot_part, dw_part, n_groups, n_strips, g);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rms_coef_kernel, dim3(static_cast<unsigned>((n_tokens + 255) / 256)), dim3(256), 0, stream,
                     dot_part, rms_scale, n_tokens, n_groups, d_model, coef);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned sb = static_cast<unsigned>(std::min<int64_t>(n_tokens, 256 * 64));
  if (dy_bf16) {
    hipLaunchKernelGGL(rms_ds_stream_kernel<true>, dim3(sb), dim3(256), 0, stream, sums, dy, rms_weight, rms_scale,
                       coef, n_tokens, d_model, ds);
  } else {
    hipLaunchKernelGGL(rms_ds_stream_kernel<false>, dim3(sb), dim3(256), 0, stream, sums, dy, rms_weight, rms_scale,
                       coef, n_tokens, d_model, ds);
  }
  if ((e = hipGetLastError()) != hipSuccess || dweight == nullptr) return e;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((d_model + 255) / 256), dim3(256), 0, stream, dw_part, tblocks, d_model,
                     dweight, accumulate_dweight ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dmel
