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
//
// Other layouts (a config with n_mel_bins <= 80 bins of mel_vocab_size <= 16
// rows each, table row n_levels * bin + level) run in the same 80 x 16 row
// space: table row V * b + l is staged at LDS row 16 * b + l, every other LDS
// row holds -0.0, and the bins past n_bins select level 0 of their (empty)
// block.  Adding -0.0 leaves every fp32 value unchanged (x + -0 = x, also for
// x = +0 and -0), so the padded sum is bit-identical to the sum over the
// n_bins real bins.
#include "embed_core.h"

namespace dmel {
namespace {

// The (strip group, token block) of this workgroup, for a grid of
// n_groups x token blocks.  Workgroup b runs on XCD b % 8.  With a multiple
// of 8 strip groups, XCD x takes group x for every token block, then group
// x + 8, and so on, so its L2 holds one group's table slices at a time (1.97 MB
// for 48 strips) while the output streams through it; otherwise consecutive
// workgroups take the groups of one token block.  (The backward's recompute
// passes keep the second order: they stream dy per token block, and measured
// slower with the first.)
__device__ __forceinline__ void block_tile(int n_groups, int& grp, int64_t& tb) {
  if (n_groups % 8 == 0) {
    const unsigned x = blockIdx.x & 7u, r = blockIdx.x >> 3;
    const unsigned tblocks = gridDim.x / static_cast<unsigned>(n_groups);
    grp = static_cast<int>(8u * (r / tblocks) + x);
    tb = r % tblocks;
  } else {
    grp = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_groups));
    tb = blockIdx.x / static_cast<unsigned>(n_groups);
  }
}

// kAny = false: the released layout (levels [n, 80], 16-byte aligned, table
// [1280, d]); true: any n_bins <= 80, n_levels <= 16 (see the top of the file).
// kSums: also write each token's fp32 sums (before the RMSNorm) to sums_out.
template <bool kAny, bool kSums>
__global__ void __launch_bounds__(kEmbThreads)
embed_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
             const uint16_t* __restrict__ table, int d_model, const float* __restrict__ rms_weight,
             const float* __restrict__ rms_scale, void* __restrict__ out, int out_f32, int64_t out_row_stride,
             const int64_t* __restrict__ out_rows, int n_groups, int n_strips, int strips_per_group,
             float* __restrict__ sums_out) {
  __shared__ float4 tab4[kRows * kPitch / 4];
  float* tab = reinterpret_cast<float*>(tab4);

  const int tid = threadIdx.x;
  int grp;
  int64_t tb;
  block_tile(n_groups, grp, tb);
  const int64_t t = tb * kEmbThreads + tid;
  const bool active = t < n_tokens;
  const int s_first = grp * strips_per_group;
  const int s_end = min(n_strips, s_first + strips_per_group);

  uint4 st[kStagePer];
  stage_load<kAny>(st, table, d_model, s_first * kStrip, 0, tid, n_bins, n_levels);

  uint32_t lv[20];
  if (active && kAny) {
    load_levels_any(lv, levels, t, n_bins, static_cast<uint32_t>(n_levels - 1));
  } else if (active) {
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
  // Byte offset of the row each bin selects, relative to its half's base (bins
  // 0..39 from the slice start, 40..79 from bin 40), two 16-bit offsets per
  // register: one VALU op per bin then forms the read address.
  uint32_t offs[40];
#pragma unroll
  for (int i = 0; i < 40; ++i) {
    const int j0 = 2 * i, j1 = 2 * i + 1;
    const uint32_t L0 = (lv[j0 >> 2] >> (8 * (j0 & 3))) & 0xFFu;
    const uint32_t L1 = (lv[j1 >> 2] >> (8 * (j1 & 3))) & 0xFFu;
    const uint32_t o0 = (kLevels * (j0 % 40) + L0) * kPitch * 4;
    const uint32_t o1 = (kLevels * (j1 % 40) + L1) * kPitch * 4;
    offs[i] = o0 | (o1 << 16);
  }
  stage_store(tab, st, 0, tid);
  __syncthreads();

  // Per strip: bins 0..39 come from the first half of the LDS slice and bins
  // 40..79 from the second.  The global reads of the half needed next are
  // issued before the adds of the current half, so the table staging overlaps
  // the arithmetic; each half is written once its previous contents are dead.
  for (int strip = s_first; strip < s_end; ++strip) {
    const int col0 = strip * kStrip;
    // make the offsets look modified here so that the 80 unpacked row offsets
    // are not hoisted out of the strip loop (keeping them live would spill)
#pragma unroll
    for (int i = 0; i < 40; ++i) asm volatile("" : "+v"(offs[i]));
    stage_load<kAny>(st, table, d_model, col0, 1, tid, n_bins, n_levels);
    float acc[kStrip];
    add_bins<0, kMels / 2>(acc, tab, offs);
    stage_store(tab, st, 1, tid);
    __syncthreads();
    const bool more = strip + 1 < s_end;
    if (more) stage_load<kAny>(st, table, d_model, col0 + kStrip, 0, tid, n_bins, n_levels);
    // (a layout of at most 40 bins has nothing but -0.0 rows in this half)
    if (!kAny || n_bins > kMels / 2) add_bins<kMels / 2, kMels>(acc, tab, offs);

    if (active) {
      if (kSums) {
        // the fp32 sums themselves, for a backward that does not recompute them
        float4* so = reinterpret_cast<float4*>(sums_out + t * d_model + col0);
        so[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        so[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        so[2] = make_float4(acc[8], acc[9], acc[10], acc[11]);
        so[3] = make_float4(acc[12], acc[13], acc[14], acc[15]);
      }
      if (rms_weight != nullptr) {
#pragma unroll
        for (int c = 0; c < kStrip; ++c) acc[c] = (acc[c] * scale) * rms_weight[col0 + c];
      }
      // Plain stores: the strips of a workgroup complete each token's
      // 128-byte lines in L2 before they are written back.  (Non-temporal
      // stores, which would keep the output from evicting the table slices,
      // send the 32-byte pieces to memory one by one and nearly double the
      // bytes written.)
      if (out_f32) {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + orow * out_row_stride + col0);
        o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        o[2] = make_float4(acc[8], acc[9], acc[10], acc[11]);
        o[3] = make_float4(acc[12], acc[13], acc[14], acc[15]);
      } else {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = pack_bf16(acc[2 * i], acc[2 * i + 1]);
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + orow * out_row_stride + col0);
        o[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
    }
    // the first half was last read before the barrier above
    if (more) stage_store(tab, st, 0, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Gram matrix G = E E^T in fp64.  A product of two bf16 entries is exact in
// fp64; the products are summed over the columns in fp64 on the matrix cores
// (v_mfma_f64_16x16x4_f64).  G is indexed in the 80 x 16 row space (16 * bin
// + level) for every layout; rows outside the n_bins x n_levels layout are 0.
// One workgroup per 64 x 64 block of the upper triangle (20 x 20 blocks of
// 4 bins each); each wavefront owns a 32 x 32 quarter as 2 x 2 MFMA tiles.
// The columns pass through LDS in chunks of 64, converted to fp64 and stored
// column by column; the next chunk is read into registers while the current
// one is multiplied.
// ---------------------------------------------------------------------------
constexpr int kGTile = 64;
constexpr int kGTiles = kRows / kGTile;  // 20
constexpr int kGK = 64;                  // columns per chunk
constexpr int kGPitchD = kGTile + 2;     // doubles per staged column

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// A block's 64 rows x 64 columns as 512 pieces of 8 bf16: piece p = tid +
// 256 i is row p / 8, columns c0 + 8 (p % 8) .. + 7 (d_model is a multiple
// of 16, so a piece lies wholly inside or wholly past the last column).
__device__ __forceinline__ void gram_fetch(uint4 (&v)[2], const uint16_t* __restrict__ table, int d_model,
                                           int n_bins, int n_levels, int blk, int c0, int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i, row = p >> 3, col = c0 + 8 * (p & 7);
    const int r = kGTile * blk + row, bin = r >> 4, lev = r & 15;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (bin < n_bins && lev < n_levels && col < d_model)
      v[i] = *reinterpret_cast<const uint4*>(table + static_cast<int64_t>(n_levels * bin + lev) * d_model + col);
  }
}

__device__ __forceinline__ void gram_stage(double* s, const uint4 (&v)[2], int tid) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = tid + 256 * i, row = p >> 3, c = 8 * (p & 7);
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s[(c + 2 * q) * kGPitchD + row] = static_cast<double>(bf16_to_f32(w[q] & 0xFFFFu));
      s[(c + 2 * q + 1) * kGPitchD + row] = static_cast<double>(bf16_to_f32(w[q] >> 16));
    }
  }
}

__global__ void __launch_bounds__(256)
gram_kernel(const uint16_t* __restrict__ table, int n_bins, int n_levels, int d_model, double* __restrict__ gram) {
  __shared__ double a_s[kGK * kGPitchD];
  __shared__ double b_s[kGK * kGPitchD];
  // blockIdx.x enumerates the upper-triangle block pairs (J, J')
  int idx = blockIdx.x;
  int bj = 0;
  while (idx >= kGTiles - bj) {
    idx -= kGTiles - bj;
    ++bj;
  }
  const int bjp = bj + idx;
  const bool diag = bj == bjp;
  const double* bsrc = diag ? a_s : b_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wr = (wv >> 1) * 32, wc = (wv & 1) * 32;
  f64x4_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  uint4 va[2], vb[2];
  gram_fetch(va, table, d_model, n_bins, n_levels, bj, 0, tid);
  if (!diag) gram_fetch(vb, table, d_model, n_bins, n_levels, bjp, 0, tid);
  for (int c0 = 0; c0 < d_model; c0 += kGK) {
    __syncthreads();
    gram_stage(a_s, va, tid);
    if (!diag) gram_stage(b_s, vb, tid);
    __syncthreads();
    if (c0 + kGK < d_model) {
      gram_fetch(va, table, d_model, n_bins, n_levels, bj, c0 + kGK, tid);
      if (!diag) gram_fetch(vb, table, d_model, n_bins, n_levels, bjp, c0 + kGK, tid);
    }
    // MFMA operands: lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]
#pragma unroll 4
    for (int k = 0; k < kGK; k += 4) {
      const int c = k + (lane >> 4);
      const double a0 = a_s[c * kGPitchD + wr + (lane & 15)];
      const double a1 = a_s[c * kGPitchD + wr + 16 + (lane & 15)];
      const double b0 = bsrc[c * kGPitchD + wc + (lane & 15)];
      const double b1 = bsrc[c * kGPitchD + wc + 16 + (lane & 15)];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
  // result: lane l, element e holds row l / 16 + 4 e, column l % 16 of a tile
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = kGTile * bj + wr + 16 * a + (lane >> 4) + 4 * e;
        const int cc = kGTile * bjp + wc + 16 * b + (lane & 15);
        gram[static_cast<int64_t>(r) * kRows + cc] = acc[a][b][e];
        if (!diag) gram[static_cast<int64_t>(cc) * kRows + r] = acc[a][b][e];
      }
}

// ---------------------------------------------------------------------------
// RMSNorm scale from the Gram matrix.  For a token with rows r_0 .. r_79
// (r_j = 16 j + L_j), |s|^2 = sum_j (d_j + 2 o_j) with d_j = G[r_j][r_j] and
// o_j = sum_{j' > j} G[r_j][r_j'].  Every kernel below evaluates it in fp64
// in the same order: o_j from +0 in increasing j', the total from +0 adding
// d_j then 2 o_j for j = 0 .. 79; then r = 1 / sqrt(total / d_model + eps)
// in fp64, rounded to fp32.  A masked term adds +0.0, which leaves a sum that
// started at +0.0 unchanged (such a sum is never -0.0), so the kernels give a
// token the same bits whichever of them runs.
//
// The levels of a token are kept in registers as 80 bytes (bin j in byte
// j % 4 of word j / 4), indexed statically.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t level_byte(const uint32_t (&lw)[20], int j) {
  return (lw[j >> 2] >> (8 * (j & 3))) & 0xFFu;
}

__device__ __forceinline__ void load_token_levels(uint32_t (&lw)[20], const uint8_t* levels, int64_t t, bool active,
                                                  bool any_layout, int n_bins, int n_levels) {
  if (active && any_layout) {
    load_levels_any(lw, levels, t, n_bins, static_cast<uint32_t>(n_levels - 1));
  } else if (active) {
    const uint4* p = reinterpret_cast<const uint4*>(levels + t * kMels);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint4 q = p[i];
      lw[4 * i + 0] = clamp_levels(q.x);
      lw[4 * i + 1] = clamp_levels(q.y);
      lw[4 * i + 2] = clamp_levels(q.z);
      lw[4 * i + 3] = clamp_levels(q.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 20; ++i) lw[i] = 0;
  }
}

// Rows 16 j .. 16 j + 15 of G, columns c0 .. c0 + width - 1, staged in LDS as
// g_s[r * kGPitch + c - c0] (fp64): the 16 rows of bin j over a part of the
// upper triangle.  A part spans at most kGCols columns (64 bins); bins
// 0 .. 15 take two parts.  1024 threads: 64 per row, 16-byte reads.
constexpr int kGCols = 1024;
constexpr int kGPitch = kGCols + 1;           // doubles per staged row (odd: the 16 rows start in different banks)
constexpr int kScaleThreads = 1024;
// Columns width .. zero_end - 1 of each staged row (both even) are set to
// +0.0, for lookups that run past the end of the upper triangle.
__device__ __forceinline__ void stage_gram_part(double* g_s, const double* __restrict__ gram, int j, int c0, int width,
                                                int tid, int zero_end) {
  const int r = tid >> 6;  // 0..15
  const int q = tid & 63;
  const double* src = gram + static_cast<int64_t>(kLevels * j + r) * kRows + c0;
  double* dst = g_s + r * kGPitch;
  // four reads in flight per thread, then their stores
  for (int c = 2 * q; c < width; c += 4 * 128) {
    double2 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c + 128 * i < width) v[i] = *reinterpret_cast<const double2*>(src + c + 128 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (c + 128 * i < width) {
        dst[c + 128 * i] = v[i].x;
        dst[c + 128 * i + 1] = v[i].y;
      }
    }
  }
  for (int c = width + 2 * q; c < zero_end; c += 128) {
    dst[c] = 0.0;
    dst[c + 1] = 0.0;
  }
}

// Adds the terms of bins j' = j + q, q = Q0 .. Q1 (static), of one token to
// o: the value at column 16 q + L_j' - base of the token's staged row (the
// row of level L_j, staged from column 16 j + base).  rot8 holds the levels
// times 8 (byte offsets of a double), bins j, j + 1, ... in bytes 0, 1, ...;
// so a lookup is one add of a byte to the row's LDS address, with 8 (16 q -
// base) in the read's immediate offset.  Bins past 79 (q > 79 - j) land in
// the zeroed columns after the triangle and add +0.0, which leaves the sum
// unchanged (it starts at +0.0, so it is never -0.0).  The lookups go out
// kTermBatch at a time and are then added in order, so a wavefront has that
// many LDS reads in flight.
constexpr int kTermBatch = 8;
template <int Q0, int Q1>
__device__ __forceinline__ void gram_terms(double& o, const char* row, const uint32_t (&rot8)[20], int base) {
#pragma unroll
  for (int q0 = Q0; q0 <= Q1; q0 += kTermBatch) {
    double v[kTermBatch];
#pragma unroll
    for (int i = 0; i < kTermBatch; ++i) {
      const int q = q0 + i;
      if (q <= Q1) v[i] = *reinterpret_cast<const double*>(row + level_byte(rot8, q) + 8 * (kLevels * q - base));
    }
#pragma unroll
    for (int i = 0; i < kTermBatch; ++i) {
      if (q0 + i <= Q1) o += v[i];
    }
    // keep the next batch's lookups after this batch's adds (registers)
    asm volatile("" : "+v"(o)::"memory");
  }
}

// The off-diagonal sum o_j of one token for bin j from part 1 (base 0, bins
// j .. j + 63).  QMAX bounds 79 - j for the caller's range of bins, so the
// loop is unrolled with static register indices; its terms past 79 - j read
// zeros.
template <int QMAX>
__device__ __forceinline__ void part1_terms(double& o, const char* row, const uint32_t (&rot8)[20]) {
  gram_terms<1, (QMAX < 63 ? QMAX : 63)>(o, row, rot8, 0);
}

// Large batches: a workgroup owns 3072 tokens (three per thread); for each bin
// the bin's 16 rows of G are staged part by part and every token adds its
// terms.  The token's levels are a byte string shifted down by one byte per
// bin (v_alignbyte), so that the level of bin j + q is always byte q.
constexpr int kScaleTok = 3;                            // tokens per thread
constexpr int kScaleBlock = kScaleThreads * kScaleTok;  // tokens per workgroup

__global__ void __launch_bounds__(kScaleThreads)
rms_scale_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
                 const double* __restrict__ gram, int d_model, float eps, float* __restrict__ scale) {
  __shared__ double g_s[16 * kGPitch];  // 131 KB
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kScaleBlock + tid;
  const bool any = n_bins != kMels || n_levels != kLevels;
  uint32_t rot[kScaleTok][20];
  double total[kScaleTok];
#pragma unroll
  for (int k = 0; k < kScaleTok; ++k) {
    const int64_t t = t0 + static_cast<int64_t>(k) * kScaleThreads;
    total[k] = 0.0;
    load_token_levels(rot[k], levels, t, t < n_tokens, any, n_bins, n_levels);
    // levels (at most 15) times 8, byte by byte
#pragma unroll
    for (int i = 0; i < 20; ++i) rot[k][i] <<= 3;
  }
  const char* g_b = reinterpret_cast<const char*>(g_s);
  for (int j = 0; j < kMels; ++j) {
    const int c0 = kLevels * j;
    const int width = min(kRows - c0, kGCols);
    __syncthreads();
    // zeros for the lookups of up to 9 bins past bin 79 (the QMAX groups below)
    stage_gram_part(g_s, gram, j, c0, width, tid, min(kGCols, width + 160));
    __syncthreads();
    double off[kScaleTok], diag[kScaleTok];
    const char* row[kScaleTok];
#pragma unroll
    for (int k = 0; k < kScaleTok; ++k) {
      const uint32_t lj8 = rot[k][0] & 0xFFu;   // 8 L_j
      row[k] = g_b + lj8 * kGPitch;
      diag[k] = *reinterpret_cast<const double*>(row[k] + lj8);
      off[k] = 0.0;
    }
#pragma unroll
    for (int k = 0; k < kScaleTok; ++k) {
      switch (j / 10) {
        case 0: part1_terms<79>(off[k], row[k], rot[k]); break;
        case 1: part1_terms<69>(off[k], row[k], rot[k]); break;
        case 2: part1_terms<59>(off[k], row[k], rot[k]); break;
        case 3: part1_terms<49>(off[k], row[k], rot[k]); break;
        case 4: part1_terms<39>(off[k], row[k], rot[k]); break;
        case 5: part1_terms<29>(off[k], row[k], rot[k]); break;
        case 6: part1_terms<19>(off[k], row[k], rot[k]); break;
        default: part1_terms<9>(off[k], row[k], rot[k]); break;
      }
    }
    if (j < kMels - 64) {
      // bins j + 64 .. 79 (j <= 15): columns 16 j + 1024 .. 1279, then zeros
      // up to relative column 256 for the terms past bin 79
      __syncthreads();
      stage_gram_part(g_s, gram, j, c0 + kGCols, kRows - c0 - kGCols, tid, 256);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kScaleTok; ++k) gram_terms<64, 79>(off[k], row[k], rot[k], kGCols);
    }
#pragma unroll
    for (int k = 0; k < kScaleTok; ++k) {
      total[k] += diag[k];
      total[k] += 2.0 * off[k];
      // shift the byte string down by one byte
#pragma unroll
      for (int i = 0; i < 19; ++i) rot[k][i] = __builtin_amdgcn_alignbyte(rot[k][i + 1], rot[k][i], 1);
      rot[k][19] >>= 8;
    }
  }
#pragma unroll
  for (int k = 0; k < kScaleTok; ++k) {
    const int64_t t = t0 + static_cast<int64_t>(k) * kScaleThreads;
    if (t < n_tokens) {
      const double ms = total[k] / static_cast<double>(d_model);
      scale[t] = static_cast<float>(1.0 / sqrt(ms + static_cast<double>(eps)));
    }
  }
}

// Small batches without a workspace: one thread per (token, bin j) reads row
// r_j of G straight from memory and forms d_j and o_j (same terms, same
// order); the token's total is then summed in bin order by one thread.
constexpr int kDirTok = 4;                  // tokens per workgroup
constexpr int kDirThreads = kDirTok * kMels;  // 320

__global__ void __launch_bounds__(kDirThreads)
rms_scale_direct_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
                        const double* __restrict__ gram, int d_model, float eps, float* __restrict__ scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lv_s[kDirTok][kMels];
  __shared__ double d_s[kDirTok][kMels];
  __shared__ double o_s[kDirTok][kMels];
  const int tid = threadIdx.x;
  const int tok = tid / kMels;
  const int j = tid - tok * kMels;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kDirTok + tok;
  const bool active = t < n_tokens;
  if (active) {
    // bins past n_bins take level 0 of their (zero) block of G
    const uint32_t vmax = static_cast<uint32_t>(n_levels - 1);
    const uint32_t v = j < n_bins ? levels[t * n_bins + j] : 0u;
    lv_s[tok][j] = static_cast<uint8_t>(v > vmax ? vmax : v);
  }
  __syncthreads();
  if (active) {
    const int rj = kLevels * j + lv_s[tok][j];
    const double* row = gram + static_cast<int64_t>(rj) * kRows;
    uint32_t lw[20];
#pragma unroll
    for (int i = 0; i < 20; ++i) lw[i] = reinterpret_cast<const uint32_t*>(lv_s[tok])[i];
    // terms of bins jp <= j are +0.0; sixteen lookups are issued together
    double off = 0.0;
#pragma unroll
    for (int jb = 0; jb < kMels; jb += 16) {
      double v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = row[kLevels * (jb + i) + level_byte(lw, jb + i)];
#pragma unroll
      for (int i = 0; i < 16; ++i) off += jb + i > j ? v[i] : 0.0;
    }
    d_s[tok][j] = row[rj];
    o_s[tok][j] = off;
  }
  __syncthreads();
  if (active && j == 0) {
    double total = 0.0;
    for (int jj = 0; jj < kMels; ++jj) {
      total += d_s[tok][jj];
      total += 2.0 * o_s[tok][jj];
    }
    const double ms = total / static_cast<double>(d_model);
    scale[t] = static_cast<float>(1.0 / sqrt(ms + static_cast<double>(eps)));
  }
}

// Small batches with a workspace, bin-parallel: a workgroup takes one bin j
// and 1024 tokens (one per thread), stages bin j's rows of G part by part and
// writes each token's (d_j, o_j) to part[j][token]; rms_total_kernel then adds
// the 80 bins of each token in order.  The lookups are those of
// rms_scale_kernel (gram_terms), on the token's level string shifted by j
// bytes, so every byte index is static.
constexpr int kBinTok = 1024;
static_assert(kBinTok == kScaleThreads, "stage_gram_part gives each of 16 rows 64 threads");

template <bool kAny>
__global__ void __launch_bounds__(kBinTok)
rms_bin_partials_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
                        const double* __restrict__ gram, int n_chunks, double2* __restrict__ part) {
  __shared__ double g_s[16 * kGPitch];   // 131 KB
  const int tid = threadIdx.x;
  const int j = static_cast<int>(blockIdx.x / static_cast<unsigned>(n_chunks));  // heavy (small) bins first
  const int64_t t = static_cast<int64_t>(blockIdx.x % static_cast<unsigned>(n_chunks)) * kBinTok + tid;
  const bool active = t < n_tokens;
  const int c0 = kLevels * j;
  const int width = min(kRows - c0, kGCols);
  uint32_t lw[20];
  load_token_levels(lw, levels, t, active, kAny, n_bins, n_levels);
  // The token's levels from bin j on, times 8 (byte offsets of a double), as
  // a byte string whose byte q is bin j + q (zeros past bin 79): each thread
  // writes its 80 bytes (+ a zero word) to LDS and reads them back shifted by
  // j bytes (j is the same for the whole workgroup).  Only the thread itself
  // reads its words.
  typedef uint32_t __attribute__((may_alias)) lds_word_t;   // the words share the fp64 buffer
  lds_word_t* lv_s = reinterpret_cast<lds_word_t*>(g_s) + tid * 21;   // 84 KB of the 131 KB
#pragma unroll
  for (int i = 0; i < 20; ++i) lv_s[i] = lw[i] << 3;
  lv_s[20] = 0u;
  const int jw = j >> 2, jb = j & 3;
  uint32_t rot[20];
  {
    uint32_t lo = lv_s[jw];
#pragma unroll
    for (int i = 0; i < 20; ++i) {
      // words past the thread's 21 read as zero (the read itself stays inside
      // the 84 KB region)
      const uint32_t hi = jw + i + 1 <= 20 ? lv_s[jw + i + 1] : 0u;
      rot[i] = __builtin_amdgcn_alignbyte(hi, lo, static_cast<uint32_t>(jb));
      lo = hi;
    }
  }
  __syncthreads();   // every thread has its levels before G overwrites them
  // zeros for the lookups of up to 9 bins past bin 79 (the QMAX groups below)
  stage_gram_part(g_s, gram, j, c0, width, tid, min(kGCols, width + 160));
  __syncthreads();
  const char* g_b = reinterpret_cast<const char*>(g_s);
  const uint32_t lj8 = rot[0] & 0xFFu;   // 8 L_j
  const char* row = g_b + lj8 * kGPitch;
  const double diag = *reinterpret_cast<const double*>(row + lj8);
  double off = 0.0;
  switch (j / 10) {   // uniform over the workgroup
    case 0: part1_terms<79>(off, row, rot); break;
    case 1: part1_terms<69>(off, row, rot); break;
    case 2: part1_terms<59>(off, row, rot); break;
    case 3: part1_terms<49>(off, row, rot); break;
    case 4: part1_terms<39>(off, row, rot); break;
    case 5: part1_terms<29>(off, row, rot); break;
    case 6: part1_terms<19>(off, row, rot); break;
    default: part1_terms<9>(off, row, rot); break;
  }
  if (j < kMels - 64) {
    // bins j + 64 .. 79 (j <= 15): columns 16 j + 1024 .. 1279, then zeros up
    // to relative column 256 for the terms past bin 79
    __syncthreads();
    stage_gram_part(g_s, gram, j, c0 + kGCols, kRows - c0 - kGCols, tid, 256);
    __syncthreads();
    gram_terms<64, 79>(off, row, rot, kGCols);
  }
  if (active) part[static_cast<int64_t>(j) * n_tokens + t] = make_double2(diag, off);
}

__global__ void __launch_bounds__(256)
rms_total_kernel(const double2* __restrict__ part, int64_t n_tokens, int d_model, float eps, float* __restrict__ scale) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_tokens) return;
  double total = 0.0;
  for (int j = 0; j < kMels; ++j) {
    const double2 v = part[static_cast<int64_t>(j) * n_tokens + t];
    total += v.x;
    total += 2.0 * v.y;
  }
  const double ms = total / static_cast<double>(d_model);
  scale[t] = static_cast<float>(1.0 / sqrt(ms + static_cast<double>(eps)));
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

hipError_t launch_embed(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                        const uint16_t* table, int d_model, const float* rms_weight, const float* rms_scale,
                        void* out, bool out_f32, int64_t out_row_stride, const int64_t* out_rows,
                        hipStream_t stream, float* sums_out) {
  if (n_tokens <= 0) return hipSuccess;
  const int n_strips = d_model / kStrip;
  const int64_t tblocks = (n_tokens + kEmbThreads - 1) / kEmbThreads;
  // Strips per workgroup: more strips amortise the per-workgroup set-up (48 -
  // eight groups of 6144 columns, one per XCD - then 24 and 16 were the
  // fastest counts measured on a 1.5M-token batch with the XCD-ordered
  // groups), but a small batch then launches too few workgroups to fill the
  // chip.  One workgroup fits per CU (LDS), so the cost of a count g is about
  // rounds-of-256-workgroups x g; take the largest g within 5% of the
  // cheapest.
  static const int kCounts[] = {48, 24, 16, 12, 8, 6, 4, 3, 2, 1};
  constexpr int kNCounts = sizeof(kCounts) / sizeof(kCounts[0]);
  int64_t cost[kNCounts];
  int64_t min_cost = -1;
  for (int i = 0; i < kNCounts; ++i) {
    const int g = kCounts[i];
    const int64_t wgs = tblocks * ((n_strips + g - 1) / g);
    cost[i] = ((wgs + 255) / 256) * g;
    if (min_cost < 0 || cost[i] < min_cost) min_cost = cost[i];
  }
  int best = 1;
  for (int i = 0; i < kNCounts; ++i) {
    if (cost[i] * 100 <= min_cost * 105) {
      best = kCounts[i];
      break;
    }
  }
  const int n_groups = (n_strips + best - 1) / best;
  const int64_t blocks = tblocks * n_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
#define DMEL_EMBED_LAUNCH(ANY, SUMS)                                                                          \
  hipLaunchKernelGGL((embed_kernel<ANY, SUMS>), dim3(static_cast<unsigned>(blocks)), dim3(kEmbThreads), 0, stream, \
                     levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, out,              \
                     out_f32 ? 1 : 0, out_row_stride, out_rows, n_groups, n_strips, best, sums_out)
  const bool released = n_bins == kMels && n_levels == kLevels;
  if (released && sums_out == nullptr) DMEL_EMBED_LAUNCH(false, false);
  else if (released) DMEL_EMBED_LAUNCH(false, true);
  else if (sums_out == nullptr) DMEL_EMBED_LAUNCH(true, false);
  else DMEL_EMBED_LAUNCH(true, true);
#undef DMEL_EMBED_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gram(const uint16_t* table, int n_bins, int n_levels, int d_model, double* gram,
                       hipStream_t stream) {
  const int pairs = kGTiles * (kGTiles + 1) / 2;
  hipLaunchKernelGGL(gram_kernel, dim3(pairs), dim3(256), 0, stream, table, n_bins, n_levels, d_model, gram);
  return hipGetLastError();
}

size_t rms_partials_bytes(int64_t n_tokens) {
  return n_tokens > 0 && n_tokens <= kRmsDirectMax ? static_cast<size_t>(n_tokens) * kMels * sizeof(double2) : 0;
}

hipError_t launch_rms_scale(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                            const double* gram, int d_model, float eps, float* scale, void* partials,
                            hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  if (n_tokens <= kRmsDirectMax && partials != nullptr) {
    const int n_chunks = static_cast<int>((n_tokens + kBinTok - 1) / kBinTok);
    auto* part = static_cast<double2*>(partials);
    const dim3 grid(static_cast<unsigned>(n_chunks * kMels));
    if (n_bins == kMels && n_levels == kLevels) {
      hipLaunchKernelGGL(rms_bin_partials_kernel<false>, grid, dim3(kBinTok), 0, stream, levels, n_tokens, n_bins,
                         n_levels, gram, n_chunks, part);
    } else {
      hipLaunchKernelGGL(rms_bin_partials_kernel<true>, grid, dim3(kBinTok), 0, stream, levels, n_tokens, n_bins,
                         n_levels, gram, n_chunks, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rms_total_kernel, dim3(static_cast<unsigned>((n_tokens + 255) / 256)), dim3(256), 0, stream,
                       part, n_tokens, d_model, eps, scale);
    return hipGetLastError();
  }
  if (n_tokens <= kRmsDirectMax) {
    const int64_t blocks = (n_tokens + kDirTok - 1) / kDirTok;
    hipLaunchKernelGGL(rms_scale_direct_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kDirThreads), 0, stream,
                       levels, n_tokens, n_bins, n_levels, gram, d_model, eps, scale);
    return hipGetLastError();
  }
  const int64_t blocks = (n_tokens + kScaleBlock - 1) / kScaleBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rms_scale_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kScaleThreads), 0, stream,
                     levels, n_tokens, n_bins, n_levels, gram, d_model, eps, scale);
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
