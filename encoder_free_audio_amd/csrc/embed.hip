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

// kAny = false: the released layout (levels [n, 80], 16-byte aligned, table
// [1280, d]); true: any n_bins <= 80, n_levels <= 16 (see the top of the file).
template <bool kAny>
__global__ void __launch_bounds__(kEmbThreads)
embed_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
             const uint16_t* __restrict__ table, int d_model, const float* __restrict__ rms_weight,
             const float* __restrict__ rms_scale, void* __restrict__ out, int out_f32, int64_t out_row_stride,
             const int64_t* __restrict__ out_rows, int n_groups, int n_strips, int strips_per_group) {
  __shared__ float4 tab4[kRows * kPitch / 4];
  float* tab = reinterpret_cast<float*>(tab4);

  const int tid = threadIdx.x;
  const int grp = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_groups));
  const int64_t tb = blockIdx.x / static_cast<unsigned>(n_groups);
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
      if (rms_weight != nullptr) {
#pragma unroll
        for (int c = 0; c < kStrip; ++c) acc[c] = (acc[c] * scale) * rms_weight[col0 + c];
      }
      // Plain stores: the 16 strips of a workgroup complete each token's
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
// Gram matrix G = E E^T (fp64 accumulation of exact bf16 products, stored
// fp32).  One workgroup per 16 x 16 block (bin j rows x bin j' rows), j <= j'.
// G is indexed in the 80 x 16 row space (16 * bin + level) for every layout;
// rows outside the n_bins x n_levels layout are zero.
// ---------------------------------------------------------------------------
constexpr int kGramChunk = 256;

__global__ void __launch_bounds__(256)
gram_kernel(const uint16_t* __restrict__ table, int n_bins, int n_levels, int d_model, float* __restrict__ gram) {
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
      if (c < width && r < n_levels) {
        if (j < n_bins) va = bf16_to_f32(table[static_cast<int64_t>(n_levels * j + r) * d_model + c0 + c]);
        if (jp < n_bins) vb = bf16_to_f32(table[static_cast<int64_t>(n_levels * jp + r) * d_model + c0 + c]);
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
// + 2 sum_{j < j'} G[r_j][r_j'].  A workgroup owns 512 tokens (one per
// thread).  For each bin j the 16 rows 16j..16j+15 of the upper triangle
// (columns 16j..1279) are staged in LDS; the thread then adds the diagonal
// term and the 79 - j terms of its token.  The token's 80 levels live in
// registers as a byte string that is shifted by one byte per bin, so that the
// level of bin j + q is always byte q: every index in the unrolled inner loop
// is static, and the 79 - j lookups of a bin are independent loads.  Partial
// sums per bin are fp32, the total fp64.
// ---------------------------------------------------------------------------
constexpr int kScaleThreads = 1024;
constexpr int kScaleTok = 2;                            // tokens per thread
constexpr int kScaleBlock = kScaleThreads * kScaleTok;  // tokens per workgroup
constexpr int kGPitch = kRows + 17;  // staged row pitch (floats): spreads the 16 rows over the banks

// Stages rows c0 .. c0 + 15 of G, columns c0 .. 1279, at g_s[r * kGPitch +
// c - c0]: a workgroup of 1024 threads gives each row 64 threads, which read
// 4 columns per step (one 16-byte read when G is 16-byte aligned), with no
// index division.
__device__ __forceinline__ void stage_gram_rows(float* g_s, const float* __restrict__ gram, int c0, int tid) {
  const int r = tid >> 6;  // 0..15
  const int q = tid & 63;
  const float* src = gram + static_cast<int64_t>(c0 + r) * kRows + c0;
  float* dst = g_s + r * kGPitch;
  const int width = kRows - c0;  // a multiple of 16
  const bool vec = (reinterpret_cast<uintptr_t>(gram) & 15) == 0;
  for (int c = 4 * q; c < width; c += 256) {
    float4 v;
    if (vec) {
      v = *reinterpret_cast<const float4*>(src + c);
    } else {
      v = make_float4(src[c], src[c + 1], src[c + 2], src[c + 3]);
    }
    dst[c] = v.x;
    dst[c + 1] = v.y;
    dst[c + 2] = v.z;
    dst[c + 3] = v.w;
  }
}

// Off-diagonal terms q = 1..qlim of one staged row block (q = bin offset from
// the block's bin).  QMAX bounds qlim for the range of bins the caller is in,
// so the loop is fully unrolled with static register indices; terms past
// qlim are read (inside the staged row pitch) but replaced by 0 in a select.
template <int QMAX>
__device__ __forceinline__ void row_terms(float (&off)[kScaleTok], const float* const (&row)[kScaleTok],
                                          const uint32_t (&rot)[kScaleTok][20], int qlim) {
#pragma unroll
  for (int q = 1; q <= QMAX; ++q) {
    const bool use = q <= qlim;
#pragma unroll
    for (int k = 0; k < kScaleTok; ++k) {
      const float v = row[k][kLevels * q + ((rot[k][q >> 2] >> (8 * (q & 3))) & 0xFFu)];
      off[k] += use ? v : 0.0f;
    }
  }
}

__global__ void __launch_bounds__(kScaleThreads)
rms_scale_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
                 const float* __restrict__ gram, int d_model, float eps, float* __restrict__ scale) {
  __shared__ float g_s[16 * kGPitch];  // 83 KB
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kScaleBlock + tid;
  uint32_t rot[kScaleTok][20];
  double total[kScaleTok];
#pragma unroll
  for (int k = 0; k < kScaleTok; ++k) {
    const int64_t t = t0 + static_cast<int64_t>(k) * kScaleThreads;
    total[k] = 0.0;
    if (t < n_tokens && (n_bins != kMels || n_levels != kLevels)) {
      load_levels_any(rot[k], levels, t, n_bins, static_cast<uint32_t>(n_levels - 1));
    } else if (t < n_tokens) {
      const uint4* p = reinterpret_cast<const uint4*>(levels + t * kMels);
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint4 q = p[i];
        rot[k][4 * i + 0] = clamp_levels(q.x);
        rot[k][4 * i + 1] = clamp_levels(q.y);
        rot[k][4 * i + 2] = clamp_levels(q.z);
        rot[k][4 * i + 3] = clamp_levels(q.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 20; ++i) rot[k][i] = 0;
    }
  }
  for (int j = 0; j < kMels; ++j) {
    const int c0 = kLevels * j;
    __syncthreads();
    stage_gram_rows(g_s, gram, c0, tid);
    __syncthreads();
    // rot byte q = level of bin j + q; staged column of bin j + q, level L: 16 q + L
    const float* row[kScaleTok];
    float off[kScaleTok];
#pragma unroll
    for (int k = 0; k < kScaleTok; ++k) {
      const uint32_t lj = rot[k][0] & 0xFFu;
      row[k] = g_s + lj * kGPitch;
      off[k] = 0.0f;
      total[k] += static_cast<double>(row[k][lj]);  // diagonal term
    }
    const int qlim = kMels - 1 - j;
    switch (j / 10) {
      case 0: row_terms<79>(off, row, rot, qlim); break;
      case 1: row_terms<69>(off, row, rot, qlim); break;
      case 2: row_terms<59>(off, row, rot, qlim); break;
      case 3: row_terms<49>(off, row, rot, qlim); break;
      case 4: row_terms<39>(off, row, rot, qlim); break;
      case 5: row_terms<29>(off, row, rot, qlim); break;
      case 6: row_terms<19>(off, row, rot, qlim); break;
      default: row_terms<9>(off, row, rot, qlim); break;
    }
#pragma unroll
    for (int k = 0; k < kScaleTok; ++k) {
      total[k] += 2.0 * static_cast<double>(off[k]);
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

// Same scale for small batches, without staging: one thread per (token, bin j)
// reads row r_j of G straight from memory (L2-resident) and forms the bin's
// fp32 diagonal and off-diagonal sums exactly as rms_scale_kernel does (same
// terms, same order); the token's total is then summed in bin order in fp64 by
// one thread.  The arithmetic is identical to rms_scale_kernel's, so a token
// gets the same scale whichever kernel runs, whatever the batch size.
constexpr int kDirTok = 4;                  // tokens per workgroup
constexpr int kDirThreads = kDirTok * kMels;  // 320

__global__ void __launch_bounds__(kDirThreads)
rms_scale_direct_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
                        const float* __restrict__ gram, int d_model, float eps, float* __restrict__ scale) {
  __shared__ __attribute__((aligned(16))) uint8_t lv_s[kDirTok][kMels];
  __shared__ float d_s[kDirTok][kMels];
  __shared__ float o_s[kDirTok][kMels];
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
    const float* row = gram + static_cast<int64_t>(rj) * kRows;
    const float diag = row[rj];
    // all lookups are issued at once (their addresses are independent) and
    // added in bin order; the terms of bins jp <= j are +0.0, which leave the
    // sum at +0.0 until its first real term (a sum that starts at +0.0 never
    // becomes -0.0), exactly as the staged kernel's masked terms
    uint32_t lw[20];
#pragma unroll
    for (int i = 0; i < 20; ++i) lw[i] = reinterpret_cast<const uint32_t*>(lv_s[tok])[i];
    float v[kMels];
#pragma unroll
    for (int jp = 0; jp < kMels; ++jp) {
      const uint32_t L = (lw[jp >> 2] >> (8 * (jp & 3))) & 0xFFu;
      v[jp] = jp > j ? row[kLevels * jp + L] : 0.0f;
    }
    float off = 0.0f;
#pragma unroll
    for (int jp = 0; jp < kMels; ++jp) off += v[jp];
    d_s[tok][j] = diag;
    o_s[tok][j] = off;
  }
  __syncthreads();
  if (active && j == 0) {
    double total = 0.0;
#pragma unroll 16
    for (int jj = 0; jj < kMels; ++jj) {
      total += static_cast<double>(d_s[tok][jj]);
      total += 2.0 * static_cast<double>(o_s[tok][jj]);
    }
    const double ms = total / static_cast<double>(d_model);
    scale[t] = static_cast<float>(1.0 / sqrt(ms + static_cast<double>(eps)));
  }
}

// Same scale for small batches with a workspace, bin-parallel: a workgroup
// takes one bin j and 1024 tokens (one per thread), stages the 16 rows of bin
// j of the upper triangle of G in LDS (as rms_scale_kernel does) and writes
// each token's diagonal term and fp32 off-diagonal sum of bin j (same terms,
// same order) to part[j][token]; rms_total_kernel then adds the 80 bins of
// each token in bin order in fp64.  Identical arithmetic again, so the scale
// does not depend on the kernel that computed it.  The token's levels stay in
// registers as 80 bytes; the lookups run over a static bin index jp = 0..79
// (terms of bins jp <= j are +0.0, which leave the sum at +0.0 until its first
// real term: a sum that starts at +0.0 never becomes -0.0), so every byte
// index is static and all lookups are independent.
constexpr int kBinTok = 1024;
static_assert(kBinTok == 1024 && kScaleThreads == 1024, "stage_gram_rows gives each of 16 rows 64 threads");

template <bool kAny>
__global__ void __launch_bounds__(kBinTok)
rms_bin_partials_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels,
                        const float* __restrict__ gram, int n_chunks, float2* __restrict__ part) {
  __shared__ float g_s[16 * kGPitch];              // 83 KB
  const int tid = threadIdx.x;
  const int j = static_cast<int>(blockIdx.x / static_cast<unsigned>(n_chunks));  // heavy (small) bins first
  const int64_t t = static_cast<int64_t>(blockIdx.x % static_cast<unsigned>(n_chunks)) * kBinTok + tid;
  const bool active = t < n_tokens;
  const int c0 = kLevels * j;
  stage_gram_rows(g_s, gram, c0, tid);
  uint32_t lw[20];
  if (active && kAny) {
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
  __syncthreads();
  if (!active) return;
  uint32_t lj = 0;
#pragma unroll
  for (int jp = 0; jp < kMels; ++jp) lj = jp == j ? (lw[jp >> 2] >> (8 * (jp & 3))) & 0xFFu : lj;
  const float* row = g_s + lj * kGPitch - c0;   // row[16 jp + L] = G[16 j + lj][16 jp + L]
  float v[kMels];
#pragma unroll
  for (int jp = 0; jp < kMels; ++jp) {
    const uint32_t L = (lw[jp >> 2] >> (8 * (jp & 3))) & 0xFFu;
    // (the address stays inside the staged rows for every jp)
    const float g = row[jp > j ? kLevels * jp + static_cast<int>(L) : c0];
    v[jp] = jp > j ? g : 0.0f;
  }
  float off = 0.0f;
#pragma unroll
  for (int jp = 0; jp < kMels; ++jp) off += v[jp];
  part[static_cast<int64_t>(j) * n_tokens + t] = make_float2(row[c0 + lj], off);
}

__global__ void __launch_bounds__(256)
rms_total_kernel(const float2* __restrict__ part, int64_t n_tokens, int d_model, float eps, float* __restrict__ scale) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n_tokens) return;
  double total = 0.0;
#pragma unroll 16
  for (int j = 0; j < kMels; ++j) {
    const float2 v = part[static_cast<int64_t>(j) * n_tokens + t];
    total += static_cast<double>(v.x);
    total += 2.0 * static_cast<double>(v.y);
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
                        hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int n_strips = d_model / kStrip;
  const int64_t tblocks = (n_tokens + kEmbThreads - 1) / kEmbThreads;
  // Strips per workgroup: more strips amortise the per-workgroup set-up (16 was
  // the fastest count measured on a 1.5M-token batch), but a small batch then
  // launches too few workgroups to fill the chip.  One workgroup fits per CU
  // (LDS), so the cost of a count g is about rounds-of-256-workgroups x g; take
  // the largest g within 5% of the cheapest.
  static const int kCounts[] = {16, 12, 8, 6, 4, 3, 2, 1};
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
  if (n_bins == kMels && n_levels == kLevels) {
    hipLaunchKernelGGL(embed_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kEmbThreads), 0, stream,
                       levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, out,
                       out_f32 ? 1 : 0, out_row_stride, out_rows, n_groups, n_strips, best);
  } else {
    hipLaunchKernelGGL(embed_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kEmbThreads), 0, stream,
                       levels, n_tokens, n_bins, n_levels, table, d_model, rms_weight, rms_scale, out,
                       out_f32 ? 1 : 0, out_row_stride, out_rows, n_groups, n_strips, best);
  }
  return hipGetLastError();
}

hipError_t launch_gram(const uint16_t* table, int n_bins, int n_levels, int d_model, float* gram,
                       hipStream_t stream) {
  const int pairs = kMels * (kMels + 1) / 2;
  hipLaunchKernelGGL(gram_kernel, dim3(pairs), dim3(256), 0, stream, table, n_bins, n_levels, d_model, gram);
  return hipGetLastError();
}

size_t rms_partials_bytes(int64_t n_tokens) {
  return n_tokens > 0 && n_tokens <= kRmsDirectMax ? static_cast<size_t>(n_tokens) * kMels * sizeof(float2) : 0;
}

hipError_t launch_rms_scale(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels,
                            const float* gram, int d_model, float eps, float* scale, void* partials,
                            hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  if (n_tokens <= kRmsDirectMax && partials != nullptr) {
    const int n_chunks = static_cast<int>((n_tokens + kBinTok - 1) / kBinTok);
    auto* part = static_cast<float2*>(partials);
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
