// Device building blocks of the bag-of-bins sum, shared by the forward
// embedding kernel and the backward kernels that recompute the forward sum:
// the LDS staging of a 1280 x 16 fp32 slice of the table (80-byte rows) and
// the per-lane sequential fp32 sum over the 80 bins (see embed.hip).
#pragma once

#include "internal.h"

namespace dmel {
namespace {

constexpr int kEmbThreads = 1024;   // tokens per workgroup
constexpr int kStrip = 16;          // fp32 columns per strip
constexpr int kPitch = 20;          // floats per LDS row (80 bytes)

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16 and packed (lo, hi): one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t v;
  v[0] = lo;
  v[1] = hi;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Levels of token t for any layout, as 80 bytes (bin j in byte j % 4 of word
// j / 4): read byte by byte from a [n, n_bins] array, clamped to vmax; bins
// past n_bins read as level 0.
__device__ __forceinline__ void load_levels_any(uint32_t (&lv)[20], const uint8_t* levels, int64_t t, int n_bins,
                                                uint32_t vmax) {
  const uint8_t* p = levels + t * n_bins;
#pragma unroll
  for (int i = 0; i < 20; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = 4 * i + b;
      if (j < n_bins) w |= min(static_cast<uint32_t>(p[j]), vmax) << (8 * b);
    }
    lv[i] = w;
  }
}

// Clamp each byte of x to at most 15.
__device__ __forceinline__ uint32_t clamp_levels(uint32_t x) {
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;              // nonzero nibble where byte >= 16
  const uint32_t big = ((hi + 0x0F0F0F0Fu) & 0x10101010u);  // bit 4 of each byte >= 16
  const uint32_t mask = (big >> 4) * 0xFFu;                 // 0xFF in those bytes
  return (x & ~mask) | (0x0F0F0F0Fu & mask);
}

// Adds bins J0..J1-1 of this lane's token into acc (bin 0 initialises it).
// Software pipeline: the four 16-byte reads of bin j + 1 are issued, then an
// empty asm that "modifies" the accumulators and clobbers memory pins them
// ahead of the adds of bin j, so a wave always has the next bin's reads in
// flight while it adds the current one, and no more than that (hoisting all
// the reads would exhaust the registers).  For J0 > 0 the LDS addresses are
// taken from a base rebased to bin J0 through an opaque register, so that every
// read of the range keeps its bin offset in the 16-bit immediate field (the
// offsets of bins past 51 would overflow it, and each read would then cost two
// extra VALU ops).
template <int J0, int J1>
__device__ __forceinline__ void add_bins(float (&acc)[kStrip], const float* tab, const uint32_t (&offs)[40]) {
  uint32_t rebase = J0 * kLevels * kPitch;
  if (J0 > 0) asm volatile("" : "+v"(rebase));
  const float* base = tab + rebase;
  auto row = [&](int j) {
    const uint32_t o = (offs[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    return reinterpret_cast<const float4*>(reinterpret_cast<const char*>(base) + o);
  };
  float4 cur[4];
  {
    const float4* r = row(J0);
#pragma unroll
    for (int q = 0; q < 4; ++q) cur[q] = r[q];
  }
#pragma unroll
  for (int j = J0; j < J1; ++j) {
    float4 nxt[4];
    if (j + 1 < J1) {
      const float4* r = row(j + 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) nxt[q] = r[q];
    }
    if (j == 0) {
      // the sum starts from the first row itself (not from +0)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[4 * q + 0] = cur[q].x;
        acc[4 * q + 1] = cur[q].y;
        acc[4 * q + 2] = cur[q].z;
        acc[4 * q + 3] = cur[q].w;
      }
    } else {
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                   "+v"(acc[6]), "+v"(acc[7]), "+v"(acc[8]), "+v"(acc[9]), "+v"(acc[10]), "+v"(acc[11]),
                   "+v"(acc[12]), "+v"(acc[13]), "+v"(acc[14]), "+v"(acc[15])::"memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[4 * q + 0] += cur[q].x;
        acc[4 * q + 1] += cur[q].y;
        acc[4 * q + 2] += cur[q].z;
        acc[4 * q + 3] += cur[q].w;
      }
    }
    if (j + 1 < J1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
    }
  }
}

constexpr int kHalfRows = kRows / 2;                   // bins 0..39 | bins 40..79
constexpr int kStageItems = kHalfRows * 2;             // 16-byte chunks per half strip (1280)
constexpr int kStagePer = (kStageItems + kEmbThreads - 1) / kEmbThreads;  // 2

// Global -> registers: this thread's chunks of half `half` of the strip at
// col0.  kAny: LDS row 16 b + l takes table row n_levels * b + l, or -0.0
// where (b, l) is outside the n_bins x n_levels layout.
template <bool kAny>
__device__ __forceinline__ void stage_load(uint4 (&st)[kStagePer], const uint16_t* table, int d_model, int col0,
                                           int half, int tid, int n_bins, int n_levels) {
#pragma unroll
  for (int k = 0; k < kStagePer; ++k) {
    const int i = tid + k * kEmbThreads;
    if (i < kStageItems) {
      const int row = half * kHalfRows + (i >> 1);
      int src = row;
      bool real = true;
      if (kAny) {
        const int b = row >> 4, l = row & 15;
        real = b < n_bins && l < n_levels;
        src = b * n_levels + l;
      }
      if (real) {
        st[k] = *reinterpret_cast<const uint4*>(table + static_cast<int64_t>(src) * d_model + col0 + 8 * (i & 1));
      } else {
        st[k] = make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u);  // bf16 -0.0
      }
    }
  }
}

// Registers -> LDS as fp32 (80-byte rows).
__device__ __forceinline__ void stage_store(float* tab, const uint4 (&st)[kStagePer], int half, int tid) {
#pragma unroll
  for (int k = 0; k < kStagePer; ++k) {
    const int i = tid + k * kEmbThreads;
    if (i < kStageItems) {
      const int row = half * kHalfRows + (i >> 1);
      const uint4 v = st[k];
      float4* d = reinterpret_cast<float4*>(tab + row * kPitch + 8 * (i & 1));
      d[0] = make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                         bf16_to_f32(v.y >> 16));
      d[1] = make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                         bf16_to_f32(v.w >> 16));
    }
  }
}


// Levels of token t -> the packed per-bin LDS row offsets add_bins reads (the
// same prologue as embed_kernel; bins past n_bins read level 0).
template <bool kAny>
__device__ __forceinline__ void token_offsets(uint32_t (&offs)[40], const uint8_t* levels, int64_t t, bool active,
                                              int n_bins, int n_levels) {
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
#pragma unroll
  for (int i = 0; i < 40; ++i) {
    const int j0 = 2 * i, j1 = 2 * i + 1;
    const uint32_t L0 = (lv[j0 >> 2] >> (8 * (j0 & 3))) & 0xFFu;
    const uint32_t L1 = (lv[j1 >> 2] >> (8 * (j1 & 3))) & 0xFFu;
    const uint32_t o0 = (kLevels * (j0 % 40) + L0) * kPitch * 4;
    const uint32_t o1 = (kLevels * (j1 % 40) + L1) * kPitch * 4;
    offs[i] = o0 | (o1 << 16);
  }
}

// The forward sum of strips [s_first, s_end) for the workgroup's tokens, with
// the staging and bin order of embed_kernel: epi(col0, acc) receives the exact
// fp32 sums of columns col0 .. col0 + 15 of this thread's token.  Contains
// barriers: every thread of the workgroup calls it; epi may use barriers too.
// pre(col0) runs at the start of each strip, before its adds (for reads the
// epilogue of the strip will use).
template <bool kAny, typename Pre, typename Epi>
__device__ __forceinline__ void sum_strips(float* tab, const uint16_t* table, int d_model, int s_first, int s_end,
                                           int tid, int n_bins, int n_levels, uint32_t (&offs)[40], Pre&& pre,
                                           Epi&& epi) {
  uint4 st[kStagePer];
  stage_load<kAny>(st, table, d_model, s_first * kStrip, 0, tid, n_bins, n_levels);
  stage_store(tab, st, 0, tid);
  __syncthreads();
  for (int strip = s_first; strip < s_end; ++strip) {
    const int col0 = strip * kStrip;
#pragma unroll
    for (int i = 0; i < 40; ++i) asm volatile("" : "+v"(offs[i]));
    stage_load<kAny>(st, table, d_model, col0, 1, tid, n_bins, n_levels);
    pre(col0);
    float acc[kStrip];
    add_bins<0, kMels / 2>(acc, tab, offs);
    stage_store(tab, st, 1, tid);
    __syncthreads();
    const bool more = strip + 1 < s_end;
    if (more) stage_load<kAny>(st, table, d_model, col0 + kStrip, 0, tid, n_bins, n_levels);
    if (!kAny || n_bins > kMels / 2) add_bins<kMels / 2, kMels>(acc, tab, offs);
    epi(col0, acc);
    if (more) stage_store(tab, st, 0, tid);
    __syncthreads();
  }
}

}  // namespace
}  // namespace dmel
