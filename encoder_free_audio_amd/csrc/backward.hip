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
//  * bucket_kernel - for each chunk of 128 tokens and each bin, a stable
//    counting sort of the chunk's tokens by level (one wave per (chunk, bin),
//    64 tokens per ballot): the LDS byte addresses of the tokens' gradient
//    rows, grouped by level, each group padded to a multiple of four entries
//    with the address of a row of -0.0, and the 17 group starts (32-bit
//    words, so that the scatter reads them with scalar loads).
//  * scatter_kernel - a workgroup owns 8 bins (one wave each) and 256
//    columns (4 per lane) and walks every chunk of the batch in order; per
//    chunk it stages the 128 x 256 gradient tile in LDS, then each wave walks
//    its bin's level groups in token order and adds the tile rows into
//    16 x 4 accumulators in registers (one ds_read_b128 and four v_add_f32
//    per token); the group lists are uniform, so they come through scalar
//    loads.  Every row's sum is thus one chain in token order across the
//    whole batch.  Workgroups that share a tile (the bin groups of one
//    strip) are placed on the same XCD.
//  * rms_dot_kernel / rms_ds_kernel - the RMSNorm backward: the forward sum
//    is recomputed exactly as embed_kernel computes it (embed_core.h); the
//    first pass forms sum_c w_c dy_c s_c per token and per-workgroup partial
//    sums of dy * s * r per column, the second pass writes ds.
#include <algorithm>

#include "embed_core.h"

namespace dmel {
namespace {

constexpr int kChunk = 128;                  // tokens per staged tile
constexpr int kRounds = kChunk / 64;         // waves of 64 tokens per chunk in the level sort
constexpr int kBwdCols = 256;                // columns per workgroup (4 per lane)
constexpr int kBwdBins = 8;                  // bins per workgroup (one per wave)
constexpr int kBwdThreads = 64 * kBwdBins;   // 512
constexpr int kTileItems = kChunk * kBwdCols / 4 / kBwdThreads;  // float4 per thread per tile (16)
constexpr int kListPitch = kChunk + 3 * 16;  // entries per (chunk, bin): groups padded to multiples of 4
constexpr int kOffPitch = 17;                // group starts per (chunk, bin): 16 levels + end
// LDS byte address of the tile row that holds -0.0 (after the kChunk token
// rows): adding it is an exact no-op, so level groups are padded with it to
// whole groups of four and the scatter needs no remainder loop.
constexpr uint32_t kNegZeroRow = kChunk * kBwdCols * 4;

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
bucket_kernel(const uint8_t* __restrict__ levels, int64_t n_tokens, int n_bins, int n_levels, int64_t n_pairs,
              uint32_t* __restrict__ lists, uint32_t* __restrict__ starts) {
  const int lane = threadIdx.x & 63;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= n_pairs) return;  // whole wave; no barriers in this kernel
  const int64_t chunk = pair / n_bins;
  const int j = static_cast<int>(pair - chunk * n_bins);
  uint32_t L[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t t = chunk * kChunk + r * 64 + lane;
    L[r] = 0xFFu;  // no group
    if (t < n_tokens) {
      const uint32_t v = levels[t * n_bins + j];
      L[r] = v < static_cast<uint32_t>(n_levels - 1) ? v : static_cast<uint32_t>(n_levels - 1);
    }
  }
  uint32_t* lst = lists + pair * kListPitch;
  uint32_t* st = starts + pair * kOffPitch;
  uint32_t base = 0;
  for (int l = 0; l < n_levels; ++l) {
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const uint64_t m = __ballot(L[r] == static_cast<uint32_t>(l));
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      if (L[r] == static_cast<uint32_t>(l)) lst[base + cnt + rank] = static_cast<uint32_t>((r * 64 + lane) * kBwdCols * 4);
      cnt += static_cast<uint32_t>(__popcll(m));
    }
    const uint32_t padded = (cnt + 3u) & ~3u;
    if (static_cast<uint32_t>(lane) < padded - cnt) lst[base + cnt + lane] = kNegZeroRow;
    if (lane == 0) st[l] = base;
    base += padded;
  }
  if (lane == 0) {
    for (int l = n_levels; l <= 16; ++l) st[l] = base;
  }
}

// ---------------------------------------------------------------------------
template <bool kBf16>
__device__ __forceinline__ void tile_load(float4 (&r)[kTileItems], const void* g, int64_t n_tokens, int d_model,
                                          int64_t t0, int c_strip, int tid) {
  // kChunk rows x 256 columns; item i = row * 64 + (4-column group)
#pragma unroll
  for (int k = 0; k < kTileItems; ++k) {
    const int i = tid + k * kBwdThreads;
    const int row = i >> 6, cg = i & 63;
    const int64_t t = t0 + row;
    const int c = c_strip + 4 * cg;
    r[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (t < n_tokens && c < d_model) {
      if (kBf16) {
        const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g) + t * d_model + c);
        r[k] = make_float4(bf16_to_f32(q.x & 0xFFFFu), bf16_to_f32(q.x >> 16), bf16_to_f32(q.y & 0xFFFFu),
                           bf16_to_f32(q.y >> 16));
      } else {
        r[k] = *reinterpret_cast<const float4*>(static_cast<const float*>(g) + t * d_model + c);
      }
    }
  }
}

__device__ __forceinline__ void tile_store(float4* tile, const float4 (&r)[kTileItems], int tid) {
#pragma unroll
  for (int k = 0; k < kTileItems; ++k) tile[tid + k * kBwdThreads] = r[k];
}

__device__ __forceinline__ void add4(float4& a, const float4& v) {
  a.x += v.x;
  a.y += v.y;
  a.z += v.z;
  a.w += v.w;
}

// Adds one chunk of this wave's bin: the list's groups of four entries in
// order (level l's groups, in token order, before level l + 1's), each into
// acc[l].  The scalar read of a group's entries is issued one group ahead, so
// that it is answered while the previous group's tile rows are read and each
// group waits once, for its own rows.
__device__ __forceinline__ void add_chunk(float4 (&acc)[16], const char* tile_lane, const uint32_t* __restrict__ lst,
                                          const uint32_t* __restrict__ st) {
  uint32_t bound[17];
#pragma unroll
  for (int l = 0; l <= 16; ++l) bound[l] = st[l];
  const int end = static_cast<int>(bound[16]);  // >= 4: a chunk holds at least one token
  uint4 an = *reinterpret_cast<const uint4*>(lst);
  int k = 0;
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    const int e = static_cast<int>(bound[l + 1]);
    for (; k < e; k += 4) {
      const uint4 a = an;
      // the next group's entries (the last group's again at the end: always
      // inside the list)
      an = *reinterpret_cast<const uint4*>(lst + (k + 4 < end ? k + 4 : end - 4));
      const float4 v0 = *reinterpret_cast<const float4*>(tile_lane + a.x);
      const float4 v1 = *reinterpret_cast<const float4*>(tile_lane + a.y);
      const float4 v2 = *reinterpret_cast<const float4*>(tile_lane + a.z);
      const float4 v3 = *reinterpret_cast<const float4*>(tile_lane + a.w);
      add4(acc[l], v0);
      add4(acc[l], v1);
      add4(acc[l], v2);
      add4(acc[l], v3);
    }
  }
}

// Workgroup (bin group, strip); see the file comment.  Writes
// out = acc (or fl32(out + acc) when accumulating), acc being each row's
// token-order sum over the whole batch.
template <bool kBf16>
__global__ void __launch_bounds__(kBwdThreads)
scatter_kernel(const void* __restrict__ g, int64_t n_tokens, int n_bins, int n_levels, int d_model,
               const uint32_t* __restrict__ lists, const uint32_t* __restrict__ starts, int64_t n_chunks,
               int n_groups, int n_strips, float* __restrict__ out, int accumulate) {
  __shared__ float4 tile[(kChunk + 1) * kBwdCols / 4];  // 128 KB of token rows + the -0.0 row
  // blockIdx -> (strip, bin group): workgroup b runs on XCD b % 8, and the
  // bin groups of one strip are 8 apart, so they share the strip's tiles in
  // that XCD's L2
  const int bid = static_cast<int>(blockIdx.x);
  const int local = bid >> 3;
  const int grp = local % n_groups;
  const int strip = (local / n_groups) * 8 + (bid & 7);
  if (strip >= n_strips) return;  // before any barrier: the whole workgroup leaves

  const int tid = threadIdx.x;
  // the wave index, made explicitly uniform so that the group lists come
  // through scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = grp * kBwdBins + wave;
  const bool bin_ok = j < n_bins;
  const int c_strip = strip * kBwdCols;
  const int c0 = c_strip + 4 * lane;

  float4 acc[16];
#pragma unroll
  for (int l = 0; l < 16; ++l) acc[l] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

  if (tid < kBwdCols / 4) tile[kChunk * kBwdCols / 4 + tid] = make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
  float4 r[kTileItems];
  tile_load<kBf16>(r, g, n_tokens, d_model, 0, c_strip, tid);
  const char* tile_lane = reinterpret_cast<const char*>(tile) + lane * 16;
  for (int64_t ch = 0; ch < n_chunks; ++ch) {
    tile_store(tile, r, tid);
    __syncthreads();
    if (ch + 1 < n_chunks) tile_load<kBf16>(r, g, n_tokens, d_model, (ch + 1) * kChunk, c_strip, tid);
    if (bin_ok) {
      const int64_t pair = ch * n_bins + j;
      add_chunk(acc, tile_lane, lists + pair * kListPitch, starts + pair * kOffPitch);
    }
    __syncthreads();  // the tile is overwritten next
  }

  if (!bin_ok || c0 >= d_model) return;
#pragma unroll
  for (int l = 0; l < 16; ++l) {
    if (l < n_levels) {
      const int64_t row = static_cast<int64_t>(j) * n_levels + l;
      float4* o = reinterpret_cast<float4*>(out + row * d_model + c0);
      float4 v = acc[l];
      if (accumulate) {
        v = *o;
        add4(v, acc[l]);
      }
      *o = v;
    }
  }
}

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
template <bool kDyBf16>
__device__ __forceinline__ void load_dy(float (&gr)[kStrip], const void* dy, int64_t t, int d_model, int col0,
                                        bool active) {
  if (!active) {
#pragma unroll
    for (int c = 0; c < kStrip; ++c) gr[c] = 0.0f;
    return;
  }
  if (kDyBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dy) + t * d_model + col0);
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      gr[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      gr[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(dy) + t * d_model + col0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = p[q];
      gr[4 * q] = v.x;
      gr[4 * q + 1] = v.y;
      gr[4 * q + 2] = v.z;
      gr[4 * q + 3] = v.w;
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
  sum_strips<kAny>(tab, table, d_model, s_first, s_end, tid, n_bins, n_levels, offs,
                   [&](int col0, float (&acc)[kStrip]) {
                     if (s_out != nullptr && active) {
                       float4* so = reinterpret_cast<float4*>(s_out + t * d_model + col0);
                       so[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
                       so[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
                       so[2] = make_float4(acc[8], acc[9], acc[10], acc[11]);
                       so[3] = make_float4(acc[12], acc[13], acc[14], acc[15]);
                     }
                     float gr[kStrip];
                     load_dy<kDyBf16>(gr, dy, t, d_model, col0, active);
                     float q[kStrip];
#pragma unroll
                     for (int c = 0; c < kStrip; ++c) {
                       dot = fmaf(rms_weight[col0 + c] * gr[c], acc[c], dot);
                       q[c] = (gr[c] * acc[c]) * r;
                     }
                     const float qs = wave_sum16(q, tid & 63);
                     if ((tid & 3) == 0) red[tid >> 6][(tid >> 2) & 15] = qs;
                     __syncthreads();
                     if (tid < kStrip) {
                       float v = 0.0f;
#pragma unroll
                       for (int w = 0; w < kEmbThreads / 64; ++w) v += red[w][tid];
                       dw_part[tb * d_model + col0 + tid] = v;
                     }
                   });
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
  sum_strips<kAny>(tab, table, d_model, s_first, s_end, tid, n_bins, n_levels, offs,
                   [&](int col0, float (&acc)[kStrip]) {
                     if (!active) return;
                     float gr[kStrip];
                     load_dy<kDyBf16>(gr, dy, t, d_model, col0, true);
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

size_t bwd_layout(int64_t n_tokens, int n_bins, size_t* off_starts) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t n_chunks = static_cast<size_t>((n_tokens + kChunk - 1) / kChunk);
  const size_t pairs = n_chunks * static_cast<size_t>(n_bins);
  const size_t b_lists = up(pairs * kListPitch * sizeof(uint32_t));
  const size_t b_starts = up(pairs * kOffPitch * sizeof(uint32_t));
  if (off_starts) *off_starts = b_lists;
  return b_lists + b_starts;
}

hipError_t launch_embed_backward(const uint8_t* levels, int64_t n_tokens, int n_bins, int n_levels, const void* dsum,
                                 bool dsum_bf16, int d_model, float* dtable, bool accumulate, void* workspace,
                                 hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(n_bins) * n_levels;
  if (n_tokens <= 0) {
    if (accumulate) return hipSuccess;
    return zero_fill(dtable, rows * d_model, stream);
  }
  size_t off_starts = 0;
  bwd_layout(n_tokens, n_bins, &off_starts);
  auto* lists = static_cast<uint32_t*>(workspace);
  auto* starts = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + off_starts);
  const int64_t n_chunks = (n_tokens + kChunk - 1) / kChunk;
  const int64_t n_pairs = n_chunks * n_bins;
  const int64_t bblocks = (n_pairs + 3) / 4;
  if (bblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bucket_kernel, dim3(static_cast<unsigned>(bblocks)), dim3(256), 0, stream, levels, n_tokens,
                     n_bins, n_levels, n_pairs, lists, starts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_groups = (n_bins + kBwdBins - 1) / kBwdBins;
  const int n_strips = (d_model + kBwdCols - 1) / kBwdCols;
  const int64_t blocks = static_cast<int64_t>((n_strips + 7) / 8) * 8 * n_groups;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (dsum_bf16) {
    hipLaunchKernelGGL(scatter_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kBwdThreads), 0, stream, dsum,
                       n_tokens, n_bins, n_levels, d_model, lists, starts, n_chunks, n_groups, n_strips, dtable,
                       accumulate ? 1 : 0);
  } else {
    hipLaunchKernelGGL(scatter_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kBwdThreads), 0, stream,
                       dsum, n_tokens, n_bins, n_levels, d_model, lists, starts, n_chunks, n_groups, n_strips,
                       dtable, accumulate ? 1 : 0);
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

}  // namespace dmel
