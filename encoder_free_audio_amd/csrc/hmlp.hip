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

// GELU(x) = x Phi(x) with Phi(x) = erfc(-x / sqrt(2)) / 2, branch free.  For
// z >= 0, erfc(z) = t exp(P(t) - z^2) with t = 1 / (1 + z / 2): the form of
// the Chebyshev erfc approximation in Press et al., Numerical Recipes, with a
// degree-9 polynomial P fitted to ln(erfc(z) / t) + z^2 over t in (0, 1]
// (largest fit error 8e-8).  This fp32 evaluation is within 3.8e-7 absolute
// of the exact GELU over [-9, 9] (1.3e-6 relative for x >= -3), well inside
// the accumulation tolerance of every stage.
__device__ __forceinline__ float gelu(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 1.767219591e-01f;
  p = fmaf(p, t, -8.499431527e-01f);
  p = fmaf(p, t, 1.544073511e+00f);
  p = fmaf(p, t, -1.195862089e+00f);
  p = fmaf(p, t, 3.181210659e-01f);
  p = fmaf(p, t, -2.015549787e-01f);
  p = fmaf(p, t, 1.002275065e-01f);
  p = fmaf(p, t, 3.736856663e-01f);
  p = fmaf(p, t, 1.000042885e+00f);
  p = fmaf(p, t, -1.265512293e+00f);
  const float ec = t * __builtin_amdgcn_exp2f(fmaf(-z, z, p) * 1.44269504088896341f);
  return x * (x >= 0.0f ? fmaf(-0.5f, ec, 1.0f) : 0.5f * ec);
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
        if (gelu) v = dmel::gelu(v);
        if (out_f32) {
          static_cast<float*>(C)[row * N + col] = v;
        } else {
          static_cast<uint16_t*>(C)[row * N + col] = to_bf16(v);
        }
      }
    }
  }
}

// ---- large-tile GEMM -------------------------------------------------------
// C[M, N] = A[M, K] B[N, K]^T + bias (then GELU) for N % 256 == 0 and
// K % 32 == 0.  Workgroup tile 256 x 256, four waves as 2 x 2, each owning
// 4 x 4 MFMA tiles of 32 x 32 (256 fp32 accumulators per lane: one wave per
// SIMD, accumulators in AGPRs).
//  * Operands go from global memory straight into LDS (16-byte
//    global_load_lds, no register staging) through a ring of four stages of
//    K = 32 (32 KB each); the loads of step k + 3 are issued during steps k
//    and k + 1 (a fifth stage measured no faster).
//  * LDS rows are 64 bytes (32 bf16 of K); the 16-byte chunk c of row r sits
//    in slot c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3: the fragment reads of
//    any 8 or 16 consecutive rows at one chunk then touch every bank at most
//    once (rows of equal r % 2, and of equal r % 4, get distinct slots).  A
//    lane of the DMA load writes slot lane & 3 of row lane >> 2 of its 16-row
//    block, so it fetches logical chunk (lane & 3) ^ f(row).
//  * One barrier per K step, between its two 16-deep sub-steps: it certifies
//    the next step's stage (after this wave's wait for its loads) and frees
//    the stage read in the previous step for the next loads.  The fragments of
//    the sub-step after it were read before it, so the matrix core does not
//    wait for the barrier's LDS reads.
//  * Tile order: workgroup b runs on XCD b % 8.  Each XCD takes a contiguous
//    range of tiles in row-panel-major order, so the ~32 workgroups resident on
//    one XCD share A row panels (all N / 256 column tiles of a panel) and B
//    column panels in that XCD's L2.
//  * Rows past M load row M - 1 (in bounds) and are not written.
constexpr int kBT = 256;                      // tile rows / columns
constexpr int kBTK = 32;                      // K step
constexpr int kNStages = 4;
constexpr int kRowBytes = kBTK * 2;           // 64-byte LDS rows
constexpr int kTileBytes = kBT * kRowBytes;   // 16 KB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;   // A + B

typedef __attribute__((address_space(3))) void lds_void_t;

// kWM = 4 (the one launched): eight waves (4 x 2) of 2 x 4 MFMA tiles, two
// waves per SIMD, so one wave's epilogue arithmetic, loads and barrier waits
// overlap the other's products.  kWM = 2: four waves (2 x 2) of 4 x 4 tiles,
// one wave per SIMD (fewer LDS fragment reads per product; measured slower
// for every hMLP and DFT shape).
constexpr int kEpPitch = 136;   // epilogue LDS row pitch (floats)

template <int kWM>
constexpr int smem_bytes() {
  return kNStages * kStageBytes > 2 * kWM * 32 * kEpPitch * 4 ? kNStages * kStageBytes : 2 * kWM * 32 * kEpPitch * 4;
}

template <int kWM>
struct GemmShape {
  static constexpr int TM = 8 / kWM;     // MFMA tile rows per wave
  static constexpr int RW = 128 / kWM;   // tile rows each wave loads per operand
  static constexpr int NJ = RW / 16;     // DMA instructions per operand per stage
};

template <int kWM, bool kGelu, bool kOutF32>
__global__ void __launch_bounds__(128 * kWM) __attribute__((amdgpu_waves_per_eu(kWM / 2, kWM / 2)))
gemm256_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, const float* __restrict__ bias,
               void* __restrict__ C, int64_t M, int N, int K, int tiles_n, int64_t n_tiles) {
  using G = GemmShape<kWM>;
  __shared__ __attribute__((aligned(1024))) char smem[smem_bytes<kWM>()];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t b = blockIdx.x;
  const int64_t q = n_tiles / 8, rem = n_tiles % 8;
  const int64_t x = b % 8;
  const int64_t tile = x * q + (x < rem ? x : rem) + b / 8;
  const int64_t bm = tile / tiles_n;
  const int bn = static_cast<int>(tile - bm * tiles_n);
  const int64_t row0 = bm * kBT;
  const int col0 = bn * kBT;

  // this lane's DMA sources: rows wave * G::RW + 16 j + (lane >> 2) of the A and
  // B tiles, logical chunk (lane & 3) ^ f(row); byte offsets from the tiles'
  // first rows (< 2^32: 256 rows of at most 2^21 bytes)
  const int lr = lane >> 2;
  uint32_t aoff[4], boff[4];   // (first G::NJ used; a fixed size keeps the arrays capturable by the lambdas)
#pragma unroll
  for (int j = 0; j < G::NJ; ++j) {
    const int r = wave * G::RW + 16 * j + lr;
    const int lc = (lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3);
    const int64_t ra = row0 + r < M ? r : M - 1 - row0;
    aoff[j] = static_cast<uint32_t>(ra * K * 2 + lc * 16);
    boff[j] = static_cast<uint32_t>(static_cast<int64_t>(r) * K * 2 + lc * 16);
  }
  const char* Ab = reinterpret_cast<const char*>(A + row0 * K);
  const char* Bb = reinterpret_cast<const char*>(B + static_cast<int64_t>(col0) * K);
  auto issue_half = [&](int kt, int h) {
    char* sa = smem + (kt % kNStages) * kStageBytes + wave * G::RW * kRowBytes + h * kTileBytes;
    const char* ga = (h == 0 ? Ab : Bb) + static_cast<int64_t>(kt) * (kBTK * 2);
#pragma unroll
    for (int j = 0; j < G::NJ; ++j)
      __builtin_amdgcn_global_load_lds(ga + (h == 0 ? aoff[j] : boff[j]), (lds_void_t*)(sa + j * 16 * kRowBytes), 16, 0, 0);
  };
  auto issue = [&](int kt) {
    char* sa = smem + (kt % kNStages) * kStageBytes + wave * G::RW * kRowBytes;
    char* sb = sa + kTileBytes;
    const char* ga = Ab + static_cast<int64_t>(kt) * (kBTK * 2);
    const char* gb = Bb + static_cast<int64_t>(kt) * (kBTK * 2);
#pragma unroll
    for (int j = 0; j < G::NJ; ++j)
      __builtin_amdgcn_global_load_lds(ga + aoff[j], (lds_void_t*)(sa + j * 16 * kRowBytes), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < G::NJ; ++j)
      __builtin_amdgcn_global_load_lds(gb + boff[j], (lds_void_t*)(sb + j * 16 * kRowBytes), 16, 0, 0);
  };
  // Wait until this wave's loads of the stage needed next have landed (loads
  // complete in order; `later` more steps' loads may stay in flight), then
  // meet the other waves.  One asm with a memory clobber, so no LDS access
  // moves across it and no fence adds a wait for every load in flight.
  auto sync_stage = [&](int later) {
    const int n = later * 2 * G::NJ;   // loads of `later` stages
    if (n == 24) {
      asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
    } else if (n == 16) {
      asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    } else if (n == 12) {
      asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
    } else if (n == 8) {
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    } else if (n == 4) {
      asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };

  // fragments of sub-step (k, h): rows (lane & 31) + 32 t of this wave's
  // blocks (32 G::TM rows of A, 128 rows of B), logical chunk 2 h + (lane >> 5)
  const int frow = (lane & 31) * kRowBytes;
  const int fsw = (((lane & 31) >> 1) ^ ((lane & 31) >> 3)) & 3;  // f(row): the block offsets are multiples of 32
  bf16x8_t fa[2][G::TM], fb[2][4];
  auto frag = [&](int kt, int h, int buf) {
    const char* sa = smem + (kt % kNStages) * kStageBytes + wm * 32 * G::TM * kRowBytes + frow;
    const char* sb = smem + (kt % kNStages) * kStageBytes + kTileBytes + wn * 128 * kRowBytes + frow;
    const int off = ((2 * h + (lane >> 5)) ^ fsw) << 4;
#pragma unroll
    for (int t = 0; t < G::TM; ++t) fa[buf][t] = *reinterpret_cast<const bf16x8_t*>(sa + t * 32 * kRowBytes + off);
#pragma unroll
    for (int t = 0; t < 4; ++t) fb[buf][t] = *reinterpret_cast<const bf16x8_t*>(sb + t * 32 * kRowBytes + off);
  };
  f32x16_t acc[G::TM][4];
#pragma unroll
  for (int a = 0; a < G::TM; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][c][i] = 0.0f;
  // Issue order per sub-step: wait for this sub-step's fragments, issue the
  // next sub-step's eight LDS reads, then the sixteen products, so the reads
  // return while the matrix core works (and at most eight are in flight).
  // pin(buf), an empty asm that "modifies" the fragments of buffer buf and
  // clobbers memory, makes the wave wait for them there and keeps the next
  // reads below it; scheduling barriers keep each group of products between
  // the reads before it and the wait after it.
  auto pin = [&](int buf) {
    if constexpr (G::TM == 4) {
      asm volatile("" : "+v"(fa[buf][0]), "+v"(fa[buf][1]), "+v"(fa[buf][2]), "+v"(fa[buf][3]), "+v"(fb[buf][0]),
                   "+v"(fb[buf][1]), "+v"(fb[buf][2]), "+v"(fb[buf][3])::"memory");
    } else {
      asm volatile("" : "+v"(fa[buf][0]), "+v"(fa[buf][1]), "+v"(fb[buf][0]), "+v"(fb[buf][1]), "+v"(fb[buf][2]),
                   "+v"(fb[buf][3])::"memory");
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int a = 0; a < G::TM; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][a], fb[buf][c], acc[a][c], 0, 0, 0);
  };

  // The ring always advances by one stage per K step: past the last step the
  // loads repeat the last step's data into a stage nobody reads again, so the
  // number of loads in flight (and so every wait) is the same in every step.
  const int nk = K / kBTK;
#pragma unroll
  for (int i = 0; i < kNStages - 1; ++i) issue(min(i, nk - 1));
  sync_stage(kNStages - 2);
  frag(0, 0, 0);
  // Each stage's loads are split over two sub-steps: its A half after the
  // barrier of step k (between the products of the second sub-step), its B
  // half in the first sub-step of step k + 1, so the DMA traffic is spread
  // over the whole step.  (In step 0 the B half repeats the prologue's loads of
  // stage 2 with the same data; the wait below then waits a little longer.)
  // Loads complete in order, so before the barrier of step k the loads of
  // stage k + 2 are the only ones that may still be in flight.
  for (int kt = 0; kt + 1 < nk; ++kt) {
    pin(0);
    frag(kt, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    issue_half(min(kt + kNStages - 2, nk - 1), 1);
    mma(0);
#pragma unroll
    for (int m = 0; m < G::NJ; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);            // two MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);            // one global (DMA) load
    }
    __builtin_amdgcn_sched_barrier(0);
    pin(1);
    sync_stage(kNStages - 3);
    issue_half(min(kt + kNStages - 1, nk - 1), 0);
    frag(kt + 1, 0, 0);
    mma(1);
#pragma unroll
    for (int m = 0; m < G::TM + 4; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
#pragma unroll
    for (int m = 0; m < G::NJ; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, (3 * G::TM - 4) / G::NJ, 0);  // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                // one global (DMA) load
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  pin(0);
  frag(nk - 1, 1, 1);
  __builtin_amdgcn_sched_barrier(0);
  mma(0);
  __builtin_amdgcn_sched_barrier(0);
  pin(1);
  mma(1);

  // Epilogue through LDS, a quarter of the wave's 128 x 128 block (32 rows) at
  // a time: the accumulators go to a wave-private 32 x 128 fp32 area (row
  // pitch 136 floats: the two row groups of one store land in different bank
  // halves), then each lane reads 4 consecutive columns of a row back, so a
  // half-wave writes one row's 128 outputs as one contiguous piece.  Lane
  // layout of a 32 x 32 accumulator: column lane & 31, rows
  // 8 (i / 4) + 4 (lane / 32) + i % 4.
  __syncthreads();  // every wave is done with the operand stages
  float* ep = reinterpret_cast<float*>(smem) + wave * 32 * kEpPitch;
  const int cl = 4 * (lane & 31);
  const int col = col0 + wn * 128 + cl;
  const float4 bb = make_float4(bias[col], bias[col + 1], bias[col + 2], bias[col + 3]);
#pragma unroll
  for (int a = 0; a < G::TM; ++a) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        ep[(8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)) * kEpPitch + c * 32 + (lane & 31)] = acc[a][c][i];
#pragma unroll 4
    for (int pr = 0; pr < 16; ++pr) {
      const int r = 2 * pr + (lane >> 5);
      const int64_t row = row0 + wm * 32 * G::TM + a * 32 + r;
      float4 v = *reinterpret_cast<const float4*>(ep + r * kEpPitch + cl);
      v.x += bb.x;
      v.y += bb.y;
      v.z += bb.z;
      v.w += bb.w;
      if (kGelu) {
        v.x = gelu(v.x);
        v.y = gelu(v.y);
        v.z = gelu(v.z);
        v.w = gelu(v.w);
      }
      if (row < M) {
        if (kOutF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(C) + row * N + col) = v;
        } else {
          const uint2 h = make_uint2(static_cast<uint32_t>(to_bf16(v.x)) | static_cast<uint32_t>(to_bf16(v.y)) << 16,
                                     static_cast<uint32_t>(to_bf16(v.z)) | static_cast<uint32_t>(to_bf16(v.w)) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(C) + row * N + col) = h;
        }
      }
    }
  }
}

hipError_t gemm(const uint16_t* A, const uint16_t* B, const float* bias, void* C, int64_t M, int N, int K, bool gelu,
                bool out_f32, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  // (the large-tile kernel stores 16 or 8 bytes per lane: C 16-byte aligned)
  if (N % kBT == 0 && K % kBTK == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0) {
    const int tiles_n = N / kBT;
    const int64_t n_tiles = ((M + kBT - 1) / kBT) * tiles_n;
    if (n_tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(n_tiles));
    // eight waves (two per SIMD): measured faster than four waves of 4 x 4
    // tiles for every stage shape (the stem 19.9 -> 17.8 ms)
    const dim3 block(512);
    if (gelu && !out_f32) {
      hipLaunchKernelGGL((gemm256_kernel<4, true, false>), grid, block, 0, stream, A, B, bias, C, M, N, K, tiles_n, n_tiles);
    } else if (gelu) {
      hipLaunchKernelGGL((gemm256_kernel<4, true, true>), grid, block, 0, stream, A, B, bias, C, M, N, K, tiles_n, n_tiles);
    } else if (!out_f32) {
      hipLaunchKernelGGL((gemm256_kernel<4, false, false>), grid, block, 0, stream, A, B, bias, C, M, N, K, tiles_n, n_tiles);
    } else {
      hipLaunchKernelGGL((gemm256_kernel<4, false, true>), grid, block, 0, stream, A, B, bias, C, M, N, K, tiles_n, n_tiles);
    }
    return hipGetLastError();
  }
  const int64_t blocks = ((M + kBM - 1) / kBM) * (N / kBN);
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
