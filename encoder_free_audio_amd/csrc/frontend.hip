// Front end: framing + Hann window + 1600-point real FFT + power + sparse mel
// projection + log + clamp + 16-level quantizer, fused in one kernel.  The
// filter count and the quantizer's range and level count come from the
// context's configuration (released values: 80 filters, [-7, 2], 16 levels;
// the same page's Coda gives -1.5 as the serving code's default minimum).
//
// "Inside Inkling: Audio Design", Part 1: 16 kHz mono audio becomes an
// 80-channel log-mel spectrogram (hop 800, window 1600) whose 80 values per
// frame are quantized to 16 levels; "Why this is a reasonable bet" gives the
// clamp range [-7, 2].  Open steps are read as: causal framing (frame t of a
// clip covers samples [800 t - 800, 800 t + 800), the clip's carry or zeros
// before sample 0), periodic Hann window, 1600-point FFT with 801 bins, power
// spectrum, 80 HTK triangles over 0..8000 Hz, ln(max(M, 1e-10)), and
// level = min(15, floor((clamp(l, -7, 2) + 7) * 16 / 9)) decided exactly.
//
// Work decomposition (one workgroup = 512 threads = 16 frames, fp32, LDS):
//  0. a frame's 32 threads sit in one wavefront and find its clip and first
//     sample themselves (steps 1-3 touch only the frame's own LDS buffer, so
//     the eight wavefronts run them without workgroup barriers);
//  1. the frame's 1600 samples are read as 800 complex values z[m] = x[2m] +
//     i x[2m+1] straight into registers (from the clip's carry or zeros, then
//     the audio, for a clip's first frame), while the tables read per lane
//     (window, pass-A twiddles, split twiddles, quantizer edges and the
//     filter schedule) are copied once per workgroup into LDS: read from
//     global memory by every frame, they were two thirds of the kernel's
//     vector-memory traffic;
//  2. 800-point complex FFT, 800 = 32 x 25:
//     pass A - one thread per (frame, n1 < 32): windowing, a 25-point DFT
//              (5 x 5) over z[n1 + 32 n2] in registers, then the twiddle
//              W800^(n1 k2);
//     pass B - one thread per (frame, k2 < 25): a 32-point DFT (8 x 4) over
//              n1 in registers, giving Z[k2 + 25 k1];
//     the exchanges (A to B, B to the split) go through the frame's LDS
//     buffer of rows padded to 33, real parts first, then imaginary parts:
//     half the buffer of complex exchanges, which leaves room in LDS for the
//     tables at two workgroups (16 wavefronts) per CU;
//  3. split Z into the 801-bin spectrum of the real frame and take |X|^2;
//  4. filters (after a barrier: lanes work across 8 of the block's frames):
//     a fixed schedule built on the host (FrontTables::mel_w) gives each of
//     four wavefronts a balanced share of the filters, once for frames 0..7
//     and once for frames 8..15; a lane computes one
//     filter of one frame as a weighted sum over the filter's contiguous
//     bins (weights from the schedule in LDS, 8 bins per step), then log,
//     clamp and the exact quantizer.
#include "internal.h"

namespace dmel {
namespace {

// Two halves of 8 frames; each half runs the four-round filter schedule.
constexpr int kFramesPerBlock = 16;
constexpr int kThreads = 512;
// Floats per frame in the exchange buffer: 825 used (25 rows x 33); the
// stride is 8 mod 64, so the filter step's reads (a wavefront's 8 frames x 8
// slots whose bins differ mod 8) fall in 64 distinct banks, and the buffers
// of 16 frames plus the tables fit two workgroups in a CU's LDS.
constexpr int kSlots = 840;
constexpr int kXchg = kFramesPerBlock * kSlots;  // exchange floats of a workgroup
// the filter step's powers: bin k at float kPOff + k of the frame's buffer,
// bins [-8, 0) and [801, kMelReadEnd) zero
constexpr int kPOff = 8;
static_assert(kSlots % 64 == 8, "bank spread of the filter step's reads");
static_assert(kSlots >= 25 * 33, "the FFT exchanges fit in the frame's buffer");
static_assert(kPOff + kMelReadEnd <= kSlots, "the filter step reads inside the frame's buffer");
static_assert(kPOff + kMelReadEnd - kBins <= 32, "the zero pads are written by one lane each");

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
// multiply by -i
__device__ __forceinline__ float2 mul_mi(float2 a) { return make_float2(a.y, -a.x); }

// In-place 5-point forward DFT, X_k = sum_n x_n exp(-2 pi i n k / 5).
__device__ __forceinline__ void dft5(float2& x0, float2& x1, float2& x2, float2& x3, float2& x4) {
  const float c1 = 0.30901699437494745f;   // cos(2 pi / 5)
  const float c2 = -0.8090169943749473f;   // cos(4 pi / 5)
  const float s1 = 0.9510565162951535f;    // sin(2 pi / 5)
  const float s2 = 0.5877852522924732f;    // sin(4 pi / 5)
  const float2 t1 = cadd(x1, x4), t2 = cadd(x2, x3);
  const float2 t3 = csub(x1, x4), t4 = csub(x2, x3);
  const float2 a1 = make_float2(x0.x + c1 * t1.x + c2 * t2.x, x0.y + c1 * t1.y + c2 * t2.y);
  const float2 a2 = make_float2(x0.x + c2 * t1.x + c1 * t2.x, x0.y + c2 * t1.y + c1 * t2.y);
  const float2 b1 = make_float2(s1 * t3.x + s2 * t4.x, s1 * t3.y + s2 * t4.y);
  const float2 b2 = make_float2(s2 * t3.x - s1 * t4.x, s2 * t3.y - s1 * t4.y);
  x0 = cadd(x0, cadd(t1, t2));
  // X1 = a1 - i b1, X4 = a1 + i b1, X2 = a2 - i b2, X3 = a2 + i b2
  x1 = make_float2(a1.x + b1.y, a1.y - b1.x);
  x4 = make_float2(a1.x - b1.y, a1.y + b1.x);
  x2 = make_float2(a2.x + b2.y, a2.y - b2.x);
  x3 = make_float2(a2.x - b2.y, a2.y + b2.x);
}

// In-place 4-point forward DFT.
__device__ __forceinline__ void dft4(float2& a0, float2& a1, float2& a2, float2& a3) {
  const float2 t0 = cadd(a0, a2), t1 = csub(a0, a2);
  const float2 t2 = cadd(a1, a3), t3 = csub(a1, a3);
  a0 = cadd(t0, t2);
  a2 = csub(t0, t2);
  a1 = cadd(t1, mul_mi(t3));
  a3 = csub(t1, mul_mi(t3));
}

// 8-point forward DFT of v[0..7] (in place), radix 2 over two 4-point DFTs.
__device__ __forceinline__ void dft8(float2 (&v)[8]) {
  const float h = 0.70710678118654752f;
  float2 e0 = v[0], e1 = v[2], e2 = v[4], e3 = v[6];
  float2 o0 = v[1], o1 = v[3], o2 = v[5], o3 = v[7];
  dft4(e0, e1, e2, e3);
  dft4(o0, o1, o2, o3);
  // W8^1 = h (1 - i), W8^2 = -i, W8^3 = h (-1 - i)
  const float2 w1o = make_float2(h * (o1.x + o1.y), h * (o1.y - o1.x));
  const float2 w2o = mul_mi(o2);
  const float2 w3o = make_float2(h * (o3.y - o3.x), -h * (o3.x + o3.y));
  v[0] = cadd(e0, o0);
  v[4] = csub(e0, o0);
  v[1] = cadd(e1, w1o);
  v[5] = csub(e1, w1o);
  v[2] = cadd(e2, w2o);
  v[6] = csub(e2, w2o);
  v[3] = cadd(e3, w3o);
  v[7] = csub(e3, w3o);
}

// Orders the LDS accesses of one wavefront.  Every frame's buffer is written
// and read only by its own 32 threads, which lie in one wavefront, and a
// wavefront's LDS operations complete in issue order; so between the FFT
// passes it is enough to keep the compiler from moving memory operations
// across this point, and the wavefronts of a workgroup run those passes
// without waiting for each other.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Clip of global frame g (the largest c with frame_off[c] <= g), with
// frame_off[c] and sample_off[c].  The first guess, (g + 0.5) * n_clips /
// n_frames, is the clip when every clip has the same number of frames F (the
// guess then lies at least 0.5 / F from an integer), and its three offsets
// are read together: one round of reads instead of log2(n_clips) + 1
// dependent ones for uniform batches and streaming steps.  A clip c with
// frame_off[c] <= g < frame_off[c + 1] is the answer because the offsets do
// not decrease; any other guess falls back to binary search.
struct ClipPos {
  int clip;
  int64_t frame0, sample0;
};
__device__ __forceinline__ ClipPos clip_of(const int64_t* frame_off, const int64_t* sample_off, int n_clips,
                                           double clip_rate, int64_t g) {
  int c = static_cast<int>((static_cast<double>(g) + 0.5) * clip_rate);
  c = c < 0 ? 0 : (c < n_clips - 1 ? c : n_clips - 1);
  const int64_t f0 = frame_off[c], f1 = frame_off[c + 1], s0 = sample_off[c];
  if (f0 <= g && g < f1) return {c, f0, s0};
  int lo = 0, hi = n_clips;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (frame_off[mid] <= g) lo = mid; else hi = mid;
  }
  return {lo, frame_off[lo], sample_off[lo]};
}

// Exact level of a log-mel value: the number of quantizer edges k = 1 .. V-1
// that the clamped value reaches, i.e. floor((c - lo) * V / (hi - lo)) capped
// at V - 1, decided by exact comparisons with the edges qe[0..V] (the released
// edges -7 + 9k/16 are exact in fp32; other edges are stored rounded up, see
// FrontTables), which the kernel keeps in LDS.
__device__ __forceinline__ int quantize(float l, const FrontTables& t, const float* qe) {
  const float c = fminf(fmaxf(l, t.q_lo), t.q_hi);
  const int vmax = t.n_levels - 1;
  int q = static_cast<int>((c - t.q_lo) * t.q_scale);
  q = q < 0 ? 0 : (q > vmax ? vmax : q);
  // The estimate is within one of the exact level: with t = (c - lo) V /
  // (hi - lo), the level is min(floor(t), V - 1), and the three fp32 roundings
  // (the difference, the stored V / (hi - lo), the product) move t by at most
  // 3 * 2^-24 * t <= 5e-5.  So one comparison each way decides it.
  const float e_lo = qe[q], e_hi = qe[q + 1];
  if (q > 0 && c < e_lo) return q - 1;
  if (q < vmax && c >= e_hi) return q + 1;
  return q;
}

// kMelLds: the filter schedule comes with the table image into LDS (it has
// at most kMelLdsChunks chunks); otherwise its weights are read from global
// memory.
// Four wavefronts per SIMD (two workgroups per CU) need at most 128 VGPRs;
// the compiler then spills a few values (12 bytes per lane) to scratch,
// outside the loops.
template <bool kMelLds>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
frontend_kernel(FrontTables tabs, const float* __restrict__ audio, int64_t n_samples_total,
                const int64_t* __restrict__ sample_off, const int64_t* __restrict__ frame_off,
                int n_clips, int64_t n_frames, double clip_rate, const float* __restrict__ carry,
                float* __restrict__ logmel, uint8_t* __restrict__ levels) {
  // LDS: the frames' exchange buffers (16 x 840 floats), then the table
  // image (window, twa, tw1600, quantizer edges, with kMelLds the schedule):
  // 78.6 KB (67.4 KB without the schedule), two workgroups per CU.
  constexpr int kImg = kMelLds ? kImgFull : kImgFloats;
  constexpr int kImgPieces = (kImg + 255) / 256;  // 1 KB pieces (the last one partial)
  static_assert(kImg % 4 == 0, "16-byte copies");
  __shared__ float smem[kXchg + kImg];
  float* const img = smem + kXchg;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int f = tid >> 5;      // frame within the block
  const int lane = tid & 31;   // n1 in pass A, k2 in pass B
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kFramesPerBlock;
  float* const zf = smem + f * kSlots;
  const float2* __restrict__ tw = tabs.tw800;

  // the frame's clip and first sample (each of its 32 threads finds them)
  const int64_t g = g0 + f;
  const bool valid = g < n_frames;
  int clip = 0;
  int64_t base = 0;
  bool first = false;
  if (valid) {
    const ClipPos cp = clip_of(frame_off, sample_off, n_clips, clip_rate, g);
    clip = cp.clip;
    const int64_t t = g - cp.frame0;
    base = cp.sample0 + kHop * t - kHop;
    first = (t == 0);
  }
  // Samples [0, 800) of the frame come from `lo` (the audio, or for a clip's
  // first frame its carry, or zeros without one) and [800, 1600) from `hi`
  // (the audio), whenever the frame lies inside the audio, which offsets that
  // describe the audio always give; `paired` marks the usual case of both
  // sources present and 8-byte aligned.  Other frames read every sample with
  // its own checks.
  const float* lo = nullptr;
  const float* hi = nullptr;
  if (valid && base + kHop >= 0 && base + kWindow <= n_samples_total && (first || base >= 0)) {
    hi = audio + (base + kHop);
    if (!first) lo = audio + base;
    else if (carry != nullptr) lo = carry + static_cast<int64_t>(clip) * kHop;
  }
  const bool paired = lo != nullptr && ((reinterpret_cast<uintptr_t>(lo) | reinterpret_cast<uintptr_t>(hi)) & 7) == 0;

  // ---- 1. the frame's samples as 800 pairs z[m] = x[2m] + i x[2m+1] -----
  // (pair m = lane + 32 n2; m < 400 from lo, m >= 400 from hi: n2 = 12
  // straddles, lanes 0..15 read lo), and the table image copied into LDS
  // while they are in flight
  float2 raw[25];
  if (paired) {
    const float2* l2 = reinterpret_cast<const float2*>(lo);
    const float2* h2 = reinterpret_cast<const float2*>(hi);
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
      const int m = lane + 32 * n2;
      if (n2 < 12) raw[n2] = l2[m];
      else if (n2 > 12) raw[n2] = h2[m - kHop / 2];
      else raw[n2] = lane < 16 ? l2[m] : h2[m - kHop / 2];
    }
  } else {
    const int64_t cbase = static_cast<int64_t>(clip) * kHop;
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
      const int m = lane + 32 * n2;
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = 2 * m + h;
        float val = 0.0f;
        if (valid) {
          if (first && n < kHop) {
            if (carry != nullptr) val = carry[cbase + n];
          } else {
            const int64_t sidx = base + n;
            if (sidx >= 0 && sidx < n_samples_total) val = audio[sidx];
          }
        }
        v[h] = val;
      }
      raw[n2] = make_float2(v[0], v[1]);
    }
  }
  for (int i = wave; i < kImgPieces; i += kThreads / 64) {
    if (256 * i + 4 * (tid & 63) < kImg) {
      __builtin_amdgcn_global_load_lds(tabs.lds_image + 256 * i + 4 * (tid & 63), (lds_void_t*)(img + 256 * i), 16, 0,
                                       0);
    }
  }
  // the copies into LDS are not tracked by the compiler: wait for every
  // memory read of the wave, then for the other waves
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- 2a. windowing, 25-point DFTs over n2 for each n1 ----------------
  {
    // window pair (w[2m], w[2m+1]) of pair m = lane + 32 n2: from the stored
    // half for m < 400, else (w[1600 - 2m], w[1599 - 2m]) (n2 = 12 straddles)
    const float* wh = img + kImgWindow;
    float2 x[25];
#pragma unroll
    for (int n2 = 0; n2 < 25; ++n2) {
      const int m = lane + 32 * n2;
      float2 w;
      if (n2 < 12) {
        w = *reinterpret_cast<const float2*>(wh + 2 * m);
      } else if (n2 > 12) {
        w = make_float2(wh[kWindow - 2 * m], wh[kWindow - 1 - 2 * m]);
      } else {
        const bool low = lane < 16;
        const int i0 = low ? 2 * m : kWindow - 1 - 2 * m;  // the lower of the two indices
        const float a = wh[i0], b = wh[i0 + 1];
        w = low ? make_float2(a, b) : make_float2(b, a);
      }
      x[n2] = make_float2(raw[n2].x * w.x, raw[n2].y * w.y);
    }
    // n2 = 5 a + b: 5-point DFTs over a for each b
#pragma unroll
    for (int b = 0; b < 5; ++b) dft5(x[b], x[5 + b], x[10 + b], x[15 + b], x[20 + b]);
    // twiddle W25^(b c) for slot 5 c + b  (W25^m = W800^(32 m))
#pragma unroll
    for (int c = 1; c < 5; ++c) {
#pragma unroll
      for (int b = 1; b < 5; ++b) x[5 * c + b] = cmul(x[5 * c + b], tw[32 * b * c]);
    }
    // 5-point DFTs over b for each c: output index c + 5 d
    float2 y[25];
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      float2 u0 = x[5 * c], u1 = x[5 * c + 1], u2 = x[5 * c + 2], u3 = x[5 * c + 3], u4 = x[5 * c + 4];
      dft5(u0, u1, u2, u3, u4);
      y[c] = u0;
      y[c + 5] = u1;
      y[c + 10] = u2;
      y[c + 15] = u3;
      y[c + 20] = u4;
    }
    const float2* twa = reinterpret_cast<const float2*>(img + kImgTwa);
#pragma unroll
    for (int k2 = 1; k2 < 25; ++k2) y[k2] = cmul(y[k2], twa[(k2 - 1) * 32 + lane]);

    // ---- exchange to pass B: real parts, then imaginary parts, through the
    // frame's 825 floats (rows of 33: neither side has bank conflicts)
    const bool active = lane < 25;
    const int k2 = active ? lane : 0;
    float2 a[32];
#pragma unroll
    for (int i = 0; i < 25; ++i) zf[lane + 33 * i] = y[i].x;
    wave_sync();
#pragma unroll
    for (int n1 = 0; n1 < 32; ++n1) a[n1].x = zf[n1 + 33 * k2];
    wave_sync();
#pragma unroll
    for (int i = 0; i < 25; ++i) zf[lane + 33 * i] = y[i].y;
    wave_sync();
#pragma unroll
    for (int n1 = 0; n1 < 32; ++n1) a[n1].y = zf[n1 + 33 * k2];
    wave_sync();

    // ---- 2b. 32-point DFTs over n1 for each k2 -------------------------
    // n1 = 4 p + q: 8-point DFTs over p for each q, output r
    float2 v[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int p = 0; p < 8; ++p) v[q][p] = a[4 * p + q];
      dft8(v[q]);
    }
    // twiddle W32^(q r) = W800^(25 q r)
#pragma unroll
    for (int q = 1; q < 4; ++q) {
#pragma unroll
      for (int r = 1; r < 8; ++r) v[q][r] = cmul(v[q][r], tw[25 * q * r]);
    }
    // 4-point DFTs over q for each r: output k1 = r + 8 s
#pragma unroll
    for (int r = 0; r < 8; ++r) dft4(v[0][r], v[1][r], v[2][r], v[3][r]);

    // ---- exchange to the split: Z[k2 + 25 k1], real parts then imaginary
    // parts; the frame's thread `lane` then takes k = lane + 32 m and 800 - k
    constexpr int kPairs = kHalf / 2 + 1;            // 401
    constexpr int kPer = (kPairs + 31) / 32;         // 13
    float2 zk[kPer], zm[kPer];
    if (active) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int s = 0; s < 4; ++s) zf[k2 + 25 * (r + 8 * s)] = v[s][r].x;
      }
    }
    wave_sync();
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int k = min(lane + 32 * m, kPairs - 1);
      zk[m].x = zf[k];
      zm[m].x = zf[k == 0 ? 0 : kHalf - k];
    }
    wave_sync();
    if (active) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int s = 0; s < 4; ++s) zf[k2 + 25 * (r + 8 * s)] = v[s][r].y;
      }
    }
    wave_sync();
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int k = min(lane + 32 * m, kPairs - 1);
      zk[m].y = zf[k];
      zm[m].y = zf[k == 0 ? 0 : kHalf - k];
    }
    wave_sync();

    // ---- 3. real-spectrum split and power -------------------------------
    // E[k] = (Z[k] + conj Z[800-k]) / 2, O[k] = (Z[k] - conj Z[800-k]) / 2i,
    // X[k] = E + W1600^k O and X[800-k] = conj(E - W1600^k O), k = 0..400.
    // The halves are left out (2E, 2O, so the powers are 4 |X|^2); the filter
    // weights carry the 1/4.
    const float2* t16 = reinterpret_cast<const float2*>(img + kImgTw1600);
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int k = lane + 32 * m;
      if (k < kPairs) {
        const float2 e = make_float2(zk[m].x + zm[m].x, zk[m].y - zm[m].y);
        const float2 o = make_float2(zk[m].y + zm[m].y, zm[m].x - zk[m].x);
        const float2 wo = cmul(t16[k], o);
        const float2 x1 = cadd(e, wo), x2 = csub(e, wo);
        zf[kPOff + k] = x1.x * x1.x + x1.y * x1.y;
        zf[kPOff + kHalf - k] = x2.x * x2.x + x2.y * x2.y;
      }
    }
    // the filter step reads bins [-8, kMelReadEnd) with zero weights outside a
    // filter's range; the powers it reads there must be finite: zero
    if (lane < kPOff) zf[lane] = 0.0f;
    else if (lane < kPOff + kMelReadEnd - kBins) zf[kBins + lane] = 0.0f;
  }
  // ---- 4. filters, log, clamp, quantize ----------------------------------
  // Wavefronts r and 4 + r run round r of the schedule (FrontTables::mel_w)
  // for frames 0..7 and 8..15: lane 8 * slot + f8 computes, for frame
  // ff = 8 * (wave / 4) + f8 and each side of the round, the
  // filter of `slot` as the sum over the side's 8-bin chunks of the chunk's
  // weights (the 8 lanes of a slot share each read) times the frame's powers,
  // then writes its log-mel value and level.
  __syncthreads();  // the powers of all 16 frames are in LDS
  {
    const int r = __builtin_amdgcn_readfirstlane(wave & 3);
    const int slot = (tid >> 3) & 7;
    const int ff = 8 * (wave >> 2) + (tid & 7);
    const int* rd = tabs.mel_round + 8 * r;
    const int base = rd[0], sides = rd[2];
    const float4* mw = kMelLds ? reinterpret_cast<const float4*>(img + kImgMelW) : tabs.mel_w;
    const int* mfirst = kMelLds ? reinterpret_cast<const int*>(img + kImgMelFirst) : tabs.mel_first;
    const int* mfilt = kMelLds ? reinterpret_cast<const int*>(img + kImgMelFilt) : tabs.mel_filt;
    const int n_mels = tabs.n_mels;
    const int64_t n_valid = n_frames - g0 < kFramesPerBlock ? n_frames - g0 : kFramesPerBlock;
    const float* p_frame = smem + ff * kSlots + kPOff;
    const float* qe = img + kImgEdge;
    const int64_t orow = (g0 + ff) * n_mels;
    for (int h = 0; h < sides; ++h) {
      const int i = 8 * (kMelMaxSides * r + h) + slot;
      const int j = mfilt[i];
      const int c_first = rd[3 + h], c_end = rd[4 + h];
      const float* p = p_frame + mfirst[i] - 8 * c_first;
      float a0 = 0.0f, a1 = 0.0f;
      for (int c = c_first; c < c_end; ++c) {
        const float4 u = mw[16 * (base + c) + slot];
        const float4 v = mw[16 * (base + c) + 8 + slot];
        float q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = p[8 * c + k];
        a0 = fmaf(u.x, q[0], a0);
        a1 = fmaf(u.y, q[1], a1);
        a0 = fmaf(u.z, q[2], a0);
        a1 = fmaf(u.w, q[3], a1);
        a0 = fmaf(v.x, q[4], a0);
        a1 = fmaf(v.y, q[5], a1);
        a0 = fmaf(v.z, q[6], a0);
        a1 = fmaf(v.w, q[7], a1);
      }
      if (j >= 0 && ff < n_valid) {
        // ln m = ln 2 * log2 m with the hardware log2 (about 1 ulp; m >= 1e-10 is normal)
        const float l = 0.69314718055994531f * __builtin_amdgcn_logf(fmaxf(a0 + a1, kLogFloor));
        if (logmel != nullptr) logmel[orow + j] = l;
        if (levels != nullptr) levels[orow + j] = static_cast<uint8_t>(quantize(l, tabs, qe));
      }
    }
  }
}

}  // namespace

hipError_t launch_frontend(const FrontTables& tabs, const float* audio, int64_t n_samples_total,
                           const int64_t* sample_off, const int64_t* frame_off, int n_clips,
                           int64_t n_frames, const float* carry, float* logmel, uint8_t* levels,
                           hipStream_t stream) {
  if (n_frames <= 0) return hipSuccess;
  const int64_t blocks = (n_frames + kFramesPerBlock - 1) / kFramesPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const double rate = static_cast<double>(n_clips) / static_cast<double>(n_frames);
  if (tabs.mel_in_lds) {
    hipLaunchKernelGGL(frontend_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       tabs, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames, rate, carry, logmel,
                       levels);
  } else {
    hipLaunchKernelGGL(frontend_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                       tabs, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames, rate, carry, logmel,
                       levels);
  }
  return hipGetLastError();
}

}  // namespace dmel
