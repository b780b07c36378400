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
// Work decomposition (one workgroup = 256 threads = 8 frames, fp32, LDS):
//  0. a frame's 32 threads sit in one wavefront and find its clip and first
//     sample themselves (steps 1-3 touch only the frame's own LDS rows, so
//     the four wavefronts run them without workgroup barriers);
//  1. the 1600 windowed samples of a frame are read as 800 complex values
//     z[m] = x[2m] + i x[2m+1] straight into the registers of pass A (from
//     the clip's carry or zeros, then the audio, for a clip's first frame);
//  2. 800-point complex FFT, 800 = 32 x 25:
//     pass A - one thread per (frame, n1 < 32): a 25-point DFT (5 x 5) over
//              z[n1 + 32 n2] (coalesced 8-byte reads across n1) in registers,
//              then the twiddle W800^(n1 k2);
//     pass B - one thread per (frame, k2 < 25): a 32-point DFT (8 x 4) over
//              n1 in registers, giving Z[k2 + 25 k1];
//     the exchange between the passes goes through LDS rows padded to 33
//     complex values so that neither pass has bank conflicts;
//  3. split Z into the 801-bin spectrum of the real frame and take |X|^2;
//  4. mel (work items across the block's frames, after a barrier): each bin
//     lies between two triangle edges and feeds exactly two filters (the
//     rising side of one, the falling side of the previous), so one pass
//     over the 81 segments gives per-segment sums A_s (rising) and C_s
//     (falling) and filter j is A_j + C_{j+1}; then log, clamp, quantize.
#include "internal.h"

namespace dmel {
namespace {

constexpr int kFramesPerBlock = 8;
constexpr int kThreads = 256;
constexpr int kSlots = 825;  // complex slots per frame in LDS: 25 rows x 33

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
// across this point, and the four wavefronts of a workgroup run those passes
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
// at V - 1, decided by exact comparisons (the released edges -7 + 9k/16 are
// exact in fp32; other edges are stored rounded up, see FrontTables).
__device__ __forceinline__ int quantize(float l, const FrontTables& t) {
  const float c = fminf(fmaxf(l, t.q_lo), t.q_hi);
  const int vmax = t.n_levels - 1;
  int q = static_cast<int>((c - t.q_lo) * t.q_scale);
  q = q < 0 ? 0 : (q > vmax ? vmax : q);
  // the estimate is within one or two of the exact level
  while (q > 0 && c < t.q_edge[q]) --q;
  while (q < vmax && c >= t.q_edge[q + 1]) ++q;
  return q;
}

__global__ void __launch_bounds__(kThreads)
frontend_kernel(FrontTables tabs, const float* __restrict__ audio, int64_t n_samples_total,
                const int64_t* __restrict__ sample_off, const int64_t* __restrict__ frame_off,
                int n_clips, int64_t n_frames, double clip_rate, const float* __restrict__ carry,
                float* __restrict__ logmel, uint8_t* __restrict__ levels) {
  // Only the frames' working buffer lives in LDS (52.8 KB: three workgroups
  // per CU); the constant tables are read from global memory (uniform indices
  // become scalar loads, the rest hit the L1).
  __shared__ float2 zbuf[kFramesPerBlock * kSlots];

  const int tid = threadIdx.x;
  const int f = tid >> 5;      // frame within the block
  const int lane = tid & 31;   // n1 in pass A, k2 in pass B
  const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kFramesPerBlock;
  float2* zf = zbuf + f * kSlots;
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
  // describe the audio always give; other frames check every sample.
  const float* lo = nullptr;
  const float* hi = nullptr;
  bool inside = false;
  if (valid && base + kHop >= 0 && base + kWindow <= n_samples_total && (first || base >= 0)) {
    inside = true;
    hi = audio + (base + kHop);
    if (!first) lo = audio + base;
    else if (carry != nullptr) lo = carry + static_cast<int64_t>(clip) * kHop;
  }
  // the usual case: both sources present and 8-byte aligned
  const bool paired = inside && lo != nullptr &&
                      ((reinterpret_cast<uintptr_t>(lo) | reinterpret_cast<uintptr_t>(hi)) & 7) == 0;

  // ---- 1 + 2a. windowed samples, 25-point DFTs over n2 for each n1 --------
  {
    float2 x[25];
    const float2* w2 = reinterpret_cast<const float2*>(tabs.window);
    // sample pair m < 400 comes from lo, m >= 400 from hi (n2 = 12 straddles:
    // lanes 0..15 read lo)
    if (paired) {
      const float2* l2 = reinterpret_cast<const float2*>(lo);
      const float2* h2 = reinterpret_cast<const float2*>(hi);
#pragma unroll
      for (int n2 = 0; n2 < 25; ++n2) {
        const int m = lane + 32 * n2;
        float2 a;
        if (n2 < 12) a = l2[m];
        else if (n2 > 12) a = h2[m - kHop / 2];
        else a = lane < 16 ? l2[m] : h2[m - kHop / 2];
        const float2 w = w2[m];
        x[n2] = make_float2(a.x * w.x, a.y * w.y);
      }
    } else if (inside) {
      // no carry (zeros) or unaligned sources: 4-byte reads
#pragma unroll
      for (int n2 = 0; n2 < 25; ++n2) {
        const int m = lane + 32 * n2;
        const bool from_lo = n2 < 12 || (n2 == 12 && lane < 16);
        float2 a = make_float2(0.0f, 0.0f);
        if (!from_lo) {
          a = make_float2(hi[2 * m - kHop], hi[2 * m - kHop + 1]);
        } else if (lo != nullptr) {
          a = make_float2(lo[2 * m], lo[2 * m + 1]);
        }
        const float2 w = w2[m];
        x[n2] = make_float2(a.x * w.x, a.y * w.y);
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
        const float2 w = w2[m];
        x[n2] = make_float2(v[0] * w.x, v[1] * w.y);
      }
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
#pragma unroll
    for (int k2 = 1; k2 < 25; ++k2) y[k2] = cmul(y[k2], tabs.twa[(k2 - 1) * 32 + lane]);
#pragma unroll
    for (int k2 = 0; k2 < 25; ++k2) zf[lane + 33 * k2] = y[k2];
  }
  wave_sync();

  // ---- 2b. 32-point DFTs over n1 for each k2 ---------------------------
  {
    float2 a[32];
    const bool active = lane < 25;
    const int k2 = active ? lane : 0;
#pragma unroll
    for (int n1 = 0; n1 < 32; ++n1) a[n1] = zf[n1 + 33 * k2];
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
    wave_sync();
    if (active) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int s = 0; s < 4; ++s) zf[k2 + 25 * (r + 8 * s)] = v[s][r];
      }
    }
  }
  wave_sync();

  // ---- 3. real-spectrum split and power ---------------------------------
  // E[k] = (Z[k] + conj Z[800-k]) / 2, O[k] = (Z[k] - conj Z[800-k]) / 2i,
  // X[k] = E + W1600^k O and X[800-k] = conj(E - W1600^k O), k = 0..400;
  // the frame's thread `lane` takes k = lane + 32 m.
  constexpr int kPairs = kHalf / 2 + 1;            // 401
  constexpr int kPer = (kPairs + 31) / 32;         // 13
  float p_lo[kPer], p_hi[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int k = lane + 32 * m;
    p_lo[m] = 0.0f;
    p_hi[m] = 0.0f;
    if (k < kPairs) {
      const float2 zk = zf[k];
      const float2 zm = zf[k == 0 ? 0 : kHalf - k];
      const float2 e = make_float2(0.5f * (zk.x + zm.x), 0.5f * (zk.y - zm.y));
      const float2 o = make_float2(0.5f * (zk.y + zm.y), -0.5f * (zk.x - zm.x));
      const float2 wo = cmul(tabs.tw1600[k], o);  // L1-cached table
      const float2 x1 = cadd(e, wo), x2 = csub(e, wo);
      p_lo[m] = x1.x * x1.x + x1.y * x1.y;
      p_hi[m] = x2.x * x2.x + x2.y * x2.y;
    }
  }
  wave_sync();
  {
    float* pw = reinterpret_cast<float*>(zf);  // the frame's 801 powers
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int k = lane + 32 * m;
      if (k < kPairs) {
        pw[k] = p_lo[m];
        pw[kHalf - k] = p_hi[m];
      }
    }
  }
  __syncthreads();  // the mel step works across the block's frames

  // ---- 4. mel: segment sums, then filters, log, clamp, quantize ----------
  {
    float* pf = reinterpret_cast<float*>(zbuf);
    const int n_mels = tabs.n_mels;
    const int n_seg = n_mels + 1;    // 81 segments for 80 filters
    constexpr int kAOff = 1024;      // per-frame float offsets of A_s and C_s (past the 801 powers)
    constexpr int kCOff = kAOff + kMaxMels + 8;
    static_assert(kCOff + kMaxMels + 1 <= 2 * kSlots, "segment sums must fit the frame's buffer");
    // segments s and n_seg - 1 - s are paired (a narrow low band with a wide
    // high one) so that the threads' loops are of similar length
    const int n_pairs = (n_seg + 1) / 2;  // 41: (0,80) .. (39,41), (40)
    const int* __restrict__ seg = tabs.seg_start;
    const float bin_hz = static_cast<float>(kSampleRate) / kNfft;
    // pair-major order: the lanes of a wavefront take neighbouring pairs, whose
    // segments have similar lengths, so their loops run about the same count
    static_assert(kFramesPerBlock == 8, "pair-major order assumes 8 frames");
    for (int it = tid; it < kFramesPerBlock * n_pairs; it += kThreads) {
      const int pr = it >> 3;
      const int ff = it & 7;
      const float* p = pf + 2 * ff * kSlots;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sg = h == 0 ? pr : n_seg - 1 - pr;
        if (h == 1 && sg == pr) break;
        // triangle weights of the segment's bins, from its edges
        const float inv = tabs.seg_inv[sg];
        const float lo = tabs.seg_lo[sg], hi = tabs.seg_hi[sg];
        float a = 0.0f, c = 0.0f;
        const int k0 = seg[sg], k1 = seg[sg + 1];
        float fk = bin_hz * static_cast<float>(k0);  // 10 k Hz, exact
        // four bins per step, their reads issued together, then one step over
        // the last 0..3 bins whose reads past the segment (at most index 802,
        // inside the frame's slots) are dropped
        int k = k0;
        for (; k + 4 <= k1; k += 4) {
          float q[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) q[i] = p[k + i];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a = fmaf(fk - lo, q[i], a);  // filter sg, rising side
            c = fmaf(hi - fk, q[i], c);  // filter sg - 1, falling side
            fk += bin_hz;
          }
        }
        if (k < k1) {
          float q[3];
#pragma unroll
          for (int i = 0; i < 3; ++i) q[i] = p[k + i];
#pragma unroll
          for (int i = 0; i < 3; ++i) {
            const float pk = k + i < k1 ? q[i] : 0.0f;
            a = fmaf(fk - lo, pk, a);
            c = fmaf(hi - fk, pk, c);
            fk += bin_hz;
          }
        }
        pf[2 * ff * kSlots + kAOff + sg] = a * inv;
        pf[2 * ff * kSlots + kCOff + sg] = c * inv;
      }
    }
    __syncthreads();
    // output it = ff * n_mels + j of the block; ff = floor((it + 0.5) / n_mels)
    // in fp32 is exact: it < 1024 puts the product within 1.3e-4 of the
    // quotient, whose distance to an integer is at least 0.5 / 128
    const int64_t n_valid = n_frames - g0 < kFramesPerBlock ? n_frames - g0 : kFramesPerBlock;
    const int n_out = static_cast<int>(n_valid) * n_mels;
    const float inv_n = 1.0f / static_cast<float>(n_mels);
    float* lm_out = logmel != nullptr ? logmel + g0 * n_mels : nullptr;
    uint8_t* lv_out = levels != nullptr ? levels + g0 * n_mels : nullptr;
    for (int it = tid; it < n_out; it += kThreads) {
      const int ff = static_cast<int>((static_cast<float>(it) + 0.5f) * inv_n);
      const int j = it - ff * n_mels;
      const float m = pf[2 * ff * kSlots + kAOff + j] + pf[2 * ff * kSlots + kCOff + j + 1];
      // ln m = ln 2 * log2 m with the hardware log2 (about 1 ulp; m >= 1e-10 is normal)
      const float l = 0.69314718055994531f * __builtin_amdgcn_logf(fmaxf(m, kLogFloor));
      if (lm_out != nullptr) lm_out[it] = l;
      if (lv_out != nullptr) lv_out[it] = static_cast<uint8_t>(quantize(l, tabs));
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
  hipLaunchKernelGGL(frontend_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     tabs, audio, n_samples_total, sample_off, frame_off, n_clips, n_frames,
                     static_cast<double>(n_clips) / static_cast<double>(n_frames), carry, logmel, levels);
  return hipGetLastError();
}

}  // namespace dmel
