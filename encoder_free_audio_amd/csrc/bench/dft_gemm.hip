// The log-mel front end (framing .. log) with the 1600-point DFT done as a
// matrix product on the matrix cores: the alternative that the LDS FFT of
// frontend.hip is measured against.
//
// "Inside Inkling: Audio Design", Part 1: 16 kHz audio, 1600-sample window,
// 800-sample hop, 80-channel log-mel.  The real DFT of a windowed frame f is
// X_k = sum_m f_m exp(-2 pi i k m / 1600), k = 0..800: as a product F D with
// D [1600, 1602] = [cos | -sin] columns.  bf16 matrix cores need the operands
// split: f = fh + fl and D = Dh + Dl with fh, fl, Dh, Dl bf16, and
// F D ~= Fh Dh + Fh Dl + Fl Dh (the dropped Fl Dl term and the split residues
// are ~2^-16 relative), computed as ONE product over K = 4800:
// A = [Fh | Fh | Fl] times B = [Dh | Dl | Dh]^T, fp32 accumulation.  Columns
// are padded to 1792 (a multiple of the 256-wide GEMM tile) with zero rows of B.
// A second kernel forms |X_k|^2, the mel filters, and the log.
//
// Work per frame: 2 * 1792 * 4800 = 17.2 MFLOP of matrix-core products (the
// FFT needs ~43 kFLOP), 9.6 KB of A written and read, 7.2 KB of spectrum
// written and read.
#include "bench_internal.h"

namespace dmel {
namespace {

constexpr int kDftCols = 1792;            // 801 real + 801 imaginary, padded
constexpr int kDftK = 3 * kWindow;         // 4800
constexpr int kThreadsD = 256;

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// B[j][kk]: column j of the DFT (j < 801: cos(2 pi j m / 1600); 801 <= j <
// 1602: -sin(2 pi (j - 801) m / 1600); beyond: 0) at m = kk mod 1600, as its
// bf16 high part for kk < 1600 and kk >= 3200, and its low part in between.
// The phase j m mod 1600 is exact in integers; sin and cos in fp64.
__global__ void __launch_bounds__(kThreadsD) dft_matrix_kernel(uint16_t* __restrict__ B) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreadsD + threadIdx.x;
  if (i >= static_cast<int64_t>(kDftCols) * kWindow) return;
  const int j = static_cast<int>(i / kWindow), m = static_cast<int>(i % kWindow);
  double v = 0.0;
  if (j < kBins) {
    v = cospi(static_cast<double>((j * m) % kWindow) / 800.0);
  } else if (j < 2 * kBins) {
    v = -sinpi(static_cast<double>(((j - kBins) * m) % kWindow) / 800.0);
  }
  const float vf = static_cast<float>(v);
  const uint16_t hi = bf16_rne(vf);
  const uint16_t lo = bf16_rne(static_cast<float>(v - static_cast<double>(bf16_f32(hi))));
  uint16_t* row = B + static_cast<int64_t>(j) * kDftK;
  row[m] = hi;
  row[kWindow + m] = lo;
  row[2 * kWindow + m] = hi;
}

__global__ void __launch_bounds__(kThreadsD) zero_kernel_f32(float* __restrict__ p, int n) {
  const int i = blockIdx.x * kThreadsD + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

__device__ __forceinline__ int clip_index(const int64_t* frame_off, int n_clips, int64_t g) {
  int lo = 0, hi = n_clips;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (frame_off[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// One workgroup per frame: A[g] = [fh | fh | fl] of the windowed frame
// f_n = w_n x[800 t - 800 + n] (the clip's carry, or zeros, before its first
// sample).
__global__ void __launch_bounds__(kThreadsD)
dft_frames_kernel(const float* __restrict__ window, const float* __restrict__ audio, int64_t n_samples_total,
                  const int64_t* __restrict__ sample_off, const int64_t* __restrict__ frame_off, int n_clips,
                  const float* __restrict__ carry, uint16_t* __restrict__ A) {
  __shared__ int64_t s_base;
  __shared__ int s_clip, s_first;
  const int64_t g = blockIdx.x;
  if (threadIdx.x == 0) {
    const int c = clip_index(frame_off, n_clips, g);
    const int64_t t = g - frame_off[c];
    s_clip = c;
    s_first = t == 0;
    s_base = sample_off[c] + static_cast<int64_t>(kHop) * t - kHop;
  }
  __syncthreads();
  uint16_t* row = A + g * kDftK;
  for (int n = threadIdx.x; n < kWindow; n += kThreadsD) {
    float x = 0.0f;
    if (s_first && n < kHop) {
      if (carry != nullptr) x = carry[static_cast<int64_t>(s_clip) * kHop + n];
    } else {
      const int64_t si = s_base + n;
      if (si >= 0 && si < n_samples_total) x = audio[si];
    }
    const float f = window[n] * x;
    const uint16_t hi = bf16_rne(f);
    const uint16_t lo = bf16_rne(f - bf16_f32(hi));
    row[n] = hi;
    row[kWindow + n] = hi;
    row[2 * kWindow + n] = lo;
  }
}

// One workgroup per frame: power of the 801 bins, the mel filters by
// triangle segment (as in frontend.hip), log with the 1e-10 floor.
__global__ void __launch_bounds__(kThreadsD)
dft_mel_kernel(FrontTables tabs, const float* __restrict__ X, float* __restrict__ logmel) {
  __shared__ float p[kBins];
  __shared__ float sa[kMaxMels + 1], sc[kMaxMels + 1];
  const int64_t g = blockIdx.x;
  const float* x = X + g * kDftCols;
  for (int k = threadIdx.x; k < kBins; k += kThreadsD) {
    const float re = x[k], im = x[kBins + k];
    p[k] = re * re + im * im;
  }
  __syncthreads();
  const int n_mels = tabs.n_mels, n_seg = n_mels + 1;
  const float bin_hz = static_cast<float>(kSampleRate) / kNfft;
  for (int sg = threadIdx.x; sg < n_seg; sg += kThreadsD) {
    const float inv = tabs.seg_inv[sg], lo = tabs.seg_lo[sg], hi = tabs.seg_hi[sg];
    float a = 0.0f, c = 0.0f;
    for (int k = tabs.seg_start[sg]; k < tabs.seg_start[sg + 1]; ++k) {
      const float fk = bin_hz * static_cast<float>(k);
      a = fmaf((fk - lo) * inv, p[k], a);
      c = fmaf((hi - fk) * inv, p[k], c);
    }
    sa[sg] = a;
    sc[sg] = c;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < n_mels; j += kThreadsD)
    logmel[g * n_mels + j] = logf(fmaxf(sa[j] + sc[j + 1], kLogFloor));
}

}  // namespace

// The matrix buffer: B bf16 [1792, 4800], then 1792 fp32 zeros (the GEMM's bias).
constexpr size_t kMatBytes = static_cast<size_t>(kDftCols) * kDftK * 2;

size_t dft_matrix_bytes() { return kMatBytes + kDftCols * 4; }

size_t dft_gemm_workspace_bytes(int64_t n_frames) {
  const size_t n = static_cast<size_t>(n_frames);
  return (n * kDftK * 2 + 255) / 256 * 256 + n * kDftCols * 4;
}

hipError_t launch_dft_matrix(uint16_t* B, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(kDftCols) * kWindow;
  hipLaunchKernelGGL(dft_matrix_kernel, dim3(static_cast<unsigned>((n + kThreadsD - 1) / kThreadsD)), dim3(kThreadsD), 0,
                     stream, B);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_kernel_f32, dim3((kDftCols + kThreadsD - 1) / kThreadsD), dim3(kThreadsD), 0, stream,
                     reinterpret_cast<float*>(reinterpret_cast<char*>(B) + kMatBytes), kDftCols);
  return hipGetLastError();
}

hipError_t launch_dft_gemm_frames(const FrontTables& tabs, const float* audio, int64_t n_samples_total,
                                  const int64_t* sample_off, const int64_t* frame_off, int n_clips, int64_t n_frames,
                                  const float* carry, const uint16_t* B, float* logmel, void* workspace,
                                  hipStream_t stream) {
  const auto* zero_bias = reinterpret_cast<const float*>(reinterpret_cast<const char*>(B) + kMatBytes);
  if (n_frames <= 0) return hipSuccess;
  if (n_frames > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto* A = static_cast<uint16_t*>(workspace);
  auto* X = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                     (static_cast<size_t>(n_frames) * kDftK * 2 + 255) / 256 * 256);
  const dim3 grid(static_cast<unsigned>(n_frames));
  hipLaunchKernelGGL(dft_frames_kernel, grid, dim3(kThreadsD), 0, stream, tabs.window, audio, n_samples_total,
                     sample_off, frame_off, n_clips, carry, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_gemm_bf16(A, B, zero_bias, X, n_frames, kDftCols, kDftK, false, true, stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(dft_mel_kernel, grid, dim3(kThreadsD), 0, stream, tabs, X, logmel);
  return hipGetLastError();
}

}  // namespace dmel
