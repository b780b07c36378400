// Host construction of the front end's constant tables, in fp64, stored fp32.
//
// Readings of the open steps ("Inside Inkling: Audio Design", Part 1 names an
// 80-channel log-mel over a 1600-sample window; the page gives no window shape,
// FFT size or mel formula):
//  * periodic Hann window w[n] = 0.5 - 0.5 cos(2 pi n / 1600);
//  * 1600-point FFT computed as an 800-point complex FFT of the even/odd
//    sample pairs, so the twiddles needed are exp(-2 pi i m / 800) and, for the
//    final real-spectrum split, exp(-2 pi i k / 1600);
//  * 80 triangular filters on the HTK mel scale m(f) = 2595 log10(1 + f / 700),
//    82 edges equally spaced in mel from 0 Hz to 8000 Hz (outer edges set to
//    exactly 0 and 8000 Hz), unit peak, evaluated at bin frequencies 10 k Hz
//    (n_mel_bins filters and n_mel_bins + 2 edges in general);
//  * uniform quantizer over the clamp range [lo, hi] in n_levels steps, whose
//    edges are lo + ((hi - lo) * k) / n_levels evaluated in fp64.
#include <cmath>

#include "internal.h"

namespace dmel {

namespace {
double hz_to_mel(double f) { return 2595.0 * std::log10(1.0 + f / 700.0); }
double mel_to_hz(double m) { return 700.0 * (std::pow(10.0, m / 2595.0) - 1.0); }
}  // namespace

void build_host_tables(HostTables* t, int n_mels, int n_levels, float lo, float hi) {
  const double two_pi = 2.0 * M_PI;
  for (int n = 0; n < kWindow; ++n) {
    t->window[n] = static_cast<float>(0.5 - 0.5 * std::cos(two_pi * n / kWindow));
  }
  for (int m = 0; m < kHalf; ++m) {
    t->tw800[2 * m] = static_cast<float>(std::cos(two_pi * m / kHalf));
    t->tw800[2 * m + 1] = static_cast<float>(-std::sin(two_pi * m / kHalf));
  }
  for (int k = 0; k <= kHalf / 2; ++k) {
    t->tw1600[2 * k] = static_cast<float>(std::cos(two_pi * k / kNfft));
    t->tw1600[2 * k + 1] = static_cast<float>(-std::sin(two_pi * k / kNfft));
  }
  // pass-A twiddles of the 800 = 32 x 25 decomposition, transposed so that the
  // 32 threads of a frame read consecutive entries
  for (int k2 = 1; k2 < 25; ++k2) {
    for (int n1 = 0; n1 < 32; ++n1) {
      const int m = (n1 * k2) % kHalf;
      t->twa[2 * ((k2 - 1) * 32 + n1)] = static_cast<float>(std::cos(two_pi * m / kHalf));
      t->twa[2 * ((k2 - 1) * 32 + n1) + 1] = static_cast<float>(-std::sin(two_pi * m / kHalf));
    }
  }
  // mel filter edges
  double edges[kMaxMels + 2];
  const double mel_hi = hz_to_mel(kSampleRate / 2.0);
  for (int i = 0; i < n_mels + 2; ++i) edges[i] = mel_to_hz(mel_hi * i / (n_mels + 1));
  edges[0] = 0.0;
  edges[n_mels + 1] = kSampleRate / 2.0;
  // bin k (frequency f = 10 k Hz) lies in segment s when edges[s] <= f <
  // edges[s+1]; the last bin, at exactly 8000 Hz, closes the last segment.
  // Inside segment s the triangle of filter s rises and that of filter s - 1
  // falls.
  int s = 0;
  t->seg_start[0] = 0;
  for (int k = 0; k < kBins; ++k) {
    const double f = static_cast<double>(k) * kSampleRate / kNfft;
    while (s < n_mels && f >= edges[s + 1]) {
      ++s;
      t->seg_start[s] = k;
    }
  }
  while (s < n_mels + 1) t->seg_start[++s] = kBins;
  for (int g = 0; g <= n_mels; ++g) {
    t->seg_lo[g] = static_cast<float>(edges[g]);
    t->seg_hi[g] = static_cast<float>(edges[g + 1]);
    t->seg_inv[g] = static_cast<float>(1.0 / (edges[g + 1] - edges[g]));
  }
  // quantizer edges, rounded up to fp32 so that an fp32 comparison with them
  // is the exact comparison with the fp64 edge
  const double dlo = lo, dhi = hi;
  t->q_edge[0] = lo;
  for (int k = 1; k < n_levels; ++k) {
    const double e = dlo + ((dhi - dlo) * k) / n_levels;
    float f = static_cast<float>(e);
    if (static_cast<double>(f) < e) f = std::nextafter(f, INFINITY);
    t->q_edge[k] = f;
  }
  t->q_edge[n_levels] = hi;
}

}  // namespace dmel
