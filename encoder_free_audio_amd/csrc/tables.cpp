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
#include <algorithm>
#include <cmath>
#include <cstring>

#include "internal.h"

namespace dmel {

namespace {
double hz_to_mel(double f) { return 2595.0 * std::log10(1.0 + f / 700.0); }
double mel_to_hz(double m) { return 700.0 * (std::pow(10.0, m / 2595.0) - 1.0); }
}  // namespace

bool build_host_tables(HostTables* t, int n_mels, int n_levels, float lo, float hi) {
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

  // the LDS image: window (its first half and middle), twa, tw1600 and the
  // quantizer edges
  std::memset(t->lds_image, 0, sizeof(t->lds_image));
  std::memcpy(t->lds_image + kImgWindow, t->window, sizeof(float) * (kWindow / 2 + 1));
  std::memcpy(t->lds_image + kImgTwa, t->twa, sizeof(t->twa));
  std::memcpy(t->lds_image + kImgTw1600, t->tw1600, sizeof(t->tw1600));
  std::memcpy(t->lds_image + kImgEdge, t->q_edge, sizeof(float) * (n_levels + 1));

  // Filter schedule (FrontTables::mel_w).  Filter j is the weighted sum over
  // its bins [seg_start[j], seg_start[j + 2]): rising (f - e_j) / (e_{j+1} - e_j)
  // over segment j, falling (e_{j+2} - f) / (e_{j+2} - e_{j+1}) over segment
  // j + 1, each weight times 1/4 (exact) for the kernel's 4 |X|^2 powers.
  // Filters are taken longest first in sets of 8 (one side each).  Inside a
  // set, longest first, each filter takes the free slot s that needs the
  // fewest chunks once its reads start at the bin = s mod 8 at or below its
  // range (never below bin -8).  A side costs the chunks of its costliest
  // slot, and the sets go, costliest first, to the round with the least work
  // so far that has a side free.
  static_assert(kMelMaxSides + 4 <= 8, "a round's entries must fit 8 ints");
  int order[kMaxMels], len[kMaxMels];
  for (int j = 0; j < n_mels; ++j) {
    order[j] = j;
    len[j] = t->seg_start[j + 2] - t->seg_start[j];
  }
  std::stable_sort(order, order + n_mels, [&](int a, int b) { return len[a] > len[b]; });
  const int n_sets = (n_mels + 7) / 8;
  const int max_sides = (n_mels + 31) / 32;
  constexpr int kSets = (kMaxMels + 7) / 8;
  int set_filt[kSets][8], set_first[kSets][8], set_cost[kSets];
  for (int s = 0; s < n_sets; ++s) {
    bool used[8] = {false, false, false, false, false, false, false, false};
    set_cost[s] = 0;
    for (int slot = 0; slot < 8; ++slot) {
      set_filt[s][slot] = -1;
      set_first[s][slot] = slot - 8;
    }
    for (int i = 8 * s; i < 8 * s + 8 && i < n_mels; ++i) {
      const int j = order[i];
      const int first = t->seg_start[j];
      int best = -1, best_chunks = 0, best_pad = 0;
      for (int slot = 0; slot < 8; ++slot) {
        if (used[slot]) continue;
        const int pad = ((first - slot) % 8 + 8) % 8;
        if (first - pad < -8) continue;
        const int chunks = (len[j] + pad + 7) / 8;
        if (best < 0 || chunks < best_chunks || (chunks == best_chunks && pad < best_pad)) {
          best = slot;
          best_chunks = chunks;
          best_pad = pad;
        }
      }
      used[best] = true;
      set_filt[s][best] = j;
      set_first[s][best] = first - best_pad;
      if (best_chunks > set_cost[s]) set_cost[s] = best_chunks;
    }
  }
  int set_order[kSets];
  for (int s = 0; s < n_sets; ++s) set_order[s] = s;
  std::stable_sort(set_order, set_order + n_sets, [&](int a, int b) { return set_cost[a] > set_cost[b]; });
  int load[4] = {0, 0, 0, 0}, sides[4] = {0, 0, 0, 0};
  int set_of[4][kMelMaxSides];
  for (int i = 0; i < n_sets; ++i) {
    const int s = set_order[i];
    int best = -1;
    for (int r = 0; r < 4; ++r) {
      if (sides[r] < max_sides && (best < 0 || load[r] < load[best])) best = r;
    }
    set_of[best][sides[best]++] = s;
    load[best] += set_cost[s];
  }
  std::memset(t->mel_w, 0, sizeof(t->mel_w));
  std::memset(t->mel_round, 0, sizeof(t->mel_round));
  for (int i = 0; i < 4 * kMelMaxSides * 8; ++i) {
    t->mel_filt[i] = -1;
    t->mel_first[i] = (i % 8) - 8;
  }
  int base = 0;  // chunks so far
  for (int r = 0; r < 4; ++r) {
    int* rd = t->mel_round + 8 * r;
    rd[0] = base;
    rd[2] = sides[r];
    int c0 = 0;  // chunk of the round where the side starts
    for (int h = 0; h < sides[r]; ++h) {
      const int s = set_of[r][h];
      const int chunks = set_cost[s];
      if (base + c0 + chunks > kMelChunks) return false;
      rd[3 + h] = c0;
      for (int slot = 0; slot < 8; ++slot) {
        const int j = set_filt[s][slot];
        const int pb = set_first[s][slot];
        t->mel_filt[8 * (kMelMaxSides * r + h) + slot] = j;
        t->mel_first[8 * (kMelMaxSides * r + h) + slot] = pb;
        if (pb + 8 * chunks > kMelReadEnd) return false;
        if (j < 0) continue;
        for (int k = t->seg_start[j]; k < t->seg_start[j + 2]; ++k) {
          const double f = static_cast<double>(k) * kSampleRate / kNfft;
          const double w = k < t->seg_start[j + 1] ? (f - edges[j]) / (edges[j + 1] - edges[j])
                                                   : (edges[j + 2] - f) / (edges[j + 2] - edges[j + 1]);
          const int i = k - pb;  // position in the slot's chunks
          const int c = base + c0 + i / 8;
          t->mel_w[4 * (16 * c + 8 * ((i % 8) / 4) + slot) + (i % 4)] = static_cast<float>(0.25 * w);
        }
      }
      c0 += chunks;
    }
    rd[3 + sides[r]] = c0;
    rd[1] = c0;
    base += c0;
  }
  // the schedule in the LDS image, when it fits
  t->mel_in_lds = base <= kMelLdsChunks ? 1 : 0;
  if (t->mel_in_lds) {
    std::memcpy(t->lds_image + kImgMelW, t->mel_w, sizeof(float) * 64 * base);
    std::memcpy(t->lds_image + kImgMelFirst, t->mel_first, sizeof(t->mel_first));
    std::memcpy(t->lds_image + kImgMelFilt, t->mel_filt, sizeof(t->mel_filt));
  }
  return true;
}

}  // namespace dmel
