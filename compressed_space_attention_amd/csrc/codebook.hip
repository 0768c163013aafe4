// Host-side quantiser codebooks of the record widths.
//
// 3 bits: the eight Gaussian Lloyd-Max levels the specification of this path
// fixes (the pages name 3-bit scalar quantisation but print no levels),
// held in iq_device.h.
// 4 bits (FreeToken issue #141, Proposed Solution: the rotation-based KV
// quantisers listed there span 3 and 4 bits): the 16-level Lloyd-Max quantiser of
// N(0, 1), computed here once per process by Lloyd's iteration.  The density
// is symmetric, so the iteration runs on the eight positive levels with the
// middle threshold fixed at 0: thresholds = midpoints of adjacent levels,
// each level = the mean of N(0, 1) over its cell.
#include <math.h>
#include <stdint.h>

#include "iq_device.h"
#include "iq_internal.h"

namespace iq {
namespace {

double std_pdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * M_PI); }

// P(a <= X < b) for a < b, from erfc (no cancellation in the tails)
double std_mass(double a, double b) {
  const double r = 1.0 / sqrt(2.0);
  return 0.5 * (erfc(a * r) - (isinf(b) ? 0.0 : erfc(b * r)));
}

// f16 rounding (round to nearest even) of x in the normal f16 range.
double round_to_f16(double x) {
  int e = 0;
  frexp(x, &e);                       // x = f 2^e, f in [0.5, 1)
  const double ulp = ldexp(1.0, e - 11);  // 11 significant bits
  return nearbyint(x / ulp) * ulp;
}

uint16_t f16_bits(double h) {  // h: a positive normal f16 value
  int e = 0;
  const double f = frexp(h, &e);  // h = (2f) 2^(e-1), 2f in [1, 2)
  const int mant = (int)lrint((2.0 * f - 1.0) * 1024.0);
  return (uint16_t)(((e - 1 + 15) << 10) | mant);
}

Codebook4 make_codebook4() {
  Codebook4 cb{};
  // positive levels c[0..7]; thresholds b[0] = 0, b[k] = (c[k-1] + c[k]) / 2, b[8] = inf
  double c[8];
  for (int k = 0; k < 8; ++k) c[k] = 0.35 * (k + 0.5);
  for (int it = 0; it < 1000000; ++it) {
    double b[9];
    b[0] = 0.0;
    for (int k = 1; k < 8; ++k) b[k] = 0.5 * (c[k - 1] + c[k]);
    b[8] = INFINITY;
    double moved = 0.0;
    for (int k = 0; k < 8; ++k) {
      const double nk = (std_pdf(b[k]) - std_pdf(b[k + 1])) / std_mass(b[k], b[k + 1]);
      moved = fmax(moved, fabs(nk - c[k]));
      c[k] = nk;
    }
    if (moved <= 1e-16) break;
  }
  for (int k = 0; k < 8; ++k) {
    cb.level[8 + k] = c[k];
    cb.level[7 - k] = -c[k];
  }
  for (int j = 0; j < 15; ++j) cb.thr[j] = (float)(0.5 * (cb.level[j] + cb.level[j + 1]));
  cb.thr[7] = 0.0f;
  for (int k = 0; k < 7; ++k) cb.lv.t[k] = cb.thr[8 + k];

  // alpha in [1, 2) putting the eight alpha-scaled magnitudes closest (in the
  // worst relative error) to f16 values
  double best = INFINITY, best_alpha = 1.0;
  for (int i = 0; i < (1 << 20); ++i) {
    const double a = 1.0 + ldexp((double)i, -20);
    double worst = 0.0;
    for (int k = 7; k >= 0 && worst < best; --k) {
      const double v = a * c[k];
      worst = fmax(worst, fabs(round_to_f16(v) - v) / v);
    }
    if (worst < best) {
      best = worst;
      best_alpha = a;
    }
  }
  cb.alpha = (float)best_alpha;
  cb.alpha_rel_err = best;
  uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
  for (int k = 0; k < 8; ++k) {
    const uint16_t h = f16_bits(round_to_f16((double)cb.alpha * c[k]));
    cb.level_f16[k] = h;
    lo[k / 4] |= (uint32_t)(h & 0xFF) << (8 * (k % 4));
    hi[k / 4] |= (uint32_t)(h >> 8) << (8 * (k % 4));
  }
  cb.lv.lo0123 = lo[0];
  cb.lv.lo4567 = lo[1];
  cb.lv.hi0123 = hi[0];
  cb.lv.hi4567 = hi[1];
  return cb;
}

}  // namespace

const Codebook4& codebook4() {
  static const Codebook4 cb = make_codebook4();  // thread-safe one-time initialisation
  return cb;
}

}  // namespace iq
