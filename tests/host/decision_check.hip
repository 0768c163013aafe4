// Host check of the kernels' quantiser decisions (no GPU): code_of (3-bit) and
// nibble_of (4-bit) search the thresholds by bisection; here they are compared
// with plain threshold counting (the quantiser's definition: a code is the
// number of thresholds u reaches, ties going up) on every float within 64 ulps
// of every threshold, at the signed zeros and infinities, and on 2e7 normal
// samples.  Exit status 0 when every decision agrees.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "../../compressed_space_attention_amd/csrc/iq_device.h"

using iq::Levels4;

static unsigned count3(float u) {
  const float t[7] = {-iq::kThr3[2], -iq::kThr3[1], -iq::kThr3[0], 0.f, iq::kThr3[0], iq::kThr3[1], iq::kThr3[2]};
  unsigned c = 0;
  for (float x : t) c += (u >= x);
  return c;
}
static unsigned count4_nibble(float u, const Levels4& lv) {
  unsigned c = 0;  // code over the 15 thresholds -t6 .. -t0, 0, t0 .. t6
  for (int k = 6; k >= 0; --k) c += (u >= -lv.t[k]);
  c += (u >= 0.f);
  for (int k = 0; k < 7; ++k) c += (u >= lv.t[k]);
  return c >= 8 ? c - 8 : 15 - c;  // stored sign-magnitude nibble
}
static float step(float x, int n) {
  unsigned b;
  memcpy(&b, &x, 4);
  b += (unsigned)n;
  memcpy(&x, &b, 4);
  return x;
}

int main(int argc, char** argv) {
  // the 4-bit thresholds (fp32 midpoints of the 16-level Gaussian codebook)
  Levels4 lv{{0.25822166f, 0.5224037f, 0.79954976f, 1.0992858f, 1.4371388f, 1.8435318f, 2.4008033f}, 0, 0, 0, 0};
  long n = 0, bad = 0;
  auto test = [&](float u) {
    ++n;
    if (iq::code_of(u) != count3(u) || iq::nibble_of(u, lv) != count4_nibble(u, lv)) {
      if (bad < 5) printf("u=%.9g code %u/%u nibble %u/%u\n", u, iq::code_of(u), count3(u),
                          iq::nibble_of(u, lv), count4_nibble(u, lv));
      ++bad;
    }
  };
  std::vector<float> ts = {iq::kThr3[0], iq::kThr3[1], iq::kThr3[2]};
  for (float t : lv.t) ts.push_back(t);
  for (float t : ts)
    for (int sgn = -1; sgn <= 1; sgn += 2)
      for (int d = -64; d <= 64; ++d) test(step(sgn * t, d));
  for (int d = 0; d <= 64; ++d) {
    test(step(0.f, d));
    test(-step(0.f, d));
  }
  test(INFINITY);
  test(-INFINITY);
  const long samples = argc > 1 ? atol(argv[1]) : 20000000;
  std::mt19937 rng(1);
  std::normal_distribution<float> nd(0.f, 1.5f);
  for (long i = 0; i < samples; ++i) test(nd(rng));
  printf("%ld decisions, %ld disagree\n", n, bad);
  return bad != 0;
}
