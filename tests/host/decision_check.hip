// Host check of the kernels' quantiser decisions (no GPU): code_of (3-bit: a
// magnitude count with a sign fix-up) and nibble_of (4-bit: bisection) are
// compared with plain threshold counting (the quantiser's definition: a code
// is the number of thresholds u reaches, ties going up) on every float within
// 64 ulps of every threshold, at the signed zeros and infinities, on normal
// samples, and (code_of, argument "all") on every float that is not a NaN;
// and the placement of a selector's codes in a packed group.  Exit status 0
// when everything agrees.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <random>
#include <thread>
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

// The two placements of a selector's fields in a group (shifts and masks, or
// a switch) agree, and the fields of selectors 0..7 OR-ed together are the
// group that selectors_to_group packs.
static long check_fields(std::mt19937& rng) {
  long bad = 0;
  for (int it = 0; it < 200000; ++it) {
    uint32_t z[8], a0 = 0, a1 = 0, a2 = 0;
    for (int s = 0; s < 8; ++s) {
      z[s] = 0;
      for (int b = 0; b < 4; ++b) z[s] |= (uint32_t)(rng() & 7u) << (8 * b);
      uint32_t p0, p1, p2, q0, q1, q2;
      iq::selector_fields<true>(s, z[s], p0, p1, p2);
      iq::selector_fields<false>(s, z[s], q0, q1, q2);
      if (p0 != q0 || p1 != q1 || p2 != q2) ++bad;
      a0 |= p0;
      a1 |= p1;
      a2 |= p2;
    }
    uint32_t g0, g1, g2;
    iq::selectors_to_group(z, g0, g1, g2);
    if (a0 != g0 || a1 != g1 || a2 != g2) ++bad;
  }
  return bad;
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
  if (argc > 2 && strcmp(argv[2], "all") == 0) {
    // every bit pattern but the NaNs, split over threads
    std::atomic<long> bad_all{0}, n_all{0};
    const unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> pool;
    for (unsigned w = 0; w < nt; ++w)
      pool.emplace_back([&, w] {
        long b = 0, c = 0;
        const uint64_t lo = (1ull << 32) * w / nt, hi = (1ull << 32) * (w + 1) / nt;
        for (uint64_t i = lo; i < hi; ++i) {
          float u;
          const uint32_t bits = (uint32_t)i;
          memcpy(&u, &bits, 4);
          if (u != u) continue;
          ++c;
          b += iq::code_of(u) != count3(u);
        }
        bad_all += b;
        n_all += c;
      });
    for (auto& t : pool) t.join();
    printf("code_of on every non-NaN float: %ld values, %ld disagree\n", (long)n_all, (long)bad_all);
    bad += bad_all;
  }
  const long bad_fields = check_fields(rng);
  printf("selector fields: 200000 groups, %ld disagree\n", bad_fields);
  return bad != 0 || bad_fields != 0;
}
