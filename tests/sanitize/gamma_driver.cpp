// gamma_driver.cpp -- drives the host-only adaptive draft-length policies
// (spec_gamma_policy_init / spec_gamma_next / spec_gamma_observe) through long
// seeded histories, edge batch sizes and invalid arguments, for a build under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Exit status 0 on success.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "specverify.h"

static uint64_t state = 7;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int main() {
  int failures = 0;
  auto expect = [&](bool ok, const char *what) {
    if (!ok) {
      std::fprintf(stderr, "%s\n", what);
      ++failures;
    }
  };
  expect(spec_gamma_policy_init(nullptr, SV_GAMMA_EMA) == SV_EINVAL, "NULL policy accepted");
  sv_gamma_policy bad;
  expect(spec_gamma_policy_init(&bad, 99) == SV_EINVAL, "unknown kind accepted");
  for (int kind : {SV_GAMMA_BY_BATCH, SV_GAMMA_EMA, SV_GAMMA_RATE_WINDOW}) {
    sv_gamma_policy p;
    expect(spec_gamma_policy_init(&p, kind) == SV_OK, "init failed");
    expect(spec_gamma_next(&p, 0) == SV_EINVAL, "batch size 0 accepted");
    expect(spec_gamma_observe(&p, nullptr, 4, 3) == SV_EINVAL, "NULL counts accepted");
    for (int step = 0; step < 3000; ++step) {  // past the window's wrap-around many times
      const int B = 1 + static_cast<int>(next_u64() % 600);
      const int g = spec_gamma_next(&p, B);
      expect(g >= 0 && g <= SV_GAMMA_MAX, "draft length out of range");
      std::vector<int32_t> acc(static_cast<size_t>(B));
      for (auto &a : acc) a = g > 0 ? static_cast<int32_t>(next_u64() % static_cast<uint64_t>(g + 1)) : 0;
      expect(spec_gamma_observe(&p, acc.data(), B, g) == SV_OK, "observe failed");
    }
    // the largest and smallest batch sizes the table and buckets know of
    for (int B : {1, 2, 31, 32, 64, 65, 128, 129, 512, 513, 1 << 20})
      expect(spec_gamma_next(&p, B) >= 0, "next failed at an edge batch size");
  }
  if (failures) return 1;
  std::printf("gamma driver ok\n");
  return 0;
}
