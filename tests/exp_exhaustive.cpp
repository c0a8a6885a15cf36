// Host build of the raster kernels' exact exponentials, exp_rn(x) and the forward's exp_neg_rn(-x), checked against
// float(exp(double(x))) - the oracle's definition of the fp32 e^x - for every float x in [-5.55, 0] (the arguments
// the kernels evaluate). Prints "<floats> <mismatches of exp_rn> <mismatches of exp_neg_rn>".
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "raster_common.hpp"

int main(int argc, char** argv) {
  const int nt = argc > 1 ? std::atoi(argv[1]) : 8;
  const float lo = -5.55f;
  uint32_t last;
  std::memcpy(&last, &lo, 4);  // negative floats: the bit pattern grows with the magnitude
  std::vector<double> neg_tab(2 * gsr::kExpTabN);
  for (uint32_t k = 0; k < gsr::kExpTabN; ++k) gsr::exp_neg_entry(k, neg_tab.data() + 2 * k);
  std::atomic<uint64_t> total{0}, bad{0}, bad_neg{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&, t] {
      uint64_t n = 0, m = 0, mn = 0;
      for (uint64_t u = 0x80000000ull + t; u <= last; u += nt) {
        const uint32_t v = uint32_t(u);
        float x;
        std::memcpy(&x, &v, 4);
        const float ref = float(std::exp(double(x)));
        n += 1;
        m += gsr::exp_rn(x, gsr::kExp2Tab) != ref;
        mn += gsr::exp_neg_rn(-x, neg_tab.data()) != ref;
      }
      total += n;
      bad += m;
      bad_neg += mn;
    });
  for (auto& th : pool) th.join();
  std::printf("%llu %llu %llu\n", (unsigned long long)total.load(), (unsigned long long)bad.load(),
              (unsigned long long)bad_neg.load());
  return 0;
}
