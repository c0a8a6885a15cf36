// Host build of the raster kernels' exact exponential, checked against float(exp(double(x))) - the oracle's
// definition of the fp32 e^x - for every float x in [-5.55, 0] (the arguments the kernels evaluate). Prints
// "<floats> <mismatches>".
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
  std::atomic<uint64_t> total{0}, bad{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&, t] {
      uint64_t n = 0, m = 0;
      for (uint64_t u = 0x80000000ull + t; u <= last; u += nt) {
        const uint32_t v = uint32_t(u);
        float x;
        std::memcpy(&x, &v, 4);
        const float ref = float(std::exp(double(x)));
        n += 1;
        m += gsr::exp_rn(x, gsr::kExp2Tab) != ref;
      }
      total += n;
      bad += m;
    });
  for (auto& th : pool) th.join();
  std::printf("%llu %llu\n", (unsigned long long)total.load(), (unsigned long long)bad.load());
  return 0;
}
