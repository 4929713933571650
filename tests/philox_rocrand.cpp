// Test helper: Philox4x32-10 outputs of rocRAND's host-callable engine for
// (counter, key) lines read from stdin ("c0 c1 c2 c3 k0 k1", decimal); one
// output line "r0 r1 r2 r3" each.  Used only to pin the CPU oracle's generator
// against an independent implementation; nothing on the HIP path uses it.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

namespace {
struct Rounds : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 c, uint2 k) { return ten_rounds(c, k); }
};
}  // namespace

int main() {
  Rounds e;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint4 r = e.run(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
