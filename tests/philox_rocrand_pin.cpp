// Reads lines "c0 c1 c2 c3 k0 k1" (decimal uint32) from stdin and prints the four output words of
// rocRAND's Philox4x32-10 block function for that counter and key. Used only to pin the oracle's
// own Philox implementation against an independent one (rocRAND's open-source header).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct Block : rocrand_device::philox4x32_10_engine {
  using philox4x32_10_engine::ten_rounds;
};

int main() {
  Block e;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 r = e.ten_rounds(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
