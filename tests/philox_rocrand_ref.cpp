// Host-only driver that evaluates rocRAND's Philox4x32-10 engine (an
// independent, open-source implementation shipped with ROCm) so the tests can
// compare the oracle's Philox against it.  Reads lines "c0 c1 c2 c3 k0 k1"
// (decimal) on stdin, prints the four output words per line.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

// ten_rounds(counter, key) is a protected member of the engine; a derived class
// exposes it so any counter/key pair can be evaluated directly.
struct philox_ref : rocrand_device::philox4x32_10_engine {
  using rocrand_device::philox4x32_10_engine::ten_rounds;
};

int main() {
  unsigned int c[4], k[2];
  while (std::scanf("%u %u %u %u %u %u", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    philox_ref eng;
    uint4 ctr{c[0], c[1], c[2], c[3]};
    uint2 key{k[0], k[1]};
    uint4 r = eng.ten_rounds(ctr, key);
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
