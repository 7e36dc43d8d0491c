// Reference outputs of Philox-4x32-10 from rocRAND (the ROCm random-number
// library's own block function, reached through its engine class), for the
// oracle's Philox pin. Host code only. Reads lines "c0 c1 c2 c3 k0 k1"
// (decimal 32-bit words) on stdin and prints the four output words of each.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct PhiloxBlock : rocrand_device::philox4x32_10_engine {
  uint4 operator()(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};

int main() {
  PhiloxBlock block;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint4 o = block(make_uint4(c0, c1, c2, c3), make_uint2(k0, k1));
    std::printf("%u %u %u %u\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
