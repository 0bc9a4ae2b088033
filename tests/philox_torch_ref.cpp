// Host-side reference for Philox4x32-10 words, built from PyTorch's own engine
// (ATen/core/PhiloxRNGEngine.h). Used only by the oracle's CPU pin test.
//
// stdin: lines "c0 c1 c2 c3 k0 k1" (decimal uint32); stdout: "o0 o1 o2 o3".
// torch's engine keys on seed = k0 | k1 << 32 and counts with
// counter = (offset_lo, offset_hi, subsequence_lo, subsequence_hi).
#include <ATen/core/PhiloxRNGEngine.h>

#include <cstdint>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
    uint64_t subseq = (uint64_t)c2 | ((uint64_t)c3 << 32);
    uint64_t offset = (uint64_t)c0 | ((uint64_t)c1 << 32);
    at::philox_engine eng(seed, subseq, offset);
    uint32_t o[4];
    for (int i = 0; i < 4; ++i) o[i] = eng(10);
    std::printf("%u %u %u %u\n", o[0], o[1], o[2], o[3]);
  }
  return 0;
}
