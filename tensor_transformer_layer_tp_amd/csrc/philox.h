// Counter-based random numbers for the dropout variants.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace tpk {

// Philox4x64-10 (Salmon et al., SC 2011): ten rounds of two 64x64 -> 128-bit
// products on words 0 and 2, the key advanced by two Weyl constants between
// rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t& x0, uint64_t& x1, uint64_t& x2, uint64_t& x3, uint64_t k0,
                                              uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B97F4A7C15ull;
      k1 += 0xBB67AE8584CAA73Bull;
    }
    const uint64_t lo0 = M0 * x0, hi0 = __umul64hi(M0, x0);
    const uint64_t lo1 = M1 * x2, hi1 = __umul64hi(M1, x2);
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
  }
}

// 16-bit lane q of a Philox block (q = 0..15), in the order of the four words.
__device__ __forceinline__ uint32_t philox_lane16(const uint64_t (&w)[4], int q) {
  return (uint32_t)((w[q >> 2] >> (16 * (q & 3))) & 0xFFFFull);
}

}  // namespace tpk
