// philox_device.h -- the counter-based generator the verifier draws its
// uniforms from, shared by the library's translation units. Not part of the
// C ABI.
//
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds over a 4 x 32-bit counter; each round
// takes the two 32 x 32 -> 64-bit products of counter words 0 and 2 with the
// round multipliers, xors their high halves with the other two words and the
// key, and the key advances by the Weyl increments between rounds.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svrng {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
    #pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        const uint32_t lo0 = kPhiloxM0 * c0, hi0 = __umulhi(kPhiloxM0, c0);
        const uint32_t lo1 = kPhiloxM1 * c2, hi1 = __umulhi(kPhiloxM1, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0;
        const uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return make_uint4(c0, c1, c2, c3);
}

// The top 24 bits of a word as a uniform in [0, 1), exact in fp32 and fp64.
__device__ __forceinline__ double word_to_uniform(uint32_t w) {
    return (double)(w >> 8) * (1.0 / 16777216.0);
}

}  // namespace svrng
