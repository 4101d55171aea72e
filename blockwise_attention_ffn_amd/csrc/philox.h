// Training-mode dropout masks for the gfx950 kernels: Philox4x64-10
// (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2,
// 3", SC 2011) and the mapping of its output onto (token, channel) keep
// flags. Internal.
//
// Mask definition (element (token t, channel j) of dropout site z under a
// 64-bit seed): key (seed, z), counter (t, j / 16, 0, 0); the four 64-bit
// output words hold sixteen 16-bit uniforms, channel j takes number j % 16
// (word (j % 16) / 4, bits 16·(j % 4) upwards); the element is dropped iff
// its uniform is below the threshold T = round(p·65536).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {
namespace dev {

// Philox4x64 with 10 rounds, in place on c[0..3]. A round maps
// (c0, c1, c2, c3) to (hi(M1·c2) ^ c1 ^ k0, lo(M1·c2), hi(M0·c0) ^ c3 ^ k1,
// lo(M0·c0)); the key is bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Keep flags of the 16 channels 16·j16 .. 16·j16 + 15 of token t: bit i set
// iff channel 16·j16 + i is kept.
__device__ __forceinline__ uint32_t dropout_keep16(uint64_t seed, uint32_t site, uint64_t t,
                                                   uint64_t j16, uint32_t threshold) {
  uint64_t c[4] = {t, j16, 0, 0};
  philox4x64_10(c, seed, site);
  uint32_t keep = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t u = (uint32_t)(c[i >> 2] >> (16 * (i & 3))) & 0xFFFFu;
    keep |= (u >= threshold ? 1u : 0u) << i;
  }
  return keep;
}

} // namespace dev
} // namespace bpt
