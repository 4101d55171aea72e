// Keep masks of the training-mode dropout, written out for testing: the
// generator and mapping of csrc/philox.h, which the GEMM epilogues apply
// inline.
#include "bpt_internal.h"
#include "philox.h"

namespace bpt {
namespace {

// one thread per (token, 16-channel block): 16 bytes of flags
__global__ __launch_bounds__(256) void dropout_keep_kernel(uint8_t *__restrict__ keep, int64_t tokens,
                                                           int64_t blocks, int64_t token0,
                                                           uint64_t seed, uint32_t site,
                                                           uint32_t threshold) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= tokens * blocks) return;
  const int64_t t = i / blocks, j16 = i - t * blocks;
  const uint32_t k = dev::dropout_keep16(seed, site, (uint64_t)(token0 + t), (uint64_t)j16, threshold);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[q] |= ((k >> (q * 4 + e)) & 1u) << (8 * e);
  }
  uint4 v;
  v.x = w[0];
  v.y = w[1];
  v.z = w[2];
  v.w = w[3];
  *reinterpret_cast<uint4 *>(keep + i * 16) = v;
}

} // namespace

hipError_t launch_dropout_keep(uint8_t *keep, int64_t tokens, int64_t channels, int64_t token0,
                               uint64_t seed, uint32_t site, uint32_t threshold, hipStream_t stream) {
  if (tokens <= 0 || channels <= 0) return hipSuccess;
  if (channels % 16 != 0) return hipErrorInvalidValue;
  const int64_t blocks = channels / 16, n = tokens * blocks;
  const int64_t grid = (n + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dropout_keep_kernel, dim3((unsigned)grid), dim3(256), 0, stream, keep, tokens,
                     blocks, token0, seed, site, threshold);
  return hipGetLastError();
}

} // namespace bpt
