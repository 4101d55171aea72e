// Keep masks of the training-mode dropout, written out for testing, and
// applied to a gradient for the backward: the generator and mapping of
// csrc/philox.h, which the GEMM epilogues apply inline in the forward.
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

// one thread per (row, 16-column block): out = in ∘ keep · scale, rounded
// to bf16 once (the backward's gradient of a dropped branch)
__global__ __launch_bounds__(256) void dropout_scale_kernel(const __bf16 *__restrict__ in,
                                                            __bf16 *__restrict__ out, int64_t rows,
                                                            int64_t blocks, int64_t ld,
                                                            int64_t token0, uint64_t seed,
                                                            uint32_t site, uint32_t threshold,
                                                            float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * blocks) return;
  const int64_t r = i / blocks, j16 = i - r * blocks;
  const uint32_t k = dev::dropout_keep16(seed, site, (uint64_t)(token0 + r), (uint64_t)j16, threshold);
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  const bf16x8 *src = reinterpret_cast<const bf16x8 *>(in + r * ld + j16 * 16);
  bf16x8 *dst = reinterpret_cast<bf16x8 *>(out + r * ld + j16 * 16);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const bf16x8 v = src[half];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      o[e] = (k >> (half * 8 + e)) & 1u ? (__bf16)((float)v[e] * scale) : (__bf16)0.f;
    dst[half] = o;
  }
}

} // namespace

hipError_t launch_dropout_scale_bf16(const void *in, void *out, int64_t rows, int64_t cols,
                                     int64_t ld, int64_t token0, uint64_t seed, uint32_t site,
                                     uint32_t threshold, float scale, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 16 != 0 || ld % 8 != 0 || ld < cols) return hipErrorInvalidValue;
  const int64_t blocks = cols / 16, n = rows * blocks;
  const int64_t grid = (n + 255) / 256;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dropout_scale_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const __bf16 *>(in), reinterpret_cast<__bf16 *>(out), rows,
                     blocks, ld, token0, seed, site, threshold, scale);
  return hipGetLastError();
}

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
