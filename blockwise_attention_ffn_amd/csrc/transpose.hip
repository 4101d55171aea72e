// bf16 matrix transpose [R, C] -> [C, R] through LDS.
//
// The layer's weights arrive in the [in, out] layout of the x·W convention;
// the MFMA GEMM wants both operands contiguous along the reduction axis, so
// each weight is turned to [out, in] once per call (an HBM-bound pass over
// the weights, small next to the GEMMs that use them).
#include "bpt_internal.h"

namespace bpt {
namespace {

typedef unsigned short u16;

constexpr int TT = 64;

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const u16 *__restrict__ in,
                                                             u16 *__restrict__ out, int64_t R,
                                                             int64_t C) {
  __shared__ u16 tile[TT][TT + 2];
  const int64_t r0 = (int64_t)blockIdx.y * TT, c0 = (int64_t)blockIdx.x * TT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < TT; i += 4) {
    const int64_t r = r0 + ty + i, c = c0 + tx;
    if (r < R && c < C) tile[ty + i][tx] = in[r * C + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TT; i += 4) {
    const int64_t c = c0 + ty + i, r = r0 + tx;
    if (r < R && c < C) out[c * R + r] = tile[tx][ty + i];
  }
}

} // namespace

hipError_t launch_transpose_bf16(const void *in, void *out, int64_t R, int64_t C,
                                 hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  const int64_t gx = (C + TT - 1) / TT, gy = (R + TT - 1) / TT;
  if (gy > 65535 || gx > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)gx, (unsigned)gy), block(256);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, block, 0, stream,
                     reinterpret_cast<const u16 *>(in), reinterpret_cast<u16 *>(out), R, C);
  return hipGetLastError();
}

} // namespace bpt
