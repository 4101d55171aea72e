// Blockwise attention kernels for head dim 64 (the template in attn_bf16.h),
// one translation unit per head dim so that they compile in parallel.
#include "attn_bf16.h"

namespace bpt {
hipError_t launch_attention_bf16_d64(const void *Q, const void *K, const void *Vt, void *A,
                                      int64_t batch, int64_t seq, int64_t heads, int causal,
                                      int rows, int keys, hipStream_t stream, float *nlse) {
  return attn::launch_d<64>(Q, K, Vt, A, batch, seq, heads, causal, rows, keys, stream, nlse);
}
} // namespace bpt
