// Dispatch of the bf16 blockwise attention (kernels in attn_bf16.h, one
// translation unit per head dim: attn_bf16_d32.hip, _d64.hip, _d128.hip).
#include "bpt_internal.h"

namespace bpt {

hipError_t launch_attention_bf16_d32(const void *, const void *, const void *, void *, int64_t,
                                     int64_t, int64_t, int, int, int, hipStream_t, float *);
hipError_t launch_attention_bf16_d64(const void *, const void *, const void *, void *, int64_t,
                                     int64_t, int64_t, int, int, int, hipStream_t, float *);
hipError_t launch_attention_bf16_d128(const void *, const void *, const void *, void *, int64_t,
                                      int64_t, int64_t, int, int, int, hipStream_t, float *);

int attention_tile_rows(int64_t B_q) {
  for (int r = 256; r > 16; r /= 2)
    if (B_q % r == 0) return r;
  return 16;
}

int attention_stage_keys(int64_t B_kv) {
  for (int k = 64; k > 16; k /= 2)
    if (B_kv % k == 0) return k;
  return 16;
}

hipError_t launch_attention_bf16(const void *Q, const void *K, const void *Vt, void *A,
                                 int64_t batch, int64_t seq, int64_t heads, int64_t head_dim,
                                 int causal, hipStream_t stream, float *nlse, int rows, int keys) {
  if (batch <= 0 || seq <= 0) return hipSuccess;
  if (seq % 16 != 0 || seq * head_dim > ((int64_t)1 << 30)) return hipErrorInvalidValue;
  switch (head_dim) {
  case 32:
    return launch_attention_bf16_d32(Q, K, Vt, A, batch, seq, heads, causal, rows, keys, stream,
                                     nlse);
  case 64:
    return launch_attention_bf16_d64(Q, K, Vt, A, batch, seq, heads, causal, rows, keys, stream,
                                     nlse);
  case 128:
    return launch_attention_bf16_d128(Q, K, Vt, A, batch, seq, heads, causal, rows, keys, stream,
                                      nlse);
  default:
    return hipErrorInvalidValue;
  }
}

} // namespace bpt
