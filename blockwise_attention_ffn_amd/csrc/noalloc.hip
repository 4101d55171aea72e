// bpt_layer_fwd_noalloc: the layer forward for callers that cannot allocate
// device memory. Its workspace (Q, K, V^T, A and the FFN group's H, the
// layout bpt_layer_workspace_bytes_ex describes) lives in `scratch`, a
// file-scope device array of fixed size that the code object carries: each
// GPU the library runs on holds its own copy from the module's load until
// the process ends.
//
// In host code `scratch` names a host-side stand-in, not the array's device
// address. The address is obtained once per device, with that device
// current, through hipGetSymbolAddress, and kept in g_scratch[]; only that
// pointer is ever handed to the layer.
#include "../../include/bpt.h"
#include "bpt_internal.h"

#include <hip/hip_runtime.h>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = BPT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices]; // device address of `scratch` per device, once known
std::mutex g_scratch_mu;

// the scratch's device address on the current device
int scratch_here(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BPT_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return BPT_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return BPT_OK;
}

} // namespace

extern "C" int bpt_layer_fwd_noalloc(const bpt_shape *shape, const void *x, const void *Wqkv,
                                     const void *bqkv, const void *Wo, const void *bo,
                                     const void *W1, const void *b1, const void *W2,
                                     const void *b2, int64_t B_q, int64_t B_kv, int causal,
                                     int64_t ffn_rows, void *out, bpt_stream_t stream) {
  size_t need = 0;
  int st = bpt_layer_workspace_bytes_ex(shape, B_q, B_kv, causal, ffn_rows, &need);
  if (st) return st;
  if (need > kScratchBytes) return BPT_ERR_SCRATCH;
  if ((st = bpt::check_device())) return st;
  void *ws = nullptr;
  if ((st = scratch_here(&ws))) return st;
  return bpt_layer_fwd_ex(shape, x, Wqkv, bqkv, Wo, bo, W1, b1, W2, b2, B_q, B_kv, causal,
                          ffn_rows, out, ws, kScratchBytes, stream);
}
