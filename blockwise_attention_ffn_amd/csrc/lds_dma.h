// Device helpers shared by the gfx950 kernels: buffer descriptors, loads from
// memory straight into LDS, and explicit wait / barrier forms. Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {
namespace dev {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor over n bytes at p (stride 0, 32-bit data format
// word, unswizzled). Loads at byte offsets >= n return zeros. The fields
// pass through readfirstlane so that the descriptor is wave-uniform and
// lives in SGPRs (a descriptor in VGPRs costs a waterfall loop per load).
__device__ __forceinline__ i32x4 make_rsrc(const void *p, uint32_t n) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 r;
  r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = (int)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  r[2] = (int)__builtin_amdgcn_readfirstlane(n);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane L's bytes land at LDS address lds_dst + 16·L (the wave-uniform
// LDS address goes in M0). Written as inline asm with no outputs because
// the compiler's wait-count pass, seeing a load into LDS, makes every later
// LDS read wait for it (and for the FLAT form, global_load_lds, waits for
// every LDS read at each use). The kernels order each read of a loaded
// buffer after its load with their own explicit waits (wait_vm, barrier_vm);
// any wait the compiler adds is only stricter. The s_nop separates the M0
// write from the load.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t byte_off, const void *lds_dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void *)lds_dst;
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(byte_off), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// 4 bytes per lane (buffer_load_dword ... lds): lane L's word lands at LDS
// address lds_dst + 4·L. Same conventions as load_lds16.
__device__ __forceinline__ void load_lds4(i32x4 rsrc, uint32_t byte_off, const void *lds_dst) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lds_void *)lds_dst;
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(byte_off), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// s_waitcnt immediate: vmcnt(n) expcnt(7) lgkmcnt(0)
constexpr int waitcnt_vm_lgkm0(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }

// wait until at most VM of this wave's vector-memory loads are outstanding
// and all its LDS operations are done
template <int VM> __device__ __forceinline__ void wait_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));
  asm volatile("" ::: "memory");
}

// wait_vm<VM>, then s_barrier. Unlike __syncthreads it leaves up to VM of
// this wave's loads into LDS in flight.
template <int VM> __device__ __forceinline__ void barrier_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate: vmcnt(n) expcnt(7) lgkmcnt(15), i.e. no LDS wait
constexpr int waitcnt_vm_only(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// wait until at most VM of this wave's vector-memory loads are outstanding,
// then s_barrier; this wave's LDS reads may still be in flight (for callers
// whose every LDS read is consumed before the buffer it reads can be reused)
template <int VM> __device__ __forceinline__ void barrier_vm_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_only(VM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

} // namespace dev
} // namespace bpt
