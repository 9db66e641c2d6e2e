// sync.hpp — explicit waits and a fence-free workgroup barrier for gfx950 kernels that keep
// direct-to-LDS loads in flight across a barrier.
#pragma once

#include <hip/hip_runtime.h>

namespace i8ql {

// s_waitcnt immediate (gfx9 encoding): vmcnt(vm) lgkmcnt(lgkm), expcnt left at its maximum.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Barrier with no memory fence.  A fence would wait for every load in flight; instead the
// waits before it are explicit, and the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Barrier that publishes LDS writes only: each wavefront waits for its own LDS operations
// (and scalar loads), not for the global loads and stores it has in flight, which a fence
// (__syncthreads) would wait for as well.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace i8ql
