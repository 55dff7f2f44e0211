// coherent.h -- device-scope handoff between workgroups of one kernel.
//
// On gfx950 each XCD has its own L2, so a plain store made by one workgroup
// is not guaranteed visible to a workgroup on another XCD until the kernel
// ends, and a release/acquire fence writes back or invalidates a whole L2.
// For small handoffs (partial results consumed by the last workgroup to
// finish) we instead store and load the handed-over values with
// device-scope relaxed atomics (sc1 accesses, coherent per access), wait for
// the stores to complete, then count arrivals with an atomic add.
#pragma once

#include "kernels.h"

namespace moe {

__device__ inline void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float load_coherent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void store_coherent64(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t load_coherent64(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this thread's earlier stores have completed (vmcnt(0)).  The
// signal fence keeps the compiler from moving memory operations across it.
__device__ inline void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), no wait on lgkm/exp
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace moe
