// Stores of results that only a later kernel reads, in whole 256-byte row
// segments (the logits): relaxed device-scope atomic stores, which write
// through the XCD's L2 (`sc1`), so a kernel that writes hundreds of MB ends
// without dirty L2 lines to write back.  (Scattered 4-byte results, such as
// top-k indices or packed Q words, measured slower this way: 70 -> 106 us
// and 21 -> 33 us on prefill.)  FP4IDX_STORE_THROUGH 0 turns them into plain
// stores (measurement builds).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef FP4IDX_STORE_THROUGH
#define FP4IDX_STORE_THROUGH 1
#endif

namespace fp4idx {

template <typename T>
__device__ __forceinline__ void store_through(T* p, T v) {
#if FP4IDX_STORE_THROUGH
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#else
  *p = v;
#endif
}

}  // namespace fp4idx
