// Device helpers shared by the Markov chain kernels: the running-argmax key
// and the previous-token lookup.
#pragma once

#include "common.h"
#include "internal.h"

namespace dspark {

// Running argmax of one (request, position) as a 64-bit key whose unsigned
// order is (score ascending, then index descending): the largest key holds
// the best score with ties on the lowest index, in whatever order the tiles
// arrive.
__device__ __forceinline__ unsigned long long best_key(float score, int idx) {
  if (score == 0.f) score = 0.f;                   // -0 ranks equal to +0
  uint32_t u = __float_as_uint(score);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(idx));
}

__device__ __forceinline__ int best_index(unsigned long long key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}

// Raise the key; the relaxed read first skips atomics that cannot change it
// (keys only grow, so a stale read only costs an unneeded atomic).
__device__ __forceinline__ void push_best(unsigned long long* slot, float score, int idx) {
  const unsigned long long k = best_key(score, idx);
  const unsigned long long cur = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (k > cur) atomicMax(slot, k);
}

// x_{j-1} of request b: the anchor for j == 0, else the final key of j-1
__device__ __forceinline__ int prev_token(const StepArgs& a, int b, int j) {
  return j == 0 ? a.anchor[b] : best_index(a.best[b * a.gamma + j - 1]);
}

}  // namespace dspark
