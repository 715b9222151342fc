// arrival.h -- how the workgroups that share one row tile (split-K pieces,
// the gate and up halves of a pair) hand their results to the last of them
// to arrive, inside one launch.
//
// Each workgroup puts its values into a workspace with device-scope atomic
// swaps, which are performed at the device's coherence point like the
// tile's arrival counter itself (device-scope atomics are coherent across
// the eight XCDs' L2s), waits for them to complete, then increments the
// counter.  The workgroup that sees the count n-1 takes every value back
// with atomic swaps that also zero them, and resets the counter: the
// workspace is all zero between calls.  No workgroup waits for another.
//
// Plain stores published by a device-scope release fence would also work,
// but that fence writes back the whole L2 of the XCD; with hundreds of
// workgroups fencing, it cost more than the launch it was meant to save.
#pragma once

#include <hip/hip_runtime.h>

namespace qg {

__device__ inline void put(float *p, float v) {
  (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The value stored at p, which is left zero.
__device__ inline float take(float *p) {
  return __hip_atomic_exchange(p, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: expcnt and
// lgkmcnt at their maxima, i.e. not waited for).
constexpr int kArriveVm0 = 0x0F70;

// Counts this workgroup's arrival on the tile's counter once its put()s
// have completed (called by one whole wavefront, the one that put); true
// for the last of n arrivals, whose take()s are issued after it and so see
// every earlier arrival's values.
__device__ inline bool arrive_last(int *cnt, int n) {
  // The swaps must be performed before the count: wait for every vector
  // memory operation of this wave (the compiler does not order relaxed
  // atomics to different addresses, nor wait for a swap whose result is
  // unused).
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kArriveVm0);
  asm volatile("" ::: "memory");
  int prev = 0;
  if ((threadIdx.x & 63) == 0) prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  return prev == n - 1;
}

// Sets the tile's counter back to zero (after the last arrival's take()s).
__device__ inline void arrive_reset(int *cnt) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qg
