// la_ctl.h -- device side of the workspace control block (la_internal.h,
// struct Ctl): how a launch whose workgroups hand data to each other through
// flags takes its epoch, and how bounded waits report that they gave up.
//
// Epochs.  A flag is a 64-bit word set to the epoch of the call that
// published it; a reader waits until the flag equals its own call's epoch.
// A call launched directly takes its epoch from the host (a process-wide
// counter with the top bits 0xFFF8, passed as a kernel argument).  A call
// captured into a graph cannot: every replay would repeat the captured
// argument.  Its kernel gets 0 instead and takes the epoch from the
// generation word gen of the control block: each workgroup loads gen at its
// start and takes epoch_of(gen) (top bits 0xFFF4); once that value is in a
// register it counts itself in (arrive), and the workgroup that arrives
// last -- when every other workgroup of the grid has already loaded gen --
// stores gen = epoch and resets the counter, ready for the next replay or
// call on the stream.  The two kinds of epoch never equal each other, both
// are NaN patterns (no float or index a workspace region held before can
// equal one), and each kind increases call after call.  (The counter costs
// one same-address atomic per workgroup, which is why direct calls do not
// use it.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_internal.h"

namespace la_ctl {

using la_internal::Ctl;

__device__ __forceinline__ uint64_t epoch_of(uint64_t gen) {
  return 0xFFF4000000000000ull | ((gen + 1) & 0x0000FFFFFFFFFFFFull);
}

// The control words a workgroup needs, loaded once at its start.
struct CtlView {
  uint64_t gen;
  uint32_t limit, skew;
};
__device__ __forceinline__ CtlView ctl_load(const Ctl* c) {
  CtlView v;
  v.gen = __hip_atomic_load(&c->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.limit = __hip_atomic_load(&c->wait_limit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.skew = __hip_atomic_load(&c->wait_skew, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
__device__ __forceinline__ uint32_t wait_limit(const CtlView& v) {
  return v.limit ? v.limit : la_internal::kDefaultWaitLimit;
}

// Count the calling workgroup in.  The asm statement takes the loaded
// generation as an operand, so the load has returned before it, and its
// memory clobber keeps the counter's atomic after it: gen is read before
// this workgroup can be the one that advances it.  Returns the counter's
// previous value, for ctl_leave (the caller need not wait for it before).
__device__ __forceinline__ uint32_t ctl_arrive(Ctl* c, const CtlView& v) {
  asm volatile("" ::"v"(v.gen) : "memory");
  return __hip_atomic_fetch_add(&c->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The last workgroup of the grid (of every dimension) to arrive stores the
// new generation and resets the counter (called by the thread that arrived,
// after its last use of the epoch).
__device__ __forceinline__ void ctl_leave(Ctl* c, uint32_t old, uint64_t epoch) {
  if (old == gridDim.x * gridDim.y * gridDim.z - 1) {
    __hip_atomic_store(&c->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c->gen, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void ctl_fail(Ctl* c, uint32_t bit) {
  __hip_atomic_fetch_or(&c->err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace la_ctl
