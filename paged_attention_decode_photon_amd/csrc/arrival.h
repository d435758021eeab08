// Arrival counters for work split over several wavefronts or workgroups,
// tagged with the epoch of the call that uses them.
//
// Several producers compute partial results of one output segment; the one
// whose arrival completes the segment's count merges them.  The counter is a
// 64-bit word in caller-provided workspace memory: the high half holds the
// epoch of the call that owns it, the low half the units counted so far.
// The host library numbers its calls (never 0).  A word holding 0, or a
// value tagged with the current epoch, is valid for the current call; any
// other value is stale: memory that was never cleared, or an earlier call
// that stopped before its last arrival.
//
// Claim.  Before counting, a producer swaps the word from 0 to (epoch, 0)
// with a compare-and-swap, issued together with its partial-record stores so
// that the wait for those stores also covers it (or earlier, where the
// decode kernel measured that faster).  If the swap returns a
// stale value, a second swap replaces exactly that value; when it fails,
// another producer of this call has claimed the word already.  Every
// producer claims before it counts, and the claim precedes its count in the
// word's modification order (same thread, same address), so no count ever
// lands on a stale value, whatever the memory held before the call.
//
// Release.  The producer that completes the count merges and stores 0, so a
// call that finishes leaves every counter at 0 and the next call needs no
// second swap.
//
// A stale value whose high half equals the current epoch is not detected:
// one chance in 2^32 for arbitrary memory contents.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace photon {

__device__ __forceinline__ uint64_t epoch_tag(uint32_t epoch) { return (uint64_t)epoch << 32; }

// First swap of a claim: returns the value the word held (0 on success).
__device__ __forceinline__ uint64_t claim_counter(uint64_t *ctr, uint32_t epoch)
{
    uint64_t seen = 0;
    __hip_atomic_compare_exchange_strong(ctr, &seen, epoch_tag(epoch), __ATOMIC_RELAXED,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return seen;
}

// Count `units` arrivals on a claimed word (`seen` is what claim_counter
// returned) and return the units counted before them in this call.
__device__ __forceinline__ uint32_t arrive_counter(uint64_t *ctr, uint32_t epoch, uint64_t seen,
                                                   uint32_t units)
{
    if (seen != 0 && (uint32_t)(seen >> 32) != epoch) {
        // stale contents: replace exactly them, then let the swap finish
        // before counting
        uint64_t expected = seen;
        __hip_atomic_compare_exchange_strong(ctr, &expected, epoch_tag(epoch), __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    const uint64_t old =
        __hip_atomic_fetch_add(ctr, (uint64_t)units, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)old;
}

// The producer that completed the count, after merging.
__device__ __forceinline__ void release_counter(uint64_t *ctr)
{
    __hip_atomic_store(ctr, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace photon
