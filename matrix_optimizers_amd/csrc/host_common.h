// Host-side helpers shared by the entry points of the C ABI: argument
// checks, the work-list upload and the optional per-launch timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <vector>

#include "../../include/mo.h"

namespace mo_host {

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

inline bool finite(float x) { return std::isfinite(x); }

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
    int writable;
};

inline int64_t elem_size(int32_t dt) { return dt == MO_BF16 ? 2 : 4; }

// Byte range touched by a rows x cols row-major matrix with stride ld.
inline Range matrix_range(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t es,
                          int writable) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    uintptr_t hi = lo + uintptr_t(((rows - 1) * ld + cols) * es);
    return Range{lo, hi, writable};
}

// Any overlap between a writable range and any other range?  (Sorts rs.)
bool ranges_conflict(std::vector<Range>& rs);

// Copies `bytes` of host memory to the device buffer `dst`, ordered on s,
// through a pinned staging buffer owned by the calling thread.
hipError_t upload(const void* src, size_t bytes, void* dst, hipStream_t s);

// Per-launch timing (mo_profile_enable): whether it is on for the calling
// thread, and the record of one launch bracketed by events a and b.  At most
// kTimingCap pairs are pending per thread; past that the oldest are read into
// per-phase sums (timing_ring.h), so a long timed run holds a bounded number
// of live events.
constexpr size_t kTimingCap = 512;
bool profiling_on();
void profile_push(int phase, hipEvent_t a, hipEvent_t b);
// A timing event on the current device, reused from the thread's free list
// when one is there, so timing adds two event records per launch and, after
// the first kTimingCap launches, no event creation.
hipError_t profile_event(hipEvent_t* ev);
// Returns an event taken by profile_event that was never pushed.
void profile_giveback(hipEvent_t ev);

// Debug mode (environment variable MO_DEBUG_SYNC=1, read once per process):
// every launch is followed by a stream synchronisation and an error check, so
// a failing kernel is named by its phase instead of surfacing at a later sync.
bool debug_sync_on();
hipError_t debug_sync_check(int phase, hipStream_t s, hipError_t launch_status);

template <typename F>
hipError_t timed_launch(int phase, hipStream_t s, F&& launch) {
    if (!profiling_on()) {
        const hipError_t le = launch();
        return debug_sync_on() ? debug_sync_check(phase, s, le) : le;
    }
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e;
    if ((e = profile_event(&a)) != hipSuccess) return e;
    if ((e = profile_event(&b)) != hipSuccess) {
        profile_giveback(a);
        return e;
    }
    if ((e = hipEventRecord(a, s)) != hipSuccess) {
        profile_giveback(a);
        profile_giveback(b);
        return e;
    }
    hipError_t le = launch();
    if ((e = hipEventRecord(b, s)) != hipSuccess) {
        // a was recorded; both go back unread
        profile_giveback(a);
        profile_giveback(b);
        return e;
    }
    profile_push(phase, a, b);
    return debug_sync_on() ? debug_sync_check(phase, s, le) : le;
}

}  // namespace mo_host
