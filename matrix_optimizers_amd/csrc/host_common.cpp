// Host-side helpers shared by the entry points of the C ABI: the alias check,
// the pinned staging upload of a work list, and the per-launch timing record.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/mo.h"
#include "host_common.h"
#include "timing_ring.h"

namespace mo_host {

// Any overlap between a writable range and any other range?
bool ranges_conflict(std::vector<Range>& rs) {
    std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) {
        return a.lo < b.lo || (a.lo == b.lo && a.hi < b.hi);
    });
    // Sweep: keep the furthest end seen so far among writable and among all.
    uintptr_t max_hi_any = 0, max_hi_w = 0;
    bool have = false;
    for (const Range& r : rs) {
        if (r.hi == r.lo) continue;
        if (have) {
            if (r.lo < max_hi_w) return true;               // overlaps an earlier writable
            if (r.writable && r.lo < max_hi_any) return true;  // writable overlaps earlier
        }
        have = true;
        max_hi_any = std::max(max_hi_any, r.hi);
        if (r.writable) max_hi_w = std::max(max_hi_w, r.hi);
    }
    return false;
}


// ---- pinned staging for the work-list upload -----------------------------------
// The list is copied host->device on the caller's stream.  The source is a
// pinned buffer owned by the calling thread and reused by its next call once
// the previous copy has completed (an event marks that); it lives until the
// process ends.
struct Staging {
    void* buf = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    int dev = -1;
    bool pending = false;
};
namespace {
thread_local Staging g_stage;
}  // namespace

hipError_t upload(const void* src, size_t bytes, void* dst, hipStream_t s) {
    hipError_t e;
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if (g_stage.pending) {
        if ((e = hipEventSynchronize(g_stage.ev)) != hipSuccess) return e;
        g_stage.pending = false;
    }
    if (g_stage.dev != dev) {
        if (g_stage.ev) (void)hipEventDestroy(g_stage.ev);
        g_stage.ev = nullptr;
        if ((e = hipEventCreateWithFlags(&g_stage.ev, hipEventDisableTiming)) != hipSuccess) return e;
        g_stage.dev = dev;
    }
    if (g_stage.cap < bytes) {
        if (g_stage.buf) (void)hipHostFree(g_stage.buf);
        g_stage.buf = nullptr;
        g_stage.cap = 0;
        if ((e = hipHostMalloc(&g_stage.buf, bytes, hipHostMallocDefault)) != hipSuccess) return e;
        g_stage.cap = bytes;
    }
    std::memcpy(g_stage.buf, src, bytes);
    if ((e = hipMemcpyAsync(dst, g_stage.buf, bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
        return e;
    if ((e = hipEventRecord(g_stage.ev, s)) != hipSuccess) return e;
    g_stage.pending = true;
    return hipSuccess;
}

// ---- optional per-launch timing --------------------------------------------------
// The pending event pairs of the calling thread, bounded (timing_ring.h).
struct HipEventOps {
    using Event = hipEvent_t;
    int create(Event* ev) { return int(hipEventCreate(ev)); }
    void destroy(Event ev) { (void)hipEventDestroy(ev); }
    int elapsed_ms(Event a, Event b, float* ms) {
        hipError_t e = hipEventSynchronize(b);
        if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
        return int(e);
    }
};
using Ring = TimingRing<HipEventOps, MO_PHASE_COUNT>;

namespace {
thread_local bool g_prof_on = false;
// Allocated on first use and never freed: destroying events from a thread-exit
// destructor could run after the HIP runtime has shut down.
thread_local Ring* g_ring = nullptr;

Ring& ring() {
    if (!g_ring) g_ring = new Ring(HipEventOps(), kTimingCap);
    return *g_ring;
}
}  // namespace

bool profiling_on() { return g_prof_on; }

hipError_t profile_event(hipEvent_t* ev) {
    int dev = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    Ring& r = ring();
    if (dev != r.device()) {
        // pairs recorded on the previous device go into the sums first
        r.flush_pending();
        r.reset_device(dev);
    }
    return hipError_t(r.take(ev));
}

void profile_giveback(hipEvent_t ev) { ring().give_back(ev); }

void profile_push(int phase, hipEvent_t a, hipEvent_t b) { ring().push(phase, a, b); }

bool debug_sync_on() {
    static const bool on = [] {
        const char* v = std::getenv("MO_DEBUG_SYNC");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

hipError_t debug_sync_check(int phase, hipStream_t s, hipError_t launch_status) {
    hipError_t e = launch_status;
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess)
        std::fprintf(stderr, "libmo: phase %d failed: %s\n", phase, hipGetErrorString(e));
    return e;
}

}  // namespace mo_host

using namespace mo_host;

extern "C" {

mo_status mo_profile_enable(int32_t enable) {
    g_prof_on = enable != 0;
    return MO_OK;
}

mo_status mo_profile_read(double* ms, int64_t* launches) {
    if (!ms || !launches) return MO_ERR_INVALID_ARG;
    return ring().read(ms, launches) == 0 ? MO_OK : MO_ERR_HIP;
}

}  // extern "C"
