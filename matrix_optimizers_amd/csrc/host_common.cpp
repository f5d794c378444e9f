// Host-side helpers shared by the entry points of the C ABI: the alias check,
// the pinned staging upload of a work list, and the per-launch timing record.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/mo.h"
#include "host_common.h"

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
struct Timed { int phase; hipEvent_t a, b; };
thread_local bool g_prof_on = false;
thread_local std::vector<Timed> g_prof;

bool profiling_on() { return g_prof_on; }
void profile_push(int phase, hipEvent_t a, hipEvent_t b) { g_prof.push_back(Timed{phase, a, b}); }

// free timing events of the calling thread, all created on g_pool_dev
thread_local std::vector<hipEvent_t> g_pool;
thread_local int g_pool_dev = -1;

hipError_t profile_event(hipEvent_t* ev) {
    int dev = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if (dev != g_pool_dev) {
        for (hipEvent_t x : g_pool) (void)hipEventDestroy(x);
        g_pool.clear();
        g_pool_dev = dev;
    }
    if (!g_pool.empty()) {
        *ev = g_pool.back();
        g_pool.pop_back();
        return hipSuccess;
    }
    return hipEventCreate(ev);
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
    mo_status st = MO_OK;
    for (Timed& t : g_prof) {
        float f = 0.f;
        if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&f, t.a, t.b) != hipSuccess)
            st = MO_ERR_HIP;
        else if (t.phase >= 0 && t.phase < MO_PHASE_COUNT) {
            ms[t.phase] += double(f);
            launches[t.phase] += 1;
        }
        // back to the pool (events of another device than the pool's are destroyed)
        int dev = -1;
        if (hipGetDevice(&dev) == hipSuccess && dev == g_pool_dev) {
            g_pool.push_back(t.a);
            g_pool.push_back(t.b);
        } else {
            (void)hipEventDestroy(t.a);
            (void)hipEventDestroy(t.b);
        }
    }
    g_prof.clear();
    return st;
}

}  // extern "C"
