// Host-only test of the per-launch timing bookkeeping (timing_ring.h) with
// fake events: the number of pending pairs stays bounded, every recorded
// duration reaches its phase's sum exactly once, events are recycled rather
// than created per launch, and a failed read is reported once.
#include <cstdio>
#include <cstdlib>
#include <map>

#include "timing_ring.h"

struct FakeOps {
    using Event = int;
    int* created;
    int* destroyed;
    int* waits;
    std::map<int, float>* stamp;   // event -> time it was "recorded"
    int fail_event = -1;           // elapsed_ms fails when b == fail_event
    int create(Event* e) { *e = ++*created; return 0; }
    void destroy(Event) { ++*destroyed; }
    int elapsed_ms(Event a, Event b, float* ms) {
        ++*waits;
        if (b == fail_event) return 7;
        *ms = (*stamp)[b] - (*stamp)[a];
        return 0;
    }
};

#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            std::fprintf(stderr, "FAILED %s at line %d\n", #c, __LINE__); \
            return 1;                                                 \
        }                                                             \
    } while (0)

int main() {
    int created = 0, destroyed = 0, waits = 0;
    std::map<int, float> stamp;
    FakeOps ops{&created, &destroyed, &waits, &stamp};
    const size_t cap = 64;
    TimingRing<FakeOps, 3> ring(ops, cap);
    ring.reset_device(0);
    double want[3] = {0, 0, 0};
    size_t max_pending = 0;
    const int launches = 100000;
    float t = 0.f;
    for (int i = 0; i < launches; ++i) {
        int a, b;
        CHECK(ring.take(&a) == 0);
        CHECK(ring.take(&b) == 0);
        CHECK(a != b);
        const int phase = i % 3;
        const float d = float((i % 7) + 1) * 0.25f;   // exact in fp32 and fp64
        stamp[a] = t;
        stamp[b] = t + d;
        t += 8.f;
        if (t > 1000.f) t = 0.f;
        want[phase] += d;
        ring.push(phase, a, b);
        if (ring.pending() > max_pending) max_pending = ring.pending();
    }
    CHECK(max_pending <= cap + 1);
    // events in use never exceed two per pending pair plus the free list
    CHECK(size_t(created) <= 2 * (cap + 1));
    double ms[3] = {0, 0, 0};
    int64_t n[3] = {0, 0, 0};
    CHECK(ring.read(ms, n) == 0);
    CHECK(ring.pending() == 0);
    CHECK(n[0] + n[1] + n[2] == launches);
    for (int p = 0; p < 3; ++p) CHECK(ms[p] == want[p]);
    CHECK(waits == launches);
    // a second read reports nothing new
    double ms2[3] = {0, 0, 0};
    int64_t n2[3] = {0, 0, 0};
    CHECK(ring.read(ms2, n2) == 0 && n2[0] + n2[1] + n2[2] == 0);

    // a failing pair drained by push is dropped and reported by the next read only
    TimingRing<FakeOps, 3> r2(ops, 4);
    r2.reset_device(0);
    int a, b;
    r2.take(&a);
    r2.take(&b);
    stamp[a] = 0.f;
    stamp[b] = 1.f;
    r2.push(0, a, b);
    for (int i = 0; i < 10; ++i) {
        int x, y;
        r2.take(&x);
        r2.take(&y);
        stamp[x] = 0.f;
        stamp[y] = 2.f;
        r2.push(1, x, y);
    }
    double m3[3] = {0, 0, 0};
    int64_t n3[3] = {0, 0, 0};
    CHECK(r2.read(m3, n3) == 0);
    CHECK(n3[0] == 1 && n3[1] == 10 && m3[1] == 20.0);

    int fa = 1000001, fb = 1000002;
    stamp[fa] = 0.f;
    stamp[fb] = 1.f;
    TimingRing<FakeOps, 3> r4(FakeOps{&created, &destroyed, &waits, &stamp, fb}, 4);
    r4.reset_device(0);
    r4.push(2, fa, fb);
    for (int i = 0; i < 10; ++i) {
        int x, y;
        r4.take(&x);
        r4.take(&y);
        stamp[x] = 0.f;
        stamp[y] = 1.f;
        r4.push(1, x, y);   // drains the failing pair; the launch is not failed
    }
    double m4[3] = {0, 0, 0};
    int64_t n4[3] = {0, 0, 0};
    CHECK(r4.read(m4, n4) == 7);
    CHECK(n4[2] == 0 && n4[1] == 10);
    double m5[3] = {0, 0, 0};
    int64_t n5[3] = {0, 0, 0};
    CHECK(r4.read(m5, n5) == 0);

    // a device change destroys the free events
    const int before = destroyed;
    const size_t nfree = r4.free_events();
    r4.reset_device(1);
    CHECK(destroyed - before == int(nfree) && r4.free_events() == 0 && r4.device() == 1);
    std::printf("timing ring OK (max pending %zu, events created %d)\n", max_pending, created);
    return 0;
}
