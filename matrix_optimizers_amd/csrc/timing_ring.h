// Bookkeeping of the optional per-launch timing: a bounded record of event
// pairs still in flight, folded into per-phase sums once they have been read.
//
// Every timed launch leaves one pair of events (before, after) on its stream.
// Left to pile up until the caller reads them, a long run keeps every pair
// alive: a SOAP step is about 15k launches, so a 20-step pass would hold about
// 600k live events, each backed by a runtime signal.  Here at most `cap`
// pairs are outstanding.  Past that, the oldest half is drained: the host
// waits for their second event (recorded hundreds of launches ago, so the
// queue ahead of the device stays that deep), adds the elapsed time to its
// phase's sum and returns both events to a free list for reuse.
//
// The event operations are a template parameter (Ops), so the same logic runs
// with HIP events in the library and with counted fake events in a host-only
// test.  Ops provides:
//   using Event = ...;
//   int  create(Event*)                 0 on success
//   void destroy(Event)
//   int  elapsed_ms(Event a, Event b, float* ms)   waits for b; 0 on success
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <deque>
#include <vector>

template <class Ops, int NPHASE>
class TimingRing {
public:
    using Event = typename Ops::Event;

    explicit TimingRing(Ops ops = Ops(), size_t cap = 512) : ops_(ops), cap_(cap < 2 ? 2 : cap) {}
    ~TimingRing() { reset_device(-1); }

    // The free list holds events of one device; a different device drops it.
    void reset_device(int dev) {
        for (Event e : free_) ops_.destroy(e);
        free_.clear();
        dev_ = dev;
    }
    int device() const { return dev_; }

    // An event from the free list, or a new one.
    int take(Event* ev) {
        if (!free_.empty()) {
            *ev = free_.back();
            free_.pop_back();
            return 0;
        }
        return ops_.create(ev);
    }
    // Returns an event that was taken but never pushed (a failed launch path).
    void give_back(Event ev) { free_.push_back(ev); }

    // Records one timed launch; drains the oldest half once `cap` are pending.
    // A failure while draining drops that pair's time and is reported by the
    // next read(), not by the launch being recorded.
    void push(int phase, Event a, Event b) {
        pending_.push_back(Rec{phase, a, b});
        if (pending_.size() > cap_) (void)drain(pending_.size() - cap_ / 2);
    }

    // Drains every pending pair, then adds the per-phase sums to ms / launches
    // and clears them.  Returns 0, or the first failure seen since the last read.
    int read(double* ms, int64_t* launches) {
        int st = drain(pending_.size());
        if (st == 0) st = sticky_;
        for (int p = 0; p < NPHASE; ++p) {
            ms[p] += ms_[p];
            launches[p] += cnt_[p];
            ms_[p] = 0.0;
            cnt_[p] = 0;
        }
        sticky_ = 0;
        return st;
    }

    // Drains every pending pair into the sums (kept until the next read).
    void flush_pending() { (void)drain(pending_.size()); }

    size_t pending() const { return pending_.size(); }
    size_t free_events() const { return free_.size(); }
    size_t cap() const { return cap_; }

private:
    struct Rec { int phase; Event a, b; };

    int drain(size_t n) {
        int first = 0;
        for (size_t i = 0; i < n && !pending_.empty(); ++i) {
            Rec r = pending_.front();
            pending_.pop_front();
            float f = 0.f;
            const int e = ops_.elapsed_ms(r.a, r.b, &f);
            if (e != 0) {
                if (first == 0) first = e;
            } else if (r.phase >= 0 && r.phase < NPHASE) {
                ms_[r.phase] += double(f);
                cnt_[r.phase] += 1;
            }
            free_.push_back(r.a);
            free_.push_back(r.b);
        }
        if (first != 0 && sticky_ == 0) sticky_ = first;
        return first;
    }

    Ops ops_;
    size_t cap_;
    int dev_ = -1;
    std::deque<Rec> pending_;
    std::vector<Event> free_;
    double ms_[NPHASE] = {};
    int64_t cnt_[NPHASE] = {};
    int sticky_ = 0;
};
