// timing.cpp -- optional per-kernel timing with HIP events (instrumentation; off by default).
//
// While enabled, each timed launch site records an event pair on the stream the kernel is
// launched on.  tria_timing_read waits for the recorded pairs, adds their elapsed times per
// timer and returns the events to a pool.  Nothing is recorded while timing is off, so the hot
// calls then make no runtime calls of their own.
#include <mutex>
#include <vector>

#include "tria_internal.h"

namespace tria {
namespace {

struct Pending {
    int which;
    hipEvent_t start, stop;
};

struct TimingState {
    std::mutex mu;
    bool on = false;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> pool;
};

TimingState &state()
{
    static TimingState s;
    return s;
}

hipEvent_t take_event(TimingState &s)
{
    if (!s.pool.empty()) {
        hipEvent_t e = s.pool.back();
        s.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

KernelTimer::KernelTimer(int which, hipStream_t st) : which_(which), st_(st)
{
    TimingState &s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    if (!s.on) return;
    start_ = take_event(s);
    stop_ = take_event(s);
    if (!start_ || !stop_ || hipEventRecord(start_, st_) != hipSuccess) {
        if (start_) s.pool.push_back(start_);
        if (stop_) s.pool.push_back(stop_);
        start_ = stop_ = nullptr;
    }
}

KernelTimer::~KernelTimer()
{
    if (!start_) return;
    TimingState &s = state();
    std::lock_guard<std::mutex> lock(s.mu);
    if (hipEventRecord(stop_, st_) == hipSuccess) {
        s.pending.push_back({which_, start_, stop_});
    } else {
        s.pool.push_back(start_);
        s.pool.push_back(stop_);
    }
}

}  // namespace tria

extern "C" {

tria_status tria_timing_enable(int on)
{
    tria::TimingState &s = tria::state();
    std::lock_guard<std::mutex> lock(s.mu);
    s.on = on != 0;
    return TRIA_OK;
}

tria_status tria_timing_read(double *ms, int *launches)
{
    if (!ms || !launches) return TRIA_E_INVALID;
    for (int i = 0; i < TRIA_TIMER_COUNT; ++i) {
        ms[i] = 0.0;
        launches[i] = 0;
    }
    tria::TimingState &s = tria::state();
    std::lock_guard<std::mutex> lock(s.mu);
    tria_status st = TRIA_OK;
    for (const tria::Pending &p : s.pending) {
        float t = 0.f;
        if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&t, p.start, p.stop) != hipSuccess) {
            st = TRIA_E_DEVICE;
        } else if (p.which >= 0 && p.which < TRIA_TIMER_COUNT) {
            ms[p.which] += t;
            launches[p.which] += 1;
        }
        s.pool.push_back(p.start);
        s.pool.push_back(p.stop);
    }
    s.pending.clear();
    return st;
}

}  // extern "C"
