// Optional per-kernel timing: when enabled, every kernel launch of the library is
// bracketed by two HIP events recorded on the launch stream; a read-out sums the
// elapsed times per kernel kind.  Off by default (one relaxed load per launch).

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "launch.h"

namespace retn {

namespace {

constexpr int kSlots = 4096;   // launches recorded between two read-outs

struct Rec {
    hipEvent_t begin, end;
    int kind;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_pool;       // event pairs, created on the first enable
int g_used = 0;                // records taken since the last read-out
int g_dropped = 0;             // launches not recorded because the pool was full

}  // namespace

bool prof_enabled() { return g_on.load(std::memory_order_relaxed); }

ProfScope::ProfScope(int kind, hipStream_t stream) : slot_(-1), stream_(stream) {
    if (!prof_enabled()) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_used >= static_cast<int>(g_pool.size())) {
        ++g_dropped;
        return;
    }
    slot_ = g_used++;
    g_pool[slot_].kind = kind;
    if (hipEventRecord(g_pool[slot_].begin, stream_) != hipSuccess) slot_ = -1;
}

ProfScope::~ProfScope() {
    if (slot_ < 0) return;
    (void)hipEventRecord(g_pool[slot_].end, stream_);
}

hipError_t prof_enable(bool on) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (on && g_pool.empty()) {
        g_pool.resize(kSlots);
        for (Rec& r : g_pool) {
            hipError_t e = hipEventCreate(&r.begin);
            if (e == hipSuccess) e = hipEventCreate(&r.end);
            if (e != hipSuccess) {
                g_pool.clear();
                return e;
            }
        }
    }
    g_used = 0;
    g_dropped = 0;
    g_on.store(on, std::memory_order_relaxed);
    return hipSuccess;
}

hipError_t prof_read(double* ms, int* count, int nkinds, int* dropped) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (int i = 0; i < nkinds; ++i) {
        ms[i] = 0.0;
        count[i] = 0;
    }
    hipError_t err = hipSuccess;
    for (int i = 0; i < g_used; ++i) {
        Rec& r = g_pool[i];
        hipError_t e = hipEventSynchronize(r.end);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.begin, r.end);
        if (e != hipSuccess) {
            err = e;
            continue;
        }
        if (r.kind >= 0 && r.kind < nkinds) {
            ms[r.kind] += t;
            ++count[r.kind];
        }
    }
    if (dropped != nullptr) *dropped = g_dropped;
    g_used = 0;
    g_dropped = 0;
    return err;
}

}  // namespace retn
