// Per-kernel event timing (see prof.h).  Events come from a pool created when timing is
// enabled, never inside a training step; records past the pool's end are dropped and
// counted.
#include <string.h>

#include <map>
#include <string>
#include <vector>

#include "prof.h"

namespace gpt2k {

thread_local Profiler* g_prof = nullptr;

class Profiler {
   public:
    static constexpr int POOL = 16384;  // events (pairs use two)
    std::vector<hipEvent_t> ev;
    int next = 0;
    long dropped = 0;
    struct Rec {
        const char* name;
        int e0, e1;
        double flops, bytes;
    };
    std::vector<Rec> recs;
    int open = -1;
    struct Sum {
        long launches = 0;
        double ms = 0, flops = 0, bytes = 0;
    };
    std::vector<std::pair<std::string, Sum>> sums;
    bool ok = true;
    std::string only;  // record only this kernel when non-empty

    Profiler() {
        ev.resize(POOL);
        for (int i = 0; i < POOL; i++)
            if (hipEventCreate(&ev[i]) != hipSuccess) ok = false;
        recs.reserve(POOL / 2);
    }
    ~Profiler() {
        for (auto e : ev) (void)hipEventDestroy(e);
    }
};

void prof_filter(Profiler* p, const char* name) { p->only = name ? name : ""; }

void prof_begin(Profiler* p, hipStream_t st, const char* name) {
    if (!p->only.empty() && p->only != name) {
        p->open = -2;
        return;
    }
    if (p->next + 2 > Profiler::POOL) {
        p->open = -1;
        return;
    }
    p->open = p->next;
    (void)hipEventRecord(p->ev[p->next], st);
    p->next += 1;
}

void prof_end(Profiler* p, hipStream_t st, const char* name, double flops, double bytes) {
    if (p->open == -2) return;
    if (p->open < 0) {
        p->dropped++;
        return;
    }
    (void)hipEventRecord(p->ev[p->next], st);
    p->recs.push_back({name, p->open, p->next, flops, bytes});
    p->next += 1;
    p->open = -1;
}

Profiler* prof_create() {
    Profiler* p = new Profiler();
    if (!p->ok) {
        delete p;
        return nullptr;
    }
    return p;
}

void prof_destroy(Profiler* p) { delete p; }

void prof_reset(Profiler* p) {
    p->next = 0;
    p->dropped = 0;
    p->recs.clear();
    p->sums.clear();
}

// Waits for the recorded events and folds them into per-name sums.
int prof_collect(Profiler* p) {
    std::map<std::string, Profiler::Sum> m;
    for (const auto& r : p->recs) {
        if (hipEventSynchronize(p->ev[r.e1]) != hipSuccess) return -1;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p->ev[r.e0], p->ev[r.e1]) != hipSuccess) return -1;
        auto& s = m[r.name];
        s.launches++;
        s.ms += ms;
        s.flops += r.flops;
        s.bytes += r.bytes;
    }
    p->sums.assign(m.begin(), m.end());
    return (int)p->sums.size();
}

int prof_entry(Profiler* p, int i, const char** name, long* launches, double* ms, double* flops, double* bytes) {
    if (i < 0 || i >= (int)p->sums.size()) return -1;
    *name = p->sums[i].first.c_str();
    *launches = p->sums[i].second.launches;
    *ms = p->sums[i].second.ms;
    *flops = p->sums[i].second.flops;
    *bytes = p->sums[i].second.bytes;
    return 0;
}

long prof_dropped(Profiler* p) { return p->dropped; }

}  // namespace gpt2k
