// Optional per-kernel timing: HIP events recorded on the launch stream around
// individual kernel launches, with the algorithmic work (flops, bytes) of each launch.
// Off unless a handle enables it; when off, a ProfScope costs one pointer test.
#pragma once

#include <hip/hip_runtime.h>

namespace gpt2k {

class Profiler;
// The profiler of the handle whose call is running on this thread (or null).
extern thread_local Profiler* g_prof;

Profiler* prof_create();
void prof_destroy(Profiler* p);
void prof_reset(Profiler* p);
int prof_collect(Profiler* p);
int prof_entry(Profiler* p, int i, const char** name, long* launches, double* ms, double* flops, double* bytes);
long prof_dropped(Profiler* p);
void prof_filter(Profiler* p, const char* name);
void prof_begin(Profiler* p, hipStream_t st, const char* name);
void prof_end(Profiler* p, hipStream_t st, const char* name, double flops, double bytes);

struct ProfScope {
    Profiler* p;
    hipStream_t st;
    const char* name;
    double flops, bytes;
    ProfScope(hipStream_t s, const char* n, double f, double b) : p(g_prof), st(s), name(n), flops(f), bytes(b) {
        if (p) prof_begin(p, st, name);
    }
    ~ProfScope() {
        if (p) prof_end(p, st, name, flops, bytes);
    }
};

}  // namespace gpt2k
