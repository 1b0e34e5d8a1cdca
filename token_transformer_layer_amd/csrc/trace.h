// Optional per-kernel timing: when enabled through tp_trace_enable(), every
// kernel launch of the library is bracketed by two HIP events recorded on the
// launch stream, together with the kernel's name and its algorithmic work
// (flops and HBM bytes of the operation, not of the schedule).  Disabled, a
// launch costs one relaxed atomic load.
#pragma once

#include <hip/hip_runtime.h>

namespace tpk {

bool trace_enabled();
void trace_begin(hipStream_t st);
void trace_end(hipStream_t st, const char *name, double flops, double bytes);

// RAII form: records the start on construction and the end on destruction.
struct TraceScope {
    hipStream_t st;
    const char *name;
    double flops, bytes;
    bool on;
    TraceScope(hipStream_t s, const char *n, double f, double b)
        : st(s), name(n), flops(f), bytes(b), on(trace_enabled()) {
        if (on) trace_begin(st);
    }
    ~TraceScope() {
        if (on) trace_end(st, name, flops, bytes);
    }
};

}  // namespace tpk
