// Per-kernel event timing (see trace.h) and its C-ABI entry points.
#include "trace.h"

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tpshard.h"

namespace tpk {

namespace {

struct Rec {
    std::string name;
    double flops, bytes;
    hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;       // free events
thread_local hipEvent_t t_open = nullptr;  // start event of the launch in flight on this thread

hipEvent_t get_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

bool trace_enabled() { return g_on.load(std::memory_order_relaxed); }

void trace_begin(hipStream_t st) {
    std::lock_guard<std::mutex> lk(g_mu);
    t_open = get_event();
    if (t_open && hipEventRecord(t_open, st) != hipSuccess) {  // no record for this launch
        g_pool.push_back(t_open);
        t_open = nullptr;
    }
}

void trace_end(hipStream_t st, const char *name, double flops, double bytes) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!t_open) return;
    hipEvent_t b = get_event();
    if (!b || hipEventRecord(b, st) != hipSuccess) {
        g_pool.push_back(t_open);
        if (b) g_pool.push_back(b);
        t_open = nullptr;
        return;
    }
    g_recs.push_back(Rec{name, flops, bytes, t_open, b});
    t_open = nullptr;
}

}  // namespace tpk

using namespace tpk;

extern "C" {

void tp_trace_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto &r : g_recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    g_on.store(on != 0, std::memory_order_relaxed);
}

int32_t tp_trace_read(tp_trace_record *out, int32_t max) {
    std::lock_guard<std::mutex> lk(g_mu);
    int32_t n = (int32_t)g_recs.size();
    for (int32_t i = 0; i < n; ++i) {
        Rec &r = g_recs[i];
        float ms = -1.f;  // -1: the events could not be timed
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) ms = -1.f;
        if (out && i < max) {
            std::memset(&out[i], 0, sizeof(out[i]));
            std::strncpy(out[i].name, r.name.c_str(), sizeof(out[i].name) - 1);
            out[i].flops = r.flops;
            out[i].bytes = r.bytes;
            out[i].ms = ms;
        }
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    return n;
}

}  // extern "C"
