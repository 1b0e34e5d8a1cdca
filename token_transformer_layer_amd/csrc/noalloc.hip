// Forward of the layer shard for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): the work areas that tp_shard_layer_fwd takes from the
// caller's scratch buffer (split-product partial sums and split-KV attention
// partial sums) live in one file-scope device array instead.
//
// The array is a host-side name for device memory: its device address is
// read once per device with hipGetSymbolAddress and only that address is
// passed to kernels.  Every call on one device shares that device's array;
// calls that overlap on one device (other streams, other threads) race on
// it.  Nothing in it needs to start at zero: every partial sum a kernel
// reads was written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "tpshard.h"

extern "C" tp_status tp_internal_fail(tp_status s, const char *msg);
tp_status tp_internal_shard_fwd(const tp_shard_cfg *cfg, const tp_shard_weights *w, const tp_partition *part,
                                int32_t slice_begin, int32_t slice_end, int32_t phase, const void *in,
                                float *partial_out, tp_kv_cache *kv, void *saved, float *split_ws,
                                int64_t split_floats, float *attn_work, int64_t attn_floats, void *stream);
namespace tpk {
bool trace_enabled();
}

namespace {

// 128 MiB: the products' split partial sums (gemm_split_workspace_floats,
// about 48 MiB) followed by attention's split-KV partial sums (the largest a
// forward call writes is about 68 MiB, at head_dim 128).
constexpr size_t kScratchBytes = (size_t)128 << 20;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of this device's array (looked up on the first call on the
// device, with that device current).
tp_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return tp_internal_fail(TP_EHIP, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return tp_internal_fail(TP_EUNSUPPORTED, "device index out of range");
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return tp_internal_fail(TP_EHIP, "hipGetSymbolAddress of the static scratch failed");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return TP_OK;
}

}  // namespace

extern "C" {

size_t tp_noalloc_scratch_bytes(void) { return kScratchBytes; }

tp_status tp_shard_layer_fwd_noalloc(const tp_shard_cfg *cfg, const tp_shard_weights *w, const tp_partition *part,
                                     int32_t slice_begin, int32_t slice_end, int32_t phase, const void *in,
                                     float *partial_out, tp_kv_cache *kv, void *saved, void *stream) {
    // per-kernel tracing creates HIP events: not for callers that cannot allocate
    if (tpk::trace_enabled())
        return tp_internal_fail(TP_EUNSUPPORTED, "tracing is on (tp_trace_enable); the allocation-free forward "
                                                 "does not trace");
    void *base = nullptr;
    tp_status s = scratch_address(&base);
    if (s != TP_OK) return s;
    const int64_t split_floats = (int64_t)tpk::gemm_split_workspace_floats();
    const int64_t split_bytes = (split_floats * 4 + 255) / 256 * 256;
    float *split_ws = (float *)base;
    float *attn_work = (float *)((char *)base + split_bytes);
    const int64_t attn_floats = ((int64_t)kScratchBytes - split_bytes) / 4;
    return tp_internal_shard_fwd(cfg, w, part, slice_begin, slice_end, phase, in, partial_out, kv, saved, split_ws,
                                 split_floats, attn_work, attn_floats, stream);
}

}  // extern "C"
