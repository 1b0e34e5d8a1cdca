// C-ABI of the layer-shard library: argument checks, buffer layouts of the
// saved/scratch regions, and the kernel sequence of each phase.
//
// The phase split follows the two all-reduces per layer and direction of
// "Transformer Training 11: model parallelism" (tensor-parallelism slide):
// every call ends where a partial sum must be reduced across ranks, and the
// next phase starts from the reduced tensor.  Calls run over a range of token
// slices ("TeraPipe", section 3): position-wise steps (LayerNorm, the
// products, GELU) batch the rows of all slices in the range, and attention
// covers the range's queries against the cache prefix [0, end of range).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.h"
#include "tpshard.h"

using namespace tpk;

namespace {

thread_local std::string g_err;

tp_status fail(tp_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

constexpr int64_t kMaxBuffer = (int64_t)1 << 31;  // buffer loads address < 2^31 bytes

struct Dims {
    int64_t h, n, d, f, t, b, s, nt, ht, ft, T;
    int es;
    DType dt;
};

tp_status check_cfg(const tp_shard_cfg *c, Dims *o) {
    if (!c) return fail(TP_EINVAL, "cfg is NULL");
    if (c->dtype != TP_F32 && c->dtype != TP_BF16) return fail(TP_EINVAL, "dtype %d is not TP_F32 or TP_BF16", c->dtype);
    if (c->hidden <= 0 || c->heads <= 0 || c->head_dim <= 0 || c->ffn <= 0 || c->tp_size <= 0 || c->batch <= 0 ||
        c->seq_len <= 0)
        return fail(TP_ESHAPE, "every size in cfg must be positive");
    if ((int64_t)c->heads * c->head_dim != c->hidden)
        return fail(TP_ESHAPE, "hidden (%d) != heads (%d) * head_dim (%d)", c->hidden, c->heads, c->head_dim);
    if (c->heads % c->tp_size) return fail(TP_ESHAPE, "heads (%d) not divisible by tp_size (%d)", c->heads, c->tp_size);
    if (c->ffn % c->tp_size) return fail(TP_ESHAPE, "ffn (%d) not divisible by tp_size (%d)", c->ffn, c->tp_size);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(TP_EUNSUPPORTED, "head_dim %d: only 64 and 128 are implemented", c->head_dim);
    if ((c->ffn / c->tp_size) % 8) return fail(TP_ESHAPE, "ffn/tp_size (%d) must be a multiple of 8", c->ffn / c->tp_size);
    if (c->hidden > 16384) return fail(TP_EUNSUPPORTED, "hidden %d > 16384", c->hidden);
    if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps)) return fail(TP_EINVAL, "ln_eps must be positive and finite");
    Dims d;
    d.h = c->hidden; d.n = c->heads; d.d = c->head_dim; d.f = c->ffn; d.t = c->tp_size; d.b = c->batch; d.s = c->seq_len;
    d.nt = d.n / d.t; d.ht = d.h / d.t; d.ft = d.f / d.t; d.T = d.b * d.s;
    d.es = c->dtype == TP_BF16 ? 2 : 4;
    d.dt = c->dtype == TP_BF16 ? DType::BF16 : DType::F32;
    // every tensor the kernels address with 32-bit buffer offsets
    int64_t widest = d.h > 3 * d.ht ? d.h : 3 * d.ht;
    if (d.ft > widest) widest = d.ft;
    if (d.T * widest * 4 >= kMaxBuffer || d.ft * d.h * 4 >= kMaxBuffer || 3 * d.ht * d.h * 4 >= kMaxBuffer)
        return fail(TP_ESHAPE, "a tensor of this configuration exceeds 2 GiB");
    if (o) *o = d;
    return TP_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Regions of the saved buffer (full sequence, T = s*b token rows).
struct Saved {
    int64_t u1, mu1, rs1, q, o, lse, u2, mu2, rs2, gz, g, total;  // gz: GELU'(Z)
};
Saved saved_layout(const Dims &d) {
    Saved L;
    int64_t off = 0;
    auto take = [&](int64_t bytes) { int64_t r = off; off += align256(bytes); return r; };
    L.u1 = take(d.T * d.h * d.es);
    L.mu1 = take(d.T * 4);
    L.rs1 = take(d.T * 4);
    L.q = take(d.b * d.nt * d.s * d.d * d.es);
    L.o = take(d.T * d.ht * d.es);
    L.lse = take(d.b * d.nt * d.s * 4);
    L.u2 = take(d.T * d.h * d.es);
    L.mu2 = take(d.T * 4);
    L.rs2 = take(d.T * 4);
    L.gz = take(d.T * d.ft * d.es);
    L.g = take(d.T * d.ft * d.es);
    L.total = off;
    return L;
}

struct Scratch {
    int64_t dz, dO, delta, dqkv, red, red_cs, attn, split, total;  // red: LayerNorm partials; red_cs: column sums
};
Scratch scratch_layout(const Dims &d) {
    Scratch L;
    int64_t off = 0;
    auto take = [&](int64_t bytes) { int64_t r = off; off += align256(bytes); return r; };
    L.dz = take(d.T * d.ft * d.es);
    L.dO = take(d.T * d.ht * d.es);
    L.delta = take(d.b * d.nt * d.s * 4);
    L.dqkv = take(d.T * 3 * d.ht * d.es);
    int64_t red = (int64_t)layernorm_bwd_partials_floats((int)d.T, (int)d.h);
    // column sums of two matrices at once: (b1, b2) or (b_o, b_qkv)
    int64_t widest = d.ft + d.h;
    if (d.h + 3 * d.ht > widest) widest = d.h + 3 * d.ht;
    int64_t cs = (int64_t)colsum_partials_floats((int)d.T, (int)widest);
    L.red = take(red * 4);
    L.red_cs = take(cs * 4);
    L.attn = take((int64_t)attn_fwd_work_floats((int)d.b, (int)d.nt, (int)d.s, (int)d.d) * 4);
    L.split = d.dt == DType::BF16 ? take((int64_t)gemm_split_workspace_floats() * 4) : off;
    L.total = off;
    return L;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

#define NEED(ptr, name)                                                                   \
    do {                                                                                  \
        if (!(ptr)) return fail(TP_EINVAL, "%s is NULL", name);                          \
        if (!aligned16(ptr)) return fail(TP_EALIGN, "%s is not 16-byte aligned", name); \
    } while (0)

// a buffer of n elements: checked only when n > 0 (an empty one is never
// addressed and may be NULL)
#define NEED_IF(n, ptr, name)          \
    do {                               \
        if ((n) > 0) NEED(ptr, name); \
    } while (0)

// scalar fp32 arrays (LayerNorm statistics): 4-byte alignment
#define NEED4(ptr, name)                                                                 \
    do {                                                                                 \
        if (!(ptr)) return fail(TP_EINVAL, "%s is NULL", name);                         \
        if ((uintptr_t)(ptr) & 3) return fail(TP_EALIGN, "%s is not 4-byte aligned", name); \
    } while (0)

tp_status check_range(const Dims &d, const tp_partition *part, int32_t j0, int32_t j1, int64_t *o0, int64_t *o1) {
    if (!part || !part->len) return fail(TP_EINVAL, "partition is NULL");
    if (part->num_slices <= 0) return fail(TP_ESHAPE, "partition has no slices");
    int64_t sum = 0;
    for (int i = 0; i < part->num_slices; ++i) {
        if (part->len[i] <= 0) return fail(TP_ESHAPE, "slice %d has length %d (must be >= 1)", i, part->len[i]);
        sum += part->len[i];
    }
    if (sum != d.s) return fail(TP_ESHAPE, "slice lengths sum to %lld, seq_len is %lld", (long long)sum, (long long)d.s);
    if (j0 < 0 || j1 > part->num_slices || j0 >= j1)
        return fail(TP_EINVAL, "slice range [%d, %d) is not inside [0, %d)", j0, j1, part->num_slices);
    int64_t a = 0;
    for (int i = 0; i < j0; ++i) a += part->len[i];
    int64_t b = a;
    for (int i = j0; i < j1; ++i) b += part->len[i];
    *o0 = a;
    *o1 = b;
    return TP_OK;
}

tp_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return TP_OK;
    return fail(TP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCALL(expr, what)                          \
    do {                                             \
        tp_status _s = hip_status((expr), (what));   \
        if (_s != TP_OK) return _s;                  \
    } while (0)

template <typename P>
P at(const void *base, int64_t byte_off) {
    return (P)((const char *)base + byte_off);
}

}  // namespace

extern "C" {

size_t tp_shard_saved_bytes(const tp_shard_cfg *cfg) {
    Dims d;
    if (check_cfg(cfg, &d) != TP_OK) return 0;
    return (size_t)saved_layout(d).total;
}

size_t tp_shard_scratch_bytes(const tp_shard_cfg *cfg) {
    Dims d;
    if (check_cfg(cfg, &d) != TP_OK) return 0;
    return (size_t)scratch_layout(d).total;
}

const char *tp_last_error(void) { return g_err.c_str(); }

// error reporting for the library's other host sources (not exported)
__attribute__((visibility("hidden"))) tp_status tp_internal_fail(tp_status s, const char *msg) {
    if (s == TP_OK) {
        g_err.clear();
        return s;
    }
    return fail(s, "%s", msg);
}

tp_status tp_gemm_force_tile(int32_t tile) {
    if (tile < -1 || tile > 6) return fail(TP_EINVAL, "tile must be -1 (automatic) or 0..6");
    tpk::gemm_force_tile(tile);
    g_err.clear();
    return TP_OK;
}

}  // extern "C"

// The forward of one phase with its two work areas given: the split-product
// partial sums (split_floats floats at split_ws) and the split-KV partial
// sums of attention (attn_floats floats at attn_work).  A call whose
// attention needs more than attn_floats fails before anything is enqueued.
__attribute__((visibility("hidden"))) tp_status tp_internal_shard_fwd(
    const tp_shard_cfg *cfg, const tp_shard_weights *w, const tp_partition *part, int32_t slice_begin,
    int32_t slice_end, int32_t phase, const void *in, float *partial_out, tp_kv_cache *kv, void *saved,
    float *split_ws, int64_t split_floats, float *attn_work, int64_t attn_floats, void *stream) {
    Dims d;
    tp_status s = check_cfg(cfg, &d);
    if (s != TP_OK) return s;
    if (!w) return fail(TP_EINVAL, "weights is NULL");
    int64_t o0, o1;
    if ((s = check_range(d, part, slice_begin, slice_end, &o0, &o1)) != TP_OK) return s;
    if (phase < TP_FWD_ATTN || phase > TP_FWD_MLP_SP) return fail(TP_EINVAL, "forward phase %d is not valid", phase);
    // sequence-parallel phases take the gathered LayerNorm output as `in`
    const bool sp = phase == TP_FWD_ATTN_SP || phase == TP_FWD_MLP_SP;
    NEED(in, "in");
    NEED(partial_out, "partial_out");
    NEED(saved, "saved");
    if (phase == TP_FWD_ATTN || phase == TP_FWD_ATTN_SP) {
        const int64_t need = d.dt == DType::BF16
                                 ? (int64_t)attn_fwd_call_work_floats((int)d.b, (int)d.nt, (int)o0, (int)o1, (int)d.d)
                                 : 0;
        if (need > attn_floats)
            return fail(TP_ESHAPE, "attention of this call needs %lld bytes of work space, %lld are available",
                        (long long)need * 4, (long long)attn_floats * 4);
    }
    const Saved L = saved_layout(d);
    const int64_t r0 = o0 * d.b, nrows = (o1 - o0) * d.b;
    hipStream_t st = (hipStream_t)stream;
    const int es = d.es;
    // every product may split its reduction through the split workspace
    auto fresh = [&]() {
        EpiArgs x;
        x.split_ws = split_ws;
        x.split_ws_floats = d.dt == DType::BF16 ? split_floats : 0;
        return x;
    };
    EpiArgs e = fresh();
    if (phase == TP_FWD_ATTN || phase == TP_FWD_ATTN_SP) {
        if (!sp) {
            NEED(w->ln1_g, "w.ln1_g");
            NEED(w->ln1_b, "w.ln1_b");
        }
        NEED(w->w_qkv, "w.w_qkv");
        NEED(w->b_qkv, "w.b_qkv");
        NEED(w->w_o, "w.w_o");
        if (!kv) return fail(TP_EINVAL, "kv is NULL");
        NEED(kv->k, "kv.k");
        NEED(kv->v, "kv.v");
        if (kv->filled != o0)
            return fail(TP_EORDER, "slices must run in order: cache holds %d positions, call starts at %lld", kv->filled,
                        (long long)o0);
        void *u1 = at<char *>(saved, L.u1 + r0 * d.h * es);
        if (sp)
            HIPCALL(hipMemcpyAsync(u1, at<const char *>(in, r0 * d.h * es), nrows * d.h * es, hipMemcpyDeviceToDevice,
                                   st),
                    "copy of the gathered LN1 output");
        else
            HIPCALL(layernorm_fwd(d.dt, (int)nrows, (int)d.h, cfg->ln_eps, at<const char *>(in, r0 * d.h * es),
                                  w->ln1_g, w->ln1_b, u1, at<float *>(saved, L.mu1 + r0 * 4),
                                  at<float *>(saved, L.rs1 + r0 * 4), st),
                    "layernorm forward (LN1)");
        e = fresh();
        e.bias = w->b_qkv;
        e.q = at<char *>(saved, L.q);
        e.k = kv->k;
        e.v = kv->v;
        e.batch = (int)d.b; e.seq = (int)d.s; e.nt = (int)d.nt; e.d = (int)d.d; e.ht = (int)d.ht; e.row0 = (int)r0;
        HIPCALL(gemm(d.dt, (int)nrows, (int)(3 * d.ht), (int)d.h, Mat{u1, d.h, true}, Mat{w->w_qkv, d.h, true}, Epi::Qkv,
                     e, st),
                "QKV product");
        AttnArgs a{};
        a.batch = (int)d.b; a.nt = (int)d.nt; a.seq = (int)d.s; a.d = (int)d.d; a.q0 = (int)o0; a.q1 = (int)o1;
        a.scale = 1.0f / std::sqrt((float)d.d);
        a.q = at<char *>(saved, L.q); a.k = kv->k; a.v = kv->v;
        a.o = at<char *>(saved, L.o); a.lse = at<float *>(saved, L.lse);
        a.work = attn_work;
        HIPCALL(attn_fwd(d.dt, a, st), "attention forward");
        e = fresh();
        e.c = partial_out + r0 * d.h;
        e.ldc = d.h;
        HIPCALL(gemm(d.dt, (int)nrows, (int)d.h, (int)d.ht, Mat{at<char *>(saved, L.o + r0 * d.ht * es), d.ht, true},
                     Mat{w->w_o, d.ht, true}, Epi::StoreF32, e, st),
                "out-projection product");
        kv->filled = (int32_t)o1;
        return TP_OK;
    }
    if (!sp) {
        NEED(w->ln2_g, "w.ln2_g");
        NEED(w->ln2_b, "w.ln2_b");
    }
    NEED(w->w1, "w.w1");
    NEED(w->b1, "w.b1");
    NEED(w->w2, "w.w2");
    void *u2 = at<char *>(saved, L.u2 + r0 * d.h * es);
    if (sp)
        HIPCALL(hipMemcpyAsync(u2, at<const char *>(in, r0 * d.h * es), nrows * d.h * es, hipMemcpyDeviceToDevice, st),
                "copy of the gathered LN2 output");
    else
        HIPCALL(layernorm_fwd(d.dt, (int)nrows, (int)d.h, cfg->ln_eps, at<const char *>(in, r0 * d.h * es), w->ln2_g,
                              w->ln2_b, u2, at<float *>(saved, L.mu2 + r0 * 4), at<float *>(saved, L.rs2 + r0 * 4), st),
                "layernorm forward (LN2)");
    void *gz = at<char *>(saved, L.gz + r0 * d.ft * es);
    void *gg = at<char *>(saved, L.g + r0 * d.ft * es);
    e = fresh();
    e.c = gz; e.ldc = d.ft; e.c2 = gg; e.ldc2 = d.ft; e.bias = w->b1;
    HIPCALL(gemm(d.dt, (int)nrows, (int)d.ft, (int)d.h, Mat{u2, d.h, true}, Mat{w->w1, d.h, true}, Epi::BiasGelu, e, st),
            "FC1 product");
    e = fresh();
    e.c = partial_out + r0 * d.h;
    e.ldc = d.h;
    HIPCALL(gemm(d.dt, (int)nrows, (int)d.h, (int)d.ft, Mat{gg, d.ft, true}, Mat{w->w2, d.ft, true}, Epi::StoreF32, e,
                 st),
            "FC2 product");
    return TP_OK;
}

extern "C" {

tp_status tp_shard_layer_fwd(const tp_shard_cfg *cfg, const tp_shard_weights *w, const tp_partition *part,
                             int32_t slice_begin, int32_t slice_end, int32_t phase, const void *in,
                             float *partial_out, tp_kv_cache *kv, void *saved, void *scratch, void *stream) {
    Dims d;
    tp_status s = check_cfg(cfg, &d);
    if (s != TP_OK) return s;
    NEED(scratch, "scratch");
    const Scratch S = scratch_layout(d);
    return tp_internal_shard_fwd(cfg, w, part, slice_begin, slice_end, phase, in, partial_out, kv, saved,
                                 at<float *>(scratch, S.split), (int64_t)gemm_split_workspace_floats(),
                                 at<float *>(scratch, S.attn), (S.split - S.attn) / 4, stream);
}

tp_status tp_shard_layer_bwd(const tp_shard_cfg *cfg, const tp_shard_weights *w, const tp_partition *part,
                             int32_t slice_begin, int32_t slice_end, int32_t phase, const void *dy, const void *ln_in,
                             const float *reduced_in, float *partial_out, void *dh, void *dx, const tp_shard_grads *g,
                             const tp_kv_cache *kv, tp_kv_grad *kvg, const void *saved, void *scratch, void *stream) {
    Dims d;
    tp_status s = check_cfg(cfg, &d);
    if (s != TP_OK) return s;
    if (!w) return fail(TP_EINVAL, "weights is NULL");
    if (!g) return fail(TP_EINVAL, "grads is NULL");
    if (g->accumulate != 0 && g->accumulate != 1) return fail(TP_EINVAL, "grads.accumulate must be 0 or 1");
    int64_t o0, o1;
    if ((s = check_range(d, part, slice_begin, slice_end, &o0, &o1)) != TP_OK) return s;
    if (phase < TP_BWD_MLP || phase > TP_BWD_ATTN_DATA_SP)
        return fail(TP_EINVAL, "backward phase %d is not valid", phase);
    NEED(saved, "saved");
    NEED(scratch, "scratch");
    // sequence-parallel attention phases: dH is given (gathered), LN2's
    // backward ran on the caller's shard
    const bool sp = phase == TP_BWD_ATTN_SP || phase == TP_BWD_ATTN_DATA_SP;
    const bool mlp = phase == TP_BWD_MLP || phase == TP_BWD_MLP_DATA;
    const bool attn = phase == TP_BWD_ATTN || phase == TP_BWD_ATTN_DATA || sp;
    const bool mlp_w = phase == TP_BWD_MLP || phase == TP_BWD_WGRAD;
    const bool attn_w = phase == TP_BWD_ATTN || phase == TP_BWD_WGRAD || phase == TP_BWD_ATTN_SP;
    const bool acc = g->accumulate != 0;
    // every check runs before anything is enqueued
    if (mlp || attn || mlp_w || attn_w) NEED(dy, "dy");
    if (mlp || attn) NEED(partial_out, "partial_out");
    if (mlp) {
        NEED(w->w1, "w.w1");
        NEED(w->w2, "w.w2");
    }
    if (mlp_w) {
        NEED(g->w1, "g.w1");
        NEED(g->b1, "g.b1");
        NEED(g->w2, "g.w2");
        NEED(g->b2, "g.b2");
    }
    if ((attn && !sp) || phase == TP_BWD_LN1) {
        NEED(ln_in, "ln_in");
        NEED(reduced_in, "reduced_in");
    }
    if (attn || attn_w || phase == TP_BWD_LN1) NEED(dh, "dh");
    if (attn && !sp) {
        NEED(w->ln2_g, "w.ln2_g");
        NEED(g->ln2_g, "g.ln2_g");
        NEED(g->ln2_b, "g.ln2_b");
    }
    if (attn) {
        NEED(w->w_o, "w.w_o");
        if (!kv || !kvg) return fail(TP_EINVAL, "kv and kvg are required for the attention backward");
        NEED(kv->k, "kv.k");
        NEED(kv->v, "kv.v");
        NEED(kvg->dk, "kvg.dk");
        NEED(kvg->dv, "kvg.dv");
        if (kv->filled < o1)
            return fail(TP_EORDER, "the cache holds %d positions; this call needs %lld", kv->filled, (long long)o1);
        if (kvg->done_from != o1)
            return fail(TP_EORDER, "backward slices must run in reverse: done_from is %d, call ends at %lld",
                        kvg->done_from, (long long)o1);
    }
    if (attn) NEED(w->w_qkv, "w.w_qkv");
    if (attn_w) {
        NEED(g->w_o, "g.w_o");
        NEED(g->b_o, "g.b_o");
        NEED(g->w_qkv, "g.w_qkv");
        NEED(g->b_qkv, "g.b_qkv");
    }
    if (phase == TP_BWD_LN1) {
        NEED(dx, "dx");
        NEED(w->ln1_g, "w.ln1_g");
        NEED(g->ln1_g, "g.ln1_g");
        NEED(g->ln1_b, "g.ln1_b");
    }

    const Saved L = saved_layout(d);
    const Scratch S = scratch_layout(d);
    const int64_t r0 = o0 * d.b, nrows = (o1 - o0) * d.b;
    hipStream_t st = (hipStream_t)stream;
    const int es = d.es;
    float *red = at<float *>(scratch, S.red);
    float *red_cs = at<float *>(scratch, S.red_cs);
    // bias-gradient and LayerNorm-parameter reductions still to finish (their
    // first stages leave partial sums; one launch finishes up to two)
    ReduceSpec pend_ln{}, pend_cs{};
    bool has_ln = false, has_cs = false;
    const Epi wepi = acc ? Epi::AccumF32 : Epi::StoreF32;  // weight-gradient epilogue
    auto fresh = [&]() {
        EpiArgs x;
        x.split_ws = at<float *>(scratch, S.split);
        x.split_ws_floats = d.dt == DType::BF16 ? (int64_t)gemm_split_workspace_floats() : 0;
        return x;
    };
    EpiArgs e = fresh();
    // rows of the call in each per-row tensor
    const void *dyr = dy ? at<const char *>(dy, r0 * d.h * es) : nullptr;
    void *dz = at<char *>(scratch, S.dz + r0 * d.ft * es);
    void *dO = at<char *>(scratch, S.dO + r0 * d.ht * es);
    void *dqkv = at<char *>(scratch, S.dqkv + r0 * 3 * d.ht * es);
    void *dhr = dh ? at<char *>(dh, r0 * d.h * es) : nullptr;

    if (mlp) {
        // dZ = (dY W2) * GELU'(Z); dU2,r = dZ W1
        e = fresh();
        e.c = dz; e.ldc = d.ft; e.aux = at<const char *>(saved, L.gz + r0 * d.ft * es); e.ldaux = d.ft;
        HIPCALL(gemm(d.dt, (int)nrows, (int)d.ft, (int)d.h, Mat{dyr, d.h, true}, Mat{w->w2, d.ft, false}, Epi::GeluGrad,
                     e, st),
                "FC2 input-gradient product");
        e = fresh();
        e.c = partial_out + r0 * d.h; e.ldc = d.h;
        HIPCALL(gemm(d.dt, (int)nrows, (int)d.h, (int)d.ft, Mat{dz, d.ft, true}, Mat{w->w1, d.h, false}, Epi::StoreF32,
                     e, st),
                "FC1 input-gradient product");
    }
    if (mlp_w) {
        // dW2 = dY^T G, dW1 = dZ^T u2, db1 = sum dZ, db2 = sum dY
        e = fresh();
        e.c = g->w2; e.ldc = d.ft;
        HIPCALL(gemm(d.dt, (int)d.h, (int)d.ft, (int)nrows, Mat{dyr, d.h, false},
                     Mat{at<const char *>(saved, L.g + r0 * d.ft * es), d.ft, false}, wepi, e, st),
                "FC2 weight-gradient product");
        e = fresh();
        e.c = g->w1; e.ldc = d.h;
        HIPCALL(gemm(d.dt, (int)d.ft, (int)d.h, (int)nrows, Mat{dz, d.ft, false},
                     Mat{at<const char *>(saved, L.u2 + r0 * d.h * es), d.h, false}, wepi, e, st),
                "FC1 weight-gradient product");
        // db1 = sum of dZ and db2 = sum of dY over the rows: one column-sum
        // launch over both matrices, one reduction
        HIPCALL(colsum_rows(d.dt, (int)nrows, (int)d.ft, dz, d.ft, (int)d.h, dyr, d.h, red_cs, st),
                "b1 and b2 gradients");
        const ReduceSpec r = colsum_reduce_spec((int)nrows, (int)d.ft, (int)d.h, red_cs, g->b1, g->b2);
        HIPCALL(reduce_partials(&r, nullptr, acc, st), "b1 and b2 gradients");
    }
    if (attn) {
        // dH = dY + LN2^T(sum_r dU2,r) (given in the sequence-parallel form);
        // dO = dH W_o; attention backward
        if (!sp) {
            // dgamma2 and dbeta2 are finished with the phase's other reductions
            HIPCALL(layernorm_bwd_rows(d.dt, (int)nrows, (int)d.h, reduced_in + r0 * d.h, dyr,
                                       at<const char *>(ln_in, r0 * d.h * es), w->ln2_g,
                                       at<const float *>(saved, L.mu2 + r0 * 4),
                                       at<const float *>(saved, L.rs2 + r0 * 4), dhr, red, st),
                    "layernorm backward (LN2)");
            pend_ln = ln_bwd_reduce_spec((int)nrows, (int)d.h, red, g->ln2_g, g->ln2_b);
            has_ln = true;
        }
        e = fresh();
        e.c = dO; e.ldc = d.ht;
        HIPCALL(gemm(d.dt, (int)nrows, (int)d.ht, (int)d.h, Mat{dhr, d.h, true}, Mat{w->w_o, d.ht, false}, Epi::Store, e,
                     st),
                "out-projection input-gradient product");
        AttnArgs a{};
        a.batch = (int)d.b; a.nt = (int)d.nt; a.seq = (int)d.s; a.d = (int)d.d; a.q0 = (int)o0; a.q1 = (int)o1;
        a.scale = 1.0f / std::sqrt((float)d.d);
        a.q = at<const char *>(saved, L.q); a.k = kv->k; a.v = kv->v;
        a.o = const_cast<char *>(at<const char *>(saved, L.o));
        a.lse = at<float *>(saved, L.lse);
        a.dout = at<const char *>(scratch, S.dO);
        a.delta = at<float *>(scratch, S.delta);
        a.dqkv = at<char *>(scratch, S.dqkv);
        a.dk_acc = kvg->dk; a.dv_acc = kvg->dv;
        a.k_final0 = (int)o0;
        a.acc_in = kvg->done_from != d.s;
        a.work = at<float *>(scratch, S.attn);
        HIPCALL(attn_bwd(d.dt, a, st), "attention backward");
        // dU1,r = dQKV W_qkv
        e = fresh();
        e.c = partial_out + r0 * d.h; e.ldc = d.h;
        HIPCALL(gemm(d.dt, (int)nrows, (int)d.h, (int)(3 * d.ht), Mat{dqkv, 3 * d.ht, true}, Mat{w->w_qkv, d.h, false},
                     Epi::StoreF32, e, st),
                "QKV input-gradient product");
        kvg->done_from = (int32_t)o0;
    }
    if (attn_w) {
        // dW_o = dH^T O, db_o = sum dH, dW_qkv = dQKV^T u1, db_qkv = sum dQKV
        e = fresh();
        e.c = g->w_o; e.ldc = d.ht;
        HIPCALL(gemm(d.dt, (int)d.h, (int)d.ht, (int)nrows, Mat{dhr, d.h, false},
                     Mat{at<const char *>(saved, L.o + r0 * d.ht * es), d.ht, false}, wepi, e, st),
                "out-projection weight-gradient product");
        e = fresh();
        e.c = g->w_qkv; e.ldc = d.h;
        HIPCALL(gemm(d.dt, (int)(3 * d.ht), (int)d.h, (int)nrows, Mat{dqkv, 3 * d.ht, false},
                     Mat{at<const char *>(saved, L.u1 + r0 * d.h * es), d.h, false}, wepi, e, st),
                "QKV weight-gradient product");
        // db_o = sum of dH and db_qkv = sum of dQKV: one column-sum launch
        HIPCALL(colsum_rows(d.dt, (int)nrows, (int)d.h, dhr, d.h, (int)(3 * d.ht), dqkv, 3 * d.ht, red_cs, st),
                "b_o and b_qkv gradients");
        pend_cs = colsum_reduce_spec((int)nrows, (int)d.h, (int)(3 * d.ht), red_cs, g->b_o, g->b_qkv);
        has_cs = true;
    }
    if (has_ln || has_cs)
        HIPCALL(reduce_partials(has_ln ? &pend_ln : nullptr, has_cs ? &pend_cs : nullptr, acc, st),
                "attention-block parameter gradients");
    if (phase == TP_BWD_LN1) {
        HIPCALL(layernorm_bwd(d.dt, (int)nrows, (int)d.h, reduced_in + r0 * d.h, dhr,
                              at<const char *>(ln_in, r0 * d.h * es), w->ln1_g, at<const float *>(saved, L.mu1 + r0 * 4),
                              at<const float *>(saved, L.rs1 + r0 * 4), at<char *>(dx, r0 * d.h * es), g->ln1_g,
                              g->ln1_b, acc, red, st),
                "layernorm backward (LN1)");
    }
    return TP_OK;
}

tp_status tp_residual_combine(const tp_shard_cfg *cfg, int64_t rows, const void *resid, const float *reduced,
                              const void *bias, void *out, void *stream) {
    Dims d;
    tp_status s = check_cfg(cfg, &d);
    if (s != TP_OK) return s;
    if (rows < 0 || rows > d.T) return fail(TP_ESHAPE, "rows %lld outside [0, batch*seq_len]", (long long)rows);
    NEED(resid, "resid");
    NEED(reduced, "reduced");
    NEED(bias, "bias");
    NEED(out, "out");
    return hip_status(residual_combine(d.dt, rows, (int)d.h, resid, reduced, bias, out, (hipStream_t)stream),
                      "residual combine");
}

tp_status tp_cube_ffn_block(int32_t rows, int32_t hidden, int32_t ffn, const void *x, const void *w1, const void *b1,
                            const void *w2, void *hbuf, float *out, void *stream) {
    if (rows <= 0 || hidden <= 0 || ffn <= 0) return fail(TP_ESHAPE, "rows, hidden and ffn must be positive");
    if (hidden % 8 || ffn % 8) return fail(TP_ESHAPE, "hidden and ffn must be multiples of 8");
    if ((int64_t)rows * ffn * 2 >= kMaxBuffer || (int64_t)rows * hidden * 4 >= kMaxBuffer ||
        (int64_t)ffn * hidden * 2 >= kMaxBuffer)
        return fail(TP_ESHAPE, "a tensor of this block exceeds 2 GiB");
    NEED(x, "x");
    NEED(w1, "w1");
    NEED(b1, "b1");
    NEED(w2, "w2");
    NEED(hbuf, "hbuf");
    NEED(out, "out");
    hipStream_t st = (hipStream_t)stream;
    EpiArgs e;
    e.c = nullptr; e.c2 = hbuf; e.ldc2 = ffn; e.bias = b1;
    HIPCALL(gemm(DType::BF16, rows, ffn, hidden, Mat{x, hidden, true}, Mat{w1, hidden, true}, Epi::BiasGelu, e, st),
            "cube FC1 product");
    e = EpiArgs{};
    e.c = out; e.ldc = hidden;
    HIPCALL(gemm(DType::BF16, rows, hidden, ffn, Mat{hbuf, ffn, true}, Mat{w2, ffn, true}, Epi::StoreF32, e, st),
            "cube FC2 product");
    return TP_OK;
}

static tp_status check_block(const tp_attn_block_shape *b) {
    if (!b) return fail(TP_EINVAL, "shape is NULL");
    if (b->batch <= 0 || b->heads <= 0 || b->nq < 0 || b->nk < 0 || b->q_pos0 < 0 || b->k_pos0 < 0)
        return fail(TP_ESHAPE, "batch and heads must be positive; nq, nk and the positions non-negative");
    if (b->head_dim != 64 && b->head_dim != 128) return fail(TP_EUNSUPPORTED, "head_dim %d is not 64 or 128", b->head_dim);
    if ((int64_t)b->q_pos0 + b->nq > INT32_MAX || (int64_t)b->k_pos0 + b->nk > INT32_MAX)
        return fail(TP_ESHAPE, "positions exceed int32");
    const int64_t bh = (int64_t)b->batch * b->heads;
    if (bh * b->nq * b->head_dim * 4 >= kMaxBuffer || bh * b->nk * b->head_dim * 2 >= kMaxBuffer)
        return fail(TP_ESHAPE, "a tensor of this block exceeds 2 GiB");
    return TP_OK;
}

tp_status tp_attn_block_fwd(const tp_attn_block_shape *shape, const void *q, const void *k, const void *v, float *o,
                            float *lse, void *stream) {
    tp_status s = check_block(shape);
    if (s != TP_OK) return s;
    NEED_IF(shape->nq, q, "q");
    NEED_IF(shape->nk, k, "k");
    NEED_IF(shape->nk, v, "v");
    NEED_IF(shape->nq, o, "o");
    NEED_IF(shape->nq, lse, "lse");
    AttnBlockArgs a;
    a.bh = shape->batch * shape->heads;
    a.nq = shape->nq;
    a.nk = shape->nk;
    a.d = shape->head_dim;
    a.q_pos0 = shape->q_pos0;
    a.k_pos0 = shape->k_pos0;
    a.scale = 1.0f / std::sqrt((float)shape->head_dim);
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    return hip_status(attn_block_fwd(a, (hipStream_t)stream), "block attention");
}

tp_status tp_attn_merge(const tp_attn_block_shape *shape, const float *o_a, const float *lse_a, const float *o_b,
                        const float *lse_b, float *o, float *lse, void *stream) {
    tp_status s = check_block(shape);
    if (s != TP_OK) return s;
    NEED_IF(shape->nq, o_a, "o_a");
    NEED_IF(shape->nq, lse_a, "lse_a");
    NEED_IF(shape->nq, o_b, "o_b");
    NEED_IF(shape->nq, lse_b, "lse_b");
    NEED_IF(shape->nq, o, "o");
    NEED_IF(shape->nq, lse, "lse");
    const int64_t rows = (int64_t)shape->batch * shape->heads * shape->nq;
    return hip_status(attn_merge(rows, shape->head_dim, o_a, lse_a, o_b, lse_b, o, lse, (hipStream_t)stream),
                      "attention merge");
}

size_t tp_attn_block_bwd_work_bytes(const tp_attn_block_shape *shape) {
    if (check_block(shape) != TP_OK) return 0;
    const size_t n = attn_block_bwd_work_floats(shape->batch * shape->heads, shape->nq) * sizeof(float);
    return n > 0 ? (n + 255) / 256 * 256 : 256;
}

tp_status tp_attn_block_bwd(const tp_attn_block_shape *shape, const void *q, const void *k, const void *v,
                            const float *o, const float *lse, const void *dout, float *dq, float *dk, float *dv,
                            int32_t accumulate, void *work, void *stream) {
    tp_status s = check_block(shape);
    if (s != TP_OK) return s;
    if (accumulate != 0 && accumulate != 1) return fail(TP_EINVAL, "accumulate must be 0 or 1");
    NEED_IF(shape->nq, q, "q");
    NEED_IF(shape->nk, k, "k");
    NEED_IF(shape->nk, v, "v");
    NEED_IF(shape->nq, o, "o");
    NEED_IF(shape->nq, lse, "lse");
    NEED_IF(shape->nq, dout, "dout");
    NEED_IF(shape->nq, dq, "dq");
    NEED_IF(shape->nk, dk, "dk");
    NEED_IF(shape->nk, dv, "dv");
    NEED_IF(shape->nq, work, "work");
    AttnBlockBwdArgs a{};
    a.bh = shape->batch * shape->heads;
    a.nq = shape->nq;
    a.nk = shape->nk;
    a.d = shape->head_dim;
    a.q_pos0 = shape->q_pos0;
    a.k_pos0 = shape->k_pos0;
    a.accumulate = accumulate != 0;
    a.scale = 1.0f / std::sqrt((float)shape->head_dim);
    a.q = q; a.k = k; a.v = v; a.dout = dout; a.o = o; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv; a.work = (float *)work;
    return hip_status(attn_block_bwd(a, (hipStream_t)stream), "block attention backward");
}

tp_status tp_cube_matmul(int32_t form, int32_t M, int32_t N, int32_t K, const void *a, const void *b, float *c,
                         int32_t accumulate, void *stream) {
    if (form < TP_CUBE_AB || form > TP_CUBE_ATB) return fail(TP_EINVAL, "form %d is not a tp_cube_form", form);
    if (M <= 0 || N <= 0 || K <= 0) return fail(TP_ESHAPE, "M, N and K must be positive");
    if (M % 8 || N % 8 || K % 8) return fail(TP_ESHAPE, "M, N and K must be multiples of 8");
    if ((int64_t)M * K * 2 >= kMaxBuffer || (int64_t)N * K * 2 >= kMaxBuffer || (int64_t)M * N * 4 >= kMaxBuffer)
        return fail(TP_ESHAPE, "an operand exceeds 2 GiB");
    if (accumulate != 0 && accumulate != 1) return fail(TP_EINVAL, "accumulate must be 0 or 1");
    NEED(a, "a");
    NEED(b, "b");
    NEED(c, "c");
    if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return fail(TP_EALIGN, "a, b and c must be 16-byte aligned");
    EpiArgs e;
    e.c = c;
    e.ldc = N;
    Mat A, B;
    if (form == TP_CUBE_AB) {
        A = Mat{a, K, true};
        B = Mat{b, N, false};
    } else if (form == TP_CUBE_ABT) {
        A = Mat{a, K, true};
        B = Mat{b, K, true};
    } else {
        A = Mat{a, M, false};
        B = Mat{b, N, false};
    }
    return hip_status(gemm(DType::BF16, M, N, K, A, B, accumulate ? Epi::AccumF32 : Epi::StoreF32, e,
                           (hipStream_t)stream),
                      "cube product");
}

tp_status tp_cube_bias_gelu(int32_t rows, int32_t n, const float *z_sum, const void *bias, void *z, void *h,
                            void *stream) {
    if (rows <= 0 || n <= 0 || n % 8) return fail(TP_ESHAPE, "rows must be positive and n a positive multiple of 8");
    if ((int64_t)rows * n * 4 >= kMaxBuffer) return fail(TP_ESHAPE, "a tensor exceeds 2 GiB");
    NEED(z_sum, "z_sum");
    NEED(bias, "bias");
    NEED(z, "z");
    NEED(h, "h");
    if (!aligned16(z_sum) || !aligned16(bias) || !aligned16(z) || !aligned16(h))
        return fail(TP_EALIGN, "z_sum, bias, z and h must be 16-byte aligned");
    return hip_status(bias_gelu(rows, n, z_sum, bias, z, h, (hipStream_t)stream), "cube bias and GELU");
}

size_t tp_cube_work_bytes(int32_t rows, int32_t n) {
    if (rows <= 0 || n <= 0) return 0;
    return colsum_partials_floats(rows, n) * sizeof(float);
}

tp_status tp_cube_gelu_backward(int32_t rows, int32_t n, const float *dh, const void *z, void *dz, float *dbias,
                                int32_t accumulate, void *work, void *stream) {
    if (rows <= 0 || n <= 0 || n % 8) return fail(TP_ESHAPE, "rows must be positive and n a positive multiple of 8");
    if ((int64_t)rows * n * 4 >= kMaxBuffer) return fail(TP_ESHAPE, "a tensor exceeds 2 GiB");
    if (accumulate != 0 && accumulate != 1) return fail(TP_EINVAL, "accumulate must be 0 or 1");
    NEED(dh, "dh");
    NEED(z, "z");
    NEED(dz, "dz");
    NEED(dbias, "dbias");
    NEED(work, "work");
    if (!aligned16(dh) || !aligned16(z) || !aligned16(dz) || !aligned16(dbias) || !aligned16(work))
        return fail(TP_EALIGN, "dh, z, dz, dbias and work must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    HIPCALL(gelu_backward(rows, n, dh, z, dz, st), "cube GELU backward");
    HIPCALL(colsum(DType::BF16, rows, n, dz, n, dbias, accumulate != 0, (float *)work, st), "cube bias gradient");
    return TP_OK;
}

size_t tp_layernorm_work_bytes(const tp_shard_cfg *cfg, int64_t rows) {
    Dims d;
    if (check_cfg(cfg, &d) != TP_OK || rows <= 0 || rows > INT32_MAX) return 0;
    return layernorm_bwd_partials_floats((int)rows, (int)d.h) * sizeof(float);
}

static tp_status check_ln_rows(const Dims &d, int64_t rows) {
    if (rows < 0 || rows > INT32_MAX) return fail(TP_ESHAPE, "rows %lld out of range", (long long)rows);
    if (rows * d.h * 4 >= kMaxBuffer) return fail(TP_ESHAPE, "a tensor of %lld rows exceeds 2 GiB", (long long)rows);
    return TP_OK;
}

tp_status tp_layernorm_fwd(const tp_shard_cfg *cfg, int64_t rows, const void *x, const void *gamma, const void *beta,
                           void *u, float *mean, float *rstd, void *stream) {
    Dims d;
    tp_status s = check_cfg(cfg, &d);
    if (s != TP_OK) return s;
    if ((s = check_ln_rows(d, rows)) != TP_OK) return s;
    NEED(x, "x");
    NEED(gamma, "gamma");
    NEED(beta, "beta");
    NEED(u, "u");
    NEED4(mean, "mean");
    NEED4(rstd, "rstd");
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(u))
        return fail(TP_EALIGN, "x, gamma, beta and u must be 16-byte aligned");
    return hip_status(layernorm_fwd(d.dt, (int)rows, (int)d.h, cfg->ln_eps, x, gamma, beta, u, mean, rstd,
                                    (hipStream_t)stream),
                      "layernorm forward");
}

tp_status tp_layernorm_bwd(const tp_shard_cfg *cfg, int64_t rows, const float *du, const void *resid, const void *x,
                           const void *gamma, const float *mean, const float *rstd, void *dx, float *dgamma,
                           float *dbeta, int32_t accumulate, void *work, void *stream) {
    Dims d;
    tp_status s = check_cfg(cfg, &d);
    if (s != TP_OK) return s;
    if ((s = check_ln_rows(d, rows)) != TP_OK) return s;
    if (accumulate != 0 && accumulate != 1) return fail(TP_EINVAL, "accumulate must be 0 or 1");
    NEED(du, "du");
    NEED(resid, "resid");
    NEED(x, "x");
    NEED(gamma, "gamma");
    NEED4(mean, "mean");
    NEED4(rstd, "rstd");
    NEED(dx, "dx");
    NEED(dgamma, "dgamma");
    NEED(dbeta, "dbeta");
    NEED(work, "work");
    if (!aligned16(du) || !aligned16(resid) || !aligned16(x) || !aligned16(gamma) || !aligned16(dx) ||
        !aligned16(dgamma) || !aligned16(dbeta) || !aligned16(work))
        return fail(TP_EALIGN, "du, resid, x, gamma, dx, dgamma, dbeta and work must be 16-byte aligned");
    return hip_status(layernorm_bwd(d.dt, (int)rows, (int)d.h, du, resid, x, gamma, mean, rstd, dx, dgamma, dbeta,
                                    accumulate != 0, (float *)work, (hipStream_t)stream),
                      "layernorm backward");
}

}  // extern "C"
