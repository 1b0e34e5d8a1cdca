// Drives the C-ABI layer (api.cpp) and the slicing planner (slicing.cpp),
// built for the CPU under AddressSanitizer and UndefinedBehaviorSanitizer
// with the launchers replaced by the range-checking stand-ins of stubs.cpp:
// every phase of a small bf16 and fp32 layer shard over three groupings of a
// ragged partition, the split weight-gradient schedule, the sequence-parallel
// phases, the cube, block-attention and LayerNorm entry points, the slicing
// functions, and calls that must fail their checks.  Prints "sanitize ok"
// and exits 0 when every status is as expected and no stand-in saw a region
// outside the caller's buffers.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "tpshard.h"

extern "C" {
void stub_register(const void *p, size_t bytes);
int stub_bad();
long stub_calls();
}

static int g_fail = 0;

static void expect(tp_status got, tp_status want, const char *what) {
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, (int)got, (int)want, tp_last_error());
        ++g_fail;
    }
}

// a registered, 256-byte aligned host buffer
struct Buf {
    std::vector<unsigned char> mem;
    void *p;
    explicit Buf(size_t bytes) : mem(bytes + 256) {
        p = (void *)(((uintptr_t)mem.data() + 255) & ~(uintptr_t)255);
        std::memset(p, 0, bytes);
        stub_register(p, bytes);
    }
    float *f() { return (float *)p; }
};

static void run_shard(tp_dtype dt) {
    const int h = 256, heads = 4, d = 64, ffn = 1024, t = 2, b = 2, s = 70;
    const int32_t lens[] = {1, 29, 40};
    tp_shard_cfg cfg{h, heads, d, ffn, t, b, s, dt, 1e-5f};
    const int es = dt == TP_BF16 ? 2 : 4, ht = h / t, ft = ffn / t, T = b * s, nt = heads / t;
    Buf ln1g(h * es), ln1b(h * es), wqkv(3 * ht * h * es), bqkv(3 * ht * es), wo(h * ht * es), ln2g(h * es),
        ln2b(h * es), w1(ft * h * es), b1(ft * es), w2(h * ft * es);
    tp_shard_weights w{ln1g.p, ln1b.p, wqkv.p, bqkv.p, wo.p, ln2g.p, ln2b.p, w1.p, b1.p, w2.p};
    Buf gl1g(h * 4), gl1b(h * 4), gwqkv(3 * ht * h * 4), gbqkv(3 * ht * 4), gwo(h * ht * 4), gbo(h * 4), gl2g(h * 4),
        gl2b(h * 4), gw1(ft * h * 4), gb1(ft * 4), gw2(h * ft * 4), gb2(h * 4);
    tp_shard_grads g{gl1g.f(), gl1b.f(), gwqkv.f(), gbqkv.f(), gwo.f(), gbo.f(), gl2g.f(), gl2b.f(), gw1.f(), gb1.f(),
                     gw2.f(), gb2.f(), 0};
    Buf x(T * h * es), hm(T * h * es), dy(T * h * es), dh(T * h * es), dx(T * h * es);
    Buf pa(T * h * 4), pm(T * h * 4), pu2(T * h * 4), pu1(T * h * 4);
    Buf kc(b * nt * s * d * es), vc(b * nt * s * d * es), dk(b * nt * s * d * 4), dv(b * nt * s * d * 4);
    Buf saved(tp_shard_saved_bytes(&cfg)), scratch(tp_shard_scratch_bytes(&cfg));
    tp_partition part{3, lens};
    const int groupings[3][4] = {{0, 3, -1, -1}, {0, 1, 2, 3}, {0, 2, 3, -1}};  // whole, per-slice, pairs
    for (const auto &gr : groupings) {
        std::vector<std::pair<int, int>> calls;
        for (int i = 0; i + 1 < 4 && gr[i + 1] >= 0; ++i) calls.push_back({gr[i], gr[i + 1]});
        tp_kv_cache kv{kc.p, vc.p, 0};
        for (auto c : calls) {
            expect(tp_shard_layer_fwd(&cfg, &w, &part, c.first, c.second, TP_FWD_ATTN, x.p, pa.f(), &kv, saved.p,
                                      scratch.p, nullptr), TP_OK, "forward attention");
            expect(tp_shard_layer_fwd(&cfg, &w, &part, c.first, c.second, TP_FWD_MLP, hm.p, pm.f(), nullptr, saved.p,
                                      scratch.p, nullptr), TP_OK, "forward MLP");
        }
        for (int split = 0; split < 2; ++split) {
            tp_kv_grad kvg{dk.f(), dv.f(), s};
            bool first = true;
            for (auto it = calls.rbegin(); it != calls.rend(); ++it) {
                g.accumulate = first ? 0 : 1;
                expect(tp_shard_layer_bwd(&cfg, &w, &part, it->first, it->second,
                                          split ? TP_BWD_MLP_DATA : TP_BWD_MLP, dy.p, nullptr, nullptr, pu2.f(),
                                          nullptr, nullptr, &g, nullptr, nullptr, saved.p, scratch.p, nullptr),
                       TP_OK, "backward MLP");
                expect(tp_shard_layer_bwd(&cfg, &w, &part, it->first, it->second,
                                          split ? TP_BWD_ATTN_DATA : TP_BWD_ATTN, dy.p, hm.p, pu2.f(), pu1.f(), dh.p,
                                          nullptr, &g, &kv, &kvg, saved.p, scratch.p, nullptr),
                       TP_OK, "backward attention");
                expect(tp_shard_layer_bwd(&cfg, &w, &part, it->first, it->second, TP_BWD_LN1, nullptr, x.p, pu1.f(),
                                          nullptr, dh.p, dx.p, &g, nullptr, nullptr, saved.p, scratch.p, nullptr),
                       TP_OK, "backward LN1");
                first = false;
            }
            if (split) {
                g.accumulate = 0;
                expect(tp_shard_layer_bwd(&cfg, &w, &part, 0, 3, TP_BWD_WGRAD, dy.p, nullptr, nullptr, nullptr, dh.p,
                                          nullptr, &g, nullptr, nullptr, saved.p, scratch.p, nullptr),
                       TP_OK, "weight gradients");
            }
        }
    }
    // sequence-parallel phases over all slices
    {
        tp_kv_cache kv{kc.p, vc.p, 0};
        tp_kv_grad kvg{dk.f(), dv.f(), s};
        expect(tp_shard_layer_fwd(&cfg, &w, &part, 0, 3, TP_FWD_ATTN_SP, x.p, pa.f(), &kv, saved.p, scratch.p,
                                  nullptr), TP_OK, "sequence-parallel forward attention");
        expect(tp_shard_layer_fwd(&cfg, &w, &part, 0, 3, TP_FWD_MLP_SP, hm.p, pm.f(), nullptr, saved.p, scratch.p,
                                  nullptr), TP_OK, "sequence-parallel forward MLP");
        expect(tp_shard_layer_bwd(&cfg, &w, &part, 0, 3, TP_BWD_ATTN_SP, dy.p, nullptr, nullptr, pu1.f(), dh.p,
                                  nullptr, &g, &kv, &kvg, saved.p, scratch.p, nullptr),
               TP_OK, "sequence-parallel backward attention");
        Buf mu((T / t) * 4), rs((T / t) * 4), work(tp_layernorm_work_bytes(&cfg, T / t));
        expect(tp_layernorm_fwd(&cfg, T / t, x.p, ln1g.p, ln1b.p, hm.p, mu.f(), rs.f(), nullptr), TP_OK,
               "shard LayerNorm");
        expect(tp_layernorm_bwd(&cfg, T / t, pu1.f(), dh.p, x.p, ln1g.p, mu.f(), rs.f(), dx.p, gl1g.f(), gl1b.f(), 0,
                                work.p, nullptr), TP_OK, "shard LayerNorm backward");
        expect(tp_residual_combine(&cfg, T, x.p, pa.f(), ln1g.p, hm.p, nullptr), TP_OK, "combine");
    }
    // checks that must fail before anything is enqueued
    tp_kv_cache kv{kc.p, vc.p, 5};
    expect(tp_shard_layer_fwd(&cfg, &w, &part, 1, 2, TP_FWD_ATTN, x.p, pa.f(), &kv, saved.p, scratch.p, nullptr),
           TP_EORDER, "out-of-order slice");
    expect(tp_shard_layer_fwd(&cfg, &w, &part, 2, 1, TP_FWD_ATTN, x.p, pa.f(), &kv, saved.p, scratch.p, nullptr),
           TP_EINVAL, "empty slice range");
    expect(tp_shard_layer_fwd(&cfg, &w, &part, 0, 1, 9, x.p, pa.f(), &kv, saved.p, scratch.p, nullptr), TP_EINVAL,
           "bad phase");
    expect(tp_shard_layer_fwd(&cfg, &w, &part, 0, 1, TP_FWD_MLP, (char *)x.p + 2, pa.f(), nullptr, saved.p,
                              scratch.p, nullptr), TP_EALIGN, "misaligned input");
    const int32_t bad_lens[] = {10, 0, 60};
    tp_partition bad{3, bad_lens};
    expect(tp_shard_layer_fwd(&cfg, &w, &bad, 0, 1, TP_FWD_MLP, x.p, pa.f(), nullptr, saved.p, scratch.p, nullptr),
           TP_ESHAPE, "zero-length slice");
    tp_shard_cfg c2 = cfg;
    c2.head_dim = 32;
    c2.heads = 8;
    expect(tp_shard_layer_fwd(&c2, &w, &part, 0, 1, TP_FWD_MLP, x.p, pa.f(), nullptr, saved.p, scratch.p, nullptr),
           TP_EUNSUPPORTED, "head_dim 32");
}

static void run_blocks() {
    const int b = 1, n = 2, d = 128, nq = 70, nk = 50;
    tp_attn_block_shape sh{b, n, d, nq, nk, 30, 10};
    Buf q(b * n * nq * d * 2), k(b * n * nk * d * 2), v(b * n * nk * d * 2), dout(b * n * nq * d * 2);
    Buf o(b * n * nq * d * 4), lse(b * n * nq * 4), o2(b * n * nq * d * 4), lse2(b * n * nq * 4);
    Buf dq(b * n * nq * d * 4), dk(b * n * nk * d * 4), dv(b * n * nk * d * 4), work(tp_attn_block_bwd_work_bytes(&sh));
    expect(tp_attn_block_fwd(&sh, q.p, k.p, v.p, o.f(), lse.f(), nullptr), TP_OK, "block forward");
    expect(tp_attn_merge(&sh, o.f(), lse.f(), o2.f(), lse2.f(), o2.f(), lse2.f(), nullptr), TP_OK, "merge");
    expect(tp_attn_block_bwd(&sh, q.p, k.p, v.p, o.f(), lse.f(), dout.p, dq.f(), dk.f(), dv.f(), 1, work.p, nullptr),
           TP_OK, "block backward");
    expect(tp_attn_block_bwd(&sh, q.p, k.p, v.p, o.f(), lse.f(), dout.p, dq.f(), dk.f(), dv.f(), 2, work.p, nullptr),
           TP_EINVAL, "block backward accumulate flag");
    const int rows = 40, hid = 64, f = 96;
    Buf x(rows * hid * 2), w1(f * hid * 2), b1(f * 2), w2(hid * f * 2), hb(rows * f * 2), out(rows * hid * 4);
    expect(tp_cube_ffn_block(rows, hid, f, x.p, w1.p, b1.p, w2.p, hb.p, out.f(), nullptr), TP_OK, "cube block");
    Buf zs(rows * f * 4), z(rows * f * 2), hh(rows * f * 2), dz(rows * f * 2), db(f * 4), cw(tp_cube_work_bytes(rows, f));
    Buf dw(hid * f * 4);
    expect(tp_cube_matmul(TP_CUBE_ATB, hid, f, rows, x.p, hb.p, dw.f(), 1, nullptr), TP_OK, "cube ATB");
    expect(tp_cube_matmul(TP_CUBE_ATB, hid, f, rows - 4, x.p, hb.p, dw.f(), 0, nullptr), TP_ESHAPE,
           "cube reduction not a multiple of 8");
    expect(tp_cube_matmul(TP_CUBE_AB, rows, f, hid, x.p, w1.p, zs.f(), 0, nullptr), TP_OK, "cube AB");
    expect(tp_cube_bias_gelu(rows, f, zs.f(), b1.p, z.p, hh.p, nullptr), TP_OK, "cube bias GELU");
    expect(tp_cube_gelu_backward(rows, f, zs.f(), z.p, dz.p, db.f(), 0, cw.p, nullptr), TP_OK, "cube GELU backward");
}

static void run_slicing() {
    const int units = 12, W = units + 1;
    std::vector<double> fwd(W), cost(W * W);
    for (int k = 1; k <= units; ++k) fwd[k] = 0.5 + 0.1 * k;
    int32_t len[6] = {16, 32, 64, 16, 32, 64}, off[6] = {16, 16, 32, 64, 96, 128};
    double ctx[6];
    for (int i = 0; i < 6; ++i) ctx[i] = 1e-4 * len[i] * off[i] + 2e-3 * off[i] + 0.01;
    double coef[3];
    expect(tp_fit_context_model(6, len, off, ctx, coef), TP_OK, "fit");
    expect(tp_slice_cost_table(units, 16, fwd.data(), coef, cost.data()), TP_OK, "cost table");
    int32_t ends[units], n = 0;
    double lat = 0, lat2 = 0;
    for (int stages : {1, 2, 8}) {
        expect(tp_slicing_plan(units, cost.data(), stages, &n, ends, &lat), TP_OK, "plan");
        expect(tp_plan_latency(units, cost.data(), stages, n, ends, &lat2), TP_OK, "plan latency");
        if (std::fabs(lat - lat2) > 1e-9) {
            std::fprintf(stderr, "plan latency %g != %g\n", lat, lat2);
            ++g_fail;
        }
    }
    expect(tp_slicing_plan(0, cost.data(), 2, &n, ends, &lat), TP_EINVAL, "zero units");
    expect(tp_fit_context_model(2, len, off, ctx, coef), TP_EINVAL, "too few samples");
}

int main() {
    run_shard(TP_BF16);
    run_shard(TP_F32);
    run_blocks();
    run_slicing();
    if (g_fail || stub_bad()) {
        std::fprintf(stderr, "sanitize: %d unexpected statuses, %d out-of-range regions\n", g_fail, stub_bad());
        return 1;
    }
    std::printf("sanitize ok: %ld launches checked\n", stub_calls());
    return 0;
}
