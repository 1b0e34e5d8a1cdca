// Host-only stand-ins for the library's kernel launchers (the functions of
// kernels.h) and the two HIP runtime calls the C-ABI layer makes, for a CPU
// build of api.cpp and slicing.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Nothing is launched: each stand-in checks that
// every buffer region its arguments address lies inside a buffer the driver
// registered (the pointer arithmetic of the C-ABI layer stays inside the
// caller's allocations) and counts the call.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <vector>

#include "kernels.h"

namespace {

struct Range {
    const char *lo, *hi;
};
std::vector<Range> g_ranges;
int g_bad = 0;
long g_calls = 0;

void need(const void *p, double bytes, const char *what) {
    if (bytes <= 0) return;
    if (!p) {
        std::fprintf(stderr, "stub: %s is NULL\n", what);
        ++g_bad;
        return;
    }
    const char *c = (const char *)p;
    for (const Range &r : g_ranges)
        if (c >= r.lo && c + (size_t)bytes <= r.hi) return;
    std::fprintf(stderr, "stub: %s [%p, +%.0f bytes) is outside every registered buffer\n", what, p, bytes);
    ++g_bad;
}

double extent(int rows, int k, const tpk::Mat &m) {
    // elements from the base to one past the last one addressed
    return m.kcontig ? (double)(rows - 1) * m.ld + k : (double)(k - 1) * m.ld + rows;
}

}  // namespace

extern "C" {
void stub_register(const void *p, size_t bytes) { g_ranges.push_back({(const char *)p, (const char *)p + bytes}); }
int stub_bad() { return g_bad; }
long stub_calls() { return g_calls; }

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind, hipStream_t) {
    ++g_calls;
    need(dst, (double)bytes, "memcpy destination");
    need(src, (double)bytes, "memcpy source");
    return hipSuccess;
}
const char *hipGetErrorString(hipError_t) { return "stub"; }
}

namespace tpk {

hipError_t gemm(DType dt, int M, int N, int K, Mat A, Mat B, Epi kind, const EpiArgs &e, hipStream_t) {
    ++g_calls;
    const int es = dt == DType::BF16 ? 2 : 4;
    if (M <= 0 || N <= 0) return hipSuccess;
    if (K > 0) {
        need(A.p, extent(M, K, A) * es, "product operand A");
        need(B.p, extent(N, K, B) * es, "product operand B");
    }
    const double mn = (double)(M - 1) * e.ldc + N;
    switch (kind) {
    case Epi::StoreF32:
    case Epi::AccumF32: need(e.c, mn * 4, "fp32 product output"); break;
    case Epi::Store: need(e.c, mn * es, "product output"); break;
    case Epi::BiasGelu:
        if (e.c) need(e.c, mn * es, "GELU' output");
        need(e.c2, ((double)(M - 1) * e.ldc2 + N) * es, "GELU output");
        need(e.bias, (double)N * es, "bias");
        break;
    case Epi::GeluGrad:
        need(e.c, mn * es, "dZ output");
        need(e.aux, ((double)(M - 1) * e.ldaux + N) * es, "GELU' input");
        break;
    case Epi::Qkv: {
        // the last row of the call lands at position (row0 + M - 1) / batch
        const int p = (e.row0 + M - 1) / e.batch;
        if (p >= e.seq) {
            std::fprintf(stderr, "stub: QKV scatter past the sequence\n");
            ++g_bad;
        }
        const double slab = (double)e.batch * e.nt * e.seq * e.d * es;
        need(e.q, slab, "Q");
        need(e.k, slab, "K cache");
        need(e.v, slab, "V cache");
        need(e.bias, (double)N * es, "QKV bias");
        break;
    }
    }
    if (e.split_ws) need(e.split_ws, (double)e.split_ws_floats * 4, "split workspace");
    return hipSuccess;
}
void gemm_force_tile(int) {}
size_t gemm_split_workspace_floats() { return 512ull * 128 * 192; }

hipError_t layernorm_fwd(DType dt, int rows, int h, float, const void *x, const void *g, const void *b, void *u,
                         float *mean, float *rstd, hipStream_t) {
    ++g_calls;
    const int es = dt == DType::BF16 ? 2 : 4;
    need(x, (double)rows * h * es, "LN input");
    need(u, (double)rows * h * es, "LN output");
    need(g, (double)h * es, "gamma");
    need(b, (double)h * es, "beta");
    need(mean, rows * 4.0, "mean");
    need(rstd, rows * 4.0, "rstd");
    return hipSuccess;
}
static int ln_blocks(int rows) { return rows < 256 ? rows : 256; }
static int cs_chunks(int rows) {
    int c = (rows + 31) / 32;
    return c < 256 ? (c < 1 ? 1 : c) : 256;
}
size_t layernorm_bwd_partials_floats(int rows, int h) { return (size_t)ln_blocks(rows) * 2 * h; }
size_t colsum_partials_floats(int rows, int n) { return (size_t)cs_chunks(rows) * n; }

hipError_t layernorm_bwd_rows(DType dt, int rows, int h, const float *du, const void *resid, const void *x,
                              const void *g, const float *mean, const float *rstd, void *dx, float *partials,
                              hipStream_t) {
    ++g_calls;
    const int es = dt == DType::BF16 ? 2 : 4;
    need(du, (double)rows * h * 4, "LN du");
    need(resid, (double)rows * h * es, "LN residual");
    need(x, (double)rows * h * es, "LN x");
    need(dx, (double)rows * h * es, "LN dx");
    need(g, (double)h * es, "gamma");
    need(mean, rows * 4.0, "mean");
    need(rstd, rows * 4.0, "rstd");
    need(partials, (double)layernorm_bwd_partials_floats(rows, h) * 4, "LN partials");
    return hipSuccess;
}
hipError_t layernorm_bwd(DType dt, int rows, int h, const float *du, const void *resid, const void *x, const void *g,
                         const float *mean, const float *rstd, void *dx, float *dg, float *db, bool, float *partials,
                         hipStream_t st) {
    need(dg, h * 4.0, "dgamma");
    need(db, h * 4.0, "dbeta");
    return layernorm_bwd_rows(dt, rows, h, du, resid, x, g, mean, rstd, dx, partials, st);
}
hipError_t colsum_rows(DType dt, int rows, int n1, const void *a1, int64_t lda1, int n2, const void *a2, int64_t lda2,
                       float *partials, hipStream_t) {
    ++g_calls;
    const int es = dt == DType::BF16 ? 2 : 4;
    if (rows <= 0) return hipSuccess;
    need(a1, ((double)(rows - 1) * lda1 + n1) * es, "column-sum matrix 1");
    if (n2 > 0) need(a2, ((double)(rows - 1) * lda2 + n2) * es, "column-sum matrix 2");
    need(partials, (double)colsum_partials_floats(rows, n1 + n2) * 4, "column-sum partials");
    return hipSuccess;
}
hipError_t colsum(DType dt, int rows, int n, const void *a, int64_t lda, float *out, bool, float *partials,
                  hipStream_t st) {
    need(out, n * 4.0, "column sums");
    return colsum_rows(dt, rows, n, a, lda, 0, nullptr, 0, partials, st);
}
ReduceSpec ln_bwd_reduce_spec(int rows, int h, const float *partials, float *dg, float *db) {
    return ReduceSpec{ln_blocks(rows), 2 * h, h, (int64_t)2 * h, partials, dg, db};
}
ReduceSpec colsum_reduce_spec(int rows, int n1, int n2, const float *partials, float *out1, float *out2) {
    return ReduceSpec{cs_chunks(rows), n1 + n2, n1, (int64_t)(n1 + n2), partials, out1, out2};
}
hipError_t reduce_partials(const ReduceSpec *a, const ReduceSpec *b, bool, hipStream_t) {
    ++g_calls;
    for (const ReduceSpec *r : {a, b}) {
        if (!r) continue;
        need(r->partials, ((double)(r->nblk - 1) * r->stride + r->n) * 4, "partials");
        need(r->out0, r->n0 * 4.0, "reduction output 0");
        if (r->n > r->n0) need(r->out1, (r->n - r->n0) * 4.0, "reduction output 1");
    }
    return hipSuccess;
}
hipError_t residual_combine(DType dt, int64_t rows, int h, const void *resid, const float *reduced, const void *bias,
                            void *out, hipStream_t) {
    ++g_calls;
    const int es = dt == DType::BF16 ? 2 : 4;
    need(resid, (double)rows * h * es, "residual");
    need(reduced, (double)rows * h * 4, "reduced");
    need(bias, (double)h * es, "bias");
    need(out, (double)rows * h * es, "combine output");
    return hipSuccess;
}

size_t attn_fwd_work_floats(int batch, int nt, int seq, int d) {
    const int nqt = (seq + 127) / 128;
    const size_t fwd = (size_t)batch * nt * nqt * 8 * 128 * (d + 2);
    const size_t bwd = (size_t)batch * nt * ((seq + 127) / 128) * 8 * 2 * 128 * d;
    return fwd > bwd ? fwd : bwd;
}
size_t attn_fwd_call_work_floats(int batch, int nt, int q0, int q1, int d) {
    return q1 > q0 ? attn_fwd_work_floats(batch, nt, q1, d) : 0;
}
hipError_t attn_fwd(DType dt, const AttnArgs &a, hipStream_t) {
    ++g_calls;
    const int es = dt == DType::BF16 ? 2 : 4;
    const double slab = (double)a.batch * a.nt * a.seq * a.d * es;
    need(a.q, slab, "saved Q");
    need(a.k, slab, "K cache");
    need(a.v, slab, "V cache");
    need(a.o, (double)a.seq * a.batch * a.nt * a.d * es, "saved O");
    need(a.lse, (double)a.batch * a.nt * a.seq * 4, "LSE");
    if (dt == DType::BF16)
        need(a.work, (double)attn_fwd_call_work_floats(a.batch, a.nt, a.q0, a.q1, a.d) * 4, "attention work");
    return hipSuccess;
}
hipError_t attn_bwd(DType dt, const AttnArgs &a, hipStream_t st) {
    attn_fwd(dt, a, st);
    const int es = dt == DType::BF16 ? 2 : 4;
    need(a.dout, (double)a.seq * a.batch * a.nt * a.d * es, "dO");
    need(a.delta, (double)a.batch * a.nt * a.seq * 4, "delta");
    need(a.dqkv, (double)a.seq * a.batch * 3 * a.nt * a.d * es, "dQKV");
    need(a.dk_acc, (double)a.batch * a.nt * a.seq * a.d * 4, "dK accumulator");
    need(a.dv_acc, (double)a.batch * a.nt * a.seq * a.d * 4, "dV accumulator");
    return hipSuccess;
}
hipError_t bias_gelu(int64_t rows, int n, const float *z_sum, const void *bias, void *z, void *h, hipStream_t) {
    ++g_calls;
    need(z_sum, (double)rows * n * 4, "z_sum");
    need(bias, n * 2.0, "bias");
    need(z, (double)rows * n * 2, "z");
    need(h, (double)rows * n * 2, "h");
    return hipSuccess;
}
hipError_t gelu_backward(int64_t rows, int n, const float *dh, const void *z, void *dz, hipStream_t) {
    ++g_calls;
    need(dh, (double)rows * n * 4, "dh");
    need(z, (double)rows * n * 2, "z");
    need(dz, (double)rows * n * 2, "dz");
    return hipSuccess;
}
hipError_t attn_block_fwd(const AttnBlockArgs &a, hipStream_t) {
    ++g_calls;
    need(a.q, (double)a.bh * a.nq * a.d * 2, "block q");
    need(a.k, (double)a.bh * a.nk * a.d * 2, "block k");
    need(a.v, (double)a.bh * a.nk * a.d * 2, "block v");
    need(a.o, (double)a.bh * a.nq * a.d * 4, "block o");
    need(a.lse, (double)a.bh * a.nq * 4, "block lse");
    return hipSuccess;
}
hipError_t attn_merge(int64_t rows, int d, const float *oa, const float *la, const float *ob, const float *lb,
                      float *o, float *lse, hipStream_t) {
    ++g_calls;
    for (const float *p : {oa, ob, (const float *)o}) need(p, (double)rows * d * 4, "merge o");
    for (const float *p : {la, lb, (const float *)lse}) need(p, (double)rows * 4, "merge lse");
    return hipSuccess;
}
size_t attn_block_bwd_work_floats(int bh, int nq) { return (size_t)bh * (size_t)(nq > 0 ? nq : 0); }
hipError_t attn_block_bwd(const AttnBlockBwdArgs &a, hipStream_t) {
    ++g_calls;
    need(a.q, (double)a.bh * a.nq * a.d * 2, "block q");
    need(a.dout, (double)a.bh * a.nq * a.d * 2, "block dO");
    need(a.k, (double)a.bh * a.nk * a.d * 2, "block k");
    need(a.v, (double)a.bh * a.nk * a.d * 2, "block v");
    need(a.o, (double)a.bh * a.nq * a.d * 4, "block o");
    need(a.lse, (double)a.bh * a.nq * 4, "block lse");
    need(a.dq, (double)a.bh * a.nq * a.d * 4, "block dq");
    need(a.dk, (double)a.bh * a.nk * a.d * 4, "block dk");
    need(a.dv, (double)a.bh * a.nk * a.d * 4, "block dv");
    need(a.work, (double)attn_block_bwd_work_floats(a.bh, a.nq) * 4, "block work");
    return hipSuccess;
}

}  // namespace tpk
