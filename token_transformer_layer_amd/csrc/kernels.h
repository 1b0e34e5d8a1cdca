// Internal launch interface between the C-ABI layer (api.cpp) and the gfx950
// kernels.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

enum class DType { F32 = 0, BF16 = 1 };

// One GEMM operand.  The product is C[m][n] = sum_k A[m][k] B[n][k].
// kcontig: element (i, k) sits at p + i*ld + k (k contiguous); otherwise at
// p + k*ld + i (the M/N index contiguous).
struct Mat {
    const void *p;
    int64_t ld;
    bool kcontig;
};

enum class Epi {
    StoreF32,  // c fp32 [M][ldc] = acc
    AccumF32,  // c fp32 [M][ldc] += acc
    Store,     // c T [M][ldc] = acc
    BiasGelu,  // z = acc + bias[n]; c T = GELU'(z) (if c != null); c2 T = GELU(z)
    GeluGrad,  // c T = acc * aux[m][n]  (aux T [M][ldaux]: the GELU'(Z) BiasGelu stored)
    Qkv,       // acc + bias[n] scattered into q/k/v [b, n_t, s, d]
};

struct EpiArgs {
    void *c = nullptr;
    int64_t ldc = 0;
    void *c2 = nullptr;
    int64_t ldc2 = 0;
    const void *bias = nullptr;
    const void *aux = nullptr;
    int64_t ldaux = 0;
    // Qkv scatter: token row m of the call is global row row0 + m = p*batch + bi
    void *q = nullptr, *k = nullptr, *v = nullptr;
    int batch = 1, seq = 1, nt = 1, d = 64, ht = 64, row0 = 0;
    // workspace for split reductions (fp32, split_ws_floats floats); a
    // product may split its reduction over workgroups when it is given
    float *split_ws = nullptr;
    int64_t split_ws_floats = 0;
};

hipError_t gemm(DType dt, int M, int N, int K, Mat A, Mat B, Epi kind, const EpiArgs &e,
                hipStream_t st);
// -1: tile configuration chosen per shape; 0..6: forced (see tp_gemm_force_tile)
void gemm_force_tile(int tile);
// floats of split-reduction workspace that lets every product split
size_t gemm_split_workspace_floats();

// LayerNorm forward over rows [0, rows): u = LN(x) * g + b; mean/rstd fp32.
hipError_t layernorm_fwd(DType dt, int rows, int h, float eps, const void *x, const void *g,
                         const void *b, void *u, float *mean, float *rstd, hipStream_t st);

// LayerNorm backward with residual: dx = resid + LN^T(du); the parameter
// gradients go to dg/db (fp32; added when accumulate, else stored) through a
// deterministic two-stage reduction that uses `partials` (fp32,
// layernorm_bwd_partials_floats).
hipError_t layernorm_bwd(DType dt, int rows, int h, const float *du, const void *resid,
                         const void *x, const void *g, const float *mean, const float *rstd,
                         void *dx, float *dg, float *db, bool accumulate, float *partials,
                         hipStream_t st);
size_t layernorm_bwd_partials_floats(int rows, int h);

// Column sums over rows into out (fp32; added when accumulate, else
// stored), two stages via `partials`.
hipError_t colsum(DType dt, int rows, int n, const void *a, int64_t lda, float *out, bool accumulate,
                  float *partials, hipStream_t st);
size_t colsum_partials_floats(int rows, int n);

// The same two reductions split into their stages, so that one launch can
// finish several of them: the first stage writes per-block partial sums
// (LayerNorm: [blocks][2 h], dgamma then dbeta; column sums of one or two
// matrices with the same rows: [chunks][n1 + n2]); a ReduceSpec names the
// partials and their outputs (columns c < n0 to out0, the rest to out1), and
// reduce_partials finishes up to two of them in one launch.
struct ReduceSpec {
    int nblk, n, n0;
    int64_t stride;
    const float *partials;
    float *out0, *out1;
};
hipError_t layernorm_bwd_rows(DType dt, int rows, int h, const float *du, const void *resid, const void *x,
                              const void *g, const float *mean, const float *rstd, void *dx, float *partials,
                              hipStream_t st);
hipError_t colsum_rows(DType dt, int rows, int n1, const void *a1, int64_t lda1, int n2, const void *a2, int64_t lda2,
                       float *partials, hipStream_t st);
ReduceSpec ln_bwd_reduce_spec(int rows, int h, const float *partials, float *dg, float *db);
ReduceSpec colsum_reduce_spec(int rows, int n1, int n2, const float *partials, float *out1, float *out2);
hipError_t reduce_partials(const ReduceSpec *a, const ReduceSpec *b, bool accumulate, hipStream_t st);

// out = resid + reduced + bias[c]
hipError_t residual_combine(DType dt, int64_t rows, int h, const void *resid, const float *reduced,
                            const void *bias, void *out, hipStream_t st);

// Attention over the queries at positions [q0, q1) of every (batch row, head),
// against keys [0, q1) of the cache.  q: [b, nt, s, d]; k, v: cache
// [b, nt, s, d]; o: token-major [s, b, nt*d] (column head*d + j); lse fp32
// [b, nt, s].
struct AttnArgs {
    int batch, nt, seq, d;
    int q0, q1;
    float scale;
    const void *q, *k, *v;
    void *o;
    float *lse;
    // backward
    const void *dout;     // token-major [s, b, nt*d]
    float *delta;         // [b, nt, s] rowsum(dO * O)
    void *dqkv;           // token-major [s, b, 3*nt*d]: dq cols [0,ht), dk [ht,2ht), dv [2ht,3ht)
    float *dk_acc, *dv_acc;  // [b, nt, s, d] fp32 accumulators
    int k_final0;         // keys in [k_final0, q1) are complete after this call
    bool acc_in;          // accumulators hold earlier calls' contributions
    float *work;          // partial sums of split work (attn_fwd_work_floats floats; fwd and bwd)
};
size_t attn_fwd_work_floats(int batch, int nt, int seq, int d);
// floats of split-KV partial sums the forward over queries [q0, q1) writes
size_t attn_fwd_call_work_floats(int batch, int nt, int q0, int q1, int d);
hipError_t attn_fwd(DType dt, const AttnArgs &a, hipStream_t st);
hipError_t attn_bwd(DType dt, const AttnArgs &a, hipStream_t st);

// Cube-partition FFN steps (bf16 outputs, n a multiple of 8): z = z_sum +
// bias, h = GELU(z); dz = dh * GELU'(z).
hipError_t bias_gelu(int64_t rows, int n, const float *z_sum, const void *bias, void *z, void *h, hipStream_t st);
hipError_t gelu_backward(int64_t rows, int n, const float *dh, const void *z, void *dz, hipStream_t st);

// Attention of nq queries at positions q_pos0.. over one block of nk keys at
// positions k_pos0.. (key position <= query position), per (batch row, head)
// slab of bh: q [bh, nq, d], k, v [bh, nk, d] bf16 -> o [bh, nq, d] fp32
// normalised, lse [bh, nq] (-inf, o = 0, where no key is visible).
struct AttnBlockArgs {
    int bh, nq, nk, d, q_pos0, k_pos0;
    float scale;
    const void *q, *k, *v;
    float *o, *lse;
};
hipError_t attn_block_fwd(const AttnBlockArgs &a, hipStream_t st);
// Backward of attention over one key block given the merged forward result
// (o fp32 [bh, nq, d], lse [bh, nq]) and dout bf16 [bh, nq, d]: this block's
// share of dq (fp32 [bh, nq, d]) and the block's dk, dv (fp32 [bh, nk, d]),
// stored or (accumulate) added; work: attn_block_bwd_work_floats floats.
struct AttnBlockBwdArgs {
    int bh, nq, nk, d, q_pos0, k_pos0;
    bool accumulate;
    float scale;
    const void *q, *k, *v, *dout;
    const float *o, *lse;
    float *dq, *dk, *dv, *work;
};
size_t attn_block_bwd_work_floats(int bh, int nq);
hipError_t attn_block_bwd(const AttnBlockBwdArgs &a, hipStream_t st);
// merge of two partial results over disjoint key sets (rows = bh * nq)
hipError_t attn_merge(int64_t rows, int d, const float *oa, const float *la, const float *ob, const float *lb,
                      float *o, float *lse, hipStream_t st);

}  // namespace tpk
