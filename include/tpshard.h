/*
 * tpshard.h - one tensor-parallel device's share of a pre-LayerNorm GPT
 * decoder layer, run over token slices, on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Rank r of t holds a column-split QKV projection (its
 * group of n/t heads) and a column-split FC1 with GELU, and a row-split
 * output projection and FC2 whose products are partial sums that an
 * all-reduce over the t ranks would add ("Transformer Training 11: model
 * parallelism", tensor-parallelism slide).  LayerNorm is replicated on every
 * rank (same deck, sequence-parallelism slide).  The layer runs slice by
 * slice along the token dimension, each slice attending to the cached K/V of
 * the slices before it ("TeraPipe: Token-Level Pipeline Parallelism for
 * Training Large-Scale Language Models", section 3).  The backward uses the
 * product-gradient forms of "Maximizing Parallelism in Distributed Training
 * for Huge Neural Networks", section 3.1.2, and the bias/scale backward of
 * its section 3.1.3.
 *
 * Forward of one layer (x: layer input, y: layer output; sums run over the
 * t ranks and are the caller's all-reduce):
 *   TP_FWD_ATTN  : P_attn,r = Attn_r(LN1(x)) W_o,r^T           (fp32 partial)
 *   caller       : h_mid = x + sum_r P_attn,r + b_o             (tp_residual_combine)
 *   TP_FWD_MLP   : P_mlp,r = GELU(LN2(h_mid) W1,r^T + b1,r) W2,r^T
 *   caller       : y = h_mid + sum_r P_mlp,r + b2
 * Backward, given dY:
 *   TP_BWD_MLP   : dU2,r (fp32 partial), dW1,r, db1,r, dW2,r, db2
 *   caller       : dU2 = sum_r dU2,r
 *   TP_BWD_ATTN  : dH = dY + LN2^T(dU2); dU1,r (fp32 partial), dW_o,r, db_o,
 *                  dW_qkv,r, db_qkv,r, dgamma2, dbeta2
 *   caller       : dU1 = sum_r dU1,r
 *   TP_BWD_LN1   : dX = dH + LN1^T(dU1), dgamma1, dbeta1
 *
 * Readings where the pages are silent: LayerNorm with the biased variance;
 * exact erf GELU; attention scale 1/sqrt(d); the causal mask keeps the
 * diagonal; no dropout; the row-split biases b_o and b2 are not in the
 * partial sums (the caller adds them once, after the reduction).
 *
 * Layouts (row-major, element type = cfg->dtype unless marked fp32):
 *   activations       [s, b, h]   sequence-major: token row m = p*b + bi, so a
 *                                 slice is a contiguous block of rows
 *   w_qkv             [3 h_t, h]  rows [0,h_t) W_q, [h_t,2h_t) W_k, [2h_t,3h_t)
 *                                 W_v of this rank's heads (head i of the rank
 *                                 owns rows [i d, (i+1) d) of each)
 *   b_qkv             [3 h_t]
 *   w_o               [h, h_t]    columns of the full W_o for this rank's heads
 *   w1 [f_t, h], b1 [f_t], w2 [h, f_t]
 *   ln*_g, ln*_b      [h]         replicated
 *   K/V cache         [b, n_t, s, d] each
 *   dK/dV accumulators[b, n_t, s, d] fp32 each
 *   gradients         fp32, same shapes as the weights; ACCUMULATED (+=)
 * with n_t = heads/t, h_t = hidden/t, f_t = ffn/t.
 *
 * Ownership.  The caller allocates every buffer (device memory for tensors,
 * host memory for the structs and the partition) and keeps it alive until
 * the stream has run the work; the library allocates nothing and frees
 * nothing.  Structs are read (and, for the cache protocol fields, written)
 * only during the call.
 *
 * Asynchrony.  Every call enqueues kernels on the given HIP stream
 * (hipStream_t passed as void*; NULL is the default stream) and returns.
 *
 * Errors.  Argument checks run on the host before anything is enqueued; a
 * failed check returns a non-zero tp_status, enqueues nothing and leaves
 * every buffer and struct untouched.  TP_EHIP means a kernel launch failed;
 * work already enqueued by that call may have run.  tp_last_error() gives a
 * message for the calling thread's last failure.  No C++ exception crosses
 * this interface.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_EINVAL = 1,       /* null pointer, bad enum, bad slice range */
    TP_ESHAPE = 2,       /* configuration or partition inconsistent or unsupported size */
    TP_EALIGN = 3,       /* a device pointer is not 16-byte aligned */
    TP_EORDER = 4,       /* token-slice order violated (cache protocol) */
    TP_EUNSUPPORTED = 5, /* valid but not implemented (e.g. head_dim not 64/128) */
    TP_EHIP = 6          /* HIP runtime error while enqueueing */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Shape of the whole layer and of this rank's share.  hidden = heads *
 * head_dim; heads and ffn divisible by tp_size; head_dim 64 or 128; ffn/t a
 * multiple of 8; hidden <= 16384.  dtype is the storage type of activations,
 * weights, the K/V cache and saved activations; all products accumulate in
 * fp32 and all partial sums and gradients are fp32.  ln_eps is LayerNorm's
 * epsilon (1e-5 in this repository's workloads). */
typedef struct {
    int32_t hidden;
    int32_t heads;
    int32_t head_dim;
    int32_t ffn;
    int32_t tp_size;
    int32_t batch;
    int32_t seq_len;
    int32_t dtype; /* tp_dtype */
    float ln_eps;
} tp_shard_cfg;

/* This rank's parameters, device pointers of element type cfg->dtype.
 * b_o and b2 are not here: they are added by the caller after the
 * reduction (tp_residual_combine). */
typedef struct {
    const void *ln1_g, *ln1_b;
    const void *w_qkv, *b_qkv;
    const void *w_o;
    const void *ln2_g, *ln2_b;
    const void *w1, *b1;
    const void *w2;
} tp_shard_weights;

/* fp32 device gradient buffers.  accumulate = 1: every gradient a call
 * produces is added into its buffer (+=); accumulate = 0: the call
 * overwrites each gradient buffer it produces (=), as BLAS does with
 * beta = 0.  A step that runs one call per phase over all slices can use 0
 * and skip zeroing; a step over several calls passes 0 on the first call
 * that produces a given gradient and 1 afterwards.  b_o and b2 are the
 * replicated row-split biases: every rank computes the same value. */
typedef struct {
    float *ln1_g, *ln1_b;
    float *w_qkv, *b_qkv;
    float *w_o, *b_o;
    float *ln2_g, *ln2_b;
    float *w1, *b1;
    float *w2, *b2;
    int32_t accumulate;
} tp_shard_grads;

/* Token-slice partition l_1..l_M of the sequence (host memory): every
 * length >= 1 and the lengths sum to seq_len ("TeraPipe", section 3).  Slice
 * j covers positions [o_j, o_j + l_j) with o_j = l_1 + ... + l_{j-1}, i.e.
 * token rows [o_j b, (o_j + l_j) b) of every [s, b, ...] activation. */
typedef struct {
    int32_t num_slices;
    const int32_t *len;
} tp_partition;

/* Prefix K/V cache (device memory, [b, n_t, s, d] each, element type
 * cfg->dtype) and the number of positions already filled.  A forward
 * attention call over slices [j0, j1) requires filled == o_{j0} (else
 * TP_EORDER) and sets filled = o_{j1} when it returns TP_OK. */
typedef struct {
    void *k, *v;
    int32_t filled;
} tp_kv_cache;

/* dK/dV accumulators of the backward over slices (device memory, fp32,
 * [b, n_t, s, d] each).  Backward attention calls run the slices in reverse:
 * a call over [j0, j1) requires done_from == o_{j1} (else TP_EORDER) and sets
 * done_from = o_{j0}.  Start a step with done_from = seq_len; the first call
 * does not read the accumulators, so they need no zeroing.  Their contents
 * are the library's working values (dK is held without the 1/sqrt(d)
 * factor); the final dK and dV of a slice's keys are written to dqkv. */
typedef struct {
    float *dk, *dv;
    int32_t done_from;
} tp_kv_grad;

/* Forward phases.  The _SP phases are the sequence-parallel form
 * ("Transformer Training 11: model parallelism", sequence-parallelism
 * slide: LayerNorm and dropout split along the sequence, each all-reduce
 * becoming a reduce-scatter and an all-gather): LayerNorm runs on the
 * rank's sequence shard (tp_layernorm_fwd) and the caller all-gathers its
 * output, which TP_FWD_ATTN_SP / TP_FWD_MLP_SP take as `in` (LN1(x) /
 * LN2(h_mid) for the call's rows) instead of computing it; the partial sums
 * are then reduce-scattered instead of all-reduced. */
typedef enum { TP_FWD_ATTN = 0, TP_FWD_MLP = 1, TP_FWD_ATTN_SP = 2, TP_FWD_MLP_SP = 3 } tp_fwd_phase;
/* Backward phases.  TP_BWD_MLP = TP_BWD_MLP_DATA + the MLP weight and bias
 * gradients of the call's rows; TP_BWD_ATTN = TP_BWD_ATTN_DATA + the
 * attention block's weight and bias gradients.  The _DATA phases produce
 * only what the next phase needs (the partial sums, dH, dK/dV and the
 * LayerNorm parameter gradients), so a pipeline stage can run them per slice
 * and take every weight gradient afterwards in one TP_BWD_WGRAD call over all
 * slices (dW2, db1, db2, dW1, dW_o, db_o, dW_qkv, db_qkv), which reads dY, dH,
 * the saved activations and the per-row intermediates the _DATA calls left in
 * scratch. */
typedef enum {
    TP_BWD_MLP = 0,
    TP_BWD_ATTN = 1,
    TP_BWD_LN1 = 2,
    TP_BWD_MLP_DATA = 3,
    TP_BWD_ATTN_DATA = 4,
    TP_BWD_WGRAD = 5,
    /* sequence-parallel form of TP_BWD_ATTN(_DATA): dh is an input, the
     * all-gathered dH = dY + LN2^T(dU2) that the caller formed on its
     * sequence shard with tp_layernorm_bwd; ln_in and reduced_in unused */
    TP_BWD_ATTN_SP = 6,
    TP_BWD_ATTN_DATA_SP = 7
} tp_bwd_phase;

/* Bytes of the opaque "saved" buffer: activations the forward keeps for the
 * backward, for the whole sequence (u1, LN statistics, Q, O, log-sum-exp,
 * u2, GELU'(Z), GELU(Z)).  0 if cfg is invalid. */
size_t tp_shard_saved_bytes(const tp_shard_cfg *cfg);

/* Bytes of the "scratch" buffer (any call, any slice range).  The backward
 * keeps its per-row intermediates there (dZ, dO, dQKV at the call's rows) for
 * a later TP_BWD_WGRAD call over the same rows, so a step's backward calls
 * must share one scratch buffer; nothing else in it survives a call.  0 if
 * cfg is invalid. */
size_t tp_shard_scratch_bytes(const tp_shard_cfg *cfg);

/* Forward of one phase over slices [slice_begin, slice_end) of part.
 *   in           TP_FWD_ATTN: x [s, b, h]; TP_FWD_MLP: h_mid [s, b, h]
 *                (the combined residual stream).  Only the call's rows are read.
 *   partial_out  fp32 [s, b, h]: this rank's partial sum for the call's rows
 *                (P_attn,r or P_mlp,r), overwritten.
 *   kv           TP_FWD_ATTN: the cache, written at the call's positions;
 *                TP_FWD_MLP: ignored (may be NULL).
 *   saved        tp_shard_saved_bytes(cfg) bytes, written at the call's rows.
 *   scratch      tp_shard_scratch_bytes(cfg) bytes.
 * All device pointers 16-byte aligned. */
tp_status tp_shard_layer_fwd(const tp_shard_cfg *cfg, const tp_shard_weights *w,
                             const tp_partition *part, int32_t slice_begin, int32_t slice_end,
                             int32_t phase, const void *in, float *partial_out,
                             tp_kv_cache *kv, void *saved, void *scratch, void *stream);

/* tp_shard_layer_fwd without the scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same phases, arguments, checks,
 * kernels and results (bit-identical) as tp_shard_layer_fwd; its work areas
 * (split-product and split-KV attention partial sums) live in a static
 * device array of tp_noalloc_scratch_bytes() bytes (128 MiB) that each GPU
 * the library runs on holds until the process ends.  The call allocates
 * nothing.  A call whose attention needs more work space than the array
 * leaves returns TP_ESHAPE before anything is enqueued; with tracing on
 * (tp_trace_enable, which creates events) it returns TP_EUNSUPPORTED.  All
 * calls on one GPU share its array: calls that overlap on one GPU (other
 * streams or threads) race and must be serialised by the caller. */
tp_status tp_shard_layer_fwd_noalloc(const tp_shard_cfg *cfg, const tp_shard_weights *w,
                                     const tp_partition *part, int32_t slice_begin,
                                     int32_t slice_end, int32_t phase, const void *in,
                                     float *partial_out, tp_kv_cache *kv, void *saved,
                                     void *stream);
size_t tp_noalloc_scratch_bytes(void);

/* Backward of one phase over slices [slice_begin, slice_end).  Phases of one
 * slice range run in the order MLP, ATTN, LN1 (or their _DATA forms); slice
 * ranges run in reverse; TP_BWD_WGRAD runs after the _DATA calls of its rows.
 *   dy           MLP, ATTN and WGRAD phases: gradient of the layer output y
 *                [s, b, h]; TP_BWD_LN1: unused.
 *   ln_in        TP_BWD_ATTN: h_mid (the input of LN2); TP_BWD_LN1: x (the
 *                input of LN1); TP_BWD_MLP: unused.
 *   reduced_in   fp32 [s, b, h]: TP_BWD_ATTN: sum_r dU2,r; TP_BWD_LN1:
 *                sum_r dU1,r; TP_BWD_MLP: unused.
 *   partial_out  fp32 [s, b, h], overwritten at the call's rows:
 *                TP_BWD_MLP: dU2,r; TP_BWD_ATTN: dU1,r; TP_BWD_LN1: unused.
 *   dh           [s, b, h]: written by TP_BWD_ATTN(_DATA), read by TP_BWD_LN1
 *                and TP_BWD_WGRAD.
 *   dx           [s, b, h]: written by TP_BWD_LN1.
 *   g            gradients (accumulated or overwritten, see tp_shard_grads).
 *   kv, kvg      TP_BWD_ATTN only: the cache the forward filled and the
 *                dK/dV accumulators (protocol above).
 *   saved        the buffer the forward filled for these rows. */
tp_status tp_shard_layer_bwd(const tp_shard_cfg *cfg, const tp_shard_weights *w,
                             const tp_partition *part, int32_t slice_begin, int32_t slice_end,
                             int32_t phase, const void *dy, const void *ln_in,
                             const float *reduced_in, float *partial_out, void *dh, void *dx,
                             const tp_shard_grads *g, const tp_kv_cache *kv, tp_kv_grad *kvg,
                             const void *saved, void *scratch, void *stream);

/* The caller's step after an all-reduce ("Transformer Training 11",
 * tensor-parallelism slide: one all-reduce adds the partial sums):
 * out[m][c] = resid[m][c] + reduced[m][c] + bias[c] for rows m < rows.
 * resid, bias, out: element type cfg->dtype ([rows, hidden], [hidden]);
 * reduced fp32 [rows, hidden]. */
tp_status tp_residual_combine(const tp_shard_cfg *cfg, int64_t rows, const void *resid,
                              const float *reduced, const void *bias, void *out, void *stream);

/* One device's block of a 2x2x2 cube-partitioned FFN ("Maximizing
 * Parallelism ...", section 3.1.2: each processor multiplies (M/p, N/p) by
 * (N/p, K/p) sub-matrices; section 2.3: C_ij = sum_l A_il B_lj), bf16 with
 * fp32 accumulation:
 *   hbuf = GELU(x w1^T + b1)  (bf16 [rows, ffn], caller-provided)
 *   out  = hbuf w2^T          (fp32 [rows, hidden]: the block's partial sum;
 *                              the reduction across the cube is not taken)
 * x [rows, hidden], w1 [ffn, hidden], b1 [ffn], w2 [hidden, ffn], all bf16.
 * hidden and ffn multiples of 8. */
tp_status tp_cube_ffn_block(int32_t rows, int32_t hidden, int32_t ffn, const void *x,
                            const void *w1, const void *b1, const void *w2, void *hbuf,
                            float *out, void *stream);

/* One device's operations of the 3-D (cube) partition of matrix products
 * ("Maximizing Parallelism in Distributed Training for Huge Neural
 * Networks", section 3.1.2: the forms C = AB, AB^T, A^T B and their
 * gradients, dA and dB each a product of one of the three forms; every
 * device multiplies its gathered sub-blocks and the partial products are
 * reduce-scattered).  bf16 operands, row-major; fp32 result:
 *   TP_CUBE_AB:  a [M, K], b [K, N]     c = a b
 *   TP_CUBE_ABT: a [M, K], b [N, K]     c = a b^T
 *   TP_CUBE_ATB: a [K, M], b [K, N]     c = a^T b
 * c fp32 [M, N] is stored (accumulate = 0) or added to (accumulate = 1).
 * M, N, K >= 1 and multiples of 8; device pointers, 16-byte aligned; each
 * buffer below 2 GiB. */
typedef enum { TP_CUBE_AB = 0, TP_CUBE_ABT = 1, TP_CUBE_ATB = 2 } tp_cube_form;
tp_status tp_cube_matmul(int32_t form, int32_t M, int32_t N, int32_t K, const void *a, const void *b,
                         float *c, int32_t accumulate, void *stream);

/* After the reduction of the first FFN product's partial sums (the
 * nonlinearity comes after it): z = z_sum + bias[col] and h = GELU(z) (exact
 * erf form), z_sum fp32 [rows, n], bias bf16 [n], z and h bf16 [rows, n]. */
tp_status tp_cube_bias_gelu(int32_t rows, int32_t n, const float *z_sum, const void *bias, void *z,
                            void *h, void *stream);

/* dz = dh * GELU'(z) (bf16 [rows, n]; dh fp32 is the reduced gradient of h,
 * z the bf16 values tp_cube_bias_gelu stored) and the bias gradient
 * dbias[col] = sum over rows of dz ("Maximizing Parallelism ...", section
 * 3.1.3), fp32 [n], stored or (accumulate = 1) added.  work: device memory
 * of tp_cube_work_bytes(rows, n) bytes for the deterministic column sums. */
size_t tp_cube_work_bytes(int32_t rows, int32_t n);
tp_status tp_cube_gelu_backward(int32_t rows, int32_t n, const float *dh, const void *z, void *dz,
                                float *dbias, int32_t accumulate, void *work, void *stream);

/* Attention with the keys split into blocks ("Transformer Training 11:
 * model parallelism", the passage after the sequence-parallelism slide on
 * very long sequences, where the key/value blocks travel between devices and
 * the queries stay put).  One call takes the device's queries against one
 * block of keys and values; tp_attn_merge combines the results of two
 * disjoint blocks into the result over their union (log-sum-exp rule), so
 * merging the results of all blocks gives causal attention over all keys.
 *
 * Shapes (the heads are this device's heads): q [batch, heads, nq,
 * head_dim], k and v [batch, heads, nk, head_dim], bf16; queries sit at
 * positions q_pos0 .. q_pos0+nq-1 and keys at k_pos0 .. k_pos0+nk-1, and a
 * query at position p sees the keys at positions <= p.  Scores are
 * q.k / sqrt(head_dim).  head_dim is 64 or 128. */
typedef struct {
    int32_t batch, heads, head_dim;
    int32_t nq, nk;
    int32_t q_pos0, k_pos0;
} tp_attn_block_shape;

/* o fp32 [batch, heads, nq, head_dim]: softmax over the block's visible keys
 * applied to v (normalised within the block); lse fp32 [batch, heads, nq]:
 * natural log of the sum of exp(score) over those keys.  A query that sees
 * none of the block's keys gets o = 0 and lse = -inf.  All pointers device,
 * 16-byte aligned, each buffer below 2 GiB; nq or nk may be 0, and a buffer
 * sized by a count of 0 (q, o and lse by nq; k and v by nk) is not addressed
 * and may be NULL (nk = 0: every query gets o = 0 and lse = -inf). */
tp_status tp_attn_block_fwd(const tp_attn_block_shape *shape, const void *q, const void *k,
                            const void *v, float *o, float *lse, void *stream);

/* (o, lse) over the union of two disjoint key sets from (o_a, lse_a) and
 * (o_b, lse_b), each shaped as tp_attn_block_fwd's outputs for `shape`
 * (nk, q_pos0 and k_pos0 are not used): with m = max(lse_a, lse_b) and
 * w = exp(lse - m) per side (0 for -inf), o = (w_a o_a + w_b o_b) /
 * (w_a + w_b) and lse = m + log(w_a + w_b); -inf and o = 0 if both sides
 * are empty.  o may be o_a or o_b and lse may be lse_a or lse_b (in place).
 * With nq = 0 nothing is addressed and every pointer may be NULL. */
tp_status tp_attn_merge(const tp_attn_block_shape *shape, const float *o_a, const float *lse_a,
                        const float *o_b, const float *lse_b, float *o, float *lse, void *stream);

/* Backward of tp_attn_block_fwd for one key block, given the result over
 * every block (ring attention's backward step, same passage): o and lse are
 * the merged output and log-sum-exp of each query over all its keys (as
 * tp_attn_merge leaves them, fp32 [batch, heads, nq, head_dim] and [batch,
 * heads, nq]) and dout (bf16, shaped like q) the gradient of o.  With
 * P = exp(score - lse) on the block's visible keys and D = rowsum(dout * o):
 *   dq (fp32, shaped like q)  = this block's share of the query gradient,
 *                               (P * (dout v^T - D)) k / sqrt(head_dim);
 *   dk, dv (fp32, shaped like k and v) = the gradients of the block's keys
 *                               and values from these queries.
 * Summing dq over all blocks gives the full query gradient.  accumulate = 0
 * stores dq, dk and dv, accumulate = 1 adds to them (a ring sums dq over
 * blocks and dk, dv over the devices the block visits).  A query whose lse is
 * -inf (it sees no key) takes no gradient.  work: device memory of
 * tp_attn_block_bwd_work_bytes(shape) bytes (rowsum(dout * o)); every
 * pointer 16-byte aligned; same shape limits as tp_attn_block_fwd.  A buffer
 * sized by a count of 0 (q, o, lse, dout, dq and work by nq; k, v, dk and dv
 * by nk) may be NULL; with nq = 0, dk and dv are zero (stored or added), with
 * nk = 0 the dq share is. */
size_t tp_attn_block_bwd_work_bytes(const tp_attn_block_shape *shape);
tp_status tp_attn_block_bwd(const tp_attn_block_shape *shape, const void *q, const void *k,
                            const void *v, const float *o, const float *lse, const void *dout,
                            float *dq, float *dk, float *dv, int32_t accumulate, void *work,
                            void *stream);

/* Token-slicing plan of a token-level pipeline ("TeraPipe: Token-Level
 * Pipeline Parallelism ...", section 3, selecting the slicing scheme).
 * Host functions: every pointer is host memory; nothing is enqueued.
 *
 * A sequence of units * g tokens is cut into slices of whole units.  Over K
 * pipeline stages whose every stage takes t_i for slice i, the last slice
 * finishes at sum_i t_i + (K - 1) max_i t_i; tp_slicing_plan returns a plan
 * minimising that, given cost[a * (units + 1) + b] = latency of the slice
 * covering units [a, b) (entries with a >= b are ignored; +inf forbids a
 * slice).  ends (capacity units) receives the slice ends in units
 * (increasing, last = units), num_slices their count and latency the plan's
 * latency.  units in [1, 4096], stages >= 1; costs >= 0.  The search takes
 * each distinct cost as a candidate largest slice latency and finds the least
 * total under it by dynamic programming over prefixes. */
tp_status tp_slicing_plan(int32_t units, const double *cost, int32_t stages, int32_t *num_slices,
                          int32_t *ends, double *latency);

/* The latency of a given plan (slice ends in units, increasing, the last one
 * = units) under the same cost table and pipeline model as tp_slicing_plan:
 * sum_i t_i + (stages - 1) max_i t_i with t_i = cost[a_i * (units + 1) + b_i]. */
tp_status tp_plan_latency(int32_t units, const double *cost, int32_t stages, int32_t num_slices,
                          const int32_t *ends, double *latency);

/* Slice-latency model: the context overhead of a slice of l tokens after o
 * tokens of context is modelled as ctx = coef[0] * l * o + coef[1] * o +
 * coef[2], fitted by least squares to n >= 3 measured samples (len[i],
 * offset[i], ctx[i]); at least one sample needs offset > 0. */
tp_status tp_fit_context_model(int32_t n, const int32_t *len, const int32_t *offset, const double *ctx,
                               double coef[3]);

/* cost[a * (units + 1) + b] = fwd[b - a] + (a > 0 ? max(0, ctx((b - a) g, a g)) : 0)
 * for a < b (+inf otherwise), with fwd[k] the measured latency of a slice of
 * k units without context (fwd has units + 1 entries; fwd[0] unused) and ctx
 * the model above, taken as 0 where the fitted line extrapolates below zero
 * (it is a latency): the cost table of tp_slicing_plan. */
tp_status tp_slice_cost_table(int32_t units, int32_t granularity, const double *fwd, const double coef[3],
                              double *cost);

/* LayerNorm over `rows` rows of width cfg->hidden (a sequence shard in the
 * sequence-parallel form; "Transformer Training 11", sequence-parallelism
 * slide), element type cfg->dtype, statistics fp32, eps cfg->ln_eps:
 *   tp_layernorm_fwd: u = (x - mean) * rstd * gamma + beta, biased variance;
 *   tp_layernorm_bwd: dx = resid + LN^T(du) for the saved mean and rstd
 *     (du fp32, the reduced gradient of u), dgamma = sum over the rows of
 *     du * xhat and dbeta = sum of du (fp32 [hidden]; stored or, with
 *     accumulate = 1, added: a shard's share, which the caller all-reduces).
 * work: tp_layernorm_work_bytes(cfg, rows) bytes of device memory.  mean
 * and rstd (fp32 [rows]) need 4-byte alignment, every other pointer 16. */
size_t tp_layernorm_work_bytes(const tp_shard_cfg *cfg, int64_t rows);
tp_status tp_layernorm_fwd(const tp_shard_cfg *cfg, int64_t rows, const void *x, const void *gamma,
                           const void *beta, void *u, float *mean, float *rstd, void *stream);
tp_status tp_layernorm_bwd(const tp_shard_cfg *cfg, int64_t rows, const float *du, const void *resid,
                           const void *x, const void *gamma, const float *mean, const float *rstd,
                           void *dx, float *dgamma, float *dbeta, int32_t accumulate, void *work,
                           void *stream);

/* Per-kernel timing.  tp_trace_enable(1) discards earlier records and makes
 * every later kernel launch of the library (from any thread) record two HIP
 * events on its launch stream, with the kernel's name and the algorithmic
 * work of its operation (flops: 2*M*N*K for a product, the matmul flops the
 * kernel executes for attention; bytes: each operand read or written once);
 * tp_trace_enable(0) stops recording.  tp_trace_read() waits for the
 * recorded events, writes the first `max` records to `out` (which may be
 * NULL), releases all records and returns how many there were.  ms is the
 * event-measured duration (-1 if the events could not be read); a launch
 * whose events could not be created or recorded has no record. */
typedef struct {
    char name[64];
    double flops;
    double bytes;
    float ms;
} tp_trace_record;

void tp_trace_enable(int32_t on);
int32_t tp_trace_read(tp_trace_record *out, int32_t max);

/* Tile configuration of the bf16 matrix products, for tests and tuning.
 * -1 (the default) lets the library choose per product shape; 0..6 force
 * one configuration for every later bf16 product of the process: 0 = 128x128
 * tiles, 1 = 128x128 tiles with software-pipelined fragment reads, 2 =
 * 256x128 tiles (two workgroups per compute unit), 3 = 256x256 tiles, 4 =
 * 256x192 tiles, 5 = 128x192 tiles (two workgroups per compute unit), 6 =
 * 256x256 tiles of 8 waves.  All
 * give identical results (each output element sums its products in the
 * same K order).  Returns TP_EINVAL for any other value. */
tp_status tp_gemm_force_tile(int32_t tile);

/* Message for the calling thread's last non-OK status ("" if none). */
const char *tp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
