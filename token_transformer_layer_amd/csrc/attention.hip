// Causal attention of one slice of queries over the prefix K/V cache, and
// its backward, on gfx950.
//
// A slice's queries at positions [q0, q1) attend to cache positions
// [0, q1): a token needs only the keys and values of earlier positions and
// its own ("TeraPipe: Token-Level Pipeline Parallelism for Training
// Large-Scale Language Models", section 3), and the heads of a rank are
// independent ("Transformer Training 11: model parallelism",
// tensor-parallelism slide).  Scores are q.k / sqrt(d), masked for keys after
// the query; the softmax is taken online (running maximum and sum per query)
// so K and V stream once per query tile from HBM through LDS.
//
// bf16 kernels use v_mfma_f32_32x32x16_bf16 with K/V (forward, dQ) or Q/dO
// (dK, dV) tiles staged by direct-to-LDS loads; their layouts are described
// with each kernel below.  The backward recomputes P from the saved
// log-sum-exp and uses two kernels so that no floating-point atomics are
// needed and results are deterministic: one per key block (dK, dV, looping
// over the queries that see those keys) and one per query block (dQ, looping
// over the keys the queries see).  dK and dV of keys before the call's first
// query are accumulated in fp32 across calls, because the backward runs the
// slices in reverse and later slices' queries also see earlier keys.
//
// fp32 kernels are plain one-wave-per-row loops (used for the fp32 storage
// configuration only).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace tpk {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Work items of a split launch: a 1-D grid of 8 * ceil(n_items / 8)
// workgroups whose linear ids are dealt round-robin to the 8 XCDs; the items
// of one XCD are made consecutive (id % 8 picks a range of n_items / 8 items)
// so that the items of one (batch row, head), which share its K/V or Q/dO
// tiles, stay in one XCD's L2.  Returns -1 for a padding workgroup.
__device__ __forceinline__ int xcd_item(int n_items) {
    const int id = blockIdx.x, per_xcd = gridDim.x >> 3;
    const int item = (id & 7) * per_xcd + (id >> 3);
    return item < n_items ? item : -1;
}
static inline unsigned xcd_grid(long n_items) { return (unsigned)(8 * ((n_items + 7) / 8)); }

struct AttnP {
    int batch, nt, seq, q0, q1, k_final0, acc_in;
    int chunk_tiles, max_chunks, nblocks;  // work split of the backward (tiles per chunk)
    int n_items, items_bh;                  // work items in all and per (batch row, head)
    float *part;                            // partial sums of split blocks
    float scale;
    const bf16 *q, *k, *v, *o, *dout;
    bf16 *out;  // forward: O; backward: dQKV
    float *lse, *delta, *dk_acc, *dv_acc;
    uint32_t kv_bytes, q_bytes;
};

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

// delta[bh][p] = sum_j dO[p][j] O[p][j] for the queries [q0, q1).
template <typename T>
__global__ __launch_bounds__(256) void attn_delta_kernel(int batch, int nt, int seq, int d, int q0, int q1,
                                                         const T *__restrict__ o, const T *__restrict__ dout,
                                                         float *__restrict__ delta) {
    const int64_t n = (int64_t)(q1 - q0) * batch * nt;
    const int64_t i = blockIdx.x * 256LL + threadIdx.x;
    if (i >= n) return;
    const int head = (int)(i % nt);
    const int64_t r = i / nt;  // call-local token row
    const int bi = (int)(r % batch);
    const int p = q0 + (int)(r / batch);
    const int64_t base = ((int64_t)p * batch + bi) * nt * d + (int64_t)head * d;
    float s = 0.f;
    for (int j = 0; j < d; ++j) s += to_f32(o[base + j]) * to_f32(dout[base + j]);
    delta[((int64_t)bi * nt + head) * seq + p] = s;
}

// ---------------------------------------------------------------------------
// fp32 kernels: one wavefront per query (forward, dQ) or per key (dK, dV)
// ---------------------------------------------------------------------------

struct AttnF {
    int batch, nt, seq, d, q0, q1, k_final0, acc_in;
    float scale;
    const float *q, *k, *v, *o, *dout;
    float *out, *lse, *delta, *dk_acc, *dv_acc;
};

__global__ __launch_bounds__(64) void attn_fwd_f32(AttnF a) {
    __shared__ float qs[128], ps[64];
    const int lane = threadIdx.x, bh = blockIdx.y, bi = bh / a.nt, head = bh % a.nt;
    const int p = a.q0 + blockIdx.x, d = a.d;
    const int64_t slab = (int64_t)bh * a.seq * d;
    for (int j = lane; j < d; j += 64) qs[j] = a.q[slab + (int64_t)p * d + j];
    __syncthreads();
    float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int c0 = 0; c0 <= p; c0 += 64) {
        int key = c0 + lane;
        float s = -INFINITY;
        if (key <= p) {
            float acc = 0.f;
            for (int j = 0; j < d; ++j) acc = fmaf(qs[j], a.k[slab + (int64_t)key * d + j], acc);
            s = acc * a.scale;
        }
        float mn = fmaxf(m, wave_max(s));
        float alpha = expf(m - mn);
        float pr = key <= p ? expf(s - mn) : 0.f;
        l = l * alpha + wave_sum(pr);
        o0 *= alpha;
        o1 *= alpha;
        m = mn;
        ps[lane] = pr;
        __syncthreads();
        int cnt = min(64, p + 1 - c0);
        for (int t = 0; t < cnt; ++t) {
            const float *vr = a.v + slab + (int64_t)(c0 + t) * d;
            o0 = fmaf(ps[t], vr[lane], o0);
            if (lane + 64 < d) o1 = fmaf(ps[t], vr[lane + 64], o1);
        }
        __syncthreads();
    }
    float *orow = a.out + ((int64_t)p * a.batch + bi) * (a.nt * d) + head * d;
    if (lane < d) orow[lane] = o0 / l;
    if (lane + 64 < d) orow[lane + 64] = o1 / l;
    if (lane == 0) a.lse[(int64_t)bh * a.seq + p] = m + logf(l);
}

__global__ __launch_bounds__(64) void attn_bwd_dq_f32(AttnF a) {
    __shared__ float qs[128], dos[128], dss[64];
    const int lane = threadIdx.x, bh = blockIdx.y, bi = bh / a.nt, head = bh % a.nt;
    const int p = a.q0 + blockIdx.x, d = a.d, ht = a.nt * d;
    const int64_t slab = (int64_t)bh * a.seq * d;
    const float *dor = a.dout + ((int64_t)p * a.batch + bi) * ht + head * d;
    for (int j = lane; j < d; j += 64) {
        qs[j] = a.q[slab + (int64_t)p * d + j];
        dos[j] = dor[j];
    }
    __syncthreads();
    const float lse = a.lse[(int64_t)bh * a.seq + p], del = a.delta[(int64_t)bh * a.seq + p];
    float dq0 = 0.f, dq1 = 0.f;
    for (int c0 = 0; c0 <= p; c0 += 64) {
        int key = c0 + lane;
        float ds = 0.f;
        if (key <= p) {
            float s = 0.f, dp = 0.f;
            for (int j = 0; j < d; ++j) {
                s = fmaf(qs[j], a.k[slab + (int64_t)key * d + j], s);
                dp = fmaf(dos[j], a.v[slab + (int64_t)key * d + j], dp);
            }
            float pr = expf(s * a.scale - lse);
            ds = pr * (dp - del);
        }
        dss[lane] = ds;
        __syncthreads();
        int cnt = min(64, p + 1 - c0);
        for (int t = 0; t < cnt; ++t) {
            const float *kr = a.k + slab + (int64_t)(c0 + t) * d;
            dq0 = fmaf(dss[t], kr[lane], dq0);
            if (lane + 64 < d) dq1 = fmaf(dss[t], kr[lane + 64], dq1);
        }
        __syncthreads();
    }
    float *dst = a.out + ((int64_t)p * a.batch + bi) * (3 * ht) + head * d;
    if (lane < d) dst[lane] = dq0 * a.scale;
    if (lane + 64 < d) dst[lane + 64] = dq1 * a.scale;
}

__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32(AttnF a) {
    __shared__ float ks[128], vs[128], pss[64], dss[64];
    const int lane = threadIdx.x, bh = blockIdx.y, bi = bh / a.nt, head = bh % a.nt;
    const int key = blockIdx.x, d = a.d, ht = a.nt * d;
    const int64_t slab = (int64_t)bh * a.seq * d;
    for (int j = lane; j < d; j += 64) {
        ks[j] = a.k[slab + (int64_t)key * d + j];
        vs[j] = a.v[slab + (int64_t)key * d + j];
    }
    __syncthreads();
    float dk0 = 0.f, dk1 = 0.f, dv0 = 0.f, dv1 = 0.f;
    const int pstart = max(a.q0, key);
    for (int c0 = pstart; c0 < a.q1; c0 += 64) {
        int p = c0 + lane;
        float pr = 0.f, ds = 0.f;
        if (p < a.q1) {
            const float *dor = a.dout + ((int64_t)p * a.batch + bi) * ht + head * d;
            float s = 0.f, dp = 0.f;
            for (int j = 0; j < d; ++j) {
                s = fmaf(a.q[slab + (int64_t)p * d + j], ks[j], s);
                dp = fmaf(dor[j], vs[j], dp);
            }
            pr = expf(s * a.scale - a.lse[(int64_t)bh * a.seq + p]);
            ds = pr * (dp - a.delta[(int64_t)bh * a.seq + p]);
        }
        pss[lane] = pr;
        dss[lane] = ds;
        __syncthreads();
        int cnt = min(64, a.q1 - c0);
        for (int t = 0; t < cnt; ++t) {
            int pp = c0 + t;
            const float *dor = a.dout + ((int64_t)pp * a.batch + bi) * ht + head * d;
            const float *qr = a.q + slab + (int64_t)pp * d;
            dv0 = fmaf(pss[t], dor[lane], dv0);
            dk0 = fmaf(dss[t], qr[lane], dk0);
            if (lane + 64 < d) {
                dv1 = fmaf(pss[t], dor[lane + 64], dv1);
                dk1 = fmaf(dss[t], qr[lane + 64], dk1);
            }
        }
        __syncthreads();
    }
    // the accumulators hold dK unscaled; final keys are scaled on output
    const int64_t arow = slab + (int64_t)key * d;
    if (a.acc_in) {
        if (lane < d) { dk0 += a.dk_acc[arow + lane]; dv0 += a.dv_acc[arow + lane]; }
        if (lane + 64 < d) { dk1 += a.dk_acc[arow + lane + 64]; dv1 += a.dv_acc[arow + lane + 64]; }
    }
    if (key >= a.k_final0) {
        float *dst = a.out + ((int64_t)key * a.batch + bi) * (3 * ht) + head * d;
        if (lane < d) { dst[ht + lane] = dk0 * a.scale; dst[2 * ht + lane] = dv0; }
        if (lane + 64 < d) { dst[ht + lane + 64] = dk1 * a.scale; dst[2 * ht + lane + 64] = dv1; }
    } else {
        if (lane < d) { a.dk_acc[arow + lane] = dk0; a.dv_acc[arow + lane] = dv0; }
        if (lane + 64 < d) { a.dk_acc[arow + lane + 64] = dk1; a.dv_acc[arow + lane + 64] = dv1; }
    }
}


// ---------------------------------------------------------------------------
// Forward, MFMA 32x32x16 with direct-to-LDS K/V tiles and split-KV
//
// A workgroup of 4 waves owns 128 queries (32 per wave) of one (batch row,
// head) and a chunk of its key tiles (64 keys each).  K and V tiles travel
// from HBM straight into LDS in their natural [key][d] layout (16-byte chunks
// XOR-swizzled by key), two stages deep.  S^T = K Q^T leaves one query's 32
// scores of a 32-key block in one lane (rows 8(v/4) + 4g + v%4), so eight
// consecutive registers are the B operand of a 16-key step of O^T += V^T P^T;
// V^T comes from LDS through transposed reads in the same key order.  When a
// query tile's keys are split over several workgroups, each writes its
// unnormalised O with its running maximum and sum, and a combine kernel
// merges them (the merge of partial softmaxes over disjoint key blocks).
// ---------------------------------------------------------------------------

constexpr int kFwdBQ = 128;  // queries per workgroup
constexpr int kFwdMaxChunks = 8;

struct AttnFwdP {
    int batch, nt, seq, q0, q1, nqt, chunk_tiles, max_chunks;
    int n_items, items_bh;  // work items in all and per (batch row, head)
    float sl2;  // scale * log2(e)
    const bf16 *q, *k, *v;
    bf16 *o;
    float *lse;
    float *part;  // [bh][nqt][max_chunks][BQ][D] unnormalised O, then [..][BQ][2] (m, l)
    uint32_t kv_bytes;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte chunk swizzle of a [rows][D] bf16 LDS tile: chunk c of row r sits
// at chunk c ^ kv_swz<D>(r) of that row.  The two read patterns of the
// kernels are then free of bank conflicts (64 banks of 4 bytes): one chunk of
// 16 consecutive rows over 16 lanes (ds_read_b128), and four chunks of 4
// consecutive rows over 32 lanes (ds_read_b64_tr_b16).  For D = 128 a row
// spans all banks, so rows r..r+3 go to different 64-byte quarters (bits
// 2-3 from r%4) and the 16 rows of a b128 read to different chunks; for
// D = 64 two rows share the banks and the pattern is the solution of the same
// two conditions.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

template <int D>
__device__ __forceinline__ int kv_chunk_off(int row, int c) {
    return row * (D * 2) + ((c ^ kv_swz<D>(row)) << 4);
}

// one 64-key tile of K or V (rows [key0, key0+64), rows >= kend zero) into LDS
template <int D>
__device__ __forceinline__ void kv_tile_dma(__amdgpu_buffer_rsrc_t r, char *dst, int64_t slab, int key0, int kend,
                                            int wave, int lane) {
    constexpr int INSTR = 64 * D * 2 / 1024, PER_WAVE = INSTR / 4;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
        const int I = wave * PER_WAVE + q;
        const int byte = I * 1024 + lane * 16;
        const int row = byte / (D * 2);
        const int c = ((byte % (D * 2)) >> 4) ^ kv_swz<D>(row);
        const int key = key0 + row;
        const uint32_t off = key < kend ? (uint32_t)((slab + (int64_t)key * D + c * 8) * 2) : kOOB;
        lds_dma16(r, dst + I * 1024, off);
    }
}

// One 64-key tile of the online softmax of the forward: scores of the tile's
// keys (LDS [64][D] at ks, positions key0 .. key0+63) for this lane's query
// (Q in qreg as the B operand), O^T += V^T P^T accumulated (V at vs) and the
// running sum l += sum of P taken by the matrix cores as one more block of
// the same product with a V^T of ones (accl: every row holds the lane's
// query's sum), so the sum costs 4 MFMAs instead of 32 vector adds and
// matches the bf16 P that O is built from.  MASK: some key of the tile is
// after a query of the wave (position > q_pos) or at or past kmax, and those
// scores are dropped; other tiles skip the test.
//
// The exponentials are taken against a reference maximum m_ref per query
// (scaled, log2 units) that is raised only when a score exceeds it by more
// than 2^8: weights stay below 256, which bf16 P and the fp32 sums hold
// without loss, and the rescaling of O and the sum (alpha = 2^(m_old - m_new))
// runs only on the tiles where some query of the wave needs it.  The result
// O / l and the log-sum-exp m_ref + log2(l) do not depend on which reference
// was used.
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile(const char *ks, const char *vs, const bf16x8 (&qreg)[D / 16],
                                         f32x16 (&acc)[D / 32], f32x16 &accl, float &m_ref, int key0, int q_pos,
                                         int kmax, float sl2, int lane) {
    constexpr int KS = D / 16, DB = D / 32;
    const int g = lane >> 5, li = lane & 31;
    f32x16 sc[2] = {f32x16{}, f32x16{}};
    // the two key blocks' products interleaved (independent accumulators)
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            sc[kb] = mfma32(*(const bf16x8 *)(ks + kv_chunk_off<D>(kb * 32 + li, 2 * st + g)), qreg[st], sc[kb]);
    // sc[kb][v]: raw score of key key0 + 32 kb + 8(v/4) + 4g + v%4 for the lane's query
    float mk[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            if constexpr (MASK) {
                const int key = key0 + 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
                if (!(key <= q_pos && key < kmax)) sc[kb][v] = -INFINITY;
            }
            mk[kb] = fmaxf(mk[kb], sc[kb][v]);
        }
    float mt = fmaxf(mk[0], mk[1]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * sl2;  // sl2 > 0: the scaled maximum
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + 8.f)) {  // wave-uniform
        const float m_new = fmaxf(m_ref, mt);
        // a query that has seen no key yet keeps m = -inf (weights 0, nothing to rescale)
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        accl *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
    const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[kb][v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][v], sl2, nm));
    // P^T for key step ks (16 keys): registers 8h..8h+7 of block ks/2, h = ks%2
    bf16x8 pb[4];
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
        const f32x16 &src = sc[ks4 >> 1];
        const int h = (ks4 & 1) * 8;
        u32x4 wv{pack_bf2(src[h], src[h + 1]), pack_bf2(src[h + 2], src[h + 3]), pack_bf2(src[h + 4], src[h + 5]),
                 pack_bf2(src[h + 6], src[h + 7])};
        pb[ks4] = __builtin_bit_cast(bf16x8, wv);
    }
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const int G = lane >> 4, L = lane & 15;
    // key steps outer, the D/32 output blocks (and the sum block) inner:
    // consecutive MFMAs go to independent accumulators
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
        const int r0 = 16 * ks4 + 4 * g + (L >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + 16 * (G & 1) + 4 * (L & 3);
            const int cc = col >> 3, within = (col & 7) * 2;
            u32x2 lo = lds_read_tr16(vs + kv_chunk_off<D>(r0, cc) + within);
            u32x2 hi = lds_read_tr16(vs + kv_chunk_off<D>(r0 + 8, cc) + within);
            acc[db] = mfma32(__builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]}), pb[ks4], acc[db]);
        }
        accl = mfma32(ones, pb[ks4], accl);
    }
}

// One tile step with the mask test only where the tile needs it (a wave-
// uniform choice): keys past the wave's first query position or at or past
// kmax.
template <int D>
__device__ __forceinline__ void fwd_tile_step(const char *ks, const char *vs, const bf16x8 (&qreg)[D / 16],
                                              f32x16 (&acc)[D / 32], f32x16 &accl, float &m_ref, int key0,
                                              int q_pos, int wave_first_pos, int kmax, float sl2, int lane) {
    if (key0 + 63 > wave_first_pos || key0 + 64 > kmax)
        fwd_tile<D, true>(ks, vs, qreg, acc, accl, m_ref, key0, q_pos, kmax, sl2, lane);
    else
        fwd_tile<D, false>(ks, vs, qreg, acc, accl, m_ref, key0, q_pos, kmax, sl2, lane);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_mfma32(AttnFwdP a) {
    constexpr int KS = D / 16;  // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    constexpr int TILE = 64 * D * 2;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, li = lane & 31;
    // item -> (batch row and head, query tile, key chunk); a head's query
    // tiles go longest first
    const int item = xcd_item(a.n_items);
    if (item < 0) return;  // whole workgroup
    const int bh = item / a.items_bh;
    int c = item - bh * a.items_bh, qi = a.nqt - 1;
    for (; qi > 0; --qi) {
        const int n = (min(a.q1, a.q0 + (qi + 1) * kFwdBQ) + 63) / 64;
        const int nc = (n + a.chunk_tiles - 1) / a.chunk_tiles;
        if (c < nc) break;
        c -= nc;
    }
    const int qt0 = a.q0 + qi * kFwdBQ;
    const int kend = min(a.q1, qt0 + kFwdBQ);
    const int ntiles = (kend + 63) / 64;
    const int nch = (ntiles + a.chunk_tiles - 1) / a.chunk_tiles;
    if (c >= nch) return;  // (not reached: the host counts the items the same way)
    const int t0 = c * a.chunk_tiles, t1 = min(ntiles, t0 + a.chunk_tiles);
    const int bi = bh / a.nt, head = bh % a.nt;
    const int my_q = qt0 + w * 32 + li;
    const int q_eff = min(my_q, a.q1 - 1);  // padding queries act as the last query
    const int wave_first = min(qt0 + w * 32, a.q1 - 1);
    const int64_t slab = (int64_t)bh * a.seq * D;

    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, a.kv_bytes);

    // B operand of S^T = K Q^T: lane (query li, g) holds Q[query][16 s + 8 g + j]
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t off = my_q < a.q1 ? (uint32_t)((slab + (int64_t)my_q * D + s * 16 + g * 8) * 2) : kOOB;
        qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    }
    f32x16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
    f32x16 accl = f32x16{};
    float m_run = -INFINITY;

    kv_tile_dma<D>(rk, smem, slab, t0 * 64, kend, w, lane);
    kv_tile_dma<D>(rv, smem + TILE, slab, t0 * 64, kend, w, lane);
    for (int t = t0; t < t1; ++t) {
        // this tile's loads are done for this wave; the barrier (with its LDS
        // fences, which keep the compiler from moving LDS reads across it)
        // makes them done for all waves
        wait_vmcnt<0>();
        __syncthreads();
        const char *ks = smem + ((t - t0) & 1) * 2 * TILE;
        const char *vs = ks + TILE;
        if (t + 1 < t1) {
            char *nx = smem + ((t + 1 - t0) & 1) * 2 * TILE;
            kv_tile_dma<D>(rk, nx, slab, (t + 1) * 64, kend, w, lane);
            kv_tile_dma<D>(rv, nx + TILE, slab, (t + 1) * 64, kend, w, lane);
        }
        const int key0 = t * 64;
        if (key0 > qt0 + w * 32 + 31) continue;  // every key of the tile is after this wave's queries
        fwd_tile_step<D>(ks, vs, qreg, acc, accl, m_run, key0, q_eff, wave_first, kend, a.sl2, lane);
    }
    const float l_tot = accl[0];
    if (my_q >= a.q1) return;
    if (nch == 1) {
        const float inv = 1.0f / l_tot;
        const int ht = a.nt * D;
        bf16 *orow = a.o + ((int64_t)my_q * a.batch + bi) * ht + head * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = db * 32 + 8 * r + 4 * g;
                *(u32x2 *)(orow + d) = u32x2{pack_bf2(acc[db][4 * r] * inv, acc[db][4 * r + 1] * inv),
                                             pack_bf2(acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv)};
            }
        if (g == 0) a.lse[(int64_t)bh * a.seq + my_q] = (m_run + __log2f(l_tot)) * kLn2;
    } else {
        const int64_t item = ((int64_t)bh * a.nqt + qi) * a.max_chunks + c;
        float *po = a.part + (item * kFwdBQ + (w * 32 + li)) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *(f32x4 *)(po + db * 32 + 8 * r + 4 * g) =
                    f32x4{acc[db][4 * r], acc[db][4 * r + 1], acc[db][4 * r + 2], acc[db][4 * r + 3]};
        if (g == 0) {
            float *pml = a.part + (int64_t)a.batch * a.nt * a.nqt * a.max_chunks * kFwdBQ * D +
                         (item * kFwdBQ + (w * 32 + li)) * 2;
            pml[0] = m_run;
            pml[1] = l_tot;
        }
    }
}

// Merges the partial softmaxes of the key chunks of one query tile:
// m = max_c m_c, l = sum_c 2^(m_c - m) l_c, O = sum_c 2^(m_c - m) O_c / l.
// One thread per 8 columns of a query (D/8 threads per query), so a query
// tile spans kFwdBQ * D / 2048 workgroups (grid.x = query tile * that +
// part); every chunk's loads are issued before the sums.
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_combine(AttnFwdP a) {
    constexpr int TPQ = D / 8, QPW = 256 / TPQ, PARTS = kFwdBQ / QPW;
    const int qi = blockIdx.x / PARTS, part = blockIdx.x % PARTS, bh = blockIdx.y;
    const int qt0 = a.q0 + qi * kFwdBQ;
    const int kend = min(a.q1, qt0 + kFwdBQ);
    const int ntiles = (kend + 63) / 64;
    const int nch = (ntiles + a.chunk_tiles - 1) / a.chunk_tiles;
    if (nch == 1) return;
    const int bi = bh / a.nt, head = bh % a.nt;
    const int ql = part * QPW + threadIdx.x / TPQ, j = (threadIdx.x % TPQ) * 8;
    const int q = qt0 + ql;
    if (q >= a.q1) return;
    const int64_t item0 = ((int64_t)bh * a.nqt + qi) * a.max_chunks;
    const float *pml = a.part + (int64_t)a.batch * a.nt * a.nqt * a.max_chunks * kFwdBQ * D;
    float mc[kFwdMaxChunks], lc[kFwdMaxChunks], x[kFwdMaxChunks][8];
#pragma unroll
    for (int cc = 0; cc < kFwdMaxChunks; ++cc) {
        if (cc < nch) {
            const float *e = pml + ((item0 + cc) * kFwdBQ + ql) * 2;
            mc[cc] = e[0];
            lc[cc] = e[1];
            load8(a.part + ((item0 + cc) * kFwdBQ + ql) * D + j, x[cc]);
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < kFwdMaxChunks; ++cc)
        if (cc < nch) m = fmaxf(m, mc[cc]);
    float l = 0.f, o[8] = {};
#pragma unroll
    for (int cc = 0; cc < kFwdMaxChunks; ++cc) {
        if (cc < nch) {
            const float wgt = mc[cc] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc[cc] - m);
            l += wgt * lc[cc];
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] += wgt * x[cc][u];
        }
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] *= inv;
    store8(a.o + ((int64_t)q * a.batch + bi) * (a.nt * D) + head * D + j, o);
    if (j == 0) a.lse[(int64_t)bh * a.seq + q] = (m + __log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Backward on 32x32x16 MFMAs
//
// dK, dV: a workgroup owns 128 keys of one (batch row, head), 32 per wave,
// held in registers; the query tiles that see them (64 queries each: Q and
// dO rows, and the tile's log-sum-exp and rowsum(dO * O)) stream through LDS
// by direct-to-LDS loads, three stages deep (two tiles in flight while one
// is worked on).  Per query tile a wave forms
// S = Q K^T and dP = dO V^T with keys along the lanes and queries along the
// registers, which is already the B operand (keys as columns, queries as the
// reduction) of dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T fragments
// come from the same LDS tiles through transposing reads.
//
// dQ: a workgroup owns 128 queries, 32 per wave, Q and dO in registers; the
// key tiles before the queries stream through LDS; S^T = K Q^T and
// dP^T = V dO^T put queries along the lanes, so dS^T is the B operand of
// dQ^T += K^T dS^T (K^T through transposing reads), as in the forward.
// ---------------------------------------------------------------------------

constexpr int kBwdBK = 128;  // keys per dK/dV workgroup
constexpr int kBwdMaxChunks = 8;  // chunks a split block may have
constexpr int kBwdKvStages = 3;   // LDS stages of the dK/dV kernel
// vector-memory loads one wave issues per query tile of the dK/dV kernel
// (the Q and dO DMAs, 1 KB per instruction over 4 waves)
template <int D> constexpr int kBwdTileLoads = 2 * (64 * D * 2 / 1024) / 4;
constexpr int kBwdBQ = 128;  // queries per dQ workgroup

// one 64-row tile of a [rows][D] bf16 matrix whose rows are `ld` elements
// apart (rows [row0, row0 + 64), rows >= rend zero) into LDS [64][D], 16-byte
// chunks swizzled by row
template <int D>
__device__ __forceinline__ void rows_tile_dma(__amdgpu_buffer_rsrc_t r, char *dst, int64_t base, int64_t ld,
                                              int row0, int rend, int wave, int lane) {
    constexpr int INSTR = 64 * D * 2 / 1024, PER_WAVE = INSTR / 4;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
        const int I = wave * PER_WAVE + q;
        const int byte = I * 1024 + lane * 16;
        const int row = byte / (D * 2);
        const int c = ((byte % (D * 2)) >> 4) ^ kv_swz<D>(row);
        const int gr = row0 + row;
        const uint32_t off = gr < rend ? (uint32_t)((base + (int64_t)gr * ld + c * 8) * 2) : kOOB;
        lds_dma16(r, dst + I * 1024, off);
    }
}

// A operand of a 32x32x16 MFMA taken transposed from a [64][D] LDS tile: lane
// l gets column db*32 + l%32 at rows r0..r0+3 and r0+8..r0+11 of the tile,
// r0 = row_base + 4*(l/32) (the order in which a score block's registers
// 8h..8h+7 hold their rows).
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char *tile, int row_base, int db, int lane) {
    const int G = lane >> 4, L = lane & 15, g = lane >> 5;
    const int col = db * 32 + 16 * (G & 1) + 4 * (L & 3);
    const int cc = col >> 3, within = (col & 7) * 2;
    const int r0 = row_base + 4 * g + (L >> 2);
    const u32x2 lo = lds_read_tr16(tile + kv_chunk_off<D>(r0, cc) + within);
    const u32x2 hi = lds_read_tr16(tile + kv_chunk_off<D>(r0 + 8, cc) + within);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// registers 8h..8h+7 of a 32x32 score block as bf16 (the B operand of one
// 16-step of the reduction over the block's rows)
__device__ __forceinline__ bf16x8 pack_half(const f32x16 &s, int h) {
    const int b = 8 * h;
    return __builtin_bit_cast(bf16x8, u32x4{pack_bf2(s[b], s[b + 1]), pack_bf2(s[b + 2], s[b + 3]),
                                            pack_bf2(s[b + 4], s[b + 5]), pack_bf2(s[b + 6], s[b + 7])});
}

// One 64-query tile of the dK/dV kernels for one wave's 32 keys (K and V
// fragments in kreg, vreg; the tile's Q, dO, log2-domain log-sum-exp and
// delta in LDS at st): S and dP of the tile's two 32-query blocks, P and
// dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS.  `full` (wave-
// uniform): every query of the tile sees every key of the wave, so no mask
// is applied, and the second block's products are issued before the first
// block's exponentials so the matrix cores work during them.  Otherwise a
// block is skipped when skip(qb) (every query precedes every key of the
// wave) and each probability is masked by vis(query index in the tile).
template <int D, class Skip, class Vis>
__device__ __forceinline__ void dkdv_tile(const char *st, const bf16x8 (&kreg)[D / 16], const bf16x8 (&vreg)[D / 16],
                                          f32x16 (&acc_dk)[D / 32], f32x16 (&acc_dv)[D / 32], float sl2, int lane,
                                          bool full, Skip skip, Vis vis) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE = 64 * D * 2;
    const int g = lane >> 5, li = lane & 31;
    const float *lse_s = (const float *)(st + 2 * TILE);
    const float *del_s = lse_s + 64;
    auto scores = [&](int qb, f32x16 &sc, f32x16 &dp) __attribute__((always_inline)) {
        sc = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int off = kv_chunk_off<D>(qb * 32 + li, 2 * s + g);
            sc = mfma32(*(const bf16x8 *)(st + off), kreg[s], sc);
            dp = mfma32(*(const bf16x8 *)(st + TILE + off), vreg[s], dp);
        }
    };
    // register v: query 32 qb + 8(v/4) + 4g + v%4 of the tile
    auto probs = [&](int qb, f32x16 &sc, f32x16 &dp, bf16x8 (&pb)[2], bf16x8 (&sb)[2], auto mask)
        __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ql = qb * 32 + 8 * r + 4 * g;
            const f32x4 l4 = *(const f32x4 *)(lse_s + ql);
            const f32x4 d4 = *(const f32x4 *)(del_s + ql);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float pr = __builtin_amdgcn_exp2f(sc[4 * r + u] * sl2 - l4[u]);
                if constexpr (decltype(mask)::value) pr = vis(ql + u) ? pr : 0.f;
                sc[4 * r + u] = pr;
                dp[4 * r + u] = pr * (dp[4 * r + u] - d4[u]);
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            pb[h] = pack_half(sc, h);
            sb[h] = pack_half(dp, h);
        }
    };
    auto grads = [&](int qb, const bf16x8 (&pb)[2], const bf16x8 (&sb)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                acc_dv[db] = mfma32(tr_frag<D>(st + TILE, qb * 32 + 16 * h, db, lane), pb[h], acc_dv[db]);
                acc_dk[db] = mfma32(tr_frag<D>(st, qb * 32 + 16 * h, db, lane), sb[h], acc_dk[db]);
            }
    };
    if (full) {
        f32x16 sc0, dp0, sc1, dp1;
        bf16x8 pb0[2], sb0[2], pb1[2], sb1[2];
        scores(0, sc0, dp0);
        scores(1, sc1, dp1);
        probs(0, sc0, dp0, pb0, sb0, std::false_type{});
        grads(0, pb0, sb0);
        probs(1, sc1, dp1, pb1, sb1, std::false_type{});
        grads(1, pb1, sb1);
        // keep the fragment reads of the score products six ahead of the
        // MFMAs that use them (left to itself the scheduler issues each read
        // just before its MFMA, which then waits out an LDS round trip)
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < 2 * 2 * KS - 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    } else {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            if (skip(qb)) continue;
            f32x16 sc, dp;
            bf16x8 pb[2], sb[2];
            scores(qb, sc, dp);
            probs(qb, sc, dp, pb, sb, std::true_type{});
            grads(qb, pb, sb);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_mfma32(AttnP a) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE = 64 * D * 2;
    constexpr int STAGE = 2 * TILE + 1024;  // Q, dO, lse * log2(e) and delta (64 floats each), 1 KB aligned
    constexpr int NST = kBwdKvStages;        // two query tiles in flight during a tile's work
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, li = lane & 31;
    // item -> (batch row and head, key block, query chunk); a head's key
    // blocks go longest first (the first block sees every query)
    const int item = xcd_item(a.n_items);
    if (item < 0) return;  // whole workgroup
    const int bh = item / a.items_bh, bi = bh / a.nt, head = bh % a.nt;
    int chunk = item - bh * a.items_bh, kb = 0;
    for (; kb < a.nblocks - 1; ++kb) {
        const int qs = max(a.q0, kb * kBwdBK);
        const int nc = max(1, ((qs < a.q1 ? (a.q1 - qs + 63) / 64 : 0) + a.chunk_tiles - 1) / a.chunk_tiles);
        if (chunk < nc) break;
        chunk -= nc;
    }
    const int kb0 = kb * kBwdBK;
    const int kw0 = kb0 + w * 32;
    const int my_k = kw0 + li;
    const int ht = a.nt * D;
    const int64_t slab = (int64_t)bh * a.seq * D;
    const float sl2 = a.scale * kLog2e;

    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q, a.q_bytes);
    __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, a.kv_bytes);
    const uint32_t do_bytes = (uint32_t)(((int64_t)a.seq * a.batch * ht) * 2);
    __amdgpu_buffer_rsrc_t rdo = make_rsrc(a.dout, do_bytes);

    // B operands of S = Q K^T and dP = dO V^T: lane holds key my_k, d = 16 s + 8 g + j
    bf16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t off = my_k < a.q1 ? (uint32_t)((slab + (int64_t)my_k * D + s * 16 + g * 8) * 2) : kOOB;
        kreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
        vreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
    }
    const int qstart = max(a.q0, kb0);
    const int nqt_all = qstart < a.q1 ? (a.q1 - qstart + 63) / 64 : 0;
    // this workgroup's chunk of the query tiles that see the key block
    const int nch = max(1, (nqt_all + a.chunk_tiles - 1) / a.chunk_tiles);
    if (chunk >= nch) return;  // (not reached: the host counts the items the same way)
    // acc[db] register v: d = db*32 + 8(v/4) + 4g + v%4 of key my_k.  An
    // unsplit block starts from the earlier calls' contributions (the
    // accumulators hold dK unscaled), loaded with the K/V fragments; split
    // blocks add them in the combine.
    const int64_t arow = slab + (int64_t)my_k * D;
    f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) { acc_dk[i] = f32x16{}; acc_dv[i] = f32x16{}; }
    if (a.acc_in && nch == 1 && my_k < a.q1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = db * 32 + 8 * r + 4 * g;
                const f32x4 pk = *(const f32x4 *)(a.dk_acc + arow + j);
                const f32x4 pv = *(const f32x4 *)(a.dv_acc + arow + j);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    acc_dk[db][4 * r + u] = pk[u];
                    acc_dv[db][4 * r + u] = pv[u];
                }
            }
    }
    const int t_first = chunk * a.chunk_tiles;
    const int nqt = max(0, min(nqt_all - t_first, a.chunk_tiles));
    const int64_t do_base = (int64_t)bi * ht + head * D;  // dO row p at do_base + p * batch * ht
    const int64_t do_ld = (int64_t)a.batch * ht;
    const int64_t stat0 = (int64_t)bh * a.seq;

    auto issue = [&](int t, char *st) {
        const int p0 = qstart + (t_first + t) * 64;
        rows_tile_dma<D>(rq, st, slab, D, p0, a.q1, w, lane);
        rows_tile_dma<D>(rdo, st + TILE, do_base, do_ld, p0, a.q1, w, lane);
    };
    // the tile's statistics go through registers of the first two waves
    float stat = 0.f;
    auto load_stat = [&](int t) {
        if (tid < 128) {
            const int p = qstart + (t_first + t) * 64 + (tid & 63);
            stat = p < a.q1 ? (tid < 64 ? a.lse[stat0 + p] * kLog2e : a.delta[stat0 + p]) : 0.f;
        }
    };
    auto store_stat = [&](char *st) {
        if (tid < 128) ((float *)(st + 2 * TILE))[tid] = stat;
    };
    // tile t sits in stage t % NST; tiles t + 1 and t + 2 are in flight while
    // tile t is worked on (each tile's statistics load precedes its DMA, so
    // waiting for the statistics leaves the DMA outstanding)
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) {
        if (t < nqt) {
            load_stat(t);
            issue(t, smem + t * STAGE);
            store_stat(smem + t * STAGE);
        }
    }
    for (int t = 0; t < nqt; ++t) {
        // tile t has landed once at most tile t+1's loads are outstanding;
        // the barrier then also frees the stage of tile t-1
        if (t + 1 < nqt) wait_vmcnt<kBwdTileLoads<D>>();
        else wait_vmcnt<0>();
        __syncthreads();
        const char *st = smem + (t % NST) * STAGE;
        char *nx = smem + ((t + NST - 1) % NST) * STAGE;
        if (t + NST - 1 < nqt) {
            load_stat(t + NST - 1);
            issue(t + NST - 1, nx);
        }
        const int p0 = qstart + (t_first + t) * 64;
        dkdv_tile<D>(st, kreg, vreg, acc_dk, acc_dv, sl2, lane, p0 >= kw0 + 31 && p0 + 63 < a.q1,
                     [&](int qb) { return p0 + qb * 32 + 31 < kw0; },
                     [&](int ql) { const int q = p0 + ql; return my_k <= q && q < a.q1; });
        if (t + NST - 1 < nqt) store_stat(nx);
    }
    if (my_k >= a.q1) return;
    if (nch > 1) {
        // partial sums of this chunk (unscaled), [2][128 keys][D] per item
        float *pk = a.part + (((int64_t)bh * a.nblocks + kb) * a.max_chunks + chunk) * (2 * kBwdBK * D) +
                    (int64_t)(w * 32 + li) * D;
        float *pv = pk + kBwdBK * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = db * 32 + 8 * r + 4 * g;
                *(f32x4 *)(pk + j) = f32x4{acc_dk[db][4 * r], acc_dk[db][4 * r + 1], acc_dk[db][4 * r + 2],
                                           acc_dk[db][4 * r + 3]};
                *(f32x4 *)(pv + j) = f32x4{acc_dv[db][4 * r], acc_dv[db][4 * r + 1], acc_dv[db][4 * r + 2],
                                           acc_dv[db][4 * r + 3]};
            }
        return;
    }
    // final keys: dK = scale * acc in bf16; others: the accumulators (dK unscaled)
    const bool final_key = my_k >= a.k_final0;
    bf16 *dst = a.out + ((int64_t)my_k * a.batch + bi) * (3 * ht) + head * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = db * 32 + 8 * r + 4 * g;
            f32x4 dk{acc_dk[db][4 * r], acc_dk[db][4 * r + 1], acc_dk[db][4 * r + 2], acc_dk[db][4 * r + 3]};
            f32x4 dv{acc_dv[db][4 * r], acc_dv[db][4 * r + 1], acc_dv[db][4 * r + 2], acc_dv[db][4 * r + 3]};
            if (final_key) {
                dk *= a.scale;
                *(u32x2 *)(dst + ht + j) = u32x2{pack_bf2(dk[0], dk[1]), pack_bf2(dk[2], dk[3])};
                *(u32x2 *)(dst + 2 * ht + j) = u32x2{pack_bf2(dv[0], dv[1]), pack_bf2(dv[2], dv[3])};
            } else {
                *(f32x4 *)(a.dk_acc + arow + j) = dk;
                *(f32x4 *)(a.dv_acc + arow + j) = dv;
            }
        }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_dq_mfma32(AttnP a) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE = 64 * D * 2;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, li = lane & 31;
    // item -> (batch row and head, query block, key chunk); a head's query
    // blocks go longest first
    const int item = xcd_item(a.n_items);
    if (item < 0) return;  // whole workgroup
    const int bh = item / a.items_bh, bi = bh / a.nt, head = bh % a.nt;
    int chunk = item - bh * a.items_bh, qb = a.nblocks - 1;
    for (; qb > 0; --qb) {
        const int n = (min(a.q1, a.q0 + (qb + 1) * kBwdBQ) + 63) / 64;
        const int nc = max(1, (n + a.chunk_tiles - 1) / a.chunk_tiles);
        if (chunk < nc) break;
        chunk -= nc;
    }
    const int qt0 = a.q0 + qb * kBwdBQ;
    const int my_q = qt0 + w * 32 + li;
    const int q_eff = min(my_q, a.q1 - 1);
    const int kend = min(a.q1, qt0 + kBwdBQ);
    const int ntiles_all = (kend + 63) / 64;
    // this workgroup's chunk of the key tiles its queries see
    const int nch = max(1, (ntiles_all + a.chunk_tiles - 1) / a.chunk_tiles);
    if (chunk >= nch) return;  // (not reached: the host counts the items the same way)
    const int t0 = chunk * a.chunk_tiles, t1 = min(ntiles_all, t0 + a.chunk_tiles);
    const int ht = a.nt * D;
    const int64_t slab = (int64_t)bh * a.seq * D;
    const float sl2 = a.scale * kLog2e;

    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q, a.q_bytes);
    __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, a.kv_bytes);
    const uint32_t do_bytes = (uint32_t)(((int64_t)a.seq * a.batch * ht) * 2);
    __amdgpu_buffer_rsrc_t rdo = make_rsrc(a.dout, do_bytes);

    // B operands of S^T = K Q^T and dP^T = V dO^T: lane holds query my_q, d = 16 s + 8 g + j
    bf16x8 qreg[KS], doreg[KS];
    const bool qok = my_q < a.q1;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t off = qok ? (uint32_t)((slab + (int64_t)my_q * D + s * 16 + g * 8) * 2) : kOOB;
        qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
        const uint32_t offd =
            qok ? (uint32_t)((((int64_t)my_q * a.batch + bi) * ht + head * D + s * 16 + g * 8) * 2) : kOOB;
        doreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rdo, offd));
    }
    const float lse2 = qok ? a.lse[(int64_t)bh * a.seq + my_q] * kLog2e : INFINITY;
    const float del = qok ? a.delta[(int64_t)bh * a.seq + my_q] : 0.f;
    f32x16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

    kv_tile_dma<D>(rk, smem, slab, t0 * 64, kend, w, lane);
    kv_tile_dma<D>(rv, smem + TILE, slab, t0 * 64, kend, w, lane);
    for (int t = t0; t < t1; ++t) {
        wait_vmcnt<0>();
        __syncthreads();
        const char *ks = smem + ((t - t0) & 1) * 2 * TILE;
        const char *vs = ks + TILE;
        if (t + 1 < t1) {
            char *nx = smem + ((t + 1 - t0) & 1) * 2 * TILE;
            kv_tile_dma<D>(rk, nx, slab, (t + 1) * 64, kend, w, lane);
            kv_tile_dma<D>(rv, nx + TILE, slab, (t + 1) * 64, kend, w, lane);
        }
        const int key0 = t * 64;
        if (key0 > qt0 + w * 32 + 31) continue;  // every key of the tile is after this wave's queries
        bf16x8 sb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 sc = f32x16{}, dp = f32x16{};
            const int row = kb * 32 + li;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int off = kv_chunk_off<D>(row, 2 * s + g);
                sc = mfma32(*(const bf16x8 *)(ks + off), qreg[s], sc);
                dp = mfma32(*(const bf16x8 *)(vs + off), doreg[s], dp);
            }
            // register v: key key0 + 32 kb + 8(v/4) + 4g + v%4, query my_q
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int key = key0 + 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
                const float pr = key <= q_eff ? __builtin_amdgcn_exp2f(sc[v] * sl2 - lse2) : 0.f;
                dp[v] = pr * (dp[v] - del);
            }
            sb[2 * kb] = pack_half(dp, 0);
            sb[2 * kb + 1] = pack_half(dp, 1);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) acc[db] = mfma32(tr_frag<D>(ks, 16 * k4, db, lane), sb[k4], acc[db]);
        // each key block's score fragments read four ahead of their MFMAs
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * KS - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    }
    if (!qok) return;
    if (nch > 1) {
        // partial dQ of this chunk (unscaled), [128 queries][D] per item
        float *pq = a.part + (((int64_t)bh * a.nblocks + qb) * a.max_chunks + chunk) * (kBwdBQ * D) +
                    (int64_t)(w * 32 + li) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *(f32x4 *)(pq + db * 32 + 8 * r + 4 * g) =
                    f32x4{acc[db][4 * r], acc[db][4 * r + 1], acc[db][4 * r + 2], acc[db][4 * r + 3]};
        return;
    }
    bf16 *dst = a.out + ((int64_t)my_q * a.batch + bi) * (3 * ht) + head * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = db * 32 + 8 * r + 4 * g;
            *(u32x2 *)(dst + j) = u32x2{pack_bf2(acc[db][4 * r] * a.scale, acc[db][4 * r + 1] * a.scale),
                                        pack_bf2(acc[db][4 * r + 2] * a.scale, acc[db][4 * r + 3] * a.scale)};
        }
}

// Split backward blocks: the partial sums of a block's chunks are added in
// chunk order, then finished as the unsplit kernels finish them (earlier
// calls' contributions added; final rows in bf16 with dK scaled, others back
// to the fp32 accumulators, which hold dK unscaled).  One thread per 8 columns of a row
// (grid.x = block * rows-per-block * D / 2048 + part), every chunk's loads
// issued before the sums.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_combine(AttnP a) {
    constexpr int TPR = D / 8, RPW = 256 / TPR, PARTS = kBwdBK / RPW;
    const int kb = blockIdx.x / PARTS, part = blockIdx.x % PARTS;
    const int bh = blockIdx.y, bi = bh / a.nt, head = bh % a.nt;
    const int kb0 = kb * kBwdBK;
    const int qstart = max(a.q0, kb0);
    const int nqt_all = qstart < a.q1 ? (a.q1 - qstart + 63) / 64 : 0;
    const int nch = max(1, (nqt_all + a.chunk_tiles - 1) / a.chunk_tiles);
    if (nch == 1) return;
    const int kl = part * RPW + threadIdx.x / TPR, j = (threadIdx.x % TPR) * 8;
    const int key = kb0 + kl;
    if (key >= a.q1) return;
    const int ht = a.nt * D;
    const int64_t slab = (int64_t)bh * a.seq * D;
    const float *base = a.part + ((int64_t)bh * a.nblocks + kb) * a.max_chunks * (2 * kBwdBK * D) + kl * D + j;
    float x[kBwdMaxChunks][8], y[kBwdMaxChunks][8];
#pragma unroll
    for (int c = 0; c < kBwdMaxChunks; ++c) {
        if (c < nch) {
            load8(base + (int64_t)c * (2 * kBwdBK * D), x[c]);
            load8(base + (int64_t)c * (2 * kBwdBK * D) + kBwdBK * D, y[c]);
        }
    }
    float dk[8] = {}, dv[8] = {};
#pragma unroll
    for (int c = 0; c < kBwdMaxChunks; ++c) {
        if (c < nch) {
#pragma unroll
            for (int u = 0; u < 8; ++u) { dk[u] += x[c][u]; dv[u] += y[c][u]; }
        }
    }
    const int64_t arow = slab + (int64_t)key * D + j;
    if (a.acc_in) {
        float xa[8], ya[8];
        load8(a.dk_acc + arow, xa);
        load8(a.dv_acc + arow, ya);
#pragma unroll
        for (int u = 0; u < 8; ++u) { dk[u] += xa[u]; dv[u] += ya[u]; }
    }
    // the accumulators hold dK unscaled; final keys are scaled on output
    if (key >= a.k_final0) {
        bf16 *dst = a.out + ((int64_t)key * a.batch + bi) * (3 * ht) + head * D + j;
#pragma unroll
        for (int u = 0; u < 8; ++u) dk[u] *= a.scale;
        store8(dst + ht, dk);
        store8(dst + 2 * ht, dv);
    } else {
        store8(a.dk_acc + arow, dk);
        store8(a.dv_acc + arow, dv);
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dq_combine(AttnP a) {
    constexpr int TPR = D / 8, RPW = 256 / TPR, PARTS = kBwdBQ / RPW;
    const int qb = blockIdx.x / PARTS, part = blockIdx.x % PARTS;
    const int bh = blockIdx.y, bi = bh / a.nt, head = bh % a.nt;
    const int qt0 = a.q0 + qb * kBwdBQ;
    const int kend = min(a.q1, qt0 + kBwdBQ);
    const int ntiles_all = (kend + 63) / 64;
    const int nch = max(1, (ntiles_all + a.chunk_tiles - 1) / a.chunk_tiles);
    if (nch == 1) return;
    const int ql = part * RPW + threadIdx.x / TPR, j = (threadIdx.x % TPR) * 8;
    const int q = qt0 + ql;
    if (q >= a.q1) return;
    const int ht = a.nt * D;
    const float *base = a.part + ((int64_t)bh * a.nblocks + qb) * a.max_chunks * (kBwdBQ * D) + ql * D + j;
    float x[kBwdMaxChunks][8];
#pragma unroll
    for (int c = 0; c < kBwdMaxChunks; ++c)
        if (c < nch) load8(base + (int64_t)c * (kBwdBQ * D), x[c]);
    float dq[8] = {};
#pragma unroll
    for (int c = 0; c < kBwdMaxChunks; ++c) {
        if (c < nch) {
#pragma unroll
            for (int u = 0; u < 8; ++u) dq[u] += x[c][u];
        }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) dq[u] *= a.scale;
    store8(a.out + ((int64_t)q * a.batch + bi) * (3 * ht) + head * D + j, dq);
}

// delta[bh][p] = sum_j dO[p][j] O[p][j]: D/8 lanes per (query, head), 8
// columns each, reduced by shuffles within the lane group.
template <int D>
__global__ __launch_bounds__(256) void attn_delta_bf16(int batch, int nt, int seq, int q0, int q1,
                                                       const bf16 *__restrict__ o, const bf16 *__restrict__ dout,
                                                       float *__restrict__ delta) {
    constexpr int LPG = D / 8;
    const int64_t n = (int64_t)(q1 - q0) * batch * nt;
    const int64_t i = (blockIdx.x * 256LL + threadIdx.x) / LPG;
    const int part = threadIdx.x % LPG;
    float s = 0.f;
    int64_t base = 0;
    if (i < n) {
        base = i * D + part * 8;  // token-major rows: (call row, head) pairs are contiguous D-blocks
        base += (int64_t)q0 * batch * nt * D;
        float x[8], y[8];
        load8(o + base, x);
        load8(dout + base, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) s += x[j] * y[j];
    }
#pragma unroll
    for (int m = LPG / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
    if (i < n && part == 0) {
        const int head = (int)(i % nt);
        const int64_t r = i / nt;
        const int bi = (int)(r % batch);
        const int p = q0 + (int)(r / batch);
        delta[((int64_t)bi * nt + head) * seq + p] = s;
    }
}

// ---------------------------------------------------------------------------
// Attention of queries over one block of keys and values at given positions
// (the per-block step of attention with the keys passed round a ring), and
// the merge of two partial results.
//
// A workgroup owns 128 queries of one (batch row, head) and streams the
// block's keys that its queries can see through LDS, with the forward's tile
// step; the result is the block's normalised O in fp32 and its log-sum-exp
// (-inf, with O = 0, for a query that sees none of the block's keys).
// ---------------------------------------------------------------------------

struct AttnBlockP {
    int nq, nk, q_pos0, k_pos0;
    float sl2;
    const bf16 *q, *k, *v;
    float *o, *lse;
    uint32_t q_bytes, kv_bytes;
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_block_fwd_mfma32(AttnBlockP a) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE = 64 * D * 2;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, li = lane & 31;
    const int bh = blockIdx.y;
    const int lq0 = blockIdx.x * kFwdBQ;
    const int my_lq = lq0 + w * 32 + li;  // query index within the block's queries
    const bool qok = my_lq < a.nq;
    const int q_pos = a.q_pos0 + min(my_lq, a.nq - 1);  // padding queries act as the last query
    // keys past the workgroup's last query position are never seen
    const int last_pos = a.q_pos0 + min(lq0 + kFwdBQ - 1, a.nq - 1);
    const int kend = max(0, min(a.nk, last_pos - a.k_pos0 + 1));
    const int ntiles = (kend + 63) / 64;
    const int64_t qslab = (int64_t)bh * a.nq * D, kslab = (int64_t)bh * a.nk * D;

    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q, a.q_bytes);
    __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, a.kv_bytes);
    bf16x8 qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t off = qok ? (uint32_t)((qslab + (int64_t)my_lq * D + s * 16 + g * 8) * 2) : kOOB;
        qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    }
    f32x16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16{};
    f32x16 accl = f32x16{};
    float m_run = -INFINITY;

    if (ntiles > 0) {
        kv_tile_dma<D>(rk, smem, kslab, 0, kend, w, lane);
        kv_tile_dma<D>(rv, smem + TILE, kslab, 0, kend, w, lane);
    }
    const int wave_last_pos = a.q_pos0 + lq0 + w * 32 + 31;
    const int wave_first_pos = a.q_pos0 + min(lq0 + w * 32, a.nq - 1);
    for (int t = 0; t < ntiles; ++t) {
        wait_vmcnt<0>();
        __syncthreads();
        const char *ks = smem + (t & 1) * 2 * TILE;
        const char *vs = ks + TILE;
        if (t + 1 < ntiles) {
            char *nx = smem + ((t + 1) & 1) * 2 * TILE;
            kv_tile_dma<D>(rk, nx, kslab, (t + 1) * 64, kend, w, lane);
            kv_tile_dma<D>(rv, nx + TILE, kslab, (t + 1) * 64, kend, w, lane);
        }
        const int key0 = a.k_pos0 + t * 64;
        if (key0 > wave_last_pos) continue;  // every key of the tile is after this wave's queries
        fwd_tile_step<D>(ks, vs, qreg, acc, accl, m_run, key0, q_pos, wave_first_pos, a.k_pos0 + kend, a.sl2, lane);
    }
    const float l_tot = accl[0];
    if (!qok) return;
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.0f / l_tot : 0.f;
    float *orow = a.o + qslab + (int64_t)my_lq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *(f32x4 *)(orow + db * 32 + 8 * r + 4 * g) =
                f32x4{acc[db][4 * r] * inv, acc[db][4 * r + 1] * inv, acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv};
    if (g == 0) a.lse[(int64_t)bh * a.nq + my_lq] = seen ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Backward of attention over one key block (the per-block step of ring
// attention's backward): queries at positions q_pos0.., keys at k_pos0..,
// with the merged forward result's log-sum-exp and rowsum(dO * O) of every
// query.  Two kernels as for the prefix form: per 128 keys (dK, dV, looping
// over the query tiles that see them; K and V in registers, Q and dO tiles
// through LDS, three stages) and per 128 queries (this block's share of dQ,
// looping over the visible key tiles).  Results are fp32, stored or added to
// the caller's buffers (a ring sums dQ shares over blocks and dK, dV over
// devices).  A query whose merged log-sum-exp is -inf sees no key anywhere
// and takes no gradient.
// ---------------------------------------------------------------------------

struct AttnBlockBwdP {
    int nq, nk, q_pos0, k_pos0, accumulate;
    float scale;
    const bf16 *q, *k, *v, *dout;   // q, dout [bh][nq][D]; k, v [bh][nk][D]
    const float *o;                 // merged O [bh][nq][D]
    const float *lse;               // merged log-sum-exp [bh][nq]
    float *delta;                   // rowsum(dO * O) [bh][nq]
    float *dq, *dk, *dv;            // dq [bh][nq][D]; dk, dv [bh][nk][D]
    uint32_t q_bytes, kv_bytes;
};

// log2-domain log-sum-exp of a query for P = exp2(s * scale * log2 e - it):
// +inf for a query that sees no key (so P = 0)
__device__ __forceinline__ float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// delta[row] = sum_j dO[row][j] O[row][j]; D/8 lanes per row, 8 columns each
template <int D>
__global__ __launch_bounds__(256) void attn_block_delta(int64_t rows, const bf16 *__restrict__ dout,
                                                        const float *__restrict__ o, float *__restrict__ delta) {
    constexpr int LPG = D / 8;
    const int64_t row = (blockIdx.x * 256LL + threadIdx.x) / LPG;
    const int part = threadIdx.x % LPG;
    float s = 0.f;
    if (row < rows) {
        float x[8], y[8];
        load8(dout + row * D + part * 8, x);
        load8(o + row * D + part * 8, y);
#pragma unroll
        for (int j = 0; j < 8; ++j) s += x[j] * y[j];
    }
#pragma unroll
    for (int m = LPG / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
    if (row < rows && part == 0) delta[row] = s;
}

// fp32 result rows: stored, or added to what the buffer holds
__device__ __forceinline__ void put4(float *p, f32x4 v, bool add) {
    if (add) v += *(const f32x4 *)p;
    *(f32x4 *)p = v;
}

template <int D>
__global__ __launch_bounds__(256) void attn_block_bwd_dkdv_mfma32(AttnBlockBwdP a) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE = 64 * D * 2;
    constexpr int STAGE = 2 * TILE + 1024;  // Q, dO, lse (log2 units) and delta of 64 queries
    constexpr int NST = kBwdKvStages;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, li = lane & 31;
    const int bh = blockIdx.y;
    const int kb0 = blockIdx.x * kBwdBK;  // first key (block-local index) of the workgroup
    const int kw0 = kb0 + w * 32;
    const int my_k = kw0 + li;
    const bool kok = my_k < a.nk;
    const int my_kpos = a.k_pos0 + my_k;
    const int64_t qslab = (int64_t)bh * a.nq * D, kslab = (int64_t)bh * a.nk * D;
    const float sl2 = a.scale * kLog2e;

    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q, a.q_bytes);
    __amdgpu_buffer_rsrc_t rdo = make_rsrc(a.dout, a.q_bytes);
    __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, a.kv_bytes);

    // B operands of S = Q K^T and dP = dO V^T: lane holds key my_k, d = 16 s + 8 g + j
    bf16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t off = kok ? (uint32_t)((kslab + (int64_t)my_k * D + s * 16 + g * 8) * 2) : kOOB;
        kreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
        vreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
    }
    f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) { acc_dk[i] = f32x16{}; acc_dv[i] = f32x16{}; }

    // the first query (block-local) that sees a key of this workgroup
    const int qstart = max(0, a.k_pos0 + kb0 - a.q_pos0);
    const int nqt = qstart < a.nq ? (a.nq - qstart + 63) / 64 : 0;
    const int64_t stat0 = (int64_t)bh * a.nq;

    auto issue = [&](int t, char *st) {
        const int p0 = qstart + t * 64;
        rows_tile_dma<D>(rq, st, qslab, D, p0, a.nq, w, lane);
        rows_tile_dma<D>(rdo, st + TILE, qslab, D, p0, a.nq, w, lane);
    };
    float stat = 0.f;
    auto load_stat = [&](int t) {
        if (tid < 128) {
            const int p = qstart + t * 64 + (tid & 63);
            stat = p < a.nq ? (tid < 64 ? lse2_of(a.lse[stat0 + p]) : a.delta[stat0 + p]) : 0.f;
        }
    };
    auto store_stat = [&](char *st) {
        if (tid < 128) ((float *)(st + 2 * TILE))[tid] = stat;
    };
#pragma unroll
    for (int t = 0; t < NST - 1; ++t) {
        if (t < nqt) {
            load_stat(t);
            issue(t, smem + t * STAGE);
            store_stat(smem + t * STAGE);
        }
    }
    for (int t = 0; t < nqt; ++t) {
        if (t + 1 < nqt) wait_vmcnt<kBwdTileLoads<D>>();
        else wait_vmcnt<0>();
        __syncthreads();
        const char *st = smem + (t % NST) * STAGE;
        char *nx = smem + ((t + NST - 1) % NST) * STAGE;
        if (t + NST - 1 < nqt) {
            load_stat(t + NST - 1);
            issue(t + NST - 1, nx);
        }
        const int p0 = qstart + t * 64;
        const bool full = kw0 + 31 < a.nk && p0 + 63 < a.nq && a.q_pos0 + p0 >= a.k_pos0 + kw0 + 31;
        dkdv_tile<D>(st, kreg, vreg, acc_dk, acc_dv, sl2, lane, full,
                     [&](int qb) { return a.q_pos0 + p0 + qb * 32 + 31 < a.k_pos0 + kw0; },
                     [&](int ql) { const int q = p0 + ql; return kok && q < a.nq && my_kpos <= a.q_pos0 + q; });
        if (t + NST - 1 < nqt) store_stat(nx);
    }
    if (!kok) return;
    float *pk = a.dk + kslab + (int64_t)my_k * D, *pv = a.dv + kslab + (int64_t)my_k * D;
    const bool add = a.accumulate != 0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = db * 32 + 8 * r + 4 * g;
            put4(pk + j, f32x4{acc_dk[db][4 * r], acc_dk[db][4 * r + 1], acc_dk[db][4 * r + 2],
                               acc_dk[db][4 * r + 3]} * a.scale, add);
            put4(pv + j, f32x4{acc_dv[db][4 * r], acc_dv[db][4 * r + 1], acc_dv[db][4 * r + 2],
                               acc_dv[db][4 * r + 3]}, add);
        }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_block_bwd_dq_mfma32(
    AttnBlockBwdP a) {
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int TILE = 64 * D * 2;
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, li = lane & 31;
    const int bh = blockIdx.y;
    const int lq0 = blockIdx.x * kBwdBQ;
    const int my_q = lq0 + w * 32 + li;  // block-local query
    const bool qok = my_q < a.nq;
    const int q_pos = a.q_pos0 + min(my_q, a.nq - 1);
    // keys after the workgroup's last query position are never seen
    const int last_pos = a.q_pos0 + min(lq0 + kBwdBQ - 1, a.nq - 1);
    const int kend = max(0, min(a.nk, last_pos - a.k_pos0 + 1));
    const int ntiles = (kend + 63) / 64;
    const int64_t qslab = (int64_t)bh * a.nq * D, kslab = (int64_t)bh * a.nk * D;
    const float sl2 = a.scale * kLog2e;

    __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q, a.q_bytes);
    __amdgpu_buffer_rsrc_t rdo = make_rsrc(a.dout, a.q_bytes);
    __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k, a.kv_bytes);
    __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v, a.kv_bytes);

    // B operands of S^T = K Q^T and dP^T = V dO^T: lane holds query my_q, d = 16 s + 8 g + j
    bf16x8 qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint32_t off = qok ? (uint32_t)((qslab + (int64_t)my_q * D + s * 16 + g * 8) * 2) : kOOB;
        qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
        doreg[s] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
    }
    const float lse2 = qok ? lse2_of(a.lse[(int64_t)bh * a.nq + my_q]) : INFINITY;
    const float del = qok ? a.delta[(int64_t)bh * a.nq + my_q] : 0.f;
    f32x16 acc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

    if (ntiles > 0) {
        kv_tile_dma<D>(rk, smem, kslab, 0, kend, w, lane);
        kv_tile_dma<D>(rv, smem + TILE, kslab, 0, kend, w, lane);
    }
    const int wave_last_pos = a.q_pos0 + lq0 + w * 32 + 31;
    for (int t = 0; t < ntiles; ++t) {
        wait_vmcnt<0>();
        __syncthreads();
        const char *ks = smem + (t & 1) * 2 * TILE;
        const char *vs = ks + TILE;
        if (t + 1 < ntiles) {
            char *nx = smem + ((t + 1) & 1) * 2 * TILE;
            kv_tile_dma<D>(rk, nx, kslab, (t + 1) * 64, kend, w, lane);
            kv_tile_dma<D>(rv, nx + TILE, kslab, (t + 1) * 64, kend, w, lane);
        }
        const int key0 = t * 64;  // block-local
        if (a.k_pos0 + key0 > wave_last_pos) continue;  // every key of the tile is after this wave's queries
        bf16x8 sb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 sc = f32x16{}, dp = f32x16{};
            const int row = kb * 32 + li;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int off = kv_chunk_off<D>(row, 2 * s + g);
                sc = mfma32(*(const bf16x8 *)(ks + off), qreg[s], sc);
                dp = mfma32(*(const bf16x8 *)(vs + off), doreg[s], dp);
            }
            // register v: key key0 + 32 kb + 8(v/4) + 4g + v%4, query my_q
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int kl = key0 + 32 * kb + 8 * (v >> 2) + 4 * g + (v & 3);
                const bool vis = kl < kend && a.k_pos0 + kl <= q_pos;
                const float pr = vis ? __builtin_amdgcn_exp2f(sc[v] * sl2 - lse2) : 0.f;
                dp[v] = pr * (dp[v] - del);
            }
            sb[2 * kb] = pack_half(dp, 0);
            sb[2 * kb + 1] = pack_half(dp, 1);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) acc[db] = mfma32(tr_frag<D>(ks, 16 * k4, db, lane), sb[k4], acc[db]);
        // each key block's score fragments read four ahead of their MFMAs
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * KS - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    }
    if (!qok) return;
    float *pq = a.dq + qslab + (int64_t)my_q * D;
    const bool add = a.accumulate != 0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            put4(pq + db * 32 + 8 * r + 4 * g,
                 f32x4{acc[db][4 * r], acc[db][4 * r + 1], acc[db][4 * r + 2], acc[db][4 * r + 3]} * a.scale, add);
}

// o = (w_a o_a + w_b o_b) / (w_a + w_b), lse = m + log(w_a + w_b) with
// m = max(lse_a, lse_b) and w_x = exp(lse_x - m) (0 for lse_x = -inf); D/8
// threads per row, each on 8 columns (a row's threads share one wave, so the
// outputs may overwrite either input).
__global__ __launch_bounds__(256) void attn_merge_kernel(int64_t rows, int d, const float *oa, const float *la,
                                                         const float *ob, const float *lb, float *o, float *lse) {
    const int per = d >> 3;
    const int64_t i = blockIdx.x * 256LL + threadIdx.x;
    const int64_t row = i / per;
    const int part = (int)(i % per);
    if (row >= rows) return;
    const float lA = la[row], lB = lb[row];
    const float m = fmaxf(lA, lB);
    const bool empty = m == -INFINITY;
    const float wa = lA == -INFINITY ? 0.f : expf(lA - m);
    const float wb = lB == -INFINITY ? 0.f : expf(lB - m);
    const float tot = wa + wb;
    const float inv = empty ? 0.f : 1.0f / tot;
    float x[8], y[8], r[8];
    load8(oa + row * d + part * 8, x);
    load8(ob + row * d + part * 8, y);
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (wa * x[j] + wb * y[j]) * inv;
    store8(o + row * d + part * 8, r);
    if (part == 0) lse[row] = empty ? -INFINITY : m + logf(tot);
}

}  // namespace

// Raises a kernel's dynamic LDS limit (above the 64 KB default) before its
// launch; the caller returns the error, if any, before launching.
static hipError_t set_lds(const void *fn, int bytes) {
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// (query, key) pairs of the causal product for queries [q0, q1) of every
// (batch row, head): query p sees p + 1 keys.
static double causal_pairs(const AttnArgs &x) {
    double q0 = x.q0, q1 = x.q1;
    return (q1 * (q1 + 1) - q0 * (q0 + 1)) / 2 * x.batch * x.nt;
}

// Key-chunk size of the split forward: the smallest chunk (at least two
// tiles, at most kFwdMaxChunks chunks per query tile) whose work items all
// fit in one round of the chip (two 64 KB workgroups on each of the 256
// compute units); when even unsplit query tiles need more than one round,
// the tiles are not split.
constexpr int kFwdSlots = 2 * 256;
static void fwd_split(const AttnArgs &x, AttnFwdP &p) {
    const int nq = x.q1 - x.q0;
    p.nqt = (nq + kFwdBQ - 1) / kFwdBQ;
    const int max_tiles = (x.q1 + 63) / 64;
    const int bh = x.batch * x.nt;
    auto items = [&](int ct) {
        long n = 0;
        for (int i = 0; i < p.nqt; ++i) n += ((std::min(x.q1, x.q0 + (i + 1) * kFwdBQ) + 63) / 64 + ct - 1) / ct;
        return n * bh;
    };
    int ct = std::min(max_tiles, std::max(2, (max_tiles + kFwdMaxChunks - 1) / kFwdMaxChunks));
    while (ct < max_tiles && items(ct) > kFwdSlots) ++ct;
    if (items(ct) > kFwdSlots) ct = max_tiles;
    p.chunk_tiles = ct;
    p.max_chunks = (max_tiles + ct - 1) / ct;
    p.items_bh = (int)(items(ct) / bh);
    p.n_items = p.items_bh * bh;
}

size_t attn_fwd_call_work_floats(int batch, int nt, int q0, int q1, int d) {
    if (q1 <= q0) return 0;
    AttnArgs x{};
    x.batch = batch; x.nt = nt; x.q0 = q0; x.q1 = q1; x.d = d;
    AttnFwdP p{};
    fwd_split(x, p);
    if (p.max_chunks <= 1) return 0;  // no query tile is split: nothing is written
    return (size_t)batch * nt * p.nqt * p.max_chunks * kFwdBQ * (d + 2);
}

size_t attn_fwd_work_floats(int batch, int nt, int seq, int d) {
    const int nqt = (seq + kFwdBQ - 1) / kFwdBQ;
    const size_t fwd = (size_t)batch * nt * nqt * kFwdMaxChunks * kFwdBQ * (d + 2);
    // the backward's partial sums of split blocks: dK and dV per 128 keys,
    // or dQ per 128 queries, up to kBwdMaxChunks chunks per block
    const int nb = (seq + kBwdBK - 1) / kBwdBK;
    const size_t bwd = (size_t)batch * nt * nb * kBwdMaxChunks * 2 * kBwdBK * d;
    return fwd > bwd ? fwd : bwd;
}

// Tiles per chunk of a split backward launch: enough work items for the
// chip (`target`), at most kBwdMaxChunks chunks per block, at least two
// tiles per chunk.  Both backward kernels take about 448 items: on the 175B
// shard (3264 tile pairs over 12 heads) chunks of 8 tiles, measured best
// against targets of 256-768 (backward 120 us against 122-144).
constexpr int kBwdItemTarget = 448;
static int bwd_chunk_tiles(double total_tiles, int max_tiles, int target) {
    int ct = (int)std::ceil(total_tiles / target);
    ct = std::max(ct, (max_tiles + kBwdMaxChunks - 1) / kBwdMaxChunks);
    return std::max(ct, 2);
}

hipError_t attn_fwd(DType dt, const AttnArgs &x, hipStream_t st) {
    const int nq = x.q1 - x.q0;
    if (nq <= 0) return hipSuccess;
    const int bh = x.batch * x.nt;
    const int es = dt == DType::BF16 ? 2 : 4;
    // algorithmic: 4d flops per pair (Q K^T and P V); Q and O once, the K/V
    // prefix once per (batch row, head)
    TraceScope ts(st, dt == DType::BF16 ? "attn_fwd_bf16" : "attn_fwd_f32", 4.0 * x.d * causal_pairs(x),
                  (double)bh * x.d * es * (2.0 * nq + 2.0 * x.q1) + 4.0 * bh * nq);
    if (dt == DType::BF16) {
        AttnFwdP p{};
        p.batch = x.batch; p.nt = x.nt; p.seq = x.seq; p.q0 = x.q0; p.q1 = x.q1;
        p.sl2 = x.scale * kLog2e;
        p.q = (const bf16 *)x.q; p.k = (const bf16 *)x.k; p.v = (const bf16 *)x.v;
        p.o = (bf16 *)x.o; p.lse = x.lse; p.part = x.work;
        p.kv_bytes = (uint32_t)((int64_t)bh * x.seq * x.d * 2);
        fwd_split(x, p);
        const int lds = 2 * 2 * 64 * x.d * 2;
        dim3 grid(xcd_grid(p.n_items));
        if (x.d == 128) {
            if (hipError_t e = set_lds((const void *)attn_fwd_mfma32<128>, lds); e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_fwd_mfma32<128>, grid, dim3(256), lds, st, p);
        } else {
            if (hipError_t e = set_lds((const void *)attn_fwd_mfma32<64>, lds); e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_fwd_mfma32<64>, grid, dim3(256), lds, st, p);
        }
        if (p.max_chunks > 1) {
            const unsigned parts = (unsigned)(kFwdBQ * x.d / 2048);
            if (x.d == 128) hipLaunchKernelGGL(attn_fwd_combine<128>, dim3(p.nqt * parts, bh), dim3(256), 0, st, p);
            else hipLaunchKernelGGL(attn_fwd_combine<64>, dim3(p.nqt * parts, bh), dim3(256), 0, st, p);
        }
    } else {
        AttnF p{};
        p.batch = x.batch; p.nt = x.nt; p.seq = x.seq; p.d = x.d; p.q0 = x.q0; p.q1 = x.q1; p.scale = x.scale;
        p.q = (const float *)x.q; p.k = (const float *)x.k; p.v = (const float *)x.v;
        p.out = (float *)x.o; p.lse = x.lse;
        hipLaunchKernelGGL(attn_fwd_f32, dim3(nq, bh), dim3(64), 0, st, p);
    }
    return hipGetLastError();
}

hipError_t attn_bwd(DType dt, const AttnArgs &x, hipStream_t st) {
    const int nq = x.q1 - x.q0;
    if (nq <= 0) return hipSuccess;
    const int bh = x.batch * x.nt;
    const int64_t nd = (int64_t)nq * x.batch * x.nt;
    const unsigned dgrid = (unsigned)((nd + 255) / 256);
    const int es = dt == DType::BF16 ? 2 : 4;
    const double pairs = causal_pairs(x);
    // dK/dV kernel: S, dP, dV, dK (8d flops per pair); dQ kernel: S, dP, dQ (6d)
    const double kv_bytes = (double)bh * x.d * (4.0 * x.q1 * es + 2.0 * nq * es * 2);
    const double q_bytes = (double)bh * x.d * (4.0 * nq * es + 2.0 * x.q1 * es);
    if (dt == DType::BF16) {
        {
            TraceScope ts(st, "attn_delta_bf16", 2.0 * x.d * nd, 2.0 * nd * x.d * es + 4.0 * nd);
            const int64_t threads = nd * (x.d / 8);
            const unsigned dg = (unsigned)((threads + 255) / 256);
            if (x.d == 128)
                hipLaunchKernelGGL(attn_delta_bf16<128>, dim3(dg), dim3(256), 0, st, x.batch, x.nt, x.seq, x.q0, x.q1,
                                   (const bf16 *)x.o, (const bf16 *)x.dout, x.delta);
            else
                hipLaunchKernelGGL(attn_delta_bf16<64>, dim3(dg), dim3(256), 0, st, x.batch, x.nt, x.seq, x.q0, x.q1,
                                   (const bf16 *)x.o, (const bf16 *)x.dout, x.delta);
        }
        AttnP p{};
        p.batch = x.batch; p.nt = x.nt; p.seq = x.seq; p.q0 = x.q0; p.q1 = x.q1; p.scale = x.scale;
        p.k_final0 = x.k_final0; p.acc_in = x.acc_in ? 1 : 0;
        p.q = (const bf16 *)x.q; p.k = (const bf16 *)x.k; p.v = (const bf16 *)x.v; p.o = (const bf16 *)x.o;
        p.dout = (const bf16 *)x.dout; p.out = (bf16 *)x.dqkv; p.lse = x.lse; p.delta = x.delta;
        p.dk_acc = x.dk_acc; p.dv_acc = x.dv_acc;
        p.kv_bytes = p.q_bytes = (uint32_t)((int64_t)bh * x.seq * x.d * 2);
        p.part = x.work;
        const int tile = 64 * x.d * 2;
        const int lds_kv = kBwdKvStages * (2 * tile + 1024), lds_q = 2 * 2 * tile;
        {
            // dK, dV: key block kb sees the query tiles from max(q0, 128 kb)
            const int nkb = (x.q1 + kBwdBK - 1) / kBwdBK;
            double total = 0;
            int max_t = 1;
            for (int kb = 0; kb < nkb; ++kb) {
                const int qs = std::max(x.q0, kb * kBwdBK);
                const int n = qs < x.q1 ? (x.q1 - qs + 63) / 64 : 0;
                total += n;
                max_t = std::max(max_t, n);
            }
            p.chunk_tiles = bwd_chunk_tiles(total * bh, max_t, kBwdItemTarget);
            p.max_chunks = (max_t + p.chunk_tiles - 1) / p.chunk_tiles;
            p.nblocks = nkb;
            p.items_bh = 0;
            for (int kb = 0; kb < nkb; ++kb) {
                const int qs = std::max(x.q0, kb * kBwdBK);
                const int n = qs < x.q1 ? (x.q1 - qs + 63) / 64 : 0;
                p.items_bh += std::max(1, (n + p.chunk_tiles - 1) / p.chunk_tiles);
            }
            p.n_items = p.items_bh * bh;
            dim3 gk(xcd_grid(p.n_items));
            TraceScope ts(st, "attn_bwd_dkdv_bf16", 8.0 * x.d * pairs, kv_bytes);
            if (x.d == 128) {
                if (hipError_t e = set_lds((const void *)attn_bwd_dkdv_mfma32<128>, lds_kv); e != hipSuccess) return e;
                hipLaunchKernelGGL(attn_bwd_dkdv_mfma32<128>, gk, dim3(256), lds_kv, st, p);
                if (p.max_chunks > 1) hipLaunchKernelGGL(attn_bwd_dkdv_combine<128>, dim3(nkb * (kBwdBK * x.d / 2048), bh), dim3(256), 0, st, p);
            } else {
                if (hipError_t e = set_lds((const void *)attn_bwd_dkdv_mfma32<64>, lds_kv); e != hipSuccess) return e;
                hipLaunchKernelGGL(attn_bwd_dkdv_mfma32<64>, gk, dim3(256), lds_kv, st, p);
                if (p.max_chunks > 1) hipLaunchKernelGGL(attn_bwd_dkdv_combine<64>, dim3(nkb * (kBwdBK * x.d / 2048), bh), dim3(256), 0, st, p);
            }
        }
        {
            // dQ: query block qb sees the key tiles before min(q1, its end)
            const int nqb = (nq + kBwdBQ - 1) / kBwdBQ;
            double total = 0;
            int max_t = 1;
            for (int qb = 0; qb < nqb; ++qb) {
                const int n = (std::min(x.q1, x.q0 + (qb + 1) * kBwdBQ) + 63) / 64;
                total += n;
                max_t = std::max(max_t, n);
            }
            p.chunk_tiles = bwd_chunk_tiles(total * bh, max_t, kBwdItemTarget);
            p.max_chunks = (max_t + p.chunk_tiles - 1) / p.chunk_tiles;
            p.nblocks = nqb;
            p.items_bh = 0;
            for (int qb = 0; qb < nqb; ++qb) {
                const int n = (std::min(x.q1, x.q0 + (qb + 1) * kBwdBQ) + 63) / 64;
                p.items_bh += std::max(1, (n + p.chunk_tiles - 1) / p.chunk_tiles);
            }
            p.n_items = p.items_bh * bh;
            dim3 gq(xcd_grid(p.n_items));
            TraceScope ts(st, "attn_bwd_dq_bf16", 6.0 * x.d * pairs, q_bytes);
            if (x.d == 128) {
                if (hipError_t e = set_lds((const void *)attn_bwd_dq_mfma32<128>, lds_q); e != hipSuccess) return e;
                hipLaunchKernelGGL(attn_bwd_dq_mfma32<128>, gq, dim3(256), lds_q, st, p);
                if (p.max_chunks > 1) hipLaunchKernelGGL(attn_bwd_dq_combine<128>, dim3(nqb * (kBwdBQ * x.d / 2048), bh), dim3(256), 0, st, p);
            } else {
                if (hipError_t e = set_lds((const void *)attn_bwd_dq_mfma32<64>, lds_q); e != hipSuccess) return e;
                hipLaunchKernelGGL(attn_bwd_dq_mfma32<64>, gq, dim3(256), lds_q, st, p);
                if (p.max_chunks > 1) hipLaunchKernelGGL(attn_bwd_dq_combine<64>, dim3(nqb * (kBwdBQ * x.d / 2048), bh), dim3(256), 0, st, p);
            }
        }
    } else {
        TraceScope ts(st, "attn_bwd_f32", 14.0 * x.d * pairs, kv_bytes + q_bytes);
        hipLaunchKernelGGL(attn_delta_kernel<float>, dim3(dgrid), dim3(256), 0, st, x.batch, x.nt, x.seq, x.d, x.q0,
                           x.q1, (const float *)x.o, (const float *)x.dout, x.delta);
        AttnF p{};
        p.batch = x.batch; p.nt = x.nt; p.seq = x.seq; p.d = x.d; p.q0 = x.q0; p.q1 = x.q1; p.scale = x.scale;
        p.k_final0 = x.k_final0; p.acc_in = x.acc_in ? 1 : 0;
        p.q = (const float *)x.q; p.k = (const float *)x.k; p.v = (const float *)x.v; p.o = (const float *)x.o;
        p.dout = (const float *)x.dout; p.out = (float *)x.dqkv; p.lse = x.lse; p.delta = x.delta;
        p.dk_acc = x.dk_acc; p.dv_acc = x.dv_acc;
        hipLaunchKernelGGL(attn_bwd_dkdv_f32, dim3(x.q1, bh), dim3(64), 0, st, p);
        hipLaunchKernelGGL(attn_bwd_dq_f32, dim3(nq, bh), dim3(64), 0, st, p);
    }
    return hipGetLastError();
}

// Visible (query, key) pairs of a block: query at position p sees the keys
// at positions k_pos0 .. min(p, k_pos0 + nk - 1).
static double block_pairs(const AttnBlockArgs &x) {
    double n = 0;
    for (int i = 0; i < x.nq; ++i) {
        const int64_t p = (int64_t)x.q_pos0 + i;
        const int64_t c = std::min<int64_t>(x.nk, p - x.k_pos0 + 1);
        if (c > 0) n += (double)c;
    }
    return n * x.bh;
}

hipError_t attn_block_fwd(const AttnBlockArgs &x, hipStream_t st) {
    if (x.nq <= 0 || x.bh <= 0) return hipSuccess;
    TraceScope ts(st, "attn_block_fwd_bf16", 4.0 * x.d * block_pairs(x),
                  (double)x.bh * x.d * (2.0 * x.nq + 4.0 * x.nk + 4.0 * x.nq) + 4.0 * x.bh * x.nq);
    AttnBlockP p{};
    p.nq = x.nq; p.nk = x.nk; p.q_pos0 = x.q_pos0; p.k_pos0 = x.k_pos0;
    p.sl2 = x.scale * kLog2e;
    p.q = (const bf16 *)x.q; p.k = (const bf16 *)x.k; p.v = (const bf16 *)x.v;
    p.o = x.o; p.lse = x.lse;
    p.q_bytes = (uint32_t)((int64_t)x.bh * x.nq * x.d * 2);
    p.kv_bytes = (uint32_t)((int64_t)x.bh * x.nk * x.d * 2);
    const int lds = 2 * 2 * 64 * x.d * 2;
    dim3 grid((x.nq + kFwdBQ - 1) / kFwdBQ, x.bh);
    if (x.d == 128) {
        if (hipError_t e = set_lds((const void *)attn_block_fwd_mfma32<128>, lds); e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_block_fwd_mfma32<128>, grid, dim3(256), lds, st, p);
    } else {
        if (hipError_t e = set_lds((const void *)attn_block_fwd_mfma32<64>, lds); e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_block_fwd_mfma32<64>, grid, dim3(256), lds, st, p);
    }
    return hipGetLastError();
}

hipError_t attn_merge(int64_t rows, int d, const float *oa, const float *la, const float *ob, const float *lb,
                      float *o, float *lse, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    TraceScope ts(st, "attn_merge_f32", 3.0 * rows * d, (double)rows * (3.0 * d * 4 + 12));
    const int64_t threads = rows * (d / 8);
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, rows, d, oa, la,
                       ob, lb, o, lse);
    return hipGetLastError();
}

size_t attn_block_bwd_work_floats(int bh, int nq) { return (size_t)bh * (size_t)(nq > 0 ? nq : 0); }

hipError_t attn_block_bwd(const AttnBlockBwdArgs &x, hipStream_t st) {
    if (x.bh <= 0) return hipSuccess;
    AttnBlockBwdP p{};
    p.nq = x.nq; p.nk = x.nk; p.q_pos0 = x.q_pos0; p.k_pos0 = x.k_pos0; p.accumulate = x.accumulate ? 1 : 0;
    p.scale = x.scale;
    p.q = (const bf16 *)x.q; p.k = (const bf16 *)x.k; p.v = (const bf16 *)x.v; p.dout = (const bf16 *)x.dout;
    p.o = x.o; p.lse = x.lse; p.delta = x.work; p.dq = x.dq; p.dk = x.dk; p.dv = x.dv;
    p.q_bytes = (uint32_t)((int64_t)x.bh * x.nq * x.d * 2);
    p.kv_bytes = (uint32_t)((int64_t)x.bh * x.nk * x.d * 2);
    const int64_t rows = (int64_t)x.bh * x.nq;
    if (rows > 0) {
        TraceScope ts(st, "attn_block_delta", 2.0 * x.d * rows, (double)rows * x.d * 6 + 4.0 * rows);
        const unsigned grid = (unsigned)((rows * (x.d / 8) + 255) / 256);
        if (x.d == 128) hipLaunchKernelGGL(attn_block_delta<128>, dim3(grid), dim3(256), 0, st, rows, p.dout, p.o, p.delta);
        else hipLaunchKernelGGL(attn_block_delta<64>, dim3(grid), dim3(256), 0, st, rows, p.dout, p.o, p.delta);
    }
    AttnBlockArgs fw{};
    fw.bh = x.bh; fw.nq = x.nq; fw.nk = x.nk; fw.d = x.d; fw.q_pos0 = x.q_pos0; fw.k_pos0 = x.k_pos0;
    const double pairs = block_pairs(fw);
    const int tile = 64 * x.d * 2;
    const int lds_kv = kBwdKvStages * (2 * tile + 1024), lds_q = 2 * 2 * tile;
    // dK/dV: workgroups of 128 keys (every key block, also one that no query
    // sees: its gradients are zero and are stored or added as such)
    if (x.nk > 0) {
        TraceScope ts(st, "attn_block_bwd_dkdv_bf16", 8.0 * x.d * pairs,
                      (double)x.bh * x.d * (4.0 * x.nk + 4.0 * x.nq + 8.0 * x.nk));
        dim3 grid((x.nk + kBwdBK - 1) / kBwdBK, x.bh);
        if (x.d == 128) {
            if (hipError_t e = set_lds((const void *)attn_block_bwd_dkdv_mfma32<128>, lds_kv); e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_block_bwd_dkdv_mfma32<128>, grid, dim3(256), lds_kv, st, p);
        } else {
            if (hipError_t e = set_lds((const void *)attn_block_bwd_dkdv_mfma32<64>, lds_kv); e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_block_bwd_dkdv_mfma32<64>, grid, dim3(256), lds_kv, st, p);
        }
    }
    if (x.nq > 0) {
        TraceScope ts(st, "attn_block_bwd_dq_bf16", 6.0 * x.d * pairs,
                      (double)x.bh * x.d * (4.0 * x.nq + 4.0 * x.nk + 4.0 * x.nq));
        dim3 grid((x.nq + kBwdBQ - 1) / kBwdBQ, x.bh);
        if (x.d == 128) {
            if (hipError_t e = set_lds((const void *)attn_block_bwd_dq_mfma32<128>, lds_q); e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_block_bwd_dq_mfma32<128>, grid, dim3(256), lds_q, st, p);
        } else {
            if (hipError_t e = set_lds((const void *)attn_block_bwd_dq_mfma32<64>, lds_q); e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_block_bwd_dq_mfma32<64>, grid, dim3(256), lds_q, st, p);
        }
    }
    return hipGetLastError();
}

}  // namespace tpk
