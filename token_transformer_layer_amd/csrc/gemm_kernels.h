// Kernels and launch templates of the bf16/fp32 products (see gemm.hip for
// the design); included by the per-layout translation units and gemm.hip.
#pragma once

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tpk {

// ---------------------------------------------------------------------------
// Epilogues.  operator()(m, n, v) handles one output element (fp32 kernel);
// row8(m, n, v[8]) handles 8 consecutive columns n..n+7 of row m with vector
// loads and stores (bf16 kernel; every N the layer uses is a multiple of 8).
// ---------------------------------------------------------------------------

// Epilogues with fp32 outputs also take 4 columns at a time (row4), so that
// consecutive lanes store consecutive 16-byte chunks of a row (see
// store_tile).
template <typename T>
struct EpiStoreF32 {
    float *c;
    int64_t ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v) const { c[m * ldc + n] = v; }
    __device__ __forceinline__ void row8(int m, int n, const float v[8]) const { store8(c + m * ldc + n, v); }
    __device__ __forceinline__ void row4(int m, int n, float4 v) const { *(float4 *)(c + m * ldc + n) = v; }
};

template <typename T>
struct EpiAccumF32 {
    float *c;
    int64_t ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v) const { c[m * ldc + n] += v; }
    __device__ __forceinline__ void row8(int m, int n, const float v[8]) const {
        float o[8];
        load8(c + m * ldc + n, o);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] += v[i];
        store8(c + m * ldc + n, o);
    }
    __device__ __forceinline__ void row4(int m, int n, float4 v) const {
        float4 *p = (float4 *)(c + m * ldc + n);
        const float4 o = *p;
        *p = float4{o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w};
    }
};

template <typename T>
struct EpiStore {
    T *c;
    int64_t ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v) const { c[m * ldc + n] = from_f32<T>(v); }
    __device__ __forceinline__ void row8(int m, int n, const float v[8]) const { store8(c + m * ldc + n, v); }
};

template <typename T>
struct EpiBiasGelu {
    T *gz;  // GELU'(z), for the backward; may be null
    int64_t ldgz;
    T *g;
    int64_t ldg;
    const T *bias;
    __device__ __forceinline__ void operator()(int m, int n, float v) const {
        float gg, gp;
        gelu_and_grad(v + to_f32(bias[n]), gg, gp);
        if (gz) gz[m * ldgz + n] = from_f32<T>(gp);
        g[m * ldg + n] = from_f32<T>(gg);
    }
    __device__ __forceinline__ void row8(int m, int n, const float v[8]) const {
        float b[8], gp[8], gg[8];
        load8(bias + n, b);
        if (gz) {
#pragma unroll
            for (int i = 0; i < 8; ++i) gelu_and_grad(v[i] + b[i], gg[i], gp[i]);
            store8(gz + m * ldgz + n, gp);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) gg[i] = gelu_f(v[i] + b[i]);
        }
        store8(g + m * ldg + n, gg);
    }
};

template <typename T>
struct EpiGeluGrad {
    T *c;
    int64_t ldc;
    const T *gz;  // GELU'(Z) saved by the forward's EpiBiasGelu
    int64_t ldgz;
    __device__ __forceinline__ void operator()(int m, int n, float v) const {
        c[m * ldc + n] = from_f32<T>(v * to_f32(gz[m * ldgz + n]));
    }
    __device__ __forceinline__ void row8(int m, int n, const float v[8]) const {
        float d[8], o[8];
        load8(gz + m * ldgz + n, d);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = v[i] * d[i];
        store8(c + m * ldc + n, o);
    }
};

template <typename T>
struct EpiQkv {
    const T *bias;
    T *q, *k, *v;
    FastDiv bdiv;  // token row -> (position, batch row)
    int nt, seq, dshift, ht, row0;
    __device__ __forceinline__ void operator()(int m, int n, float acc) const {
        float val = acc + to_f32(bias[n]);
        uint32_t gm = (uint32_t)(row0 + m);
        uint32_t p = fdiv(gm, bdiv);
        uint32_t bi = gm - p * bdiv.d;
        int which = (n >= ht) + (n >= 2 * ht);
        int c = n - which * ht;
        int head = c >> dshift;
        int j = c & ((1 << dshift) - 1);
        size_t off = ((((size_t)bi * nt + head) * seq + p) << dshift) + j;
        T *dst = which == 0 ? q : (which == 1 ? k : v);
        dst[off] = from_f32<T>(val);
    }
    // the 8 columns lie in one head of one of Q, K, V (d is a multiple of 8),
    // so they land on 8 consecutive elements of the destination
    __device__ __forceinline__ void row8(int m, int n, const float acc[8]) const {
        float b[8], o[8];
        load8(bias + n, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = acc[i] + b[i];
        uint32_t gm = (uint32_t)(row0 + m);
        uint32_t p = fdiv(gm, bdiv);
        uint32_t bi = gm - p * bdiv.d;
        int which = (n >= ht) + (n >= 2 * ht);
        int c = n - which * ht;
        int head = c >> dshift;
        int j = c & ((1 << dshift) - 1);
        size_t off = ((((size_t)bi * nt + head) * seq + p) << dshift) + j;
        T *dst = which == 0 ? q : (which == 1 ? k : this->v);
        store8(dst + off, o);
    }
};

// Partial products of a split reduction: split blockIdx.y writes its fp32
// tile to ws + blockIdx.y * stride (rows of ldc floats).
struct EpiSplit {
    float *ws;
    int64_t ldc, stride;
    __device__ __forceinline__ void operator()(int m, int n, float v) const {
        ws[blockIdx.y * stride + m * ldc + n] = v;
    }
    __device__ __forceinline__ void row8(int m, int n, const float v[8]) const {
        store8(ws + blockIdx.y * stride + m * ldc + n, v);
    }
    __device__ __forceinline__ void row4(int m, int n, float4 v) const {
        *(float4 *)(ws + blockIdx.y * stride + m * ldc + n) = v;
    }
};

struct GemmArgs {
    int M, N, K;
    int kc;      // reduction length per split: workgroup row blockIdx.y covers [y*kc, min(K, (y+1)*kc))
    int nsplit;  // number of splits (gridDim.y)
    const void *a;
    int64_t lda;
    uint32_t a_bytes;
    const void *b;
    int64_t ldb;
    uint32_t b_bytes;
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }

// ---------------------------------------------------------------------------
// bf16 MFMA kernel with direct-to-LDS loads
//
// Tiles travel from HBM to LDS by buffer loads that write LDS directly (each
// lane's 16 bytes land at the instruction's LDS base + 16 * lane), so no
// registers stage them and several K-tiles can be in flight (S LDS stages).
// A K-contiguous operand is stored [rows][64 k] with its 16-byte chunks
// XOR-swizzled by row (the permutation is applied to the global addresses,
// since the LDS side of the copy is fixed); fragments are read with
// ds_read_b128.  An M/N-contiguous operand is stored as it lies in memory,
// [64 k][rows], with 16-byte units XOR-swizzled by k, and its fragments are
// read transposed with ds_read_b64_tr_b16: in a group of 16 lanes, lane i
// receives element i%4 of the 8-byte pieces addressed by lanes i/4 + 4j
// (j = 0..3), which gives each lane 4 consecutive k of one row of the tile.
// Loads outside the matrix write zeros to LDS, which masks ragged edges.
// ---------------------------------------------------------------------------

// One operand tile of ROWS (M or N) x BK (K, 32 or 64) bf16 in LDS:
// ROWS * BK * 2 bytes.
template <int ROWS, bool KCONTIG, int NWAVES, int BK>
struct DlOperand {
    static_assert(BK == 32 || BK == 64, "K-tile of 32 or 64");
    static constexpr int kRowBytes = BK * 2;              // [ROWS][BK] layout: bytes per row
    static constexpr int kChunks = BK / 8;                // 16-byte chunks per [ROWS][BK] row
    static constexpr int kBytes = ROWS * kRowBytes;
    static constexpr int kInstr = kBytes / 1024;          // 1 KB per wave-wide load
    static_assert(kInstr % NWAVES == 0, "tile must split evenly over the waves");
    static constexpr int kPerWave = kInstr / NWAVES;      // loads per wave per K-tile
    static constexpr int kPitch = ROWS * 2;               // row pitch of the [BK][ROWS] layout
    static constexpr int kUnits = ROWS / 8;               // 16-byte units per [BK][ROWS] row

    // chunk swizzle of the [ROWS][BK] layout: the rows that one MFMA fragment
    // read touches together (same logical chunk) land on distinct banks
    __device__ static __forceinline__ int swz_row(int r) {
        if constexpr (BK == 64) return lds_swz(r);
        else return (r >> 2) & 3;
    }
    // [BK][ROWS] layout: the 16-byte unit u of row k sits at position
    // unit_pos(u, k), so that the 4 rows x 4 units (256 bytes) that half a
    // wave's transposing read touches cover all 64 banks once.  Power-of-two
    // widths XOR the unit with 4 (k % 4).  A 24-unit row (192 columns, 384
    // bytes: consecutive rows start 32 banks apart) swaps neighbouring 4-unit
    // blocks in the rows with k % 4 >= 2 (the rotation by 4 (k % 4) that
    // preceded it wrapped past the row's end and conflicted up to 5-way,
    // 23% of the LDS cycles of the input-gradient products).  Both are XORs:
    // their own inverse.
    static constexpr bool kPow2Units = (kUnits & (kUnits - 1)) == 0;
    static_assert(kPow2Units || kUnits % 8 == 0, "non-power-of-two rows pair their 4-unit blocks");
    __device__ static __forceinline__ int unit_pos(int u, int k) {
        if constexpr (kPow2Units) return u ^ ((k & 3) * 4 % kUnits);
        else return u ^ (((k >> 1) & 1) << 2);
    }
    __device__ static __forceinline__ int unit_src(int pos, int k) { return unit_pos(pos, k); }

    __device__ static __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, char *stage, int mn0, int k0, int MN,
                                                 int K, int64_t ld, int wave, int lane) {
#pragma unroll
        for (int q = 0; q < kPerWave; ++q) {
            const int I = wave * kPerWave + q;
            uint32_t off;
            if constexpr (KCONTIG) {
                const int row = I * (1024 / kRowBytes) + lane / kChunks;
                const int c = (lane % kChunks) ^ swz_row(row);
                const int gm = mn0 + row, gk = k0 + c * 8;
                off = (gm < MN && gk < K) ? (uint32_t)((gm * ld + gk) * 2) : kOOB;
            } else {
                const int byte = I * 1024 + lane * 16;
                const int k = byte / kPitch;
                const int u = unit_src((byte % kPitch) >> 4, k);
                const int gk = k0 + k, gm = mn0 + u * 8;
                off = (gm < MN && gk < K) ? (uint32_t)((gk * ld + gm) * 2) : kOOB;
            }
            lds_dma16<true>(r, stage + I * 1024, off);
        }
    }

    // Whole K-tiles (K and the split length multiples of BK): the lane's part
    // of each load offset is the same for every K-tile of the reduction, and
    // a K-tile adds one uniform byte advance to it.  base[q] is the lane's
    // offset at k = 0, or kOOB for rows (columns) past MN: kOOB plus an
    // advance inside the buffer (below 2 GiB) stays past its end and reads
    // zeros.
    struct Lanes {
        uint32_t base[kPerWave];
    };
    __device__ static __forceinline__ Lanes lanes(int mn0, int MN, int64_t ld, int wave, int lane) {
        Lanes L;
#pragma unroll
        for (int q = 0; q < kPerWave; ++q) {
            const int I = wave * kPerWave + q;
            if constexpr (KCONTIG) {
                const int row = I * (1024 / kRowBytes) + lane / kChunks;
                const int c = (lane % kChunks) ^ swz_row(row);
                const int gm = mn0 + row;
                L.base[q] = gm < MN ? (uint32_t)((gm * ld + c * 8) * 2) : kOOB;
            } else {
                const int byte = I * 1024 + lane * 16;
                const int k = byte / kPitch;
                const int u = unit_src((byte % kPitch) >> 4, k);
                const int gm = mn0 + u * 8;
                L.base[q] = gm < MN ? (uint32_t)((k * ld + gm) * 2) : kOOB;
            }
        }
        return L;
    }
    // The loads of the K-tile at k0 into the stage at LDS address stage_lds
    // (uniform).  A tile at or past kend is never consumed: its offsets are
    // shifted by kOOB (any offset is checked against the buffer's size, so
    // such a load reads zeros or bytes of the operand, never other memory).
    __device__ static __forceinline__ void issue_whole(__amdgpu_buffer_rsrc_t r, uint32_t stage_lds, const Lanes &L,
                                                       int k0, int kend, int64_t ld, int wave) {
        const uint32_t adv = KCONTIG ? (uint32_t)k0 * 2u : (uint32_t)((int64_t)k0 * ld * 2);
        const uint32_t step = k0 < kend ? adv : kOOB;
#pragma unroll
        for (int q = 0; q < kPerWave; ++q)
            lds_dma16_at(r, stage_lds + (uint32_t)((wave * kPerWave + q) * 1024), L.base[q] + step);
    }

    // MFMA 32x32x16 operand: row (M or N index) `mn` = base + lane % 32 of
    // the fragment, k = kk*16 + 8*(lane/32) + j for j = 0..7.
    __device__ static __forceinline__ bf16x8 frag(const char *stage, int base, int kk, int lane) {
        if constexpr (KCONTIG) {
            const int row = base + (lane & 31);
            const int c = kk * 2 + (lane >> 5);
            return *(const bf16x8 *)(stage + row * kRowBytes + ((c ^ swz_row(row)) << 4));
        } else {
            const int L = lane & 15;
            const int mn = base + 16 * ((lane >> 4) & 1) + 4 * (L & 3);
            const int k = kk * 16 + 8 * (lane >> 5) + (L >> 2);
            const int u = mn >> 3, within = (mn & 7) * 2;
            const char *p0 = stage + k * kPitch + (unit_pos(u, k) << 4) + within;
            const char *p1 = stage + (k + 4) * kPitch + (unit_pos(u, k + 4) << 4) + within;
            u32x2 a = lds_read_tr16(p0), b = lds_read_tr16(p1);
            return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
        }
    }
};

// Maps the linear workgroup index to a (tile row, tile column) pair.
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2), so consecutive indices are first regrouped so that every XCD gets a
// contiguous range of tiles; that range is then walked in groups of GM tile
// rows, column by column, so the tiles resident on one XCD share A rows and
// B columns.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int gm_rows, int &tm, int &tn) {
    const int L = tiles_m * tiles_n, L8 = L & ~7;
    int t = bid;
    if (bid < L8) t = (bid & 7) * (L8 >> 3) + (bid >> 3);
    const int per_group = gm_rows * tiles_n;
    const int group = t / per_group, first = group * gm_rows;
    const int rows = min(tiles_m - first, gm_rows);
    const int r = t - group * per_group;
    tm = first + r % rows;
    tn = r / rows;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK = 64, int OCC = 1>
struct DlCfg {
    static constexpr int kBM = BM, kBN = BN, kBK = BK, kWM = WAVES_M, kWN = WAVES_N, kStages = STAGES;
    static constexpr int kOcc = OCC;  // workgroups per compute unit the register budget is sized for
    static constexpr int kThreads = WAVES_M * WAVES_N * 64;
    static constexpr int kLds = STAGES * (BM + BN) * BK * 2;
};

// Whether an epilogue takes 4 columns at a time (row4).
template <class E, class = void>
struct HasRow4 : std::false_type {};
template <class E>
struct HasRow4<E, std::void_t<decltype(&E::row4)>> : std::true_type {};

// Epilogue through LDS, 32 tile rows at a time: the waves holding those
// rows write their fp32 accumulators (32x32 layout: register v of lane l is
// row 8*(v/4) + 4*(l/32) + v%4, column l%32 of a block) into a [32][BN + 8]
// buffer, then all threads apply the epilogue to 8 consecutive columns each
// (4 for the fp32-output epilogues, row4) with vector loads and stores.  The
// caller has synchronised the workgroup (the LDS stages are free).
template <class C, int FM, int FN, class Epi>
__device__ __forceinline__ void store_tile(f32x16 (&acc)[FM][FN], char *smem, Epi &epi, const GemmArgs &g, int m0,
                                           int n0, int wm, int wn, int tid, int lane) {
    constexpr int BM = C::kBM, BN = C::kBN;
    constexpr int WTN = BN / C::kWN;
    constexpr int EP = BN + 8;  // row pitch in floats: the two half-waves' rows land 32 banks apart
    float *ep = (float *)smem;
#pragma unroll
    for (int c = 0; c < BM / 32; ++c) {
        if (wm == c / FM) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    ep[r * EP + wn * WTN + j * 32 + (lane & 31)] = acc[c % FM][j][v];
                }
        }
        __syncthreads();
        if constexpr (HasRow4<Epi>::value) {
            // 4 columns per item: consecutive lanes store consecutive 16-byte
            // chunks of a row (with 8 per item each store instruction covers
            // twice the span at half density: 3% slower on the fp32 weight
            // gradients)
#pragma unroll
            for (int q = tid; q < 32 * BN / 4; q += C::kThreads) {
                const int r = q / (BN / 4), cv = q % (BN / 4);
                const int gm = m0 + c * 32 + r, gn = n0 + cv * 4;
                if (gm < g.M && gn < g.N) epi.row4(gm, gn, *(const float4 *)(ep + r * EP + cv * 4));
            }
            __syncthreads();
            continue;
        }
#pragma unroll
        for (int q = tid; q < 32 * BN / 8; q += C::kThreads) {
            const int r = q / (BN / 8), cv = q % (BN / 8);
            const int gm = m0 + c * 32 + r, gn = n0 + cv * 8;
            if (gm < g.M && gn < g.N) {
                float v[8];
                const float4 a = *(const float4 *)(ep + r * EP + cv * 8);
                const float4 b = *(const float4 *)(ep + r * EP + cv * 8 + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
                epi.row8(gm, gn, v);
            }
        }
        __syncthreads();
    }
}

template <class C, bool AK, bool BK_, class Epi>
__global__ __launch_bounds__(C::kThreads) void gemm_bf16_dl_kernel(GemmArgs g, Epi epi, int gm_rows) {
    constexpr int BM = C::kBM, BN = C::kBN, BK = C::kBK, S = C::kStages;
    constexpr int NW = C::kWM * C::kWN;
    constexpr int WTM = BM / C::kWM, WTN = BN / C::kWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KSTEPS = BK / 16;
    using OpA = DlOperand<BM, AK, NW, BK>;
    using OpB = DlOperand<BN, BK_, NW, BK>;
    constexpr int STAGE = OpA::kBytes + OpB::kBytes;
    constexpr int LPT = OpA::kPerWave + OpB::kPerWave;  // loads per wave per K-tile
    static_assert(LPT * (S - 2) < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / C::kWN, wn = wid % C::kWN;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, gm_rows, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, g.a_bytes);
    __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, g.b_bytes);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int kbase = blockIdx.y * g.kc, kend = min(g.K, kbase + g.kc);
    const int nkt = kend > kbase ? (kend - kbase + BK - 1) / BK : 0;
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
        if (s < nkt) {
            OpA::issue(ra, smem + s * STAGE, m0, kbase + s * BK, g.M, kend, g.lda, wid, lane);
            OpB::issue(rb, smem + s * STAGE + OpA::kBytes, n0, kbase + s * BK, g.N, kend, g.ldb, wid, lane);
        }
    }
    for (int kt = 0; kt < nkt; ++kt) {
        // tile kt must have landed; the tiles after it that are already in
        // flight (at most S-2) may still be pending
        const int later = min(S - 2, nkt - 1 - kt);
        if constexpr (S >= 4) {
            if (later >= 2) wait_vmcnt<LPT * 2 < 64 ? LPT * 2 : 63>();
            else if (later == 1) wait_vmcnt<LPT>();
            else wait_vmcnt<0>();
        } else if constexpr (S == 3) {
            if (later >= 1) wait_vmcnt<LPT>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // no LDS read moves above the barrier
        if (kt + S - 1 < nkt) {
            char *st = smem + ((kt + S - 1) % S) * STAGE;
            OpA::issue(ra, st, m0, kbase + (kt + S - 1) * BK, g.M, kend, g.lda, wid, lane);
            OpB::issue(rb, st + OpA::kBytes, n0, kbase + (kt + S - 1) * BK, g.N, kend, g.ldb, wid, lane);
        }
        const char *cur = smem + (kt % S) * STAGE;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            bf16x8 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = OpA::frag(cur, wm * WTM + i * 32, kk, lane);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = OpB::frag(cur + OpA::kBytes, wn * WTN + j * 32, kk, lane);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        // every wave is done reading this stage before any wave refills it
        // (the refill is issued after the next iteration's barrier)
    }

    wait_vmcnt<0>();
    __syncthreads();
    store_tile<C>(acc, smem, epi, g, m0, n0, wm, wn, tid, lane);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel, software-pipelined
//
// Same LDS layout and direct-to-LDS staging as above, with the work of each
// wave ordered so that the matrix cores never wait on LDS: the fragments of
// k-step ks+1 are read into a second register set while the MFMAs of k-step
// ks run, and the hand-over between K-tiles (wait for the next tile's DMA,
// workgroup barrier, refill of the stage just consumed) happens before the
// MFMAs of a tile's last k-step, so those MFMAs cover the barrier and the
// first fragment reads of the next tile.  All S stages are filled ahead; the
// stage of tile kt is refilled with tile kt + S once every wave has its last
// fragments of tile kt in registers.  Scheduling-group barriers interleave
// the LDS reads (and the DMA issues) with the MFMAs.
// ---------------------------------------------------------------------------

template <int NR, int NM, int NV>
__device__ __forceinline__ void sched_interleave() {
    // NM MFMAs with NR LDS reads and NV VMEM issues spread between them
    constexpr int RPM = (NR + NM - 1) / NM;
    constexpr int VPM = (NV + NM - 1) / NM;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        if constexpr (RPM > 0) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
        if constexpr (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x020, VPM, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
}

// The vector-memory bookkeeping of gemm_bf16_pp_kernel replayed at compile
// time for LPT loads per wave per K-tile (the direct-to-LDS loads one
// issue() or issue_whole() makes: the two operands' kPerWave), S stages and
// the two wait counts the kernel passes to wait_vmcnt (W0 before the first
// tile, WH at each hand-over).  Loads retire in issue order, so a wait until
// at most N are outstanding completes every load but the last N issued.  The
// kernel issues S K-tiles ahead, waits to W0, and at each hand-over waits to
// WH and then refills one stage; the replay checks that every wait completes
// exactly the tile about to be read (all of its loads, none of a later
// tile's) and that the counts fit the 6-bit vmcnt field.
template <int LPT, int S, int W0, int WH>
constexpr bool pp_waits_complete_next_tile(int nkt = 12) {
    if (LPT <= 0 || S < 2 || W0 >= 64 || WH >= 64 || W0 < 0 || WH < 0 || nkt > 60) return false;
    long issued = 0, last_of[64] = {};
    int next = 0;
    for (int s = 0; s < S; ++s) {
        issued += LPT;
        last_of[next++] = issued;  // count of loads issued when tile s's last load was
    }
    long completed = issued - W0;
    if (completed != last_of[0]) return false;
    for (int kt = 0; kt + 1 < nkt; ++kt) {
        const long now = issued - WH;
        if (now > completed) completed = now;
        if (completed < last_of[kt + 1]) return false;          // the next tile would be read too early
        if (S > 2 && completed > last_of[kt + 1]) return false;  // a later tile's loads would be waited for
        issued += LPT;
        last_of[next++] = issued;
    }
    return true;
}

template <class C, bool AK, bool BK_, class Epi, bool WHOLE>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::kOcc * C::kThreads / 256)))
void gemm_bf16_pp_kernel(GemmArgs g, Epi epi, int gm_rows) {
    constexpr int BM = C::kBM, BN = C::kBN, BK = C::kBK, S = C::kStages;
    constexpr int NW = C::kWM * C::kWN;
    constexpr int WTM = BM / C::kWM, WTN = BN / C::kWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KSTEPS = BK / 16;
    static_assert(KSTEPS % 2 == 0, "register sets alternate by k-step parity");
    using OpA = DlOperand<BM, AK, NW, BK>;
    using OpB = DlOperand<BN, BK_, NW, BK>;
    constexpr int STAGE = OpA::kBytes + OpB::kBytes;
    constexpr int LPT = OpA::kPerWave + OpB::kPerWave;  // DMA issues per wave per K-tile
    constexpr int NREAD = (AK ? 1 : 2) * FM + (BK_ ? 1 : 2) * FN;
    static_assert(LPT * (S - 1) < 64, "vmcnt range");
    static_assert(OpA::kPerWave * NW * 1024 == OpA::kBytes && OpB::kPerWave * NW * 1024 == OpB::kBytes,
                  "the loads of one K-tile cover its stage exactly once");
    constexpr int W0 = LPT * (S - 1), WH = LPT * (S - 2);  // the kernel's two wait counts
    static_assert(pp_waits_complete_next_tile<LPT, S, W0, WH>(), "the waits do not match the loads issued per K-tile");
    extern __shared__ __attribute__((aligned(1024))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / C::kWN, wn = wid % C::kWN;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, gm_rows, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, g.a_bytes);
    __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, g.b_bytes);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    const int kbase = blockIdx.y * g.kc, kend = min(g.K, kbase + g.kc);
    const int nkt = kend > kbase ? (kend - kbase + BK - 1) / BK : 0;
    if (nkt > 0) {
        [[maybe_unused]] typename OpA::Lanes la;
        [[maybe_unused]] typename OpB::Lanes lb;
        [[maybe_unused]] uint32_t smem_lds = 0;
        if constexpr (WHOLE) {
            la = OpA::lanes(m0, g.M, g.lda, wid, lane);
            if constexpr (!(AK && BK_)) lb = OpB::lanes(n0, g.N, g.ldb, wid, lane);
            smem_lds = lds_addr_of(smem);
        }
        auto issue = [&](int s, int k0) __attribute__((always_inline)) {
            if constexpr (WHOLE && AK && BK_) {
                // two K-contiguous operands: B keeps the per-load test (with
                // both operands on fixed offsets these products ran 3-9%
                // slower, with A alone on them 2-3% faster)
                OpA::issue_whole(ra, smem_lds + s * STAGE, la, k0, kend, g.lda, wid);
                OpB::issue(rb, smem + s * STAGE + OpA::kBytes, n0, k0, g.N, kend, g.ldb, wid, lane);
            } else if constexpr (WHOLE) {
                OpA::issue_whole(ra, smem_lds + s * STAGE, la, k0, kend, g.lda, wid);
                OpB::issue_whole(rb, smem_lds + s * STAGE + OpA::kBytes, lb, k0, kend, g.ldb, wid);
            } else {
                OpA::issue(ra, smem + s * STAGE, m0, k0, g.M, kend, g.lda, wid, lane);
                OpB::issue(rb, smem + s * STAGE + OpA::kBytes, n0, k0, g.N, kend, g.ldb, wid, lane);
            }
        };
        // Stages are always filled S tiles ahead: loads past the end of K
        // read as zeros (their stages are never consumed), so the number of
        // loads in flight is the same at every hand-over and the loop body
        // has no branches for the scheduler to stop at.
#pragma unroll
        for (int s = 0; s < S; ++s) issue(s, kbase + s * BK);
        wait_vmcnt<W0>();  // tile 0 has landed
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

        bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[0][i] = OpA::frag(smem, wm * WTM + i * 32, 0, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = OpB::frag(smem + OpA::kBytes, wn * WTN + j * 32, 0, lane);

        auto mfmas = [&](int set) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
        };
        auto reads = [&](const char *stage, int kk, int set) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[set][i] = OpA::frag(stage, wm * WTM + i * 32, kk, lane);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[set][j] = OpB::frag(stage + OpA::kBytes, wn * WTN + j * 32, kk, lane);
        };
        // k-steps 0 .. KSTEPS-2 of a tile: next k-step's fragments are read
        // while this one's MFMAs run
        auto inner = [&](const char *cur) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk + 1 < KSTEPS; ++kk) {
                reads(cur, kk + 1, (kk + 1) & 1);
                mfmas(kk & 1);
                sched_interleave<NREAD, FM * FN, 0>();
            }
        };

        int stage = 0;
        for (int kt = 0; kt + 1 < nkt; ++kt) {
            const char *cur = smem + stage * STAGE;
            inner(cur);
            // hand-over to tile kt + 1 (last k-step's fragments are in
            // registers once lgkmcnt drains; tiles kt + 2 .. kt + S - 1 may
            // still be in flight)
            wait_lgkm0();
            wait_vmcnt<WH>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            // the next tile's first fragments are read before the refill is
            // issued: no load is then in flight for the compiler to wait on
            const int next = stage + 1 == S ? 0 : stage + 1;
            reads(smem + next * STAGE, 0, 0);
            issue(stage, kbase + (kt + S) * BK);
            stage = next;
            mfmas((KSTEPS - 1) & 1);
            sched_interleave<NREAD, FM * FN, LPT>();
        }
        inner(smem + stage * STAGE);
        mfmas((KSTEPS - 1) & 1);
    }
    wait_vmcnt<0>();
    __syncthreads();
    store_tile<C>(acc, smem, epi, g, m0, n0, wm, wn, tid, lane);
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain FMA)
// ---------------------------------------------------------------------------

template <bool AK, bool BK_, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, Epi epi) {
    constexpr int T = 64, KT = 16;
    __shared__ float As[KT][T + 4], Bs[KT][T + 4];
    const float *A = (const float *)g.a, *B = (const float *)g.b;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < g.K; k0 += KT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int e = tid + i * 256;
            int r, kk;
            if (AK) { r = e / KT; kk = e % KT; } else { kk = e / T; r = e % T; }
            int gm = m0 + r, gk = k0 + kk;
            As[kk][r] = (gm < g.M && gk < g.K) ? (AK ? A[gm * g.lda + gk] : A[gk * g.lda + gm]) : 0.f;
            if (BK_) { r = e / KT; kk = e % KT; } else { kk = e / T; r = e % T; }
            int gn = n0 + r;
            gk = k0 + kk;
            Bs[kk][r] = (gn < g.N && gk < g.K) ? (BK_ ? B[gn * g.ldb + gk] : B[gk * g.ldb + gn]) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < g.M && n < g.N) epi(m, n, acc[i][j]);
        }
}

// Sums the nsplit partial products of each output element in split order and
// applies the product's epilogue to 8 consecutive columns per thread.
template <class Epi>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ ws, int nsplit, int M, int N,
                                                            Epi epi) {
    const int64_t i = blockIdx.x * 256LL + threadIdx.x;
    const int n8 = N >> 3;
    if (i >= (int64_t)M * n8) return;
    const int m = (int)(i / n8), n = (int)(i % n8) * 8;
    const int64_t stride = (int64_t)M * N;
    float v[8];
    load8(ws + (int64_t)m * N + n, v);
    for (int sp = 1; sp < nsplit; ++sp) {
        float x[8];
        load8(ws + sp * stride + (int64_t)m * N + n, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += x[j];
    }
    epi.row8(m, n, v);
}

// The same for partial products stored transposed (a product computed as
// C^T = B A^T: split sp holds element (m, n) at ws[sp * stride + n * ldm + m]).
// Consecutive threads take consecutive rows m, so every partial-sum load of a
// wave reads one contiguous run.
template <class Epi>
__global__ __launch_bounds__(256) void splitk_reduce_t_kernel(const float *__restrict__ ws, int nsplit, int M,
                                                              int ldm, int N, Epi epi) {
    const int64_t i = blockIdx.x * 256LL + threadIdx.x;
    if (i >= (int64_t)M * (N >> 3)) return;
    const int m = (int)(i % M), n = (int)(i / M) * 8;
    const int64_t stride = (int64_t)N * ldm;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ws[(int64_t)(n + j) * ldm + m];
    for (int sp = 1; sp < nsplit; ++sp) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] += ws[sp * stride + (int64_t)(n + j) * ldm + m];
    }
    epi.row8(m, n, v);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Tile rows per group of the XCD-aware tile order (see tile_of): 8 measured
// best or within noise of it on every product of the layer (4 and 16 lose up
// to 5% on the long-K products).
constexpr int kGroupRows = 8;

// The dynamic-LDS limit of one kernel, raised once per device (a function
// attribute is per device; the flags are atomic so concurrent first calls
// only repeat an idempotent call).
struct AttrOnce {
    static constexpr int kMaxDev = 64;
    std::atomic<bool> done[kMaxDev] = {};
    hipError_t set(const void *fn, int lds) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < kMaxDev && done[dev].load(std::memory_order_acquire)) return hipSuccess;
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess && dev >= 0 && dev < kMaxDev) done[dev].store(true, std::memory_order_release);
        return e;
    }
};

template <class C, bool AK, bool BK_, class E>
static hipError_t launch_dl(const GemmArgs &g, const E &epi, hipStream_t st) {
    static AttrOnce once;
    hipError_t e = once.set((const void *)gemm_bf16_dl_kernel<C, AK, BK_, E>, C::kLds);
    if (e != hipSuccess) return e;
    const int tiles = ((g.M + C::kBM - 1) / C::kBM) * ((g.N + C::kBN - 1) / C::kBN);
    hipLaunchKernelGGL((gemm_bf16_dl_kernel<C, AK, BK_, E>), dim3(tiles, g.nsplit), dim3(C::kThreads), C::kLds, st, g,
                       epi, kGroupRows);
    return hipGetLastError();
}

template <class C, bool AK, bool BK_, class E, bool WHOLE>
static hipError_t launch_pp_as(const GemmArgs &g, const E &epi, hipStream_t st) {
    static AttrOnce once;
    hipError_t e = once.set((const void *)gemm_bf16_pp_kernel<C, AK, BK_, E, WHOLE>, C::kLds);
    if (e != hipSuccess) return e;
    const int tiles = ((g.M + C::kBM - 1) / C::kBM) * ((g.N + C::kBN - 1) / C::kBN);
    hipLaunchKernelGGL((gemm_bf16_pp_kernel<C, AK, BK_, E, WHOLE>), dim3(tiles, g.nsplit), dim3(C::kThreads), C::kLds,
                       st, g, epi, kGroupRows);
    return hipGetLastError();
}

// Reductions of whole K-tiles (every split too) take the kernel whose load
// offsets are fixed per lane; others test every load against the end of K.
// (Measured in the layer step: weight gradients 2%, the input-gradient
// products 2-5%, the forward products 2-3% faster.)
template <class C, bool AK, bool BK_, class E>
static hipError_t launch_pp(const GemmArgs &g, const E &epi, hipStream_t st) {
    const bool whole = g.K % C::kBK == 0 && (g.nsplit == 1 || g.kc % C::kBK == 0);
    return whole ? launch_pp_as<C, AK, BK_, E, true>(g, epi, st) : launch_pp_as<C, AK, BK_, E, false>(g, epi, st);
}

using Dl128 = DlCfg<128, 128, 2, 2, 2>;              // 64 KB of LDS: two workgroups per compute unit
using Pp256 = DlCfg<256, 256, 2, 2, 2, 64>;          // 128 KB, one workgroup per compute unit
using Pp256x192 = DlCfg<256, 192, 2, 2, 2, 64>;      // 112 KB, one workgroup per compute unit
using Pp128x192 = DlCfg<128, 192, 2, 2, 2, 64, 2>;   // 80 KB, two workgroups per compute unit
using Pp256x128 = DlCfg<256, 128, 2, 2, 3, 32, 2>;   // 72 KB, two workgroups per compute unit
// eight waves (two per SIMD) on one large tile: the latency hiding of two
// workgroups per compute unit with the operand reuse of the large tile
using Pp256w8 = DlCfg<256, 256, 2, 4, 2, 64>;        // 128 KB; waves 2x4 (128x64 each)
// the same with four stages of 32-deep K-tiles, three in flight, for the
// products with an M/N-contiguous operand, whose K-rows stay 512-byte runs
// at any depth (a K-contiguous operand's 64-byte rows would split every
// 128-byte line in two): 1.5% faster on the weight gradients in the step
using Pp256w8k32 = DlCfg<256, 256, 2, 4, 4, 32>;     // 128 KB
// products of at most 128 token rows computed transposed (C^T = W X^T): 256
// weight rows by the 128 token rows, three stages (two K-tiles in flight);
// 8 waves measured 1-3% ahead of 4 (128x64 each) on the forward products
using Sk256x128 = DlCfg<256, 128, 4, 2, 3, 64>;      // 144 KB; waves 4x2 (64x64 each)
// 192x192 tiles of 4 waves (96x96 each), four stages of 32-deep K-tiles:
// weight gradients whose 256x256 tiles leave most of a round idle
using Pp192k32 = DlCfg<192, 192, 2, 2, 4, 32>;       // 96 KB, one workgroup per compute unit

// Tile configurations, chosen per product shape from measurements on MI355X
// (TFLOP/s of each candidate on the GPT-3 175B t=8 shard's products and on
// large square products).  A 128x128 tile needs 64 bytes of operand per
// clock per compute unit to keep the matrix cores busy, close to what the
// load path delivers, so larger tiles win wherever there are enough of them
// to fill the 256 compute units; the plain (non-pipelined) 128x128 kernel
// is the best fit for short reductions and narrow outputs.
enum class Tile { Dl128, Pp128, Pp256x128, Pp256, Pp256x192, Pp128x192, Pp256w8, Sk256x128, Pp192 };

template <typename T, bool AK, bool BK_, class E>
static hipError_t launch(const GemmArgs &g, const E &epi, Tile tile, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        switch (tile) {
        case Tile::Pp256: return launch_pp<Pp256, AK, BK_>(g, epi, st);
        case Tile::Pp256x192: return launch_pp<Pp256x192, AK, BK_>(g, epi, st);
        case Tile::Pp128x192: return launch_pp<Pp128x192, AK, BK_>(g, epi, st);
        case Tile::Pp256w8:
            if constexpr (AK && BK_) return launch_pp<Pp256w8, AK, BK_>(g, epi, st);
            else return launch_pp<Pp256w8k32, AK, BK_>(g, epi, st);
        case Tile::Pp256x128: return launch_pp<Pp256x128, AK, BK_>(g, epi, st);
        case Tile::Pp128: return launch_pp<Dl128, AK, BK_>(g, epi, st);
        case Tile::Sk256x128: return launch_pp<Sk256x128, AK, BK_>(g, epi, st);
        case Tile::Pp192:
            if constexpr (!AK && !BK_) return launch_pp<Pp192k32, AK, BK_>(g, epi, st);
            else return launch_pp<Pp128x192, AK, BK_>(g, epi, st);
        case Tile::Dl128: break;
        }
        return launch_dl<Dl128, AK, BK_>(g, epi, st);
    } else {
        dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
        hipLaunchKernelGGL((gemm_f32_kernel<AK, BK_, E>), grid, dim3(256), 0, st, g, epi);
        return hipGetLastError();
    }
}

// Calls f with the epilogue functor of `kind`.
template <typename T, class F>
static hipError_t with_epi(Epi kind, const EpiArgs &e, F &&f) {
    switch (kind) {
    case Epi::StoreF32: return f(EpiStoreF32<T>{(float *)e.c, e.ldc});
    case Epi::AccumF32: return f(EpiAccumF32<T>{(float *)e.c, e.ldc});
    case Epi::Store: return f(EpiStore<T>{(T *)e.c, e.ldc});
    case Epi::BiasGelu: return f(EpiBiasGelu<T>{(T *)e.c, e.ldc, (T *)e.c2, e.ldc2, (const T *)e.bias});
    case Epi::GeluGrad: return f(EpiGeluGrad<T>{(T *)e.c, e.ldc, (const T *)e.aux, e.ldaux});
    case Epi::Qkv: {
        int dshift = 0;
        while ((1 << dshift) < e.d) ++dshift;
        return f(EpiQkv<T>{(const T *)e.bias, (T *)e.q, (T *)e.k, (T *)e.v, make_fastdiv((uint32_t)e.batch), e.nt,
                           e.seq, dshift, e.ht, e.row0});
    }
    }
    return hipErrorInvalidValue;
}

// The product kernels of one operand layout with every epilogue: split
// partial sums to split_ws when it is given, else the product's epilogue.
template <typename T, bool AK, bool BK_>
static hipError_t dispatch_epi(const GemmArgs &g, Epi kind, const EpiArgs &e, float *split_ws, Tile tile,
                               hipStream_t st) {
    if (split_ws) return launch<T, AK, BK_>(g, EpiSplit{split_ws, g.N, (int64_t)g.M * g.N}, tile, st);
    return with_epi<T>(kind, e, [&](auto epi) { return launch<T, AK, BK_>(g, epi, tile, st); });
}

// One translation unit per operand layout instantiates its kernels (they
// dominate the build): forward (A and B K-contiguous), input gradient (B
// N-contiguous), weight gradient (A and B M/N-contiguous).
hipError_t gemm_layout_nt(bool is_bf16, const GemmArgs &g, Epi kind, const EpiArgs &e, float *split_ws, Tile tile,
                          hipStream_t st);
hipError_t gemm_layout_nn(bool is_bf16, const GemmArgs &g, Epi kind, const EpiArgs &e, float *split_ws, Tile tile,
                          hipStream_t st);
hipError_t gemm_layout_tn(bool is_bf16, const GemmArgs &g, Epi kind, const EpiArgs &e, float *split_ws, Tile tile,
                          hipStream_t st);
// A M-contiguous, B K-contiguous: the input-gradient products computed
// transposed (split partial sums only)
hipError_t gemm_layout_mk_split(const GemmArgs &g, float *split_ws, int64_t ldc, Tile tile, hipStream_t st);

}  // namespace tpk
