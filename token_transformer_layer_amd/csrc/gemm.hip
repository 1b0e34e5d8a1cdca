// GEMMs of the layer shard on gfx950.
//
// C[m][n] = sum_k A[m][k] B[n][k] with fp32 accumulation and a fused
// epilogue.  The three operand forms the layer needs are the ones of
// "Maximizing Parallelism in Distributed Training for Huge Neural Networks",
// section 3.1.2: the forward Y = X W^T (both operands K-contiguous), the
// input gradient dX = dY W (W read along its rows: B is N-contiguous) and the
// weight gradient dW = dY^T X (a reduction over tokens: both operands are
// M/N-contiguous).
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on LDS-staged tiles.  Each workgroup of
// 4 waves computes a BM x BN tile; each wave a (BM/2) x (BN/2) sub-tile as a
// grid of 32x32 MFMA blocks.  Global loads are raw buffer loads (16 bytes per
// lane, zero-filled outside the matrix), prefetched one K-tile ahead into
// registers while the MFMAs run on the current LDS buffer (two LDS buffers,
// one barrier per K-tile).  LDS rows hold 8 chunks of 16 bytes (BK = 64);
// chunk c of row r is stored at c ^ ((r ^ (r >> 3)) & 7), which keeps both
// the MFMA fragment reads (8 consecutive rows, same chunk) and the
// transposing stores (rows 8 apart) free of bank conflicts.  An operand that
// is M/N-contiguous in memory is transposed in registers on its way to LDS.
//
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tiles, 4 x 4 per thread).
#include <cmath>
#include <cstdio>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace tpk {

// ---------------------------------------------------------------------------
// Epilogues: called once per output element (m, n) inside the matrix.
// ---------------------------------------------------------------------------

template <typename T>
struct EpiStoreF32 {
    float *c;
    int64_t ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v) const { c[m * ldc + n] = v; }
};

template <typename T>
struct EpiAccumF32 {
    float *c;
    int64_t ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v) const { c[m * ldc + n] += v; }
};

template <typename T>
struct EpiStore {
    T *c;
    int64_t ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v) const { c[m * ldc + n] = from_f32<T>(v); }
};

template <typename T>
struct EpiBiasGelu {
    T *z;  // may be null
    int64_t ldz;
    T *g;
    int64_t ldg;
    const T *bias;
    __device__ __forceinline__ void operator()(int m, int n, float v) const {
        float zz = v + to_f32(bias[n]);
        if (z) z[m * ldz + n] = from_f32<T>(zz);
        g[m * ldg + n] = from_f32<T>(gelu_f(zz));
    }
};

template <typename T>
struct EpiGeluGrad {
    T *c;
    int64_t ldc;
    const T *z;
    int64_t ldz;
    __device__ __forceinline__ void operator()(int m, int n, float v) const {
        c[m * ldc + n] = from_f32<T>(v * gelu_grad_f(to_f32(z[m * ldz + n])));
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
};

struct GemmArgs {
    int M, N, K;
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

// Loads a ROWS x BK tile (ROWS along M or N) of one bf16 operand into
// registers and stores it to LDS as [ROWS][BK] with the chunk swizzle.
template <int ROWS, int BK, int NT, bool KCONTIG>
struct TileLoader {
    static constexpr int VEC = ROWS * BK / 8 / NT;  // 16-byte vectors per thread
    static_assert(VEC >= 1, "tile too small for the thread count");
    u32x4 r[VEC];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int mn0, int k0, int MN, int K,
                                         int64_t ld, int tid) {
        if constexpr (KCONTIG) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                int v = tid + i * NT;
                int row = v / (BK / 8), ch = v % (BK / 8);
                int gm = mn0 + row, gk = k0 + ch * 8;
                uint32_t off = (gm < MN && gk < K) ? (uint32_t)((gm * ld + gk) * 2) : kOOB;
                r[i] = buf_load16(rs, off);
            }
        } else {
            static_assert(VEC == 4 || VEC == 8, "transposing loader needs 4 or 8 vectors");
            int mnb = tid % (ROWS / 8), kg = tid / (ROWS / 8);
            int gm = mn0 + mnb * 8;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                int gk = k0 + kg * VEC + i;
                uint32_t off = (gm < MN && gk < K) ? (uint32_t)((gk * ld + gm) * 2) : kOOB;
                r[i] = buf_load16(rs, off);
            }
        }
    }

    __device__ __forceinline__ void store(char *lds, int tid) const {
        if constexpr (KCONTIG) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                int v = tid + i * NT;
                int row = v / (BK / 8), ch = v % (BK / 8);
                *(u32x4 *)(lds + row * (BK * 2) + ((ch ^ lds_swz(row)) << 4)) = r[i];
            }
        } else {
            int mnb = tid % (ROWS / 8), kg = tid / (ROWS / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                int row = mnb * 8 + c;
                // word w of the output: element c of r[2w] (low) and of r[2w+1] (high)
                uint32_t w[VEC / 2];
#pragma unroll
                for (int ww = 0; ww < VEC / 2; ++ww) {
                    uint32_t lo = r[2 * ww][c >> 1], hi = r[2 * ww + 1][c >> 1];
                    w[ww] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                int kbyte = kg * VEC * 2;  // byte offset of this thread's k-range in the row
                int ch = kbyte >> 4, within = kbyte & 15;
                char *dst = lds + row * (BK * 2) + ((ch ^ lds_swz(row)) << 4) + within;
                if constexpr (VEC == 4) {
                    *(u32x2 *)dst = u32x2{w[0], w[1]};
                } else {
                    *(u32x4 *)dst = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
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

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct TileCfg {
    static constexpr int kBM = BM, kBN = BN, kBK = 64, kWM = WAVES_M, kWN = WAVES_N;
    static constexpr int kThreads = WAVES_M * WAVES_N * 64;
    static constexpr int kLds = 2 * (BM + BN) * 64 * 2;  // two stages of A and B tiles
};

template <class C, bool AK, bool BK_, class Epi>
__global__ __launch_bounds__(C::kThreads) void gemm_bf16_kernel(GemmArgs g, Epi epi, int gm_rows) {
    constexpr int BM = C::kBM, BN = C::kBN, BK = C::kBK, NT = C::kThreads;
    constexpr int WTM = BM / C::kWM, WTN = BN / C::kWN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / C::kWN, wn = wid % C::kWN;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, gm_rows, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, g.a_bytes);
    __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, g.b_bytes);
    TileLoader<BM, BK, NT, AK> la;
    TileLoader<BN, BK, NT, BK_> lb;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

    // per-lane LDS byte offsets of the fragment rows (the chunk is added per k-step)
    int a_row[FM], b_row[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a_row[i] = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j) b_row[j] = wn * WTN + j * 32 + (lane & 31);

    const int nkt = (g.K + BK - 1) / BK;
    la.load(ra, m0, 0, g.M, g.K, g.lda, tid);
    lb.load(rb, n0, 0, g.N, g.K, g.ldb, tid);
    la.store(smem, tid);
    lb.store(smem + A_BYTES, tid);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const char *cur = smem + (kt & 1) * (A_BYTES + B_BYTES);
        const bool more = kt + 1 < nkt;
        if (more) {
            la.load(ra, m0, (kt + 1) * BK, g.M, g.K, g.lda, tid);
            lb.load(rb, n0, (kt + 1) * BK, g.N, g.K, g.ldb, tid);
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 fa[FM], fb[FN];
            const int ch = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *(const bf16x8 *)(cur + a_row[i] * (BK * 2) + ((ch ^ lds_swz(a_row[i])) << 4));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *(const bf16x8 *)(cur + A_BYTES + b_row[j] * (BK * 2) + ((ch ^ lds_swz(b_row[j])) << 4));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            char *nxt = smem + ((kt + 1) & 1) * (A_BYTES + B_BYTES);
            la.store(nxt, tid);
            lb.store(nxt + A_BYTES, tid);
        }
        __syncthreads();
    }

    // 32x32 accumulator layout: register v of lane l holds
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32 of the block.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            int col = n0 + wn * WTN + j * 32 + (lane & 31);
            if (col < g.N) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = m0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    if (row < g.M) epi(row, col, acc[i][j][v]);
                }
            }
        }
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

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static uint32_t extent_bytes(int rows, int k, const Mat &m, int es) {
    // bytes from the base pointer to one past the last element addressed
    int64_t last = m.kcontig ? (int64_t)(rows - 1) * m.ld + k : (int64_t)(k - 1) * m.ld + rows;
    return (uint32_t)(last * es);
}

// Tile configurations of the bf16 kernel.  Wide wave tiles cut the LDS
// traffic per MFMA (128x128 per wave reads 1 KB of fragments per 32x32 block
// pair); smaller tiles give more workgroups where M or N is small.
using Cfg256x256 = TileCfg<256, 256, 2, 2>;
using Cfg256x128 = TileCfg<256, 128, 2, 2>;
using Cfg128x128 = TileCfg<128, 128, 2, 2>;

enum class TileChoice { T256x256, T256x128, T128x128 };

// Picks the tile for an M x N x K product.  Measured on MI355X: the
// 128x128 tile (up to three workgroups per compute unit hide each other's
// memory latency) is fastest for every product of the GPT-3 175B shard; the
// 256x256 tile only wins on large products whose operands are both
// K-contiguous (e.g. 8192^3, 4096x24576x6144).
static TileChoice choose_tile(int M, int N, int K, bool ak, bool bk) {
    const double tiles128 = (double)((M + 127) / 128) * ((N + 127) / 128);
    if (ak && bk && tiles128 >= 4096 && K >= 1024) return TileChoice::T256x256;
    return TileChoice::T128x128;
}

template <class C, bool AK, bool BK_, class E>
static hipError_t launch_cfg(const GemmArgs &g, const E &epi, hipStream_t st) {
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_bf16_kernel<C, AK, BK_, E>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ((g.M + C::kBM - 1) / C::kBM) * ((g.N + C::kBN - 1) / C::kBN);
    hipLaunchKernelGGL((gemm_bf16_kernel<C, AK, BK_, E>), dim3(tiles), dim3(C::kThreads), C::kLds, st, g, epi, 4);
    return hipGetLastError();
}

template <typename T, bool AK, bool BK_, class E>
static hipError_t launch(const GemmArgs &g, const E &epi, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        switch (choose_tile(g.M, g.N, g.K, AK, BK_)) {
        case TileChoice::T256x256: return launch_cfg<Cfg256x256, AK, BK_>(g, epi, st);
        case TileChoice::T256x128: return launch_cfg<Cfg256x128, AK, BK_>(g, epi, st);
        default: return launch_cfg<Cfg128x128, AK, BK_>(g, epi, st);
        }
    } else {
        dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
        hipLaunchKernelGGL((gemm_f32_kernel<AK, BK_, E>), grid, dim3(256), 0, st, g, epi);
        return hipGetLastError();
    }
}

template <typename T, bool AK, bool BK_>
static hipError_t dispatch_epi(const GemmArgs &g, Epi kind, const EpiArgs &e, hipStream_t st) {
    switch (kind) {
    case Epi::StoreF32:
        return launch<T, AK, BK_>(g, EpiStoreF32<T>{(float *)e.c, e.ldc}, st);
    case Epi::AccumF32:
        return launch<T, AK, BK_>(g, EpiAccumF32<T>{(float *)e.c, e.ldc}, st);
    case Epi::Store:
        return launch<T, AK, BK_>(g, EpiStore<T>{(T *)e.c, e.ldc}, st);
    case Epi::BiasGelu:
        return launch<T, AK, BK_>(g, EpiBiasGelu<T>{(T *)e.c, e.ldc, (T *)e.c2, e.ldc2, (const T *)e.bias}, st);
    case Epi::GeluGrad:
        return launch<T, AK, BK_>(g, EpiGeluGrad<T>{(T *)e.c, e.ldc, (const T *)e.aux, e.ldaux}, st);
    case Epi::Qkv: {
        int dshift = 0;
        while ((1 << dshift) < e.d) ++dshift;
        return launch<T, AK, BK_>(g,
                                  EpiQkv<T>{(const T *)e.bias, (T *)e.q, (T *)e.k, (T *)e.v,
                                            make_fastdiv((uint32_t)e.batch), e.nt, e.seq, dshift, e.ht,
                                            e.row0},
                                  st);
    }
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t dispatch_layout(const GemmArgs &g, bool ak, bool bk, Epi kind, const EpiArgs &e,
                                  hipStream_t st) {
    // The layer uses three operand forms: forward (K, K), input gradient
    // (K, N-contiguous) and weight gradient (M-contiguous, N-contiguous).
    if (ak && bk) return dispatch_epi<T, true, true>(g, kind, e, st);
    if (ak && !bk) return dispatch_epi<T, true, false>(g, kind, e, st);
    if (!ak && !bk) return dispatch_epi<T, false, false>(g, kind, e, st);
    return hipErrorInvalidValue;
}

hipError_t gemm(DType dt, int M, int N, int K, Mat A, Mat B, Epi kind, const EpiArgs &e, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int es = dt == DType::BF16 ? 2 : 4;
    GemmArgs g;
    g.M = M;
    g.N = N;
    g.K = K;
    g.a = A.p;
    g.lda = A.ld;
    g.b = B.p;
    g.ldb = B.ld;
    if (K <= 0) {
        // an empty reduction: run the epilogue on zeros through a K = 0 loop
        g.K = 0;
    }
    g.a_bytes = K > 0 ? extent_bytes(M, K, A, es) : 0;
    g.b_bytes = K > 0 ? extent_bytes(N, K, B, es) : 0;
    // algorithmic work: 2MNK flops; A and B read once, C written once (read
    // too when accumulated), plus the epilogue's extra operand or output
    static const char *kEpiName[] = {"store_f32", "accum_f32", "store", "bias_gelu", "gelu_grad", "qkv"};
    const char *lay = A.kcontig ? (B.kcontig ? "nt" : "nn") : "tn";
    char name[64];
    snprintf(name, sizeof name, "gemm_%s_%s_%s", dt == DType::BF16 ? "bf16" : "f32", lay, kEpiName[(int)kind]);
    const double mn = (double)M * N;
    double out_b = mn * es;
    if (kind == Epi::StoreF32) out_b = mn * 4;
    if (kind == Epi::AccumF32) out_b = mn * 8;
    if (kind == Epi::BiasGelu && e.c) out_b = 2 * mn * es;
    if (kind == Epi::GeluGrad) out_b = 2 * mn * es;
    TraceScope ts(st, name, 2.0 * mn * K, ((double)M * K + (double)N * K) * es + out_b);
    if (dt == DType::BF16) return dispatch_layout<bf16>(g, A.kcontig, B.kcontig, kind, e, st);
    return dispatch_layout<float>(g, A.kcontig, B.kcontig, kind, e, st);
}

}  // namespace tpk
