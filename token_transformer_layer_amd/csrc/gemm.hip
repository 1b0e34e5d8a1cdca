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
// bf16 path: v_mfma_f32_32x32x16_bf16.  A workgroup of 4 waves computes a
// 128x192 tile (two workgroups per compute unit; also 128x128 and, with 4
// or 8 waves, 256-row tiles), each wave its share as a grid of 32x32 MFMA
// blocks.  K-tiles of 64 travel from HBM straight into LDS (buffer loads
// that write LDS, two stages, the next K-tile in flight while the current
// one feeds the MFMAs); fragments are read from LDS with ds_read_b128
// (K-contiguous operands) or ds_read_b64_tr_b16 (M/N-contiguous operands,
// read transposed).  Tiles are mapped to workgroups XCD-aware; products too
// small to fill the chip split their reduction into fp32 partial sums that a
// second kernel adds in split order; those of at most 128 token rows against
// a weight (short slices) are computed transposed, C^T = W X^T, so that 256
// weight rows share each read of the token rows.
//
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tiles, 4 x 4 per thread).
#include <algorithm>
#include <atomic>
#include <cstdio>

#include "gemm_kernels.h"
#include "trace.h"

namespace tpk {

static uint32_t extent_bytes(int rows, int k, const Mat &m, int es) {
    // bytes from the base pointer to one past the last element addressed
    int64_t last = m.kcontig ? (int64_t)(rows - 1) * m.ld + k : (int64_t)(k - 1) * m.ld + rows;
    return (uint32_t)(last * es);
}

static std::atomic<int> g_force_tile{-1};

constexpr int64_t kSplitMaxFloats = 512LL * 128 * 192;  // 48 MB: about two rounds of 128x192 tiles

void gemm_force_tile(int tile) { g_force_tile.store(tile); }

// Fraction of the last round of a launch that its tiles fill, with `slots`
// workgroups resident on the chip at once.
static double round_fill(long tiles, long slots) {
    const long rounds = (tiles + slots - 1) / slots;
    return rounds > 0 ? (double)tiles / (double)(rounds * slots) : 0.0;
}

static Tile pick_tile(int M, int N, int K, bool ak, bool bk) {
    const int forced = g_force_tile.load(std::memory_order_relaxed);
    if (forced >= 0) return (Tile)forced;
    const long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);
    const long t128x192 = (long)((M + 127) / 128) * ((N + 191) / 192);
    // Two 128x192 workgroups per compute unit (64-wide K-tiles: whole cache
    // lines per row) are the best measured fit for the layer shards'
    // forward and input-gradient products.  An 8-wave 256x256 workgroup
    // per compute unit (one workgroup of two waves per SIMD) wins where its
    // tiles fill the last round of 256: the weight gradients (K = tokens;
    // 3% in the 175B step), large squares and the cube block's products
    // (8-10% in isolation).  (An 8-wave 256x192 tile measured 10-15% ahead
    // on the 175B forward products in isolation, with the operands resident
    // in the MALL, but not in the step, where the weights come from HBM;
    // it is not used.)  Products too small for a round of 128x192 tiles take
    // 128x128 tiles and split their reduction.
    const double f256 = round_fill(t256, 256), f128x192 = round_fill(t128x192, 512);
    if (ak && bk && K >= 4096 && f256 >= 0.97) return Tile::Pp256w8;
    // input gradients and weight gradients: the 8-wave tile also for
    // reductions of 1024-4095 and for weight gradients whose last round is
    // 60% full (measured on the 13B shard's products with the operands
    // flushed from the MALL: 4-10% over 128x192 tiles)
    if (ak && !bk && K >= 1024 && t128x192 >= 192 && f256 >= f128x192 - 0.02) return Tile::Pp256w8;
    if (!ak && !bk && K >= 1024 && f256 >= 0.6 && t256 >= 128) return Tile::Pp256w8;
    // weight gradients whose 192x192 tiles fill whole rounds of 256 where the
    // 256x256 ones do not (the 175B output projection's, 12288 x 1536: 512
    // tiles against 288): 88-89 against 92-94 us for 128x192 tiles
    const long t192 = (long)((M + 191) / 192) * ((N + 191) / 192);
    if (!ak && !bk && K >= 1024 && M % 192 == 0 && N % 192 == 0 && t192 % 256 == 0) return Tile::Pp192;
    // long reductions into outputs whose width wastes more than 15% of a
    // 192-wide tile column (640 columns: 768 computed) take 128-wide tiles
    // (7-9% faster there)
    const int n192 = (N + 191) / 192 * 192;
    if ((double)N / n192 < 0.85 && M >= 256 && K >= 4096) return Tile::Pp128;
    if (t128x192 >= 192 && K >= 512) return Tile::Pp128x192;
    // narrow outputs of a long reduction over many rows (the attention
    // output projection's input gradient): 128x192 tiles with the reduction
    // split (measured 858 against 698 TFLOP/s for split 128x128 tiles on
    // 2048x1536x12288)
    if (M >= 256 && K >= 4096) return Tile::Pp128x192;
    return Tile::Dl128;
}

static const char *tile_name(Tile t) {
    switch (t) {
    case Tile::Dl128: return "128";
    case Tile::Pp128: return "p128";
    case Tile::Pp256x128: return "256x128";
    case Tile::Pp256: return "256";
    case Tile::Pp256x192: return "256x192";
    case Tile::Pp128x192: return "128x192";
    case Tile::Pp256w8: return "256w8";
    case Tile::Sk256x128: return "sk256x128";
    case Tile::Pp192: return "192";
    }
    return "?";
}

static hipError_t dispatch_layout(bool is_bf16, const GemmArgs &g, bool ak, bool bk, Epi kind, const EpiArgs &e,
                                  float *split_ws, Tile tile, hipStream_t st) {
    // The layer uses three operand forms: forward (K, K), input gradient
    // (K, N-contiguous) and weight gradient (M-contiguous, N-contiguous).
    if (ak && bk) return gemm_layout_nt(is_bf16, g, kind, e, split_ws, tile, st);
    if (ak && !bk) return gemm_layout_nn(is_bf16, g, kind, e, split_ws, tile, st);
    if (!ak && !bk) return gemm_layout_tn(is_bf16, g, kind, e, split_ws, tile, st);
    return hipErrorInvalidValue;
}

// Number of reduction splits: a product whose 128-row tiles do not fill the
// compute units (short token ranges, narrow outputs) splits its reduction
// so that about 1.5 workgroups per compute unit run, when the caller's
// workspace holds the partial products (at most kSplitMaxFloats floats).
static int pick_splits(int M, int N, int K, Tile t, int64_t ws_floats) {
    if (t != Tile::Dl128 && t != Tile::Pp128 && t != Tile::Pp128x192) return 1;
    const int bn = t == Tile::Pp128x192 ? 192 : 128;
    const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + bn - 1) / bn);
    int sp;
    if (t == Tile::Pp128x192) {
        // two workgroups per compute unit: the largest split that keeps the
        // launch within one round of 512 (tiles filling at most half a round;
        // a product with a tile per compute unit already does not split: the
        // medium configuration's QKV product, 256 tiles over K = 1024, 37 ->
        // 25 us unsplit)
        if (tiles >= 256) return 1;
        sp = (int)(512 / tiles);
    } else {
        if (tiles >= 256) return 1;
        // about 384 workgroups (1.5 per compute unit): measured better than
        // two rounds, whose extra partial sums cost more than the fill they add
        sp = (int)((384 + tiles - 1) / tiles);
    }
    // at most 8 splits, 16 when even 8 leave most compute units idle (a
    // slice's narrow products: 12 tiles, 1.2 -> 1.5 TB/s of weights)
    sp = std::min(sp, tiles * 8 < 128 ? 16 : 8);
    sp = std::min(sp, K / 512);
    while (sp > 1 && (int64_t)sp * M * N > ws_floats) --sp;
    return std::max(sp, 1);
}

size_t gemm_split_workspace_floats() { return kSplitMaxFloats; }

static const char *const kEpiName[] = {"store_f32", "accum_f32", "store", "bias_gelu", "gelu_grad", "qkv"};

// Algorithmic bytes of a product for its trace record: A and B read once,
// C written once (read too when accumulated), plus the epilogue's extra
// operand or output.
static double product_bytes(int M, int N, int K, int es, Epi kind, const EpiArgs &e) {
    const double mn = (double)M * N;
    double out_b = mn * es;
    if (kind == Epi::StoreF32) out_b = mn * 4;
    if (kind == Epi::AccumF32) out_b = mn * 8;
    if (kind == Epi::BiasGelu && e.c) out_b = 2 * mn * es;
    if (kind == Epi::GeluGrad) out_b = 2 * mn * es;
    return ((double)M * K + (double)N * K) * es + out_b;
}

// A product of at most 128 token rows against a weight (a forward or
// input-gradient product of a short slice) computed transposed, C^T = W X^T:
// 256 weight rows per workgroup share one read of the token rows (half the
// activation reads of 128x128 tiles), and the reduction splits so that one
// round of 256 workgroups (one per compute unit) runs.  Measured on the
// 175B shard's 128-row products: the per-slice schedule 1-3.5% faster (the
// QKV product 51 -> 44 us); 128 or 192 workgroups leave compute units idle
// and two rounds (512) write twice the partial sums, both 1-12% slower.
// Returns false (nothing launched) when the product does not qualify.
static bool gemm_swapped(int M, int N, int K, const Mat &A, const Mat &B, Epi kind, const EpiArgs &e, const char *lay,
                         hipStream_t st, hipError_t &err) {
    if (M > 128 || M % 8 != 0 || N % 8 != 0 || !A.kcontig || K < 1024) return false;
    const Tile tile = Tile::Sk256x128;
    const int tiles = (N + 255) / 256;
    int sp = std::max(1, 256 / tiles);
    sp = std::min(sp, std::min(16, K / 512));
    while (sp > 1 && (int64_t)sp * M * N > e.split_ws_floats) --sp;
    if (sp < 2) return false;
    GemmArgs g{};
    g.M = N;
    g.N = M;
    g.K = K;
    g.a = B.p;
    g.lda = B.ld;
    g.b = A.p;
    g.ldb = A.ld;
    g.a_bytes = extent_bytes(N, K, B, 2);
    g.b_bytes = extent_bytes(M, K, A, 2);
    g.kc = ((K + sp - 1) / sp + 63) / 64 * 64;
    g.nsplit = (K + g.kc - 1) / g.kc;
    char name[64];
    snprintf(name, sizeof name, "gemm_bf16_%s_%s_%s_split", tile_name(tile), lay, kEpiName[(int)kind]);
    TraceScope ts(st, name, 2.0 * M * N * K, product_bytes(M, N, K, 2, kind, e));
    err = B.kcontig ? gemm_layout_nt(true, g, kind, e, e.split_ws, tile, st)
                    : gemm_layout_mk_split(g, e.split_ws, M, tile, st);
    if (err != hipSuccess) return true;
    const int64_t threads = (int64_t)M * (N / 8);
    err = with_epi<bf16>(kind, e, [&](auto epi) {
        hipLaunchKernelGGL((splitk_reduce_t_kernel<decltype(epi)>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, st, e.split_ws, g.nsplit, M, M, N, epi);
        return hipGetLastError();
    });
    return true;
}

hipError_t gemm(DType dt, int M, int N, int K, Mat A, Mat B, Epi kind, const EpiArgs &e, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int es = dt == DType::BF16 ? 2 : 4;
    GemmArgs g{};
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
    const Tile tile = pick_tile(M, N, K, A.kcontig, B.kcontig);
    // (the split reductions take 8 output columns per thread)
    const int nsplit =
        dt == DType::BF16 && e.split_ws && N % 8 == 0 ? pick_splits(M, N, g.K, tile, e.split_ws_floats) : 1;
    const char *lay = A.kcontig ? (B.kcontig ? "nt" : "nn") : "tn";
    if (nsplit > 1 && g_force_tile.load(std::memory_order_relaxed) < 0) {
        hipError_t err = hipSuccess;
        if (gemm_swapped(M, N, K, A, B, kind, e, lay, st, err)) return err;
    }
    g.nsplit = nsplit;
    g.kc = nsplit > 1 ? ((g.K + nsplit - 1) / nsplit + 63) / 64 * 64 : g.K;
    char name[64];
    if (dt == DType::BF16 && nsplit > 1)
        snprintf(name, sizeof name, "gemm_bf16_%s_%s_%s_split", tile_name(tile), lay, kEpiName[(int)kind]);
    else if (dt == DType::BF16)
        snprintf(name, sizeof name, "gemm_bf16_%s_%s_%s", tile_name(tile), lay, kEpiName[(int)kind]);
    else
        snprintf(name, sizeof name, "gemm_f32_%s_%s", lay, kEpiName[(int)kind]);
    TraceScope ts(st, name, 2.0 * M * N * K, product_bytes(M, N, K, es, kind, e));
    if (dt != DType::BF16) return dispatch_layout(false, g, A.kcontig, B.kcontig, kind, e, nullptr, tile, st);
    if (nsplit == 1) return dispatch_layout(true, g, A.kcontig, B.kcontig, kind, e, nullptr, tile, st);
    hipError_t err = dispatch_layout(true, g, A.kcontig, B.kcontig, kind, e, e.split_ws, tile, st);
    if (err != hipSuccess) return err;
    const int64_t threads = (int64_t)M * (N / 8);
    return with_epi<bf16>(kind, e, [&](auto epi) {
        hipLaunchKernelGGL((splitk_reduce_kernel<decltype(epi)>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, st, e.split_ws, nsplit, M, N, epi);
        return hipGetLastError();
    });
}

}  // namespace tpk
