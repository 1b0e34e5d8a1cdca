// LayerNorm forward/backward, bias-gradient column sums and the residual
// combine on gfx950.  All HBM-bound: each kernel reads and writes its rows
// once, with 16-byte (bf16) or 32-byte (fp32) vector accesses, and reduces
// within a row through wavefront shuffles and one LDS exchange.
//
// LayerNorm is replicated on every tensor-parallel rank ("Transformer
// Training 11: model parallelism", sequence-parallelism slide) and applies
// gamma and beta as matrix-vector ops ("Maximizing Parallelism in
// Distributed Training for Huge Neural Networks", section 3.2); its backward
// and the bias gradients follow that paper's section 3.1.3 (dA = dC * b,
// db = sum of dC * A over rows).  Parameter gradients are reduced in two
// deterministic stages (per-block partials, then one pass over the blocks),
// so repeated runs give identical bits.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace tpk {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxVec = 8;  // 8 vectors of 8 elements per thread: h <= 16384

// Sum over the 256 threads of a block; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// Rows [blockIdx.x * rpb, ...): dx = resid + rstd (gg - mean(gg) - xhat mean(gg xhat))
// with gg = du * gamma; the block's sums of du * xhat and du over its rows go
// to partials[block][0][:] and partials[block][1][:].  Each thread owns NV
// vectors of 8 columns (column vector c = threadIdx.x + i * 256) and keeps
// its gamma, its parameter-gradient sums and up to two rows' inputs in
// registers: the loads of row r + 1 are in flight while row r is reduced and
// written.
// Every row access goes through a buffer descriptor of that row, so vectors
// past the row (offset kOOB) and rows past the block's range (a descriptor
// of length zero) read zeros and drop stores without a branch: the loads are
// unconditional, and the compiler's wait before a row's arithmetic covers
// only that row's loads, not the next row's.
// 8 consecutive elements as loaded: packed bf16, or fp32.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    u32x4 w;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) { w = buf_load16(r, off); }
    __device__ __forceinline__ float operator[](int j) const { return j & 1 ? bf_hi(w[j >> 1]) : bf_lo(w[j >> 1]); }
};
template <> struct Raw8<float> {
    u32x4 a, b;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        a = buf_load16(r, off);
        b = buf_load16(r, off + 16);  // kOOB + 16 is still past every row
    }
    __device__ __forceinline__ float operator[](int j) const { return __uint_as_float(j < 4 ? a[j] : b[j - 4]); }
};

__device__ __forceinline__ void store8_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, const float v[8], float *) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                                 __float_as_uint(v[3])}, r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                                 __float_as_uint(v[7])}, r, off + 16, 0, 0);
}
__device__ __forceinline__ void store8_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, const float v[8], bf16 *) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf2(v[2 * i], v[2 * i + 1]);
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
}

// One row per block: u = (x - mean) rstd gamma + beta, two-pass statistics
// (mean, then the centred sum of squares) through wavefront sums and one LDS
// exchange each.  The row stays in registers as loaded (packed bf16: 4
// registers per 8 columns), so a block holds few registers and many rows are
// in flight per CU; loads and stores go through a buffer descriptor of the
// row (vectors past it read zeros and drop their stores).
template <typename T, int NV, bool EARLY = false>
__global__ __launch_bounds__(kThreads) void ln_fwd_kernel(int h, float eps, const T *__restrict__ x,
                                                          const T *__restrict__ g, const T *__restrict__ b,
                                                          T *__restrict__ u, float *__restrict__ mean,
                                                          float *__restrict__ rstd) {
    __shared__ float red[4];
    const int row = blockIdx.x, nv = h >> 3;
    const uint32_t row_t = (uint32_t)h * sizeof(T);
    const __amdgpu_buffer_rsrc_t px = make_rsrc(x + (size_t)row * h, row_t);
    uint32_t ot[NV];
    Raw8<T> xv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = threadIdx.x + i * kThreads;
        ot[i] = c < nv ? (uint32_t)c * (8 * sizeof(T)) : kOOB;
        xv[i].load(px, ot[i]);
    }
    // short row ranges: gamma and beta loaded with the row, one memory round
    // trip fewer per row
    [[maybe_unused]] Raw8<T> ge[EARLY ? NV : 1], be[EARLY ? NV : 1];
    if constexpr (EARLY) {
        const __amdgpu_buffer_rsrc_t pg = make_rsrc(g, row_t), pb = make_rsrc(b, row_t);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            ge[i].load(pg, ot[i]);
            be[i].load(pb, ot[i]);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += xv[i][j];  // vectors past the row are zeros
    const float mu = block_sum(s, red) / (float)h;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if ((int)threadIdx.x + i * kThreads < nv) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float dlt = xv[i][j] - mu;
                q += dlt * dlt;
            }
        }
    }
    const float var = block_sum(q, red) / (float)h;
    const float r = 1.0f / sqrtf(var + eps);
    const __amdgpu_buffer_rsrc_t pu = make_rsrc(u + (size_t)row * h, row_t);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        Raw8<T> gr, br;
        if constexpr (EARLY) {
            gr = ge[i];
            br = be[i];
        } else {
            const __amdgpu_buffer_rsrc_t pg = make_rsrc(g, row_t), pb = make_rsrc(b, row_t);
            gr.load(pg, ot[i]);
            br.load(pb, ot[i]);
        }
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (xv[i][j] - mu) * r * gr[j] + br[j];
        store8_buf(pu, ot[i], o, (T *)nullptr);
    }
    if (threadIdx.x == 0) {
        mean[row] = mu;
        rstd[row] = r;
    }
}

// Rows of at most 2048 columns: one wave per row, four rows a workgroup,
// the two row sums by wave reduction (no barrier).  Lane l owns the column
// vectors l + 64 i.
template <typename T, int NVW>
__global__ __launch_bounds__(256) void ln_fwd_wave_kernel(int rows, int h, float eps, const T *__restrict__ x,
                                                          const T *__restrict__ g, const T *__restrict__ b,
                                                          T *__restrict__ u, float *__restrict__ mean,
                                                          float *__restrict__ rstd) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (row >= rows) return;  // whole wave
    const int nv = h >> 3;
    const uint32_t row_t = (uint32_t)h * sizeof(T);
    const __amdgpu_buffer_rsrc_t px = make_rsrc(x + (size_t)row * h, row_t);
    uint32_t ot[NVW];
    Raw8<T> xv[NVW];
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
        const int c = lane + i * 64;
        ot[i] = c < nv ? (uint32_t)c * (8 * sizeof(T)) : kOOB;
        xv[i].load(px, ot[i]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NVW; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += xv[i][j];  // vectors past the row are zeros
    const float mu = wave_sum(s) / (float)h;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
        if (lane + i * 64 < nv) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float dlt = xv[i][j] - mu;
                q += dlt * dlt;
            }
        }
    }
    const float var = wave_sum(q) / (float)h;
    const float r = 1.0f / sqrtf(var + eps);
    const __amdgpu_buffer_rsrc_t pg = make_rsrc(g, row_t), pb = make_rsrc(b, row_t);
    const __amdgpu_buffer_rsrc_t pu = make_rsrc(u + (size_t)row * h, row_t);
#pragma unroll
    for (int i = 0; i < NVW; ++i) {
        Raw8<T> gr, br;
        gr.load(pg, ot[i]);
        br.load(pb, ot[i]);
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (xv[i][j] - mu) * r * gr[j] + br[j];
        store8_buf(pu, ot[i], o, (T *)nullptr);
    }
    if (lane == 0) {
        mean[row] = mu;
        rstd[row] = r;
    }
}

template <typename T>
struct LnRow {
    // one thread's share of a row: du fp32, x and resid as stored
    Raw8<float> du;
    Raw8<T> x, res;
};

template <typename T, int NV, int TPB>
__global__ __launch_bounds__(TPB) void ln_bwd_kernel(int rows, int h, int rpb, const float *__restrict__ du,
                                                          const T *__restrict__ resid, const T *__restrict__ x,
                                                          const T *__restrict__ g, const float *__restrict__ mean,
                                                          const float *__restrict__ rstd, T *__restrict__ dx,
                                                          float *__restrict__ partials) {
    constexpr int NWV = TPB / 64;
    __shared__ float red[2][2][NWV];
    const int nv = h >> 3;
    const int r0 = blockIdx.x * rpb, r1 = min(rows, r0 + rpb);
    const uint32_t row_f32 = (uint32_t)h * 4, row_t = (uint32_t)h * sizeof(T);
    // byte offsets of this thread's vectors in an fp32 row and a T row
    uint32_t o4[NV], ot[NV];
    float gg[NV][8], adg[NV][8], adb[NV][8];
    {
        const __amdgpu_buffer_rsrc_t pg = make_rsrc(g, row_t);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = threadIdx.x + i * TPB;
            o4[i] = c < nv ? (uint32_t)c * 32 : kOOB;
            ot[i] = c < nv ? (uint32_t)c * (8 * sizeof(T)) : kOOB;
            Raw8<T> gr;
            gr.load(pg, ot[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                gg[i][j] = gr[j];
                adg[i][j] = adb[i][j] = 0.f;
            }
        }
    }
    // a row's statistics are loaded with its data (before the next row's
    // loads), so waiting for them does not wait for the next row
    auto load_row = [&](int row, LnRow<T> (&d)[NV], float &mu, float &rs) __attribute__((always_inline)) {
        const bool valid = row < r1;
        const int rr = valid ? row : min(r0, rows - 1);  // a workgroup past the last row still reads in bounds
        mu = mean[rr];
        rs = rstd[rr];
        const size_t base = (size_t)rr * h;
        const __amdgpu_buffer_rsrc_t pdu = make_rsrc(du + base, valid ? row_f32 : 0u);
        const __amdgpu_buffer_rsrc_t px = make_rsrc(x + base, valid ? row_t : 0u);
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(resid + base, valid ? row_t : 0u);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            d[i].du.load(pdu, o4[i]);
            d[i].x.load(px, ot[i]);
            d[i].res.load(pr, ot[i]);
        }
    };
    auto process = [&](int row, const LnRow<T> (&cur)[NV], float mu, float rs) __attribute__((always_inline)) {
        // vectors past the row hold zeros: they add nothing to the sums
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xh = (cur[i].x[j] - mu) * rs;
                const float gd = cur[i].du[j] * gg[i][j];
                s1 += gd;
                s2 += gd * xh;
                adg[i][j] += cur[i].du[j] * xh;
                adb[i][j] += cur[i].du[j];
            }
        // both row sums in one exchange; the two LDS buffers alternate by
        // row, so a buffer is rewritten only after every thread has passed
        // the next row's barrier
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        float(*rb)[NWV] = red[row & 1];
        if ((threadIdx.x & 63) == 0) {
            rb[0][threadIdx.x >> 6] = s1;
            rb[1][threadIdx.x >> 6] = s2;
        }
        __syncthreads();
        float m1 = rb[0][0], m2 = rb[1][0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            m1 += rb[0][w];
            m2 += rb[1][w];
        }
        m1 /= (float)h;
        m2 /= (float)h;
        const __amdgpu_buffer_rsrc_t pdx = make_rsrc(dx + (size_t)row * h, row_t);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xh = (cur[i].x[j] - mu) * rs;
                o[j] = cur[i].res[j] + rs * (cur[i].du[j] * gg[i][j] - m1 - xh * m2);
            }
            store8_buf(pdx, ot[i], o, (T *)nullptr);
        }
    };
    // two register sets alternate by row while the register budget allows
    // (6 vectors per thread in bf16, 5 in fp32 at one wave per SIMD; half as
    // many at two); every load is issued, so the number in flight is the
    // same on every path through the loop
    constexpr bool kPrefetch = NV * (TPB / 256) <= (sizeof(T) == 2 ? 6 : 5);
    if constexpr (kPrefetch) {
        LnRow<T> ra[NV], rb[NV];
        float mua, rsa, mub, rsb;
        load_row(r0, ra, mua, rsa);
        // the scheduling barriers keep each row's loads ahead of the
        // previous row's arithmetic (the scheduler would otherwise sink them
        // to shorten their registers' live ranges)
        for (int row = r0; row < r1; row += 2) {
            load_row(row + 1, rb, mub, rsb);
            __builtin_amdgcn_sched_barrier(0);
            process(row, ra, mua, rsa);
            if (row + 1 >= r1) break;
            load_row(row + 2, ra, mua, rsa);
            __builtin_amdgcn_sched_barrier(0);
            process(row + 1, rb, mub, rsb);
        }
    } else {
        LnRow<T> ra[NV];
        for (int row = r0; row < r1; ++row) {
            float mu, rs;
            load_row(row, ra, mu, rs);
            process(row, ra, mu, rs);
        }
    }
    float *pb = partials + (size_t)blockIdx.x * 2 * h;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = threadIdx.x + i * TPB;
        if (c < nv) {
            store8(pb + c * 8, adg[i]);
            store8(pb + h + c * 8, adb[i]);
        }
    }
}

// Rows of at most 2048 columns: the workgroup's rows go to its four waves in
// turn (rows r0 + w, r0 + w + 4, ...), one wave per row with the row sums by
// wave reduction (no barrier per row) and, for up to 1024 columns, the
// wave's next row in flight.  Each wave keeps its own parameter-gradient
// sums; the four waves add them in wave order through LDS at the end, into
// the same per-workgroup partials as ln_bwd_kernel.
constexpr int kLnWaveMaxH = 2048;
template <typename T, int NVW>
__global__ __launch_bounds__(256) void ln_bwd_wave_kernel(int rows, int h, int rpb, const float *__restrict__ du,
                                                          const T *__restrict__ resid, const T *__restrict__ x,
                                                          const T *__restrict__ g, const float *__restrict__ mean,
                                                          const float *__restrict__ rstd, T *__restrict__ dx,
                                                          float *__restrict__ partials) {
    __shared__ float sums[2 * kLnWaveMaxH];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nv = h >> 3;
    const int r0 = blockIdx.x * rpb, r1 = min(rows, r0 + rpb);
    const uint32_t row_f32 = (uint32_t)h * 4, row_t = (uint32_t)h * sizeof(T);
    uint32_t o4[NVW], ot[NVW];
    float gg[NVW][8], adg[NVW][8], adb[NVW][8];
    {
        const __amdgpu_buffer_rsrc_t pg = make_rsrc(g, row_t);
#pragma unroll
        for (int i = 0; i < NVW; ++i) {
            const int c = lane + i * 64;
            o4[i] = c < nv ? (uint32_t)c * 32 : kOOB;
            ot[i] = c < nv ? (uint32_t)c * (8 * sizeof(T)) : kOOB;
            Raw8<T> gr;
            gr.load(pg, ot[i]);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                gg[i][j] = gr[j];
                adg[i][j] = adb[i][j] = 0.f;
            }
        }
    }
    // rows past the workgroup's range read zeros (descriptors of length zero)
    auto load_row = [&](int row, LnRow<T> (&d)[NVW], float &mu, float &rs) __attribute__((always_inline)) {
        const bool valid = row < r1;
        const int rr = valid ? row : min(r0, rows - 1);  // a workgroup past the last row still reads in bounds
        mu = mean[rr];
        rs = rstd[rr];
        const size_t base = (size_t)rr * h;
        const __amdgpu_buffer_rsrc_t pdu = make_rsrc(du + base, valid ? row_f32 : 0u);
        const __amdgpu_buffer_rsrc_t px = make_rsrc(x + base, valid ? row_t : 0u);
        const __amdgpu_buffer_rsrc_t pr = make_rsrc(resid + base, valid ? row_t : 0u);
#pragma unroll
        for (int i = 0; i < NVW; ++i) {
            d[i].du.load(pdu, o4[i]);
            d[i].x.load(px, ot[i]);
            d[i].res.load(pr, ot[i]);
        }
    };
    auto process = [&](int row, const LnRow<T> (&cur)[NVW], float mu, float rs) __attribute__((always_inline)) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NVW; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xh = (cur[i].x[j] - mu) * rs;
                const float gd = cur[i].du[j] * gg[i][j];
                s1 += gd;
                s2 += gd * xh;
                adg[i][j] += cur[i].du[j] * xh;
                adb[i][j] += cur[i].du[j];
            }
        const float m1 = wave_sum(s1) / (float)h, m2 = wave_sum(s2) / (float)h;
        const __amdgpu_buffer_rsrc_t pdx = make_rsrc(dx + (size_t)row * h, row_t);
#pragma unroll
        for (int i = 0; i < NVW; ++i) {
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xh = (cur[i].x[j] - mu) * rs;
                o[j] = cur[i].res[j] + rs * (cur[i].du[j] * gg[i][j] - m1 - xh * m2);
            }
            store8_buf(pdx, ot[i], o, (T *)nullptr);
        }
    };
    if constexpr (NVW <= 2) {
        LnRow<T> ra[NVW], rb[NVW];
        float mua, rsa, mub, rsb;
        load_row(r0 + w, ra, mua, rsa);
        for (int row = r0 + w; row < r1; row += 8) {
            load_row(row + 4, rb, mub, rsb);
            __builtin_amdgcn_sched_barrier(0);
            process(row, ra, mua, rsa);
            if (row + 4 >= r1) break;
            load_row(row + 8, ra, mua, rsa);
            __builtin_amdgcn_sched_barrier(0);
            process(row + 4, rb, mub, rsb);
        }
    } else {
        LnRow<T> ra[NVW];
        for (int row = r0 + w; row < r1; row += 4) {
            float mu, rs;
            load_row(row, ra, mu, rs);
            process(row, ra, mu, rs);
        }
    }
    // the waves' sums added in wave order
    for (int k = 0; k < 4; ++k) {
        if (w == k) {
#pragma unroll
            for (int i = 0; i < NVW; ++i) {
                const int c = lane + i * 64;
                if (c < nv) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        sums[c * 8 + j] = k == 0 ? adg[i][j] : sums[c * 8 + j] + adg[i][j];
                        sums[h + c * 8 + j] = k == 0 ? adb[i][j] : sums[h + c * 8 + j] + adb[i][j];
                    }
                }
            }
        }
        __syncthreads();
    }
    float *pb = partials + (size_t)blockIdx.x * 2 * h;
    for (int c = threadIdx.x; c < 2 * h; c += 256) pb[c] = sums[c];
}

// out[c] (+)= sum over blocks of partials[blk][c], for c < n; partial rows are
// `stride` floats apart.  A workgroup owns 32 columns; its 8 row groups each
// sum every 8th partial row, and the 8 sums are added in a fixed order.
// Columns c < n0 go to out0[c], columns n0 <= c < n to out1[c - n0] (two
// vectors reduced together).  Up to two such segments (independent partial
// arrays) share one launch: workgroups [0, seg[0].groups) take the first.
constexpr int kRedCols = 32, kRedGroups = kThreads / kRedCols;
struct RedSeg {
    int nblk, n, n0, groups;
    int64_t stride;
    const float *partials;
    float *out0, *out1;
};
__global__ __launch_bounds__(kThreads) void reduce_blocks_kernel(RedSeg s0, RedSeg s1, int accumulate) {
    __shared__ float part[kRedGroups][kRedCols];
    const bool second = (int)blockIdx.x >= s0.groups;
    const RedSeg &sg = second ? s1 : s0;
    const int gx = second ? (int)blockIdx.x - s0.groups : (int)blockIdx.x;
    const int cx = threadIdx.x % kRedCols, gy = threadIdx.x / kRedCols;
    const int c = gx * kRedCols + cx;
    const int nblk = sg.nblk, n = sg.n;
    const int64_t stride = sg.stride;
    const float *partials = sg.partials;
    float s = 0.f;
    if (c < n) {
        int k = gy;
        // four partial rows' loads in flight, added in row order
        for (; k + 3 * kRedGroups < nblk; k += 4 * kRedGroups) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = partials[(size_t)(k + u * kRedGroups) * stride + c];
#pragma unroll
            for (int u = 0; u < 4; ++u) s += v[u];
        }
        for (; k < nblk; k += kRedGroups) s += partials[(size_t)k * stride + c];
    }
    part[gy][cx] = s;
    __syncthreads();
    if (gy == 0 && c < n) {
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < kRedGroups; ++k) t += part[k][cx];
        float *o = c < sg.n0 ? sg.out0 + c : sg.out1 + (c - sg.n0);
        *o = accumulate ? *o + t : t;
    }
}

// Per-chunk column sums of one or two matrices with the same rows:
// partials[chunk][c] = sum of the chunk's rows of column c of a1 (c < n1) or
// of column c - n1 of a2 (n1 <= c < n1 + n2), over the rows of chunk
// `blockIdx.y`; each thread owns 8 columns of one matrix.
template <typename T>
__global__ __launch_bounds__(kThreads) void colsum_kernel(int rows, int n1, const T *__restrict__ a1, int64_t lda1,
                                                          int n2, const T *__restrict__ a2, int64_t lda2, int rpc,
                                                          float *__restrict__ partials) {
    const int c8 = (blockIdx.x * kThreads + threadIdx.x) * 8;
    if (c8 >= n1 + n2) return;
    const bool first = c8 < n1;
    const T *a = first ? a1 + c8 : a2 + (c8 - n1);
    const int64_t lda = first ? lda1 : lda2;
    const int r0 = blockIdx.y * rpc, r1 = min(rows, r0 + rpc);
    float s[8] = {};
    int r = r0;
    // four rows' loads in flight, added in row order
    for (; r + 4 <= r1; r += 4) {
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) load8(a + (size_t)(r + u) * lda, v[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) s[j] += v[u][j];
    }
    for (; r < r1; ++r) {
        float v[8];
        load8(a + (size_t)r * lda, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] += v[j];
    }
    store8(partials + (size_t)blockIdx.y * (n1 + n2) + c8, s);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(int64_t n8, int h, const T *__restrict__ resid,
                                                           const float *__restrict__ red, const T *__restrict__ bias,
                                                           T *__restrict__ out) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
        int64_t e = i * 8;
        int c = (int)(e % h);
        float a[8], r[8], b[8];
        load8(resid + e, a);
        load8(red + e, r);
        load8(bias + c, b);
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] += r[j] + b[j];
        store8(out + e, a);
    }
}

// Workgroups of the backward: 256 for long row ranges; a short one (a slice
// of up to 255 rows) gives each workgroup two rows, which halves the
// parameter-gradient partial sums (2 h floats a workgroup) against one row
// a workgroup (the 175B per-slice schedule 0.6% faster; four rows a
// workgroup 0.8% slower).
int ln_bwd_blocks(int rows) { return rows < 256 ? (rows + 1) / 2 : 256; }
// chunks of 32 rows, at most 256 (long token ranges keep short serial sums)
int colsum_chunks(int rows) {
    int c = (rows + 31) / 32;
    return c < 256 ? (c < 1 ? 1 : c) : 256;
}

// Cube-partition FFN elementwise steps, 8 columns per thread: Z = z_sum +
// bias[c] stored bf16 and H = GELU(Z) (of the fp32 Z); dZ = dH * GELU'(Z)
// with Z the stored bf16 values.
__global__ __launch_bounds__(kThreads) void bias_gelu_kernel(int64_t n8, int n, const float *__restrict__ zs,
                                                             const bf16 *__restrict__ bias, bf16 *__restrict__ z,
                                                             bf16 *__restrict__ h) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
        const int64_t e = i * 8;
        const int c = (int)(e % n);
        float v[8], b[8], g[8];
        load8(zs + e, v);
        load8(bias + c, b);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[j] += b[j];
            g[j] = gelu_f(v[j]);
        }
        store8(z + e, v);
        store8(h + e, g);
    }
}

__global__ __launch_bounds__(kThreads) void gelu_backward_kernel(int64_t n8, const float *__restrict__ dh,
                                                                 const bf16 *__restrict__ z, bf16 *__restrict__ dz) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n8; i += (int64_t)gridDim.x * kThreads) {
        const int64_t e = i * 8;
        float d[8], zz[8];
        load8(dh + e, d);
        load8(z + e, zz);
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] *= gelu_grad_f(zz[j]);
        store8(dz + e, d);
    }
}

}  // namespace

size_t layernorm_bwd_partials_floats(int rows, int h) { return (size_t)ln_bwd_blocks(rows) * 2 * h; }
size_t colsum_partials_floats(int rows, int n) { return (size_t)colsum_chunks(rows) * n; }

template <typename T, int NV>
static void launch_ln_fwd(int rows, int h, float eps, const void *x, const void *g, const void *b, void *u,
                          float *mean, float *rstd, hipStream_t st) {
    // fewer rows than a round of the chip (a slice): gamma and beta loaded with
    // the row (the per-slice LayerNorm forward 9.5 -> 7.2 us on 128 x 12288,
    // the schedule 0.9% faster); with many rows other rows' loads cover that
    // round trip and the registers are worth more (2048 rows: 51 -> 62 us)
    if (rows < 256)
        hipLaunchKernelGGL((ln_fwd_kernel<T, NV, true>), dim3(rows), dim3(kThreads), 0, st, h, eps, (const T *)x,
                           (const T *)g, (const T *)b, (T *)u, mean, rstd);
    else
        hipLaunchKernelGGL((ln_fwd_kernel<T, NV>), dim3(rows), dim3(kThreads), 0, st, h, eps, (const T *)x,
                           (const T *)g, (const T *)b, (T *)u, mean, rstd);
}

template <typename T, int NVW>
static void launch_ln_fwd_wave(int rows, int h, float eps, const void *x, const void *g, const void *b, void *u,
                               float *mean, float *rstd, hipStream_t st) {
    hipLaunchKernelGGL((ln_fwd_wave_kernel<T, NVW>), dim3((rows + 3) / 4), dim3(256), 0, st, rows, h, eps,
                       (const T *)x, (const T *)g, (const T *)b, (T *)u, mean, rstd);
}

template <typename T>
static void dispatch_ln_fwd(int rows, int h, float eps, const void *x, const void *g, const void *b, void *u,
                            float *mean, float *rstd, hipStream_t st) {
    if (h <= kLnWaveMaxH) {
        switch (((h >> 3) + 63) / 64) {
        case 1: launch_ln_fwd_wave<T, 1>(rows, h, eps, x, g, b, u, mean, rstd, st); return;
        case 2: launch_ln_fwd_wave<T, 2>(rows, h, eps, x, g, b, u, mean, rstd, st); return;
        case 3: launch_ln_fwd_wave<T, 3>(rows, h, eps, x, g, b, u, mean, rstd, st); return;
        default: launch_ln_fwd_wave<T, 4>(rows, h, eps, x, g, b, u, mean, rstd, st); return;
        }
    }
    static_assert(kMaxVec == 8, "the cases below cover 1..kMaxVec vectors per thread");
    switch (((h >> 3) + kThreads - 1) / kThreads) {  // vectors per thread, 1..kMaxVec
    case 1: launch_ln_fwd<T, 1>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    case 2: launch_ln_fwd<T, 2>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    case 3: launch_ln_fwd<T, 3>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    case 4: launch_ln_fwd<T, 4>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    case 5: launch_ln_fwd<T, 5>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    case 6: launch_ln_fwd<T, 6>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    case 7: launch_ln_fwd<T, 7>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    default: launch_ln_fwd<T, 8>(rows, h, eps, x, g, b, u, mean, rstd, st); break;
    }
}

hipError_t layernorm_fwd(DType dt, int rows, int h, float eps, const void *x, const void *g, const void *b,
                         void *u, float *mean, float *rstd, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const int es = dt == DType::BF16 ? 2 : 4;
    TraceScope ts(st, dt == DType::BF16 ? "ln_fwd_bf16" : "ln_fwd_f32", 0.0,
                  (double)rows * h * 2 * es + 8.0 * rows + 2.0 * h * es);
    if (dt == DType::BF16)
        dispatch_ln_fwd<bf16>(rows, h, eps, x, g, b, u, mean, rstd, st);
    else
        dispatch_ln_fwd<float>(rows, h, eps, x, g, b, u, mean, rstd, st);
    return hipGetLastError();
}

template <typename T, int NV, int TPB>
static void launch_ln_bwd(int nblk, int rows, int h, int rpb, const float *du, const void *resid, const void *x,
                          const void *g, const float *mean, const float *rstd, void *dx, float *partials,
                          hipStream_t st) {
    hipLaunchKernelGGL((ln_bwd_kernel<T, NV, TPB>), dim3(nblk), dim3(TPB), 0, st, rows, h, rpb, du,
                       (const T *)resid, (const T *)x, (const T *)g, mean, rstd, (T *)dx, partials);
}

template <typename T, int NVW>
static void launch_ln_bwd_wave(int nblk, int rows, int h, int rpb, const float *du, const void *resid, const void *x,
                               const void *g, const float *mean, const float *rstd, void *dx, float *partials,
                               hipStream_t st) {
    hipLaunchKernelGGL((ln_bwd_wave_kernel<T, NVW>), dim3(nblk), dim3(256), 0, st, rows, h, rpb, du, (const T *)resid,
                       (const T *)x, (const T *)g, mean, rstd, (T *)dx, partials);
}

template <typename T>
static void dispatch_ln_bwd(int nblk, int rows, int h, int rpb, const float *du, const void *resid, const void *x,
                            const void *g, const float *mean, const float *rstd, void *dx, float *partials,
                            hipStream_t st) {
    const int nv = h >> 3;
    if (h <= kLnWaveMaxH) {
        switch ((nv + 63) / 64) {
        case 1: launch_ln_bwd_wave<T, 1>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); return;
        case 2: launch_ln_bwd_wave<T, 2>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); return;
        case 3: launch_ln_bwd_wave<T, 3>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); return;
        default: launch_ln_bwd_wave<T, 4>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); return;
        }
    }
    // bf16 rows of 6145..12288 columns: 512 threads of 2 or 3 vectors each,
    // two waves per SIMD with the next row prefetched
    if constexpr (sizeof(T) == 2) {
        if (nv > 3 * kThreads && nv <= 2 * 512) {
            launch_ln_bwd<T, 2, 512>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st);
            return;
        }
        if (nv > 2 * 512 && nv <= 3 * 512) {
            launch_ln_bwd<T, 3, 512>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st);
            return;
        }
    }
    const int nvt = (nv + kThreads - 1) / kThreads;  // vectors per thread, 1..kMaxVec
    switch (nvt) {
    case 1: launch_ln_bwd<T, 1, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    case 2: launch_ln_bwd<T, 2, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    case 3: launch_ln_bwd<T, 3, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    case 4: launch_ln_bwd<T, 4, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    case 5: launch_ln_bwd<T, 5, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    case 6: launch_ln_bwd<T, 6, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    case 7: launch_ln_bwd<T, 7, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    default: launch_ln_bwd<T, 8, kThreads>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st); break;
    }
}

hipError_t layernorm_bwd_rows(DType dt, int rows, int h, const float *du, const void *resid, const void *x,
                              const void *g, const float *mean, const float *rstd, void *dx, float *partials,
                              hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    const int nblk = ln_bwd_blocks(rows), rpb = (rows + nblk - 1) / nblk;
    const int es = dt == DType::BF16 ? 2 : 4;
    TraceScope ts(st, dt == DType::BF16 ? "ln_bwd_bf16" : "ln_bwd_f32", 0.0,
                  (double)rows * h * (4 + 3 * es) + 8.0 * rows + (double)nblk * 2 * h * 4);
    if (dt == DType::BF16)
        dispatch_ln_bwd<bf16>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st);
    else
        dispatch_ln_bwd<float>(nblk, rows, h, rpb, du, resid, x, g, mean, rstd, dx, partials, st);
    return hipGetLastError();
}

hipError_t colsum_rows(DType dt, int rows, int n1, const void *a1, int64_t lda1, int n2, const void *a2, int64_t lda2,
                       float *partials, hipStream_t st) {
    if (rows <= 0 || n1 + n2 <= 0) return hipSuccess;
    const int nch = colsum_chunks(rows), rpc = (rows + nch - 1) / nch;
    const int n = n1 + n2;
    dim3 grid((n / 8 + kThreads - 1) / kThreads, nch);
    const int es = dt == DType::BF16 ? 2 : 4;
    TraceScope ts(st, dt == DType::BF16 ? "colsum_bf16" : "colsum_f32", (double)rows * n,
                  (double)rows * n * es + (double)nch * n * 4);
    if (dt == DType::BF16)
        hipLaunchKernelGGL(colsum_kernel<bf16>, grid, dim3(kThreads), 0, st, rows, n1, (const bf16 *)a1, lda1, n2,
                           (const bf16 *)a2, lda2, rpc, partials);
    else
        hipLaunchKernelGGL(colsum_kernel<float>, grid, dim3(kThreads), 0, st, rows, n1, (const float *)a1, lda1, n2,
                           (const float *)a2, lda2, rpc, partials);
    return hipGetLastError();
}

ReduceSpec ln_bwd_reduce_spec(int rows, int h, const float *partials, float *dg, float *db) {
    return ReduceSpec{ln_bwd_blocks(rows), 2 * h, h, (int64_t)2 * h, partials, dg, db};
}

ReduceSpec colsum_reduce_spec(int rows, int n1, int n2, const float *partials, float *out1, float *out2) {
    return ReduceSpec{colsum_chunks(rows), n1 + n2, n1, (int64_t)(n1 + n2), partials, out1, out2};
}

hipError_t reduce_partials(const ReduceSpec *a, const ReduceSpec *b, bool accumulate, hipStream_t st) {
    auto seg = [](const ReduceSpec *r) {
        RedSeg g{};
        if (r && r->n > 0 && r->nblk > 0) {
            g.nblk = r->nblk; g.n = r->n; g.n0 = r->n0; g.stride = r->stride; g.partials = r->partials;
            g.out0 = r->out0; g.out1 = r->out1; g.groups = (r->n + kRedCols - 1) / kRedCols;
        }
        return g;
    };
    RedSeg s0 = seg(a), s1 = seg(b);
    if (s0.groups == 0) std::swap(s0, s1);
    const int groups = s0.groups + s1.groups;
    if (groups == 0) return hipSuccess;
    TraceScope ts(st, "block_reduce", 0.0,
                  ((double)s0.nblk * s0.n + (double)s1.nblk * s1.n) * 4 + 8.0 * (s0.n + s1.n) * (accumulate ? 2 : 1));
    hipLaunchKernelGGL(reduce_blocks_kernel, dim3(groups), dim3(kThreads), 0, st, s0, s1, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t layernorm_bwd(DType dt, int rows, int h, const float *du, const void *resid, const void *x,
                         const void *g, const float *mean, const float *rstd, void *dx, float *dg, float *db,
                         bool accumulate, float *partials, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    hipError_t e = layernorm_bwd_rows(dt, rows, h, du, resid, x, g, mean, rstd, dx, partials, st);
    if (e != hipSuccess) return e;
    // dgamma and dbeta: the partial rows are [2][h] per block, one launch
    // reduces both halves
    const ReduceSpec r = ln_bwd_reduce_spec(rows, h, partials, dg, db);
    return reduce_partials(&r, nullptr, accumulate, st);
}

hipError_t colsum(DType dt, int rows, int n, const void *a, int64_t lda, float *out, bool accumulate,
                  float *partials, hipStream_t st) {
    if (rows <= 0 || n <= 0) return hipSuccess;
    hipError_t e = colsum_rows(dt, rows, n, a, lda, 0, nullptr, 0, partials, st);
    if (e != hipSuccess) return e;
    const ReduceSpec r = colsum_reduce_spec(rows, n, 0, partials, out, out);
    return reduce_partials(&r, nullptr, accumulate, st);
}

hipError_t residual_combine(DType dt, int64_t rows, int h, const void *resid, const float *reduced,
                            const void *bias, void *out, hipStream_t st) {
    int64_t n8 = rows * h / 8;
    if (n8 <= 0) return hipSuccess;
    int64_t blocks = (n8 + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    const int es = dt == DType::BF16 ? 2 : 4;
    TraceScope ts(st, dt == DType::BF16 ? "combine_bf16" : "combine_f32", 2.0 * rows * h,
                  (double)rows * h * (2 * es + 4) + (double)h * es);
    if (dt == DType::BF16)
        hipLaunchKernelGGL(combine_kernel<bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, st, n8, h,
                           (const bf16 *)resid, reduced, (const bf16 *)bias, (bf16 *)out);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, st, n8, h,
                           (const float *)resid, reduced, (const float *)bias, (float *)out);
    return hipGetLastError();
}

hipError_t bias_gelu(int64_t rows, int n, const float *z_sum, const void *bias, void *z, void *h, hipStream_t st) {
    const int64_t n8 = rows * n / 8;
    if (n8 <= 0) return hipSuccess;
    TraceScope ts(st, "cube_bias_gelu", 0.0, (double)rows * n * (4 + 2 + 2) + 2.0 * n);
    const int64_t blocks = std::min<int64_t>((n8 + kThreads - 1) / kThreads, 8192);
    hipLaunchKernelGGL(bias_gelu_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, n8, n, z_sum,
                       (const bf16 *)bias, (bf16 *)z, (bf16 *)h);
    return hipGetLastError();
}

hipError_t gelu_backward(int64_t rows, int n, const float *dh, const void *z, void *dz, hipStream_t st) {
    const int64_t n8 = rows * n / 8;
    if (n8 <= 0) return hipSuccess;
    TraceScope ts(st, "cube_gelu_bwd", 0.0, (double)rows * n * (4 + 2 + 2));
    const int64_t blocks = std::min<int64_t>((n8 + kThreads - 1) / kThreads, 8192);
    hipLaunchKernelGGL(gelu_backward_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, n8, dh, (const bf16 *)z,
                       (bf16 *)dz);
    return hipGetLastError();
}

}  // namespace tpk
