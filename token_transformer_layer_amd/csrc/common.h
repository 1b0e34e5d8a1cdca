// Internal helpers shared by the gfx950 kernels: element types, bf16
// conversion, buffer-resource loads and small fast-division helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Offset that lies outside every buffer the library addresses (all buffers
// are checked on the host to be smaller than 2^31 bytes): a raw buffer load
// at this offset returns zeros, which is how tile edges are masked.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    // gfx9 buffer descriptor: raw (stride 0) addressing with bounds checking
    // against num_records = bytes.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Direct-to-LDS buffer load: each lane's 16 bytes land at lds_base + 16 *
// lane (lds_base must be the same for the whole wave: it goes to M0); an
// out-of-bounds offset writes zeros.
//
// UNTRACKED issues it as inline assembly, out of sight of the compiler's
// wait insertion.  That pass treats every LDS read after a direct-to-LDS
// load it can see as possibly reading what the load writes (it cannot tell
// two stages of one LDS buffer apart) and waits for all such loads in
// flight (s_waitcnt vmcnt(0)) before the read, so a pipeline that reads
// stage s while stage s + 1 loads waits for stage s + 1 at every step.
// Hidden from it, the loads are waited for only where the kernel says: a
// caller of the untracked form waits on vmcnt for its own loads and then
// synchronises the workgroup before any wave reads what they wrote, and
// drains them before it ends.  (The compiler's own waits for other loads
// only become more conservative, as it does not count these.)  The price:
// a volatile asm statement also fences the scheduler, which cannot move LDS
// reads or other memory operations across it, so the GEMM hand-over reads
// the next tile's first fragments before it issues the refill.  Measured in
// the layer step, the GEMM kernels take the untracked form (weight
// gradients 7% faster, input-gradient products 3-16%), and the attention
// kernels, 1-3% slower with it, keep the tracked builtin.
typedef __attribute__((address_space(3))) void lds_void;
template <bool UNTRACKED = false>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, char *lds_base, uint32_t voff) {
    if constexpr (UNTRACKED) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)lds_base);
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(r)
                     : "memory", "m0");
    } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 16, voff, 0, 0, 0);
    }
}

// The untracked load with the LDS destination given as a wave-uniform LDS
// byte address (kept in scalar registers by its caller).
__device__ __forceinline__ void lds_dma16_at(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r)
                 : "memory", "m0");
}

// LDS byte address of a pointer into shared memory, as a wave-uniform value.
__device__ __forceinline__ uint32_t lds_addr_of(char *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)p);
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt with only the LDS/scalar-memory counter drained (vmcnt and
// expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8)); }

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte pieces addressed by lanes i/4 + 4j (j = 0..3), in j
// order; with lane L addressing row r0 + L/4, columns c0 + 4(L%4)..+3 of a
// row-major bf16 tile, lane i gets rows r0..r0+3 of column c0 + i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// bf16 halves of a 32-bit word
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// two values rounded to bf16 (nearest, ties to even) in one word: one
// v_cvt_pk_bf16_f32
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 8 consecutive elements (16 bytes of bf16 or 32 bytes of fp32; the address
// is aligned to that size) converted to and from fp32.
__device__ __forceinline__ void load8(const float *p, float o[8]) {
    float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16 *p, float o[8]) {
    u32x4 w = *(const u32x4 *)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf_lo(w[i]); o[2 * i + 1] = bf_hi(w[i]); }
}
__device__ __forceinline__ void store8(float *p, const float v[8]) {
    *(float4 *)p = float4{v[0], v[1], v[2], v[3]};
    *(float4 *)(p + 4) = float4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(bf16 *p, const float v[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf2(v[2 * i], v[2 * i + 1]);
    *(u32x4 *)p = w;
}

// Unsigned division by a runtime constant d >= 1 (n < 2^31): q = n / d via a
// multiply-high with a magic number prepared on the host.
struct FastDiv {
    uint32_t d, magic, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1u << s) < d) ++s;
    f.shift = s;
    // magic = floor(2^32 * (2^s - d) / d) + 1, valid for n, d < 2^31
    f.magic = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << s) - d)) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    uint32_t t = __umulhi(n, f.magic);
    return (t + n) >> f.shift;
}

// GELU as z * Phi(z) with Phi(z) = (1 + erf(z / sqrt 2)) / 2, and its
// derivative Phi(z) + z phi(z).
__device__ __forceinline__ float gelu_f(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_grad_f(float z) {
    float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
    float pdf = 0.39894228040143268f * __expf(-0.5f * z * z);
    return cdf + z * pdf;
}

// GELU and its derivative together (they share Phi(z)).
__device__ __forceinline__ void gelu_and_grad(float z, float &g, float &gp) {
    const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * __expf(-0.5f * z * z);
    g = z * cdf;
    gp = cdf + z * pdf;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace tpk
