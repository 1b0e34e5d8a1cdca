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

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// bf16 halves of a 32-bit word
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    bf16 a = (bf16)lo, b = (bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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
