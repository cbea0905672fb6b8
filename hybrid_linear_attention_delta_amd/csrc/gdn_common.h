// gdn_common.h -- device helpers shared by the gated delta-rule kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kNormEps = 1e-6f;  // q/k L2 normalisation: x / sqrt(sum x^2 + eps)

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) {           // inf / nan: keep, quiet the nan
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Element loads/stores for the two storage types of q, k, v, o.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
    // four consecutive elements starting at p[i] (i multiple of 4)
    static __device__ __forceinline__ f32x4 load4(const float* p, int64_t i)
    {
        return *reinterpret_cast<const f32x4*>(p + i);
    }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16_bits(x); }
    static __device__ __forceinline__ f32x4 load4(const uint16_t* p, int64_t i)
    {
        u16x4 b = *reinterpret_cast<const u16x4*>(p + i);
        f32x4 r;
        r.x = bf16_bits_to_f32(b.x);
        r.y = bf16_bits_to_f32(b.y);
        r.z = bf16_bits_to_f32(b.z);
        r.w = bf16_bits_to_f32(b.w);
        return r;
    }
};

// Butterfly sum over aligned groups of `W` lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

}  // namespace gdn
