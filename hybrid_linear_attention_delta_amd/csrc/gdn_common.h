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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  Widening is exact; narrowing is the gfx950 hardware convert
// (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two values -> packed bf16 pair (first value in the low half)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// hi = bf16(x), lo = bf16(x - hi) for a pair: hi + lo carries ~16 significant bits
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo)
{
    hi = pack_bf16x2(a, b);
    lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// Element loads/stores for the two storage types of q, k, v, o.
template <typename T> struct Elem;
template <> struct Elem<float> {
    typedef f32x4 Raw4;  // four stored elements, before widening
    static __device__ __forceinline__ Raw4 raw4(const float* p, int64_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
    static __device__ __forceinline__ f32x4 widen4(Raw4 r) { return r; }
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
    // four consecutive elements starting at p[i] (i multiple of 4)
    static __device__ __forceinline__ f32x4 load4(const float* p, int64_t i)
    {
        return *reinterpret_cast<const f32x4*>(p + i);
    }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
    typedef u16x4 Raw4;
    static __device__ __forceinline__ Raw4 raw4(const uint16_t* p, int64_t i) { return *reinterpret_cast<const u16x4*>(p + i); }
    static __device__ __forceinline__ f32x4 widen4(Raw4 b)
    {
        return f32x4{bf16_bits_to_f32(b.x), bf16_bits_to_f32(b.y), bf16_bits_to_f32(b.z), bf16_bits_to_f32(b.w)};
    }
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

// silu(u) = u / (1 + e^{-u}) on the hardware exp2 and reciprocal (about 1 ulp
// each): the IEEE expf and divide cost more ALU time than the streaming
// kernels that apply it can hide.  Large |u| reach the exact limits
// (e^{-u} = inf gives u * 0).
__device__ __forceinline__ float fast_silu(float u)
{
    return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * u));
}

// ---- front end (App. A.3: the short convolution before the recurrence and the
//      gates of the paragraph after Eq. 21).  Shared by the standalone front-end
//      kernels and the prefill that folds the front end into its row loads, so
//      that both round every value identically.

// silu of the 4-tap causal convolution of one channel: taps oldest first,
// x0 .. x3 the inputs of tokens t-3 .. t (explicit FMA order).
__device__ __forceinline__ float conv4_silu(const float (&w)[4], float x0, float x1, float x2, float x3)
{
    return fast_silu(fmaf(w[3], x3, fmaf(w[2], x2, fmaf(w[1], x1, w[0] * x0))));
}

// log(1 + e^u) without overflow: max(u, 0) + log1p(e^{-|u|})
__device__ __forceinline__ float softplus(float u) { return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u))); }

// g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)
__device__ __forceinline__ float gate_g(float a, float A_log, float dt_bias)
{
    return -expf(A_log) * softplus(a + dt_bias);
}
__device__ __forceinline__ float gate_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

}  // namespace gdn
