// Shared device/host helpers of the GPT-2 step library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define DEVI __device__ __forceinline__

// ---- scalar conversions -------------------------------------------------
DEVI float to_f32(float x) { return x; }
DEVI float to_f32(bf16 x) { return (float)x; }
template <typename T> DEVI T from_f32(float x);
template <> DEVI float from_f32<float>(float x) { return x; }
template <> DEVI bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

// ---- 16-byte vectors of activations --------------------------------------
// VecN<T>::N elements of T in 16 bytes, loaded/stored with one dwordx4.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    float v[4];
};
template <> struct Vec16<bf16> {
    static constexpr int N = 8;
    bf16 v[8];
};

template <typename T> DEVI Vec16<T> ld16(const T* p) {
    Vec16<T> r;
    *reinterpret_cast<uint4*>(&r) = *reinterpret_cast<const uint4*>(p);
    return r;
}
template <typename T> DEVI void st16(T* p, const Vec16<T>& r) {
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(&r);
}

// ---- wavefront reductions (64 lanes) --------------------------------------
DEVI float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
DEVI float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// tanh(x) = 1 - 2 / (exp(2x) + 1): the hardware exp and reciprocal, exact to
// a few fp32 ulps, and saturating cleanly to +-1 (exp overflows to inf or
// underflows to 0; the denominator never falls below 1)
DEVI float tanh_fast(float x) { return 1.f - __fdividef(2.f, __expf(2.f * x) + 1.f); }

// GELU, tanh approximation: 0.5 u (1 + tanh(k (u + 0.044715 u^3))), k = sqrt(2/pi)
#define GELU_K 0.7978845608028654f
DEVI float gelu_f(float u) {
    float t = tanh_fast(GELU_K * (u + 0.044715f * u * u * u));
    return 0.5f * u * (1.0f + t);
}
DEVI float gelu_grad_f(float u) {
    float t = tanh_fast(GELU_K * (u + 0.044715f * u * u * u));
    return 0.5f * (1.0f + t) + 0.5f * u * (1.0f - t * t) * GELU_K * (1.0f + 3.0f * 0.044715f * u * u);
}

static inline unsigned cdiv(size_t a, size_t b) { return (unsigned)((a + b - 1) / b); }
