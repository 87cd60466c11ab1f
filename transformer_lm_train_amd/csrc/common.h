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

// ---- streaming (non-temporal) accesses -------------------------------------
// For arrays read or written once per pass and far larger than the caches
// (optimizer state and gradients in the update, logits in the loss): the
// accesses carry the non-temporal hint, so they neither keep nor evict other
// lines.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef bf16 bf16x4_nt __attribute__((ext_vector_type(4)));
DEVI float4 ld_stream(const float* p, size_t i) {  // 16 bytes at p + 4 i
    const f32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p) + i);
    return make_float4(t.x, t.y, t.z, t.w);
}
DEVI void st_stream(float* p, size_t i, const float4& q) {
    const f32x4_nt t = {q.x, q.y, q.z, q.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4_nt*>(p) + i);
}
DEVI bf16x4_nt ld_stream(const bf16* p, size_t i) {  // 8 bytes at p + 4 i
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x4_nt*>(p) + i);
}
DEVI void st_stream(bf16* p, size_t i, const bf16x4_nt& q) {
    __builtin_nontemporal_store(q, reinterpret_cast<bf16x4_nt*>(p) + i);
}
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
template <typename T> DEVI Vec16<T> ld16_stream(const T* p) {
    Vec16<T> r;
    *reinterpret_cast<u32x4_nt*>(&r) = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return r;
}
template <typename T> DEVI void st16_stream(T* p, const Vec16<T>& r) {
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_nt*>(&r), reinterpret_cast<u32x4_nt*>(p));
}

// ---- wavefront reductions (64 lanes, all active) ---------------------------
// Within each 16-lane row through DPP lane moves (quad_perm [1,0,3,2] and
// [2,3,0,1], then row_ror 4 and 8), then the four row results, read out of
// lanes 0, 16, 32 and 48, are combined in a fixed order: the result is the
// same in every lane and from run to run.
template <int CTRL> DEVI float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
DEVI float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
DEVI float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);   // lane ^ 1
    x += dpp_mov<0x4E>(x);   // lane ^ 2: each lane holds its quad's sum
    x += dpp_mov<0x124>(x);  // + the quad 4 lanes round the row
    x += dpp_mov<0x128>(x);  // + the other two quads: lane 16r holds row r's sum
    return (lane_value(x, 0) + lane_value(x, 16)) + (lane_value(x, 32) + lane_value(x, 48));
}
DEVI float wave_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));
    x = fmaxf(x, dpp_mov<0x4E>(x));
    x = fmaxf(x, dpp_mov<0x124>(x));
    x = fmaxf(x, dpp_mov<0x128>(x));
    return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

// GELU, tanh approximation: 0.5 u (1 + tanh(v/2)) with v = 2k (u + 0.044715 u^3),
// k = sqrt(2/pi).  Since 0.5 (1 + tanh(v/2)) is the logistic sigmoid s(v),
// gelu(u) = u s(v) and gelu'(u) = s + u s (1 - s) v', each from one exp2 and
// one reciprocal: s = 1 / (1 + 2^(-v log2 e)).  At the tails 2^(..) goes to 0
// or +inf, s to 1 or 0, and both formulas stay finite (1 - s, not e s, carries
// the derivative's second term).
#define GELU_K 0.7978845608028654f
#define GELU_C 0.044715f
DEVI float gelu_sig(float u) {
    const float u2 = u * u;
    const float z = u * fmaf(-2.f * GELU_K * GELU_C * 1.4426950408889634f, u2, -2.f * GELU_K * 1.4426950408889634f);
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(z));
}
DEVI float gelu_f(float u) { return u * gelu_sig(u); }
DEVI float gelu_grad_f(float u) {
    const float s = gelu_sig(u);
    const float dv = fmaf(6.f * GELU_K * GELU_C, u * u, 2.f * GELU_K);  // v'
    return s * fmaf(u * dv, 1.f - s, 1.f);
}
// both from one sigmoid: gelu(u) into y, gelu'(u) into dy
DEVI void gelu_and_grad(float u, float& y, float& dy) {
    const float s = gelu_sig(u);
    const float dv = fmaf(6.f * GELU_K * GELU_C, u * u, 2.f * GELU_K);
    y = u * s;
    dy = s * fmaf(u * dv, 1.f - s, 1.f);
}

static inline unsigned cdiv(size_t a, size_t b) { return (unsigned)((a + b - 1) / b); }
