// Causal multi-head self-attention, forward and backward, with a row-wise
// log-sum-exp instead of a stored T x T attention matrix.
//
// Forward (llm.c lesson, section 2: attention_forward with the causal loop
// t2 <= t): per query row t of head h,
//   s_t2 = q_t . k_t2 / sqrt(hs),  p = softmax over t2 <= t,  o_t = sum p v_t2,
//   lse_t = log sum_t2 exp(s_t2)   (kept for the backward).
// Backward (the same section: "out += att * value" becomes datt += value *
// dout and dvalue += att * dout), with D_t = do_t . o_t = sum_t2 p dp_t2:
//   p = exp(s - lse_t); dp = do_t . v_t2; ds = p (dp - D_t);
//   dq_t = sum_t2 ds k_t2 / sqrt(hs); dk_t2 = sum_t ds q_t / sqrt(hs);
//   dv_t2 = sum_t p do_t.
// These kernels give one wavefront to one query row (forward, dq) or one key
// row (dk, dv); every output is written by exactly one wavefront, so there
// are no atomics and results are deterministic.
#include "kernels.h"

namespace {

constexpr int MAXT = 1024;  // longest sequence the row buffers hold
constexpr int MAXHS = 128;

template <typename T>
__global__ __launch_bounds__(64) void attn_fwd_row_kernel(T* out, float* lse, const T* qkv, int T_, int C, int NH) {
    __shared__ float q[MAXHS];
    __shared__ float p[MAXT];
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int hs = C / NH;
    const int64_t C3 = 3 * (int64_t)C;
    const float scale = rsqrtf((float)hs);
    const T* base = qkv + (int64_t)b * T_ * C3;
    for (int d = lane; d < hs; d += 64) q[d] = to_f32(base[(int64_t)t * C3 + h * hs + d]);
    __syncthreads();
    float mx = -INFINITY;
    for (int t2 = lane; t2 <= t; t2 += 64) {
        const T* k = base + (int64_t)t2 * C3 + C + h * hs;
        float s = 0.f;
        for (int d = 0; d < hs; d++) s += q[d] * to_f32(k[d]);
        s *= scale;
        p[t2] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int t2 = lane; t2 <= t; t2 += 64) {
        float e = __expf(p[t2] - mx);
        p[t2] = e;
        sum += e;
    }
    sum = wave_sum(sum);
    __syncthreads();
    float inv = 1.f / sum;
    for (int d = lane; d < hs; d += 64) {
        float acc = 0.f;
        for (int t2 = 0; t2 <= t; t2++) acc += p[t2] * to_f32(base[(int64_t)t2 * C3 + 2 * C + h * hs + d]);
        out[((int64_t)b * T_ + t) * C + h * hs + d] = from_f32<T>(acc * inv);
    }
    if (lane == 0) lse[((int64_t)b * NH + h) * T_ + t] = mx + logf(sum);
}

// D[b,h,t] = do_t . o_t over the head's channels
template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_d_kernel(float* D, const T* dout, const T* out, int T_, int C, int NH) {
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int hs = C / NH;
    int64_t o = ((int64_t)b * T_ + t) * C + h * hs;
    float s = 0.f;
    for (int d = lane; d < hs; d += 64) s += to_f32(dout[o + d]) * to_f32(out[o + d]);
    s = wave_sum(s);
    if (lane == 0) D[((int64_t)b * NH + h) * T_ + t] = s;
}

// dq for query row t
template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_dq_kernel(T* dqkv, const T* dout, const T* qkv, const float* lse,
                                                         const float* D, int T_, int C, int NH) {
    __shared__ float q[MAXHS], dO[MAXHS];
    __shared__ float ds[MAXT];
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int hs = C / NH;
    const int64_t C3 = 3 * (int64_t)C;
    const float scale = rsqrtf((float)hs);
    const T* base = qkv + (int64_t)b * T_ * C3;
    for (int d = lane; d < hs; d += 64) {
        q[d] = to_f32(base[(int64_t)t * C3 + h * hs + d]);
        dO[d] = to_f32(dout[((int64_t)b * T_ + t) * C + h * hs + d]);
    }
    __syncthreads();
    const int64_t ri = ((int64_t)b * NH + h) * T_ + t;
    const float L = lse[ri], Dt = D[ri];
    for (int t2 = lane; t2 <= t; t2 += 64) {
        const T* k = base + (int64_t)t2 * C3 + C + h * hs;
        const T* v = base + (int64_t)t2 * C3 + 2 * C + h * hs;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < hs; d++) {
            s += q[d] * to_f32(k[d]);
            dp += dO[d] * to_f32(v[d]);
        }
        float pr = __expf(s * scale - L);
        ds[t2] = pr * (dp - Dt);
    }
    __syncthreads();
    for (int d = lane; d < hs; d += 64) {
        float acc = 0.f;
        for (int t2 = 0; t2 <= t; t2++) acc += ds[t2] * to_f32(base[(int64_t)t2 * C3 + C + h * hs + d]);
        dqkv[((int64_t)b * T_ + t) * C3 + h * hs + d] = from_f32<T>(acc * scale);
    }
}

// dk, dv for key row t2 (sums over the query rows t >= t2)
template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_kernel(T* dqkv, const T* dout, const T* qkv, const float* lse,
                                                           const float* D, int T_, int C, int NH) {
    __shared__ float k[MAXHS], v[MAXHS];
    __shared__ float pr[MAXT], ds[MAXT];
    const int t2 = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int hs = C / NH;
    const int64_t C3 = 3 * (int64_t)C;
    const float scale = rsqrtf((float)hs);
    const T* base = qkv + (int64_t)b * T_ * C3;
    for (int d = lane; d < hs; d += 64) {
        k[d] = to_f32(base[(int64_t)t2 * C3 + C + h * hs + d]);
        v[d] = to_f32(base[(int64_t)t2 * C3 + 2 * C + h * hs + d]);
    }
    __syncthreads();
    for (int t = t2 + lane; t < T_; t += 64) {
        const T* q = base + (int64_t)t * C3 + h * hs;
        const T* dO = dout + ((int64_t)b * T_ + t) * C + h * hs;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < hs; d++) {
            s += to_f32(q[d]) * k[d];
            dp += to_f32(dO[d]) * v[d];
        }
        const int64_t ri = ((int64_t)b * NH + h) * T_ + t;
        float p = __expf(s * scale - lse[ri]);
        pr[t] = p;
        ds[t] = p * (dp - D[ri]);
    }
    __syncthreads();
    for (int d = lane; d < hs; d += 64) {
        float ak = 0.f, av = 0.f;
        for (int t = t2; t < T_; t++) {
            ak += ds[t] * to_f32(base[(int64_t)t * C3 + h * hs + d]);
            av += pr[t] * to_f32(dout[((int64_t)b * T_ + t) * C + h * hs + d]);
        }
        int64_t o = ((int64_t)b * T_ + t2) * C3 + h * hs + d;
        dqkv[o + C] = from_f32<T>(ak * scale);
        dqkv[o + 2 * C] = from_f32<T>(av);
    }
}

}  // namespace

template <typename T>
hipError_t attention_fwd(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s) {
    if (T_ > MAXT || C / NH > MAXHS) return hipErrorInvalidValue;
    dim3 grid(T_, NH, B);
    attn_fwd_row_kernel<T><<<grid, 64, 0, s>>>(out, lse, qkv, T_, C, NH);
    return hipGetLastError();
}

template <typename T>
hipError_t attention_bwd(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse, float* dbuf, int B,
                         int T_, int C, int NH, hipStream_t s) {
    if (T_ > MAXT || C / NH > MAXHS) return hipErrorInvalidValue;
    dim3 grid(T_, NH, B);
    attn_bwd_d_kernel<T><<<grid, 64, 0, s>>>(dbuf, dout, out, T_, C, NH);
    attn_bwd_dq_kernel<T><<<grid, 64, 0, s>>>(dqkv, dout, qkv, lse, dbuf, T_, C, NH);
    attn_bwd_dkdv_kernel<T><<<grid, 64, 0, s>>>(dqkv, dout, qkv, lse, dbuf, T_, C, NH);
    return hipGetLastError();
}

template hipError_t attention_fwd<float>(float*, float*, const float*, int, int, int, int, hipStream_t);
template hipError_t attention_fwd<bf16>(bf16*, float*, const bf16*, int, int, int, int, hipStream_t);
template hipError_t attention_bwd<float>(float*, const float*, const float*, const float*, const float*, float*, int,
                                         int, int, int, hipStream_t);
template hipError_t attention_bwd<bf16>(bf16*, const bf16*, const bf16*, const bf16*, const float*, float*, int, int,
                                        int, int, hipStream_t);
