// Generic fp32-accumulating matrix product on the vector ALUs, used by the
// fp32 mode (and any shape the MFMA kernel does not take).  64x64 output
// tile per 256-thread block, 4x4 outputs per thread, k-steps of 16 staged
// through LDS.  Handles every edge by predication.
#include "kernels.h"

template <int EPI, typename T, typename TC>
DEVI void epi_store(const GemmArgs& g, int m, int n, float acc) {
    int64_t o = (int64_t)m * g.ldo + n;
    if (EPI == EPI_ACC_F32) {
        float* out = (float*)g.out;
        out[o] += acc;
        return;
    }
    float b = (EPI != EPI_STORE && EPI != EPI_GELU_BWD && g.bias) ? g.bias[n] : 0.f;
    float y = acc + b;
    if (EPI == EPI_BIAS_RESID) y += to_f32(((const T*)g.resid)[o]);
    if (EPI == EPI_GELU_BWD) y = acc * gelu_grad_f(to_f32(((const T*)g.aux)[o]));
    ((T*)g.out)[o] = from_f32<T>(y);
    if (EPI == EPI_BIAS_GELU) ((T*)g.out2)[o] = from_f32<T>(gelu_f(y));
}

template <typename T, bool AK, bool BK, int EPI>
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmArgs g) {
    constexpr int BM = 64, BN = 64, BKK = 16;
    __shared__ float As[BKK][BM + 4];
    __shared__ float Bs[BKK][BN + 4];
    const T* A = (const T*)g.a;
    const T* B = (const T*)g.b;
    int tid = threadIdx.x;
    int tx = tid & 15, ty = tid >> 4;
    int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = 0.f;
    for (int k0 = 0; k0 < g.K; k0 += BKK) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int e = tid + i * 256;
            int r, kk;
            if (AK) { r = e >> 4; kk = e & 15; } else { kk = e >> 6; r = e & 63; }
            int m = m0 + r, k = k0 + kk;
            float v = 0.f;
            if (m < g.M && k < g.K) v = to_f32(AK ? A[(int64_t)m * g.lda + k] : A[(int64_t)k * g.lda + m]);
            As[kk][r] = v;
            if (BK) { r = e >> 4; kk = e & 15; } else { kk = e >> 6; r = e & 63; }
            int n = n0 + r;
            k = k0 + kk;
            v = 0.f;
            if (n < g.N && k < g.K) v = to_f32(BK ? B[(int64_t)n * g.ldb + k] : B[(int64_t)k * g.ldb + n]);
            Bs[kk][r] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BKK; kk++) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
            if (m < g.M && n < g.N) epi_store<EPI, T, T>(g, m, n, acc[i][j]);
        }
}

template <typename T, bool AK, bool BK>
static hipError_t launch_simt(const GemmArgs& g, hipStream_t s) {
    dim3 grid(cdiv(g.N, 64), cdiv(g.M, 64));
    switch (g.epi) {
        case EPI_STORE: gemm_simt_kernel<T, AK, BK, EPI_STORE><<<grid, 256, 0, s>>>(g); break;
        case EPI_BIAS: gemm_simt_kernel<T, AK, BK, EPI_BIAS><<<grid, 256, 0, s>>>(g); break;
        case EPI_BIAS_RESID: gemm_simt_kernel<T, AK, BK, EPI_BIAS_RESID><<<grid, 256, 0, s>>>(g); break;
        case EPI_BIAS_GELU: gemm_simt_kernel<T, AK, BK, EPI_BIAS_GELU><<<grid, 256, 0, s>>>(g); break;
        case EPI_GELU_BWD: gemm_simt_kernel<T, AK, BK, EPI_GELU_BWD><<<grid, 256, 0, s>>>(g); break;
        case EPI_ACC_F32: gemm_simt_kernel<T, AK, BK, EPI_ACC_F32><<<grid, 256, 0, s>>>(g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T> hipError_t gemm_simt(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return hipErrorInvalidValue;
    if (g.a_kcontig && g.b_kcontig) return launch_simt<T, true, true>(g, s);
    if (g.a_kcontig && !g.b_kcontig) return launch_simt<T, true, false>(g, s);
    if (!g.a_kcontig && !g.b_kcontig) return launch_simt<T, false, false>(g, s);
    return launch_simt<T, false, true>(g, s);
}

template hipError_t gemm_simt<float>(const GemmArgs&, hipStream_t);
template hipError_t gemm_simt<bf16>(const GemmArgs&, hipStream_t);
