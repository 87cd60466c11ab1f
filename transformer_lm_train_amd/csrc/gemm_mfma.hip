// bf16 matrix products on the gfx950 matrix cores.
//
// Block tile BM x BN, k-step 64, 256 threads = 4 wavefronts in a 2x2 grid,
// each wave owning a (BM/2) x (BN/2) sub-tile of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16 (8 bf16 of A and of B per lane, fp32 accumulate).
// Operand tiles are staged in LDS as [row][k] with k contiguous, so every
// MFMA fragment is one 16-byte LDS read.  An operand stored with its row
// index contiguous (the transposed operands of the backward products) is
// loaded as 8x8 blocks and transposed in registers on its way into LDS.
// Two LDS buffers: the global loads of k-step t+1 are in flight while the
// matrix cores work on step t.  Block ids are remapped so that the tiles
// one XCD (one L2) runs are neighbours sharing operand panels.
#include <algorithm>

#include "kernels.h"

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in elements (144 bytes)

// rows [r0, r0+R) x k [k0, k0+64) of X with X(r,k) = X[r*ld + k]
template <int R> struct KTile {
    static constexpr int PER = R * (BK / 8) / 256;
    uint4 v[PER];
    DEVI void load(const bf16* X, int64_t ld, int r0, int rows, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            int c = tid + i * 256;
            int row = c >> 3, kc = c & 7;
            if (r0 + row < rows)
                v[i] = *reinterpret_cast<const uint4*>(X + (int64_t)(r0 + row) * ld + k0 + kc * 8);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
    }
    DEVI void store(uint16_t* lds, int tid) {
#pragma unroll
        for (int i = 0; i < PER; i++) {
            int c = tid + i * 256;
            int row = c >> 3, kc = c & 7;
            *reinterpret_cast<uint4*>(lds + row * LDK + kc * 8) = v[i];
        }
    }
};

// same tile of X with X(r,k) = X[k*ld + r]: R/8 x 8 blocks of 8x8, one
// block per thread (threads (tid+off)%256 < R work), transposed in registers.
template <int R> struct MNTile {
    static constexpr int PER = (R + 255) / 256;
    uint4 v[PER][8];
    DEVI void load(const bf16* X, int64_t ld, int r0, int rows, int k0, int tid, int off) {
        int t = (tid + off) & 255;
#pragma unroll
        for (int p = 0; p < PER; p++) {
            int b = t + p * 256;
            if (b < R) {
                // k-block fastest: the 8 lanes of a group then write 8 different
                // 16-byte columns of one LDS row group (distinct banks), while
                // each row of 8 lanes still reads 128 contiguous bytes
                int kb = b & 7, rb = b >> 3;
                int r = r0 + rb * 8;
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    if (r < rows)
                        v[p][j] = *reinterpret_cast<const uint4*>(X + (int64_t)(k0 + kb * 8 + j) * ld + r);
                    else
                        v[p][j] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    }
    DEVI void store(uint16_t* lds, int tid, int off) {
        int t = (tid + off) & 255;
#pragma unroll
        for (int p = 0; p < PER; p++) {
            int b = t + p * 256;
            if (b < R) {
                int kb = b & 7, rb = b >> 3;
                const uint32_t* w[8];
#pragma unroll
                for (int j = 0; j < 8; j++) w[j] = reinterpret_cast<const uint32_t*>(&v[p][j]);
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    uint32_t o[4];
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        uint32_t lo = w[2 * q][i >> 1], hi = w[2 * q + 1][i >> 1];
                        o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                    }
                    *reinterpret_cast<uint4*>(lds + (rb * 8 + i) * LDK + kb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
};

constexpr int EPI_PARTIAL = 100;  // split-K partial tile into g.ws[split][M][N]

template <int EPI>
DEVI void epi_store(const GemmArgs& g, int m, int n, float acc) {
    if (EPI == EPI_PARTIAL) {
        g.ws[((int64_t)blockIdx.y * g.M + m) * g.N + n] = acc;
        return;
    }
    int64_t o = (int64_t)m * g.ldo + n;
    if (EPI == EPI_ACC_F32) {
        float* out = (float*)g.out;
        out[o] += acc;
        return;
    }
    float b = (EPI != EPI_STORE && EPI != EPI_GELU_BWD && g.bias) ? g.bias[n] : 0.f;
    float y = acc + b;
    if (EPI == EPI_BIAS_RESID) y += to_f32(((const bf16*)g.resid)[o]);
    if (EPI == EPI_GELU_BWD) y = acc * gelu_grad_f(to_f32(((const bf16*)g.aux)[o]));
    ((bf16*)g.out)[o] = (bf16)y;
    if (EPI == EPI_BIAS_GELU) ((bf16*)g.out2)[o] = (bf16)gelu_f(y);
}

template <int BM, int BN, int WAVES_M, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs g, int kchunk) {
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N, FM = TM / 32, FN = TN / 32;
    static_assert(FM >= 1 && FN >= 1 && TM % 32 == 0 && TN % 32 == 0, "wave tile");
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][(BM + BN) * LDK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // block -> tile: XCD-contiguous ranges, then groups of 8 tile-rows
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    constexpr int GM = 8;
    int group = bid / (GM * tiles_n);
    int first_m = group * GM;
    int gsz = min(tiles_m - first_m, GM);
    int in = bid % (GM * tiles_n);
    const int m0 = (first_m + in % gsz) * BM;
    const int n0 = (in / gsz) * BN;

    const bf16* A = (const bf16*)g.a;
    const bf16* B = (const bf16*)g.b;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    typename std::conditional<AK, KTile<BM>, MNTile<BM>>::type ta;
    typename std::conditional<BKC, KTile<BN>, MNTile<BN>>::type tb;

    auto load = [&](int k0) {
        if constexpr (AK) ta.load(A, g.lda, m0, g.M, k0, tid);
        else ta.load(A, g.lda, m0, g.M, k0, tid, 0);
        if constexpr (BKC) tb.load(B, g.ldb, n0, g.N, k0, tid);
        else tb.load(B, g.ldb, n0, g.N, k0, tid, 128);
    };
    auto store = [&](uint16_t* buf) {
        if constexpr (AK) ta.store(buf, tid);
        else ta.store(buf, tid, 0);
        if constexpr (BKC) tb.store(buf + BM * LDK, tid);
        else tb.store(buf + BM * LDK, tid, 128);
    };

    // this workgroup's share of the reduction (the whole of it unless split)
    const int kbeg = blockIdx.y * kchunk;
    const int nk = (min(g.K, kbeg + kchunk) - kbeg) / BK;
    load(kbeg);
    store(lds[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load(kbeg + (kt + 1) * BK);
        const uint16_t* As = lds[cur];
        const uint16_t* Bs = lds[cur] + BM * LDK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ks++) {
            bf16x8 a[FM], b[FN];
            const int koff = ks * 16 + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < FM; i++)
                a[i] = *reinterpret_cast<const bf16x8*>(As + (wm * TM + i * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
            for (int j = 0; j < FN; j++)
                b[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * TN + j * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store(lds[cur ^ 1]);
        __syncthreads();
    }

    // accumulator (i,j) register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
    // column l%32 of the 32x32 block
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int m = m0 + wm * TM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                int n = n0 + wn * TN + j * 32 + (lane & 31);
                if (m < g.M && n < g.N) epi_store<EPI>(g, m, n, acc[i][j][r]);
            }
}

template <int BM, int BN, int WAVES_M, bool AK, bool BKC, int EPI>
hipError_t launch(const GemmArgs& g, hipStream_t s, int splits = 1, int kchunk = 0) {
    dim3 grid(cdiv(g.M, BM) * cdiv(g.N, BN), splits);
    gemm_mfma_kernel<BM, BN, WAVES_M, AK, BKC, EPI><<<grid, 256, 0, s>>>(g, kchunk ? kchunk : g.K);
    return hipGetLastError();
}

// Split of the reduction for the weight-gradient products, whose outputs are
// small (C x C .. 4C x C) next to their reduction over all B*T tokens:
// enough splits to give ~512 workgroups, each at least 4 k-steps long.
void splitk_plan(int M, int N, int K, int* splits, int* kchunk) {
    int tiles = (int)(cdiv(M, 128) * cdiv(N, 128));
    int S = (512 + tiles - 1) / tiles;
    int smax = K / 256;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    int kc = (int)cdiv(K / BK, S) * BK;
    *kchunk = kc;
    *splits = (K + kc - 1) / kc;
}

__global__ void splitk_reduce_kernel(float* out, int64_t ldo, const float* ws, int S, int M, int N) {
    const int64_t n4 = (int64_t)M * N / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        int64_t e = i * 4;
        int m = (int)(e / N), n = (int)(e % N);
        float4 acc = reinterpret_cast<const float4*>(ws)[i];
        for (int sp = 1; sp < S; sp++) {
            float4 v = reinterpret_cast<const float4*>(ws + (int64_t)sp * M * N)[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        float4* o = reinterpret_cast<float4*>(out + (int64_t)m * ldo + n);
        float4 cur = *o;
        cur.x += acc.x; cur.y += acc.y; cur.z += acc.z; cur.w += acc.w;
        *o = cur;
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % BK || g.M % 8 || g.N % 8 || g.lda % 8 || g.ldb % 8)
        return hipErrorInvalidValue;
    if (!aligned16(g.a) || !aligned16(g.b)) return hipErrorInvalidValue;
    if (g.a_kcontig && g.b_kcontig) {
        switch (g.epi) {
            case EPI_STORE: return launch<128, 128, 2, true, true, EPI_STORE>(g, s);
            case EPI_BIAS: return launch<128, 128, 2, true, true, EPI_BIAS>(g, s);
            case EPI_BIAS_RESID: return launch<128, 128, 2, true, true, EPI_BIAS_RESID>(g, s);
            case EPI_BIAS_GELU: return launch<128, 128, 2, true, true, EPI_BIAS_GELU>(g, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (g.a_kcontig && !g.b_kcontig) {
        switch (g.epi) {
            case EPI_STORE: return launch<128, 128, 2, true, false, EPI_STORE>(g, s);
            case EPI_GELU_BWD: return launch<128, 128, 2, true, false, EPI_GELU_BWD>(g, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (!g.a_kcontig && !g.b_kcontig && g.epi == EPI_ACC_F32) {
        int S, kc;
        splitk_plan(g.M, g.N, g.K, &S, &kc);
        if (S > 1 && g.ws && (size_t)S * g.M * g.N * 4 <= g.ws_bytes && g.N % 4 == 0 && g.ldo % 4 == 0) {
            hipError_t e = launch<128, 128, 2, false, false, EPI_PARTIAL>(g, s, S, kc);
            if (e != hipSuccess) return e;
            int64_t n4 = (int64_t)g.M * g.N / 4;
            unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
            splitk_reduce_kernel<<<blocks, 256, 0, s>>>((float*)g.out, g.ldo, g.ws, S, g.M, g.N);
            return hipGetLastError();
        }
        return launch<128, 128, 2, false, false, EPI_ACC_F32>(g, s);
    }
    return hipErrorInvalidValue;
}

size_t gemm_splitk_ws_bytes(int M, int N, int K) {
    int S, kc;
    splitk_plan(M, N, K, &S, &kc);
    return S > 1 ? (size_t)S * M * N * 4 : 0;
}
