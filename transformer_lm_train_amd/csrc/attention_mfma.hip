// Causal flash attention for head size 64 in bf16 on the gfx950 matrix cores.
//
// The method (llm.c lesson, section 2: attention_forward / attention_backward
// with the causal loop t2 <= t; the origin-of-llm.c transcript, "Avengers":
// the mainline moved attention to a flash kernel) is computed without a
// T x T buffer: per query row a running max and sum (online softmax) in the
// forward, the row log-sum-exp kept for the backward, and P recomputed from
// it there.
//
// Layout trick: scores are produced TRANSPOSED, S^T[key][query] = K Q^T,
// with v_mfma_f32_32x32x16_bf16.  In the 32x32 accumulator layout lane l
// owns one column (l % 32), so each lane owns one query and all of that
// query's softmax statistics live in its own registers (the other half of
// the query's keys sits in lane l ^ 32: one shuffle combines them).  The
// accumulator registers 8j..8j+7 of a lane hold 8 distinct keys, which is
// exactly the B-operand shape of the next product (O^T = V^T P^T), so P
// never leaves registers; V^T is staged in LDS key-contiguous to match.
//
// Backward is two deterministic kernels, no atomics:
//   dq kernel (query blocks): recompute S^T and dP^T = V dO^T, dS^T =
//     P^T (dP^T - D), dQ^T = K^T dS^T; also writes D = rowsum(dO o O).
//   dk/dv kernel (key blocks): the untransposed S = Q K^T and dP = dO V^T
//     give each lane one key, so dV = P^T dO and dK = dS^T Q take P and dS
//     straight from registers as A operands.
#include "kernels.h"

namespace {

constexpr int HS = 64;   // head size
constexpr int QB = 128;  // rows (queries or keys) owned by one workgroup: 4 waves x 32
constexpr int KB = 64;   // rows streamed per inner step
constexpr int LP = 72;   // LDS pitch (elements) of a 64-wide bf16 row, padded
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

DEVI bf16x8 cat44(bf16x4 a, bf16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

DEVI bf16x8 to_bf16x8(const f32x16& v, int base) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (bf16)v[base + i];
    return r;
}

DEVI f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

DEVI uint4 ld_row(const bf16* p, bool ok) {
    return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}

// 8x8 bf16 transpose: in[j] holds 8 elements of row j; out[i] gets element i
// of every row.
DEVI void transpose8(const uint4 in[8], uint4 out[8]) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint32_t lo = reinterpret_cast<const uint32_t*>(&in[2 * q])[i >> 1];
            uint32_t hi = reinterpret_cast<const uint32_t*>(&in[2 * q + 1])[i >> 1];
            o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        out[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// Stage rows [r0, r0+64) x 64 channels of a [*, ld] bf16 matrix into LDS.
// 64 threads (t = 0..63) each take an 8-row x 8-channel block; nat and/or
// tr receive the natural ([row][ch]) and transposed ([ch][row]) copies.
DEVI void stage_block(const bf16* src, int64_t ld, int r0, int rows, int t, bf16* nat, bf16* tr) {
    const int rb = t >> 3, cb = t & 7;
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        int r = r0 + rb * 8 + j;
        v[j] = ld_row(src + (int64_t)r * ld + cb * 8, r < rows);
    }
    if (nat) {
#pragma unroll
        for (int j = 0; j < 8; j++) *reinterpret_cast<uint4*>(nat + (rb * 8 + j) * LP + cb * 8) = v[j];
    }
    if (tr) {
        uint4 o[8];
        transpose8(v, o);
#pragma unroll
        for (int i = 0; i < 8; i++) *reinterpret_cast<uint4*>(tr + (cb * 8 + i) * LP + rb * 8) = o[i];
    }
}

// The A operand of a 32x32x16 product whose 16 reduction slots are the keys
// (or queries) held by accumulator registers 8j..8j+7 of a lane in half hi:
// positions t32 + 8*(2j) + 4hi + 0..3 and t32 + 8*(2j+1) + 4hi + 0..3 of a
// key-contiguous LDS row.
DEVI bf16x8 a_from_tr(const bf16* row, int t32, int j, int hi) {
    bf16x4 x = *reinterpret_cast<const bf16x4*>(row + t32 + 16 * j + 4 * hi);
    bf16x4 y = *reinterpret_cast<const bf16x4*>(row + t32 + 16 * j + 8 + 4 * hi);
    return cat44(x, y);
}

// accumulator register r of lane half hi covers row 8*(r/4) + 4*hi + r%4
DEVI int acc_row(int r, int hi) { return ((r >> 2) << 3) + (hi << 2) + (r & 3); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void flash_fwd_kernel(bf16* out, float* lse, const bf16* qkv, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[KB * LP];
    __shared__ __attribute__((aligned(16))) bf16 Vt[HS * LP];
    const int nqb = (T + QB - 1) / QB;
    const int qblk = nqb - 1 - (int)blockIdx.x;  // longest rows first
    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const int q0 = qblk * QB + w * 32;
    const int q = q0 + lq;

    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        uint4 v = ld_row(base + (int64_t)q * C3 + h * HS + ks * 16 + hi * 8, q < T);
        qf[ks] = *reinterpret_cast<bf16x8*>(&v);
    }
    f32x16 o[2];
#pragma unroll
    for (int r = 0; r < 16; r++) { o[0][r] = 0.f; o[1][r] = 0.f; }
    float m_run = -INFINITY, l_run = 0.f;
    const float sc = 0.125f * LOG2E;  // 1/sqrt(64), in log2 units

    const int kend = min(T, qblk * QB + QB);
    const int nkb = (kend + KB - 1) / KB;
    for (int kb = 0; kb < nkb; kb++) {
        const int k0 = kb * KB;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; i++) {
            int c = tid + i * 256, key = c >> 3, dc = c & 7;
            uint4 v = ld_row(base + (int64_t)(k0 + key) * C3 + C + h * HS + dc * 8, k0 + key < T);
            *reinterpret_cast<uint4*>(Ks + key * LP + dc * 8) = v;
        }
        if (tid < 64) stage_block(base + 2 * C + h * HS, C3, k0, T, tid, nullptr, Vt);
        __syncthreads();
        if (k0 > q0 + 31) continue;  // every key of the block is in the future of every query of the wave

        f32x16 s[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
#pragma unroll
            for (int r = 0; r < 16; r++) s[t][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (t * 32 + lq) * LP + ks * 16 + hi * 8);
                s[t] = mfma(a, qf[ks], s[t]);
            }
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int key = k0 + t * 32 + acc_row(r, hi);
                float x = s[t][r] * sc;
                if (key > q || key >= T) x = -INFINITY;
                s[t][r] = x;
                mloc = fmaxf(mloc, x);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = exp2f(m_run - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float p = exp2f(s[t][r] - m_new);
                s[t][r] = p;
                lsum += p;
            }
        lsum += __shfl_xor(lsum, 32, 64);
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int r = 0; r < 16; r++) { o[0][r] *= alpha; o[1][r] *= alpha; }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                bf16x8 pb = to_bf16x8(s[t], 8 * j);
#pragma unroll
                for (int dt = 0; dt < 2; dt++) o[dt] = mfma(a_from_tr(Vt + (dt * 32 + lq) * LP, t * 32, j, hi), pb, o[dt]);
            }
    }
    if (q < T) {
        const float inv = 1.f / l_run;
        bf16* orow = out + ((int64_t)b * T + q) * C + h * HS;
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; i++) v[i] = (bf16)(o[dt][4 * g + i] * inv);
                *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * g + 4 * hi) = v;
            }
        if (hi == 0) lse[((int64_t)b * NH + h) * T + q] = (m_run + log2f(l_run)) * LN2;
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void flash_bwd_dq_kernel(bf16* dqkv, float* Dout, const bf16* dout, const bf16* qkv,
                                                           const bf16* out, const float* lse, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 Ks[KB * LP];
    __shared__ __attribute__((aligned(16))) bf16 Kt[HS * LP];
    __shared__ __attribute__((aligned(16))) bf16 Vs[KB * LP];
    const int nqb = (T + QB - 1) / QB;
    const int qblk = nqb - 1 - (int)blockIdx.x;
    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const int q0 = qblk * QB + w * 32;
    const int q = q0 + lq;
    const bool qok = q < T;

    bf16x8 qf[4], dof[4];
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const int d = ks * 16 + hi * 8;
        uint4 v = ld_row(base + (int64_t)q * C3 + h * HS + d, qok);
        qf[ks] = *reinterpret_cast<bf16x8*>(&v);
        uint4 g = ld_row(dout + ((int64_t)b * T + q) * C + h * HS + d, qok);
        dof[ks] = *reinterpret_cast<bf16x8*>(&g);
        uint4 ov = ld_row(out + ((int64_t)b * T + q) * C + h * HS + d, qok);
        bf16x8 of = *reinterpret_cast<bf16x8*>(&ov);
#pragma unroll
        for (int i = 0; i < 8; i++) dsum += (float)dof[ks][i] * (float)of[i];
    }
    const float Dq = dsum + __shfl_xor(dsum, 32, 64);
    const int64_t ri = ((int64_t)b * NH + h) * T + q;
    if (qok && hi == 0) Dout[ri] = Dq;
    const float lse2 = qok ? lse[ri] * LOG2E : 0.f;
    const float sc = 0.125f * LOG2E;

    f32x16 dq[2];
#pragma unroll
    for (int r = 0; r < 16; r++) { dq[0][r] = 0.f; dq[1][r] = 0.f; }
    const int kend = min(T, qblk * QB + QB);
    const int nkb = (kend + KB - 1) / KB;
    for (int kb = 0; kb < nkb; kb++) {
        const int k0 = kb * KB;
        __syncthreads();
        if (tid < 64) stage_block(base + C + h * HS, C3, k0, T, tid, Ks, Kt);
        else if (tid < 128) stage_block(base + 2 * C + h * HS, C3, k0, T, tid - 64, Vs, nullptr);
        __syncthreads();
        if (k0 > q0 + 31) continue;

        f32x16 s[2], dp[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
#pragma unroll
            for (int r = 0; r < 16; r++) { s[t][r] = 0.f; dp[t][r] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int off = (t * 32 + lq) * LP + ks * 16 + hi * 8;
                s[t] = mfma(*reinterpret_cast<const bf16x8*>(Ks + off), qf[ks], s[t]);
                dp[t] = mfma(*reinterpret_cast<const bf16x8*>(Vs + off), dof[ks], dp[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int key = k0 + t * 32 + acc_row(r, hi);
                float p = (key > q || key >= T || !qok) ? 0.f : exp2f(s[t][r] * sc - lse2);
                s[t][r] = p * (dp[t][r] - Dq);  // dS^T
            }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                bf16x8 dsb = to_bf16x8(s[t], 8 * j);
#pragma unroll
                for (int dt = 0; dt < 2; dt++) dq[dt] = mfma(a_from_tr(Kt + (dt * 32 + lq) * LP, t * 32, j, hi), dsb, dq[dt]);
            }
    }
    if (qok) {
        bf16* row = dqkv + ((int64_t)b * T + q) * C3 + h * HS;
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; i++) v[i] = (bf16)(dq[dt][4 * g + i] * 0.125f);
                *reinterpret_cast<bf16x4*>(row + dt * 32 + 8 * g + 4 * hi) = v;
            }
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void flash_bwd_dkdv_kernel(bf16* dqkv, const float* Din, const bf16* dout,
                                                             const bf16* qkv, const float* lse, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 Qs[KB * LP];
    __shared__ __attribute__((aligned(16))) bf16 Qt[HS * LP];
    __shared__ __attribute__((aligned(16))) bf16 Os[KB * LP];  // dO natural
    __shared__ __attribute__((aligned(16))) bf16 Ot[HS * LP];  // dO transposed
    __shared__ float sl[KB], sd[KB];
    const int kblk = blockIdx.x;  // the first key blocks see the most queries: launched first
    const int h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* dbase = dout + (int64_t)b * T * C;
    const int k0 = kblk * QB + w * 32;
    const int key = k0 + lq;

    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const int d = ks * 16 + hi * 8;
        uint4 v = ld_row(base + (int64_t)key * C3 + C + h * HS + d, key < T);
        kf[ks] = *reinterpret_cast<bf16x8*>(&v);
        uint4 u = ld_row(base + (int64_t)key * C3 + 2 * C + h * HS + d, key < T);
        vf[ks] = *reinterpret_cast<bf16x8*>(&u);
    }
    f32x16 dk[2], dv[2];
#pragma unroll
    for (int r = 0; r < 16; r++) { dk[0][r] = dk[1][r] = dv[0][r] = dv[1][r] = 0.f; }
    const float sc = 0.125f * LOG2E;
    const int64_t rbase = ((int64_t)b * NH + h) * T;

    for (int qs0 = (kblk * QB / KB) * KB; qs0 < T; qs0 += KB) {
        __syncthreads();
        if (tid < 64) stage_block(base + h * HS, C3, qs0, T, tid, Qs, Qt);
        else if (tid < 128) stage_block(dbase + h * HS, C, qs0, T, tid - 64, Os, Ot);
        else if (tid < 192) {
            int qq = qs0 + tid - 128;
            sl[tid - 128] = qq < T ? lse[rbase + qq] * LOG2E : 0.f;
            sd[tid - 128] = qq < T ? Din[rbase + qq] : 0.f;
        }
        __syncthreads();
        if (qs0 + KB - 1 < k0) continue;  // every query of the block precedes every key of the wave

        f32x16 s[2], dp[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
#pragma unroll
            for (int r = 0; r < 16; r++) { s[t][r] = 0.f; dp[t][r] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int off = (t * 32 + lq) * LP + ks * 16 + hi * 8;
                s[t] = mfma(*reinterpret_cast<const bf16x8*>(Qs + off), kf[ks], s[t]);
                dp[t] = mfma(*reinterpret_cast<const bf16x8*>(Os + off), vf[ks], dp[t]);
            }
        }
        // s[t][r]: query qs0 + t*32 + acc_row(r), key `key`
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                int ql = t * 32 + acc_row(r, hi);
                int qq = qs0 + ql;
                float p = (key > qq || qq >= T || key >= T) ? 0.f : exp2f(s[t][r] * sc - sl[ql]);
                s[t][r] = p;
                dp[t][r] = p * (dp[t][r] - sd[ql]);
            }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                bf16x8 pa = to_bf16x8(s[t], 8 * j);
                bf16x8 da = to_bf16x8(dp[t], 8 * j);
#pragma unroll
                for (int dt = 0; dt < 2; dt++) {
                    dv[dt] = mfma(pa, a_from_tr(Ot + (dt * 32 + lq) * LP, t * 32, j, hi), dv[dt]);
                    dk[dt] = mfma(da, a_from_tr(Qt + (dt * 32 + lq) * LP, t * 32, j, hi), dk[dt]);
                }
            }
    }
    // dk[dt][r], dv[dt][r]: key k0 + acc_row(r), channel dt*32 + lq
#pragma unroll
    for (int r = 0; r < 16; r++) {
        int kk = k0 + acc_row(r, hi);
        if (kk < T) {
            bf16* row = dqkv + ((int64_t)b * T + kk) * C3 + h * HS;
#pragma unroll
            for (int dt = 0; dt < 2; dt++) {
                row[C + dt * 32 + lq] = (bf16)(dk[dt][r] * 0.125f);
                row[2 * C + dt * 32 + lq] = (bf16)dv[dt][r];
            }
        }
    }
}

}  // namespace

hipError_t flash_attention_fwd(bf16* out, float* lse, const bf16* qkv, int B, int T, int C, int NH, hipStream_t s) {
    if (C / NH != HS || C % NH) return hipErrorInvalidValue;
    dim3 grid((T + QB - 1) / QB, NH, B);
    flash_fwd_kernel<<<grid, 256, 0, s>>>(out, lse, qkv, T, C, NH);
    return hipGetLastError();
}

hipError_t flash_attention_bwd(bf16* dqkv, const bf16* dout, const bf16* qkv, const bf16* out, const float* lse,
                               float* dbuf, int B, int T, int C, int NH, hipStream_t s) {
    if (C / NH != HS || C % NH) return hipErrorInvalidValue;
    dim3 grid((T + QB - 1) / QB, NH, B);
    flash_bwd_dq_kernel<<<grid, 256, 0, s>>>(dqkv, dbuf, dout, qkv, out, lse, T, C, NH);
    flash_bwd_dkdv_kernel<<<grid, 256, 0, s>>>(dqkv, dbuf, dout, qkv, lse, T, C, NH);
    return hipGetLastError();
}
