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

// native 4 x u32 vector (SROA-friendly, unlike the union-based uint4)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in elements (144 bytes)

// ---- operand tiles: rows [r0, r0+R) x k [k0, k0+64) of X ------------------
// Rows past the end re-read the last row (always in bounds).  They only feed
// accumulator rows/columns past M or N, which the epilogue never stores, so
// they need no zeroing and the loads carry no branches.

// k-contiguous X (X(r,k) = X[r*ld + k]): R*8 16-byte chunks, R/32 per thread
template <int R> struct KT {
    static constexpr int N = R / 32;
    static DEVI void load(u32x4 (&v)[N], const bf16* X, int64_t ld, int r0, int rows, int k0, int tid, int) {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int c = tid + i * 256;
            const int rr = min(r0 + (c >> 3), rows - 1);
            v[i] = *reinterpret_cast<const u32x4*>(X + (int64_t)rr * ld + k0 + (c & 7) * 8);
        }
    }
    static DEVI void store(const u32x4 (&v)[N], uint16_t* lds, int tid, int) {
#pragma unroll
        for (int i = 0; i < N; i++) {
            const int c = tid + i * 256;
            *reinterpret_cast<u32x4*>(lds + (c >> 3) * LDK + (c & 7) * 8) = v[i];
        }
    }
};

// mn-contiguous X (X(r,k) = X[k*ld + r]): 8 x R/8 blocks of 8x8, one block
// per thread for threads (tid+off)%256 < R (R <= 256), transposed in
// registers on the way into LDS.  The k-block index runs fastest, so the 8
// lanes of a group write 8 different 16-byte columns of one LDS row group
// (distinct banks) while every 8 lanes still read 128 contiguous bytes.
template <int R> struct MNT {
    static_assert(R <= 256, "one 8x8 block per thread");
    static constexpr int N = 8;
    static DEVI void load(u32x4 (&v)[N], const bf16* X, int64_t ld, int r0, int rows, int k0, int tid, int off) {
        const int b = (tid + off) & 255;
        if (b >= R) return;
        const int kb = b & 7, rb = b >> 3;
        const int rr = min(r0 + rb * 8, rows - 8);
#pragma unroll
        for (int j = 0; j < 8; j++) v[j] = *reinterpret_cast<const u32x4*>(X + (int64_t)(k0 + kb * 8 + j) * ld + rr);
    }
    static DEVI void store(const u32x4 (&v)[N], uint16_t* lds, int tid, int off) {
        const int b = (tid + off) & 255;
        if (b >= R) return;
        const int kb = b & 7, rb = b >> 3;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t lo = (i & 2) ? (i & 4 ? v[2 * q].w : v[2 * q].y) : (i & 4 ? v[2 * q].z : v[2 * q].x);
                const uint32_t hi = (i & 2) ? (i & 4 ? v[2 * q + 1].w : v[2 * q + 1].y)
                                            : (i & 4 ? v[2 * q + 1].z : v[2 * q + 1].x);
                o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<u32x4*>(lds + (rb * 8 + i) * LDK + kb * 8) = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
};

constexpr int EPI_PARTIAL = 100;  // split-K partial tile into g.ws[split][M][N]

// Epilogue of 4 consecutive columns n..n+3 of row m (n % 4 == 0, N % 8 == 0,
// so the 4 are all inside or all outside the matrix): 8-byte bf16 or 16-byte
// fp32 accesses.
template <int EPI>
DEVI void epi_store4(const GemmArgs& g, int m, int n, const float (&acc)[4]) {
    typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    if (EPI == EPI_PARTIAL) {
        *reinterpret_cast<float4*>(g.ws + ((int64_t)blockIdx.y * g.M + m) * g.N + n) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
        return;
    }
    const int64_t o = (int64_t)m * g.ldo + n;
    if (EPI == EPI_ACC_F32) {
        float4* p = reinterpret_cast<float4*>((float*)g.out + o);
        float4 v = *p;
        v.x += acc[0]; v.y += acc[1]; v.z += acc[2]; v.w += acc[3];
        *p = v;
        return;
    }
    float y[4] = {acc[0], acc[1], acc[2], acc[3]};
    if ((EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU) && g.bias) {
        const float4 bv = *reinterpret_cast<const float4*>(g.bias + n);
        y[0] += bv.x; y[1] += bv.y; y[2] += bv.z; y[3] += bv.w;
    }
    if (EPI == EPI_BIAS_RESID) {
        const bf16x4_t r = *reinterpret_cast<const bf16x4_t*>((const bf16*)g.resid + o);
#pragma unroll
        for (int e = 0; e < 4; e++) y[e] += (float)r[e];
    }
    if (EPI == EPI_GELU_BWD) {
        const bf16x4_t u = *reinterpret_cast<const bf16x4_t*>((const bf16*)g.aux + o);
#pragma unroll
        for (int e = 0; e < 4; e++) y[e] *= gelu_grad_f((float)u[e]);
    }
    bf16x4_t out;
#pragma unroll
    for (int e = 0; e < 4; e++) out[e] = (bf16)y[e];
    *reinterpret_cast<bf16x4_t*>((bf16*)g.out + o) = out;
    if (EPI == EPI_BIAS_GELU) {
#pragma unroll
        for (int e = 0; e < 4; e++) out[e] = (bf16)gelu_f(y[e]);
        *reinterpret_cast<bf16x4_t*>((bf16*)g.out2 + o) = out;
    }
}

// The products run the MFMA with the operands swapped, acc = B A^T: register
// r of lane l of the 32x32 block (i, j) then holds row i*32 + l % 32 and
// column j*32 + 8*(r/4) + 4*(l/32) + r%4, so each group of 4 registers is 4
// consecutive columns of one row.
template <int EPI, int FM, int FN>
DEVI void epilogue(const GemmArgs& g, const f32x16 (&acc)[FM][FN], int mrow0, int ncol0, int lane) {
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int m = mrow0 + i * 32 + (lane & 31);
                const int n = ncol0 + j * 32 + q * 8 + (lane >> 5) * 4;
                if (m < g.M && n < g.N) {
                    const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                        acc[i][j][4 * q + 3]};
                    epi_store4<EPI>(g, m, n, v);
                }
            }
}

// One k-step (64) of the wave's FM x FN block of 32x32 accumulators from an
// LDS stage holding the A tile ([BM][LDK]) followed by the B tile.
template <int BM, int FM, int FN, int TM, int TN>
DEVI void mfma_tile(f32x16 (&acc)[FM][FN], const uint16_t* As, int wm, int wn, int lane) {
    const uint16_t* Bs = As + BM * LDK;
    // fragments double-buffered in registers (see mfma_swz)
    bf16x8 a[2][FM], b[2][FN];
    auto frag = [&](int ks, bf16x8 (&fa)[FM], bf16x8 (&fb)[FN]) {
        const int koff = ks * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int i = 0; i < FM; i++)
            fa[i] = *reinterpret_cast<const bf16x8*>(As + (wm * TM + i * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
        for (int j = 0; j < FN; j++)
            fb[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * TN + j * 32 + (lane & 31)) * LDK + koff);
    };
    frag(0, a[0], b[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
        if (ks + 1 < BK / 16) frag(ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[ks & 1][j], a[ks & 1][i], acc[i][j], 0, 0, 0);
        // keep that order through scheduling: the next sub-step's LDS reads
        // (mask 0x100) issue ahead of this sub-step's MFMAs (mask 0x008)
        if (ks + 1 < BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
    }
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

    typedef typename std::conditional<AK, KT<BM>, MNT<BM>>::type TA;
    typedef typename std::conditional<BKC, KT<BN>, MNT<BN>>::type TB;
    // two register stages: the loads of k-step t+2 are issued while step t
    // computes, and step t+1 (loaded one compute phase earlier) goes to LDS
    u32x4 ra0[TA::N], ra1[TA::N], rb0[TB::N], rb1[TB::N];
    const int kbeg = blockIdx.y * kchunk;  // this workgroup's share of the reduction
    const int nk = (min(g.K, kbeg + kchunk) - kbeg) / BK;
#define GEMM_LOAD(ra, rb, k0)                                   \
    do {                                                        \
        TA::load(ra, A, g.lda, m0, g.M, (k0), tid, 0);          \
        TB::load(rb, B, g.ldb, n0, g.N, (k0), tid, 128);        \
    } while (0)
#define GEMM_STORE(ra, rb, buf)                                 \
    do {                                                        \
        TA::store(ra, (buf), tid, 0);                           \
        TB::store(rb, (buf) + BM * LDK, tid, 128);              \
    } while (0)

    // Loads are issued unconditionally (the k-step index clamped to the last
    // one; a redundant tail load is never consumed): a load under a branch
    // makes the wait-count insertion assume the worst at the join and wait
    // for every outstanding load, which would undo the prefetch.
    const int klast = kbeg + (nk - 1) * BK;
    int kt = 0;
    if constexpr (!AK && !BKC) {
        // both operands transposed through registers (16 x 16 bytes per thread):
        // one register stage keeps the kernel at two waves per SIMD
        GEMM_LOAD(ra0, rb0, kbeg);
        GEMM_STORE(ra0, rb0, lds[0]);
        __syncthreads();
        for (; kt < nk; kt++) {
            const int cur = kt & 1;
            GEMM_LOAD(ra0, rb0, min(kbeg + (kt + 1) * BK, klast));
            mfma_tile<BM, FM, FN, TM, TN>(acc, lds[cur], wm, wn, lane);
            GEMM_STORE(ra0, rb0, lds[cur ^ 1]);
            __syncthreads();
        }
    } else {
        GEMM_LOAD(ra0, rb0, kbeg);
        GEMM_LOAD(ra1, rb1, min(kbeg + BK, klast));
        GEMM_STORE(ra0, rb0, lds[0]);
        __syncthreads();
        for (; kt + 1 < nk; kt += 2) {
            // even step: compute buffer 0, refill register stage 0 with step kt+2
            GEMM_LOAD(ra0, rb0, min(kbeg + (kt + 2) * BK, klast));
            mfma_tile<BM, FM, FN, TM, TN>(acc, lds[0], wm, wn, lane);
            GEMM_STORE(ra1, rb1, lds[1]);
            __syncthreads();
            // odd step: compute buffer 1, refill register stage 1 with step kt+3;
            // buffer 0 then receives step kt+2 (unused when kt+2 == nk)
            GEMM_LOAD(ra1, rb1, min(kbeg + (kt + 3) * BK, klast));
            mfma_tile<BM, FM, FN, TM, TN>(acc, lds[1], wm, wn, lane);
            GEMM_STORE(ra0, rb0, lds[0]);
            __syncthreads();
        }
        if (kt < nk) mfma_tile<BM, FM, FN, TM, TN>(acc, lds[0], wm, wn, lane);  // odd step count: last one in buffer 0
    }
#undef GEMM_LOAD
#undef GEMM_STORE

    epilogue<EPI>(g, acc, m0 + wm * TM, n0 + wn * TN, lane);
}

// ============================================================================
// Machinery of the direct-to-LDS kernel below: global_load_lds_dwordx4 fills
// 1 KB of LDS per wave instruction, lane l's 16 bytes at base + 16*l.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt immediate (gfx9 encoding): vmcnt <= N, lgkmcnt = 0 (this wave's
// LDS writes done before a barrier publishes them), expcnt unconstrained
template <int N> constexpr int vmcnt_imm() { return (N & 15) | ((N >> 4) << 14) | (7 << 4); }

// ============================================================================
// Large-tile variant: every operand goes global -> LDS by direct loads, in the
// layout it has in memory.
//  - k-contiguous operand: LDS [row][64], 16-byte chunk c of row r in slot
//    c ^ (r & 7); fragment = one 16-byte LDS read.
//  - mn-contiguous operand: LDS [k][R] (R = tile rows), 16-byte chunk c of
//    k-row k in slot c ^ ((k & 3) << 1); fragment = two ds_read_b64_tr_b16.
//    Within each 16-lane group that instruction hands lane i element (i % 4)
//    of the 8-byte read of lane 4e + i/4 as its element e; so when lane j
//    reads X[k0 + j/4][m0 + 4(j%4) .. +3], lane i receives X[k0..k0+3][m0+i],
//    four consecutive k of one row: exactly the MFMA operand fragment.
// NW waves (2 x NW/2), each owning a (BM/2) x (BN/(NW/2)) block of 32x32
// accumulators; NS LDS stages with explicit vmcnt waits and raw barriers.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

DEVI int mn_swz(int k) { return (k & 3) << 1; }

// tile rows [r0, r0+R) x k [k0, k0+64) of X into LDS; NIW 1 KB loads per wave
template <int R, int NW, bool KCONTIG>
DEVI void dma_any(uint16_t* tile, const bf16* X, int64_t ld, int r0, int rows, int k0, int wave, int lane) {
    constexpr int NIW = R / (8 * NW);
    static_assert(NIW >= 1 && NIW * 8 * NW == R, "tile rows vs waves");
#pragma unroll
    for (int i = 0; i < NIW; i++) {
        const int blk = wave * NIW + i;  // 1 KB block of the tile
        const bf16* g;
        if constexpr (KCONTIG) {
            const int r = blk * 8 + (lane >> 3);
            const int c = (lane & 7) ^ (lane >> 3);  // = slot ^ (r & 7)
            g = X + (int64_t)min(r0 + r, rows - 1) * ld + k0 + c * 8;
        } else {
            constexpr int CPR = R / 8;  // chunks per k-row
            const int p = blk * 64 + lane;
            const int k = p / CPR;
            const int c = (p % CPR) ^ mn_swz(k);
            g = X + (int64_t)(k0 + k) * ld + min(r0 + c * 8, rows - 8);
        }
        __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)(tile + blk * 512), 16, 0, 0);
    }
}

// MFMA fragment: rows row0 + (lane & 31), k = kk + (lane >> 5) * 8 + 0..7
template <int R, bool KCONTIG>
DEVI bf16x8 frag_any(const uint16_t* tile, int row0, int kk, int lane) {
    if constexpr (KCONTIG) {
        const int r = row0 + (lane & 31);
        const int c = (kk >> 3) + (lane >> 5);
        return *reinterpret_cast<const bf16x8*>(tile + r * BK + ((c ^ (r & 7)) << 3));
    } else {
        const int j = lane & 15, g = lane >> 4;
        const int m = row0 + 16 * (g & 1) + 4 * (j & 3);
        const int k = kk + (g >> 1) * 8 + (j >> 2);
        const int o0 = k * R + ((((m >> 3) ^ mn_swz(k)) << 3) | (m & 7));
        const int o1 = (k + 4) * R + ((((m >> 3) ^ mn_swz(k + 4)) << 3) | (m & 7));
        i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o0));
        i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o1));
        i16x4 xy[2] = {x, y};
        return *reinterpret_cast<bf16x8*>(xy);
    }
}

template <int BM, int BN, int FM, int FN, int TM, int TN, bool AK, bool BKC>
DEVI void mfma_any(f32x16 (&acc)[FM][FN], const uint16_t* As, const uint16_t* Bs, int wm, int wn, int lane) {
    bf16x8 a[2][FM], b[2][FN];
#pragma unroll
    for (int i = 0; i < FM; i++) a[0][i] = frag_any<BM, AK>(As, wm * TM + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < FN; j++) b[0][j] = frag_any<BN, BKC>(Bs, wn * TN + j * 32, 0, lane);
    __builtin_amdgcn_sched_group_barrier(0x100, (FM + FN) * (AK && BKC ? 1 : 2), 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
        if (ks + 1 < BK / 16) {
#pragma unroll
            for (int i = 0; i < FM; i++) a[(ks + 1) & 1][i] = frag_any<BM, AK>(As, wm * TM + i * 32, (ks + 1) * 16, lane);
#pragma unroll
            for (int j = 0; j < FN; j++) b[(ks + 1) & 1][j] = frag_any<BN, BKC>(Bs, wn * TN + j * 32, (ks + 1) * 16, lane);
        }
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[ks & 1][j], a[ks & 1][i], acc[i][j], 0, 0, 0);
        if (ks + 1 < BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, (FM + FN) * (AK && BKC ? 1 : 2), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
    }
}

template <int BM, int BN, int NW, int NS, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_big_kernel(GemmArgs g, int kchunk) {
    constexpr int WAVES_M = 2, WAVES_N = NW / 2;
    constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N, FM = TM / 32, FN = TN / 32;
    static_assert(NS >= 2 && NS <= 3, "stages");
    __shared__ __attribute__((aligned(1024))) uint16_t sa0[BM * BK], sa1[BM * BK], sa2[NS > 2 ? BM * BK : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t sb0[BN * BK], sb1[BN * BK], sb2[NS > 2 ? BN * BK : 8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int bid = blockIdx.x;
    const int total = gridDim.x;
    if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
    constexpr int GM = 8;
    const int group = bid / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in = bid % (GM * tiles_n);
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

    const int kbeg = blockIdx.y * kchunk;
    const int nk = (min(g.K, kbeg + kchunk) - kbeg) / BK;
    const int klast = kbeg + (nk - 1) * BK;
    constexpr int LPS = (BM + BN) / (8 * NW);  // direct loads per thread per stage

#define BIG_DMA(SA, SB, K0)                                                  \
    do {                                                                     \
        dma_any<BM, NW, AK>(SA, A, g.lda, m0, g.M, (K0), wave, lane);        \
        dma_any<BN, NW, BKC>(SB, B, g.ldb, n0, g.N, (K0), wave, lane);       \
    } while (0)
#define BIG_STEP(SA, SB, NA, NB, KT)                                                     \
    do {                                                                                 \
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<(NS - 2) * LPS>());                         \
        __builtin_amdgcn_s_barrier();                                                    \
        asm volatile("" ::: "memory");                                                   \
        BIG_DMA(NA, NB, min(kbeg + ((KT) + NS - 1) * BK, klast));                        \
        mfma_any<BM, BN, FM, FN, TM, TN, AK, BKC>(acc, SA, SB, wm, wn, lane);            \
    } while (0)

    BIG_DMA(sa0, sb0, kbeg);
    if constexpr (NS > 2) BIG_DMA(sa1, sb1, min(kbeg + BK, klast));
    int kt = 0;
    if constexpr (NS == 2) {
        for (; kt + 2 <= nk; kt += 2) {
            BIG_STEP(sa0, sb0, sa1, sb1, kt);
            BIG_STEP(sa1, sb1, sa0, sb0, kt + 1);
        }
        if (kt < nk) BIG_STEP(sa0, sb0, sa1, sb1, kt);
    } else {
        for (; kt + 3 <= nk; kt += 3) {
            BIG_STEP(sa0, sb0, sa2, sb2, kt);
            BIG_STEP(sa1, sb1, sa0, sb0, kt + 1);
            BIG_STEP(sa2, sb2, sa1, sb1, kt + 2);
        }
        if (kt < nk) { BIG_STEP(sa0, sb0, sa2, sb2, kt); kt++; }
        if (kt < nk) BIG_STEP(sa1, sb1, sa0, sb0, kt);
    }
#undef BIG_DMA
#undef BIG_STEP
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());  // no load may still be writing LDS at exit

    epilogue<EPI>(g, acc, m0 + wm * TM, n0 + wn * TN, lane);
}

template <int BM, int BN, int NW, int NS, bool AK, bool BKC, int EPI>
hipError_t launch_big(const GemmArgs& g, hipStream_t s, int splits = 1, int kchunk = 0) {
    dim3 grid(cdiv(g.M, BM) * cdiv(g.N, BN), splits);
    gemm_big_kernel<BM, BN, NW, NS, AK, BKC, EPI><<<grid, NW * 64, 0, s>>>(g, kchunk ? kchunk : g.K);
    return hipGetLastError();
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
    // Tile choice per form and width, from timings at the GPT-2 shapes:
    // 256x256 (8 waves) for wide outputs and the backward-data products,
    // 128x128 direct-load tiles for mid widths, the register-staged 128x128
    // kernel for the narrow (N = C) forward products.
    if (g.a_kcontig && g.b_kcontig) {
#define NT_CASES(BIG)                                                                                   \
    switch (g.epi) {                                                                                    \
        case EPI_STORE: return BIG(EPI_STORE);                                                          \
        case EPI_BIAS: return BIG(EPI_BIAS);                                                            \
        case EPI_BIAS_RESID: return BIG(EPI_BIAS_RESID);                                                \
        case EPI_BIAS_GELU: return BIG(EPI_BIAS_GELU);                                                  \
        default: return hipErrorInvalidValue;                                                           \
    }
#define NT_256(E) launch_big<256, 256, 8, 2, true, true, E>(g, s)
#define NT_128(E) launch_big<128, 128, 4, 2, true, true, E>(g, s)
#define NT_REG(E) launch<128, 128, 2, true, true, E>(g, s)
        if (g.N >= 3072) NT_CASES(NT_256)
        if (g.N >= 1536) NT_CASES(NT_128)
        NT_CASES(NT_REG)
#undef NT_CASES
#undef NT_256
#undef NT_128
#undef NT_REG
    }
    if (g.a_kcontig && !g.b_kcontig) {
        switch (g.epi) {
            case EPI_STORE: return launch_big<256, 256, 8, 2, true, false, EPI_STORE>(g, s);
            case EPI_GELU_BWD: return launch_big<256, 256, 8, 2, true, false, EPI_GELU_BWD>(g, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (!g.a_kcontig && !g.b_kcontig && g.epi == EPI_ACC_F32) {
        if (cdiv(g.M, 256) * cdiv(g.N, 256) >= 256)  // wide output (the classifier): no split needed
            return launch_big<256, 256, 8, 2, false, false, EPI_ACC_F32>(g, s);
        int S, kc;
        splitk_plan(g.M, g.N, g.K, &S, &kc);
        if (S > 1 && g.ws && (size_t)S * g.M * g.N * 4 <= g.ws_bytes && g.N % 4 == 0 && g.ldo % 4 == 0) {
            hipError_t e = launch_big<128, 128, 4, 3, false, false, EPI_PARTIAL>(g, s, S, kc);
            if (e != hipSuccess) return e;
            int64_t n4 = (int64_t)g.M * g.N / 4;
            unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
            splitk_reduce_kernel<<<blocks, 256, 0, s>>>((float*)g.out, g.ldo, g.ws, S, g.M, g.N);
            return hipGetLastError();
        }
        return launch_big<128, 128, 4, 3, false, false, EPI_ACC_F32>(g, s);
    }
    return hipErrorInvalidValue;
}

size_t gemm_splitk_ws_bytes(int M, int N, int K) {
    int S, kc;
    splitk_plan(M, N, K, &S, &kc);
    return S > 1 ? (size_t)S * M * N * 4 : 0;
}
