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
// the query's keys sits in lane l ^ 32: one half swap combines them).  The
// accumulator registers 8j..8j+7 of a lane hold 8 distinct keys, which is
// exactly the B-operand shape of the next product (O^T = V^T P^T), so P
// never leaves registers.
//
// The softmax work per score element is what bounds these kernels (the
// exponential runs at a quarter of the FMA rate), so each element costs the
// minimum: one FMA into the raw v_exp_f32 (arguments are <= 0, so the
// denormal range handling of exp2f is not needed), the causal mask only on
// the one diagonal block of each wave, and in the forward the output is
// rescaled only when the running max grows by more than 2^8 (the final
// normalisation uses the same stale max for numerator and denominator, and
// probabilities up to 256 are harmless in fp32 and bf16).
//
// Tiles stream through LDS in their natural [row][64] layout (16-byte chunk c
// of row r in slot c ^ aswz(r), see below), loaded by global_load_lds_dwordx4 straight
// from global memory, two stages deep.  A product that needs a tile
// transposed (V^T, K^T, dO and Q as B operands) reads it with
// ds_read_b64_tr_b16: within a 16-lane group, lane i receives element i%4 of
// the 8-byte reads of lanes 4e + i/4 (e = 0..3), so lanes reading rows
// k0..k0+3 at columns m0 + 4(j%4) hand lane i the column m0 + i over those
// four rows.
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
constexpr int TILE = KB * HS;  // elements of one 64 x 64 tile
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_LOG2 = 8.f;  // lazy rescale threshold of the running max (log2 units)
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

DEVI bf16x8 to_bf16x8(const f32x16& v, int base) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (bf16)v[base + i];
    return r;
}

DEVI f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

DEVI f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; r++) z[r] = 0.f;
    return z;
}

DEVI u32x4 ld_row(const bf16* p, bool ok) {
    return ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0, 0, 0, 0};
}

// s_waitcnt immediate (gfx9 encoding): vmcnt <= N, lgkmcnt = 0, expcnt free
template <int N> constexpr int vmcnt_imm() { return (N & 15) | ((N >> 4) << 14) | (7 << 4); }

// LDS swizzle of the [row][64] tiles (64 banks of 4 bytes: two 128-byte rows
// per bank window): chunk c of row r sits in slot c ^ aswz(r), aswz(r) =
// rot(r/2 mod 8) with rot moving bit 0 to bit 2.  Sixteen rows read at one
// chunk (a 16-byte fragment read) then cover all 16 bank groups, and so do
// the four rows x four-chunk groups a transposing read touches at once
// (rows two apart differ in bit 2 of the swizzle).
DEVI int aswz(int r) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
}

// rows [r0, r0+64) x 64 channels of a [*, ld] matrix into a swizzled tile;
// each of the 4 waves issues 2 loads of 1 KB (8 rows each).  Callers stream
// whole 64-row blocks of a sequence whose length is a multiple of 64, so
// every row read exists.  The loads go through a buffer resource whose base
// is the matrix at row r0 (wave-uniform), and each lane carries the 32-bit
// byte offsets of its two 16-byte chunks, computed once (row 0 of the wave's
// 8-row blocks): measured faster than per-lane 64-bit addresses (forward
// 3%, backward 2%).  dword3 0x00020000: raw 32-bit data format;
// num_records at its maximum (every offset here is in bounds).
struct LanePtr {
    const bf16* base;
    uint32_t off[2];  // bytes from base
};
DEVI LanePtr dma_lane_ptr(const bf16* base, int ld, int wave, int lane) {
    LanePtr lp;
    lp.base = base;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int row = wave * 16 + i * 8 + (lane >> 3);  // tile row this lane lands in
        const int c = (lane & 7) ^ aswz(row);             // chunk landing in slot lane & 7
        lp.off[i] = (uint32_t)(row * ld + c * 8) * 2u;
    }
    return lp;
}
DEVI void dma_tile(bf16* tile, const LanePtr& src, int ld, int r0, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer builtins exist only in the device pass
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(src.base + (int64_t)r0 * ld), (short)0, -1, 0x00020000);
#pragma unroll
    for (int i = 0; i < 2; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(tile + (wave * 2 + i) * 512), 16, src.off[i], 0, 0,
                                                 0);
#endif
}

// 8 consecutive channels chunk*8.. of tile row `row` (one 16-byte read)
DEVI bf16x8 frag_row(const bf16* tile, int row, int chunk) {
    return *reinterpret_cast<const bf16x8*>(tile + row * HS + ((chunk ^ aswz(row)) << 3));
}

// 4 consecutive rows krow..krow+3 of column mcol + (lane % 16), transposed
// out of the tile (krow, mcol uniform over each 16-lane group)
DEVI i16x4 tr4(const bf16* tile, int krow, int mcol, int lane) {
    const int j = lane & 15;
    const int r = krow + (j >> 2), c = mcol + 4 * (j & 3);
    const int off = r * HS + ((((c >> 3) ^ aswz(r)) << 3) | (c & 7));
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off));
}

// Operand of a 32x32x16 product whose 16 reduction slots are the tile rows
// held by accumulator registers 8j..8j+7 of a lane in half hi (rows
// t32 + 16j + 4hi + 0..3 and t32 + 16j + 8 + 4hi + 0..3) and whose 32 rows or
// columns are channels dt*32 + lane%32: two transposing reads.
DEVI bf16x8 frag_tr(const bf16* tile, int t32, int j, int dt, int lane) {
    const int krow = t32 + 16 * j + 4 * (lane >> 5);
    const int mcol = dt * 32 + 16 * ((lane >> 4) & 1);
    i16x4 xy[2] = {tr4(tile, krow, mcol, lane), tr4(tile, krow + 8, mcol, lane)};
    return *reinterpret_cast<bf16x8*>(xy);
}

// accumulator register r of lane half hi covers row 8*(r/4) + 4*hi + r%4
DEVI int acc_row(int r, int hi) { return ((r >> 2) << 3) + (hi << 2) + (r & 3); }
DEVI constexpr int acc_off(int r) { return ((r >> 2) << 3) + (r & 3); }  // acc_row less the half term

DEVI float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane l's value and that of lane l ^ 32, ordered by lane half: {x of lane
// l % 32, x of lane l % 32 + 32} in every lane.  v_permlane32_swap exchanges
// the halves in the VALU, without the LDS round trip of a shuffle (forward
// 42.0 -> 40.9 us per layer at B=16, T=1024, C=768, identical outputs).
struct HalfPair { float lo, hi; };
DEVI HalfPair half_pair(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Block placement on a 1-D grid of nblk blocks per (batch, head).
// Workgroup L runs on XCD L % 8.  When the grid splits evenly, each XCD
// takes a contiguous range of heads (their K/V or Q/dO re-reads then hit
// that XCD's L2), and within it the blocks go out rank-major: rank 0 of
// every head first, then rank 1, ...; callers give rank 0 to their longest
// block, so the short blocks fill the tail of the launch.  Returns the rank
// and the head's (b, h).
DEVI int place_block(int nblk, int NH, int* h, int* b) {
    const int total = gridDim.x;
    const int L = blockIdx.x;
    int bh, rank;
    const int per_xcd = total >> 3;
    if ((total & 7) == 0 && per_xcd % nblk == 0) {
        const int heads = per_xcd / nblk;  // heads per XCD
        const int pos = L >> 3;
        rank = pos / heads;
        bh = (L & 7) * heads + pos % heads;
    } else {
        bh = L / nblk;
        rank = L % nblk;
    }
    *h = bh % NH;
    *b = bh / NH;
    return rank;
}

// Two LDS stages, distinct __shared__ arrays (so that alias analysis keeps
// the reads of one stage independent of the loads in flight into the other).
// A step waits for its own stage's loads (the only ones in flight), passes a
// raw barrier (every wave is then done with the previous step's stage), and
// requests the next step's tiles into that stage before its own products.
// Two stages measured faster than three (forward 43.6 -> 42.0, backward
// 154.6 -> 146 us per layer at B=16, T=1024, C=768): the next tile still has
// a whole step to arrive.
#define STAGE_SYNC()                                          \
    do {                                                      \
        __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());           \
        __builtin_amdgcn_s_barrier();                         \
        asm volatile("" ::: "memory");                        \
    } while (0)

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void flash_fwd_kernel(bf16* out, float* lse, const bf16* qkv, int T, int C, int NH) {
    __shared__ __attribute__((aligned(1024))) bf16 k0s[TILE], k1s[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 v0s[TILE], v1s[TILE];
    const int nqb = (T + QB - 1) / QB;
    int h, b;
    const int qblk = nqb - 1 - place_block(nqb, NH, &h, &b);  // longest rows first
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const LanePtr kbase = dma_lane_ptr(base + C + h * HS, C3, w, lane);
    const LanePtr vbase = dma_lane_ptr(base + 2 * C + h * HS, C3, w, lane);
    const int q0 = qblk * QB + w * 32;
    const int q = q0 + lq;

    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        u32x4 v = ld_row(base + (int64_t)q * C3 + h * HS + ks * 16 + hi * 8, q < T);
        qf[ks] = *reinterpret_cast<bf16x8*>(&v);
    }
    f32x16 o[2] = {zero16(), zero16()};
    float m_run = -INFINITY, l_run = 0.f;
    const float sc = 0.125f * LOG2E;  // 1/sqrt(64), in log2 units

    const int kend = min(T, qblk * QB + QB);
    const int nkb = (kend + KB - 1) / KB;
    const int klast = (nkb - 1) * KB;

    auto step = [&](const bf16* Ks, const bf16* Vs, bf16* NK, bf16* NV, int kb) {
        STAGE_SYNC();
        const int kn = min((kb + 1) * KB, klast);
        dma_tile(NK, kbase, C3, kn, w);
        dma_tile(NV, vbase, C3, kn, w);
        const int k0 = kb * KB;
        // every key of the block is in the future of every query of the wave,
        // or the wave's queries are all past the end of the sequence
        if (k0 > q0 + 31 || q0 >= T) return;
        f32x16 s[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            s[t] = zero16();
#pragma unroll
            for (int ks = 0; ks < 4; ks++) s[t] = mfma(frag_row(Ks, t * 32 + lq, ks * 2 + hi), qf[ks], s[t]);
        }
        if (k0 + KB - 1 > q0) {  // the wave's diagonal block: key k0 + t*32 + acc_row(r) > q is masked
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int thr = q - k0 - t * 32 - 4 * hi;
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (acc_off(r) > thr) s[t][r] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[t][r]);
        {
            const HalfPair p = half_pair(mx);
            mx = fmaxf(p.lo, p.hi) * sc;
        }
        if (__any(mx > m_run + RESCALE_LOG2)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2_raw(m_run - m_new);  // 0 on the first block (m_run = -inf)
            l_run *= alpha;
#pragma unroll
            for (int r = 0; r < 16; r++) { o[0][r] *= alpha; o[1][r] *= alpha; }
            m_run = m_new;
        }
        const float nm = -m_run;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float pr = exp2_raw(fmaf(s[t][r], sc, nm));
                s[t][r] = pr;
                l_run += pr;  // this half's keys only: the halves are combined at the end
            }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const bf16x8 pb = to_bf16x8(s[t], 8 * j);
#pragma unroll
                for (int dt = 0; dt < 2; dt++) o[dt] = mfma(frag_tr(Vs, t * 32, j, dt, lane), pb, o[dt]);
            }
    };
    dma_tile(k0s, kbase, C3, 0, w);
    dma_tile(v0s, vbase, C3, 0, w);
    int kb = 0;
    for (; kb + 2 <= nkb; kb += 2) {
        step(k0s, v0s, k1s, v1s, kb);
        step(k1s, v1s, k0s, v0s, kb + 1);
    }
    if (kb < nkb) step(k0s, v0s, k1s, v1s, kb);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());  // no load may still be writing LDS at exit

    {
        const HalfPair p = half_pair(l_run);
        l_run = p.lo + p.hi;
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
        if (hi == 0) lse[((int64_t)b * NH + h) * T + q] = (m_run + __log2f(l_run)) * LN2;
    }
}

// ---------------------------------------------------------------------------
// Dout[row] = -rowsum(dO o O) and Lout[row] = -lse * log2(e), for the dK/dV kernel
// bpart (optional): per-(batch, 128-row block) column sums of the dq / dk / dv
// written, one row [3C] per block: the partials of the qkv bias gradient.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_bwd_dq_kernel(bf16* dqkv, float* Dout, float* Lout, const bf16* dout,
                                                           const bf16* qkv, const bf16* out, const float* lse, int T,
                                                           int C, int NH, float* bpart) {
    __shared__ __attribute__((aligned(1024))) bf16 k0s[TILE], k1s[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 v0s[TILE], v1s[TILE];
    const int nqb = (T + QB - 1) / QB;
    int h, b;
    const int qblk = nqb - 1 - place_block(nqb, NH, &h, &b);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const LanePtr kbase = dma_lane_ptr(base + C + h * HS, C3, w, lane);
    const LanePtr vbase = dma_lane_ptr(base + 2 * C + h * HS, C3, w, lane);
    const int q0 = qblk * QB + w * 32;
    const int q = q0 + lq;
    const bool qok = q < T;

    bf16x8 qf[4], dof[4];
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const int d = ks * 16 + hi * 8;
        u32x4 v = ld_row(base + (int64_t)q * C3 + h * HS + d, qok);
        qf[ks] = *reinterpret_cast<bf16x8*>(&v);
        u32x4 g = ld_row(dout + ((int64_t)b * T + q) * C + h * HS + d, qok);
        dof[ks] = *reinterpret_cast<bf16x8*>(&g);
        u32x4 ov = ld_row(out + ((int64_t)b * T + q) * C + h * HS + d, qok);
        const bf16x8 of = *reinterpret_cast<bf16x8*>(&ov);
#pragma unroll
        for (int i = 0; i < 8; i++) dsum += (float)dof[ks][i] * (float)of[i];
    }
    const float Dq = dsum + __shfl_xor(dsum, 32, 64);
    const int64_t ri = ((int64_t)b * NH + h) * T + q;
    const float nl2 = qok ? -lse[ri] * LOG2E : 0.f;
    if (qok && hi == 0) { Dout[ri] = -Dq; Lout[ri] = nl2; }
    // dP^T - D straight out of the matrix core: its accumulators start at -D
    // (the query's, the same in every register of the lane)
    f32x16 negD;
#pragma unroll
    for (int r = 0; r < 16; r++) negD[r] = -Dq;
    const float sc = 0.125f * LOG2E;

    f32x16 dq[2] = {zero16(), zero16()};
    const int kend = min(T, qblk * QB + QB);
    const int nkb = (kend + KB - 1) / KB;
    const int klast = (nkb - 1) * KB;

    auto step = [&](const bf16* Ks, const bf16* Vs, bf16* NK, bf16* NV, int kb) {
        STAGE_SYNC();
        const int kn = min((kb + 1) * KB, klast);
        dma_tile(NK, kbase, C3, kn, w);
        dma_tile(NV, vbase, C3, kn, w);
        const int k0 = kb * KB;
        if (k0 > q0 + 31 || q0 >= T) return;
        f32x16 s[2], dp[2];
#pragma unroll
        for (int t = 0; t < 2; t++) {
            s[t] = zero16();
            dp[t] = negD;
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                s[t] = mfma(frag_row(Ks, t * 32 + lq, ks * 2 + hi), qf[ks], s[t]);
                dp[t] = mfma(frag_row(Vs, t * 32 + lq, ks * 2 + hi), dof[ks], dp[t]);
            }
        }
        if (k0 + KB - 1 > q0) {  // diagonal block
#pragma unroll
            for (int t = 0; t < 2; t++) {
                const int thr = q - k0 - t * 32 - 4 * hi;
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (acc_off(r) > thr) s[t][r] = -INFINITY;
            }
        }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float pr = exp2_raw(fmaf(s[t][r], sc, nl2));
                s[t][r] = pr * dp[t][r];  // dS^T = P^T (dP^T - D)
            }
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const bf16x8 dsb = to_bf16x8(s[t], 8 * j);
#pragma unroll
                for (int dt = 0; dt < 2; dt++) dq[dt] = mfma(frag_tr(Ks, t * 32, j, dt, lane), dsb, dq[dt]);
            }
    };
    dma_tile(k0s, kbase, C3, 0, w);
    dma_tile(v0s, vbase, C3, 0, w);
    int kb = 0;
    for (; kb + 2 <= nkb; kb += 2) {
        step(k0s, v0s, k1s, v1s, kb);
        step(k1s, v1s, k0s, v0s, kb + 1);
    }
    if (kb < nkb) step(k0s, v0s, k1s, v1s, kb);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());

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
    if (bpart) {
        // sum of the stored dq over the block's queries.  Each wave transposes
        // its 32 queries x 64 channels through its own 8 KB stage array (free
        // once every wave is past the loop): row q, float4 slot c4 ^ (q & 15),
        // so 16 lanes writing one column hit 16 distinct bank groups; then
        // lane c sums column c over the 32 rows and the 4 waves are added in
        // a fixed order.
        __shared__ float cred[4][HS];
        __syncthreads();
        float* tq = reinterpret_cast<float*>(w == 0 ? k0s : w == 1 ? k1s : w == 2 ? v0s : v1s);
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int c4 = dt * 8 + 2 * g + hi;  // channels dt*32 + 8g + 4hi .. +3
                float4 v;
                v.x = qok ? (float)(bf16)(dq[dt][4 * g + 0] * 0.125f) : 0.f;
                v.y = qok ? (float)(bf16)(dq[dt][4 * g + 1] * 0.125f) : 0.f;
                v.z = qok ? (float)(bf16)(dq[dt][4 * g + 2] * 0.125f) : 0.f;
                v.w = qok ? (float)(bf16)(dq[dt][4 * g + 3] * 0.125f) : 0.f;
                *reinterpret_cast<float4*>(tq + lq * HS + ((c4 ^ (lq & 15)) << 2)) = v;
            }
        float t = 0.f;
#pragma unroll
        for (int qq = 0; qq < 32; qq++) t += tq[qq * HS + ((((lane >> 2) ^ (qq & 15)) << 2) | (lane & 3))];
        cred[w][lane] = t;
        __syncthreads();
        if (tid < HS)
            bpart[((int64_t)b * nqb + qblk) * C3 + h * HS + tid] = cred[0][tid] + cred[1][tid] + cred[2][tid] + cred[3][tid];
    }
}

// ---------------------------------------------------------------------------
// Per-query statistics of a 64-query block, one 1 KB load per wave into the
// wave's own region: lanes 0..15 bring L[q0 .. q0+63] (-lse log2 e), lanes
// 16..31 -D[...], lanes 32..63 repeat lane 0's read (unused).  Needs T % 64 == 0.
DEVI const float* stats_lane_ptr(const float* L, const float* D, int64_t rbase, int lane) {
    return lane < 16 ? L + rbase + 4 * lane : lane < 32 ? D + rbase + 4 * (lane - 16) : L + rbase;
}
DEVI void dma_stats(float* region, const float* src, int q0) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)(src + q0), (lds_void_t*)region, 16, 0, 0);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_bwd_dkdv_kernel(
    bf16* dqkv, const float* Din, const float* Lin, const bf16* dout, const bf16* qkv, int T, int C, int NH,
    float* bpart) {
    __shared__ __attribute__((aligned(1024))) bf16 q0s[TILE], q1s[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 o0s[TILE], o1s[TILE];  // dO
    __shared__ __attribute__((aligned(1024))) float st0[4 * 256], st1[4 * 256];
    int h, b;
    const int kblk = place_block((T + QB - 1) / QB, NH, &h, &b);  // the first key blocks see the most queries
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hi = lane >> 5, lq = lane & 31;
    const int C3 = 3 * C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const LanePtr qbase = dma_lane_ptr(base + h * HS, C3, w, lane);
    const LanePtr dbase = dma_lane_ptr(dout + (int64_t)b * T * C + h * HS, C, w, lane);
    const int k0 = kblk * QB + w * 32;
    const int key = k0 + lq;

    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const int d = ks * 16 + hi * 8;
        u32x4 v = ld_row(base + (int64_t)key * C3 + C + h * HS + d, key < T);
        kf[ks] = *reinterpret_cast<bf16x8*>(&v);
        u32x4 u = ld_row(base + (int64_t)key * C3 + 2 * C + h * HS + d, key < T);
        vf[ks] = *reinterpret_cast<bf16x8*>(&u);
    }
    f32x16 dk[2] = {zero16(), zero16()}, dv[2] = {zero16(), zero16()};
    const float sc = 0.125f * LOG2E;
    const int64_t rbase = ((int64_t)b * NH + h) * T;
    const float* sbase = stats_lane_ptr(Lin, Din, rbase, lane);
    const int qstart = (kblk * QB / KB) * KB;
    const int nqb = (T - qstart + KB - 1) / KB;
    const int qlast = qstart + (nqb - 1) * KB;

    auto load = [&](bf16* Q, bf16* O, float* S, int qs0) {
        dma_tile(Q, qbase, C3, qs0, w);
        dma_tile(O, dbase, C, qs0, w);
        dma_stats(S + w * 256, sbase, qs0);
    };
    auto step = [&](const bf16* Qs, const bf16* Os, const float* S, bf16* NQ, bf16* NO, float* NS_, int i) {
        STAGE_SYNC();
        load(NQ, NO, NS_, min(qstart + (i + 1) * KB, qlast));
        const int qs0 = qstart + i * KB;
        // every query of the block precedes every key of the wave, or the
        // wave's keys are all past the end of the sequence
        if (qs0 + KB - 1 < k0 || k0 >= T) return;
        const bool diag = qs0 < k0 + 31;
        const float* sl = S + w * 256;
        const float* sd = sl + 64;
        // one 32-query half at a time keeps only 32 score registers live
#pragma unroll
        for (int t = 0; t < 2; t++) {
            // dP - D straight out of the matrix core: the accumulators start at
            // -D of each register's query (registers 4g..4g+3 cover 4
            // consecutive queries: one float4 of the stats each)
            f32x16 s = zero16(), dp;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 D4 = *reinterpret_cast<const float4*>(sd + t * 32 + 8 * g + 4 * hi);
                dp[4 * g] = D4.x; dp[4 * g + 1] = D4.y; dp[4 * g + 2] = D4.z; dp[4 * g + 3] = D4.w;
            }
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                s = mfma(frag_row(Qs, t * 32 + lq, ks * 2 + hi), kf[ks], s);
                dp = mfma(frag_row(Os, t * 32 + lq, ks * 2 + hi), vf[ks], dp);
            }
            // s[r]: query qs0 + t*32 + acc_row(r), key `key`; registers 4g..4g+3
            // cover 4 consecutive queries, so their L and D come as one float4
            if (diag) {  // query qs0 + t*32 + acc_row(r) < key is masked
                const int thr = key - qs0 - t * 32 - 4 * hi;
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (acc_off(r) < thr) s[r] = -INFINITY;
            }
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int ql0 = t * 32 + 8 * g + 4 * hi;
                const float4 L4 = *reinterpret_cast<const float4*>(sl + ql0);
                const float Lv[4] = {L4.x, L4.y, L4.z, L4.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r = 4 * g + e;
                    const float pr = exp2_raw(fmaf(s[r], sc, Lv[e]));
                    s[r] = pr;
                    dp[r] = pr * dp[r];  // dS = P (dP - D)
                }
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const bf16x8 pa = to_bf16x8(s, 8 * j);
                const bf16x8 da = to_bf16x8(dp, 8 * j);
#pragma unroll
                for (int dt = 0; dt < 2; dt++) {
                    dv[dt] = mfma(pa, frag_tr(Os, t * 32, j, dt, lane), dv[dt]);
                    dk[dt] = mfma(da, frag_tr(Qs, t * 32, j, dt, lane), dk[dt]);
                }
            }
        }
    };
    load(q0s, o0s, st0, qstart);
    int i = 0;
    for (; i + 2 <= nqb; i += 2) {
        step(q0s, o0s, st0, q1s, o1s, st1, i);
        step(q1s, o1s, st1, q0s, o0s, st0, i + 1);
    }
    if (i < nqb) step(q0s, o0s, st0, q1s, o1s, st1, i);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());

    // dk[dt][r], dv[dt][r]: key k0 + acc_row(r), channel dt*32 + lq
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int kk = k0 + acc_row(r, hi);
        if (kk < T) {
            bf16* row = dqkv + ((int64_t)b * T + kk) * C3 + h * HS;
#pragma unroll
            for (int dt = 0; dt < 2; dt++) {
                row[C + dt * 32 + lq] = (bf16)(dk[dt][r] * 0.125f);
                row[2 * C + dt * 32 + lq] = (bf16)dv[dt][r];
            }
        }
    }
    if (bpart) {
        // sums of the stored dk, dv over the block's keys: the 16 registers
        // and two halves of a lane's channel, then the 4 waves
        __shared__ float kred[4][HS], vred[4][HS];
#pragma unroll
        for (int dt = 0; dt < 2; dt++) {
            float tk = 0.f, tv = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (k0 + acc_row(r, hi) < T) {
                    tk += (float)(bf16)(dk[dt][r] * 0.125f);
                    tv += (float)(bf16)dv[dt][r];
                }
            tk += __shfl_xor(tk, 32, 64);
            tv += __shfl_xor(tv, 32, 64);
            if (hi == 0) {
                kred[w][dt * 32 + lq] = tk;
                vred[w][dt * 32 + lq] = tv;
            }
        }
        __syncthreads();
        if (tid < HS) {
            float* prow = bpart + ((int64_t)b * ((T + QB - 1) / QB) + kblk) * C3 + h * HS + tid;
            prow[C] = kred[0][tid] + kred[1][tid] + kred[2][tid] + kred[3][tid];
            prow[2 * C] = vred[0][tid] + vred[1][tid] + vred[2][tid] + vred[3][tid];
        }
    }
}

#undef STAGE_SYNC

}  // namespace

hipError_t flash_attention_fwd(bf16* out, float* lse, const bf16* qkv, int B, int T, int C, int NH, hipStream_t s) {
    if (C / NH != HS || C % NH || T % KB) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((T + QB - 1) / QB * NH * B);
    flash_fwd_kernel<<<grid, 256, 0, s>>>(out, lse, qkv, T, C, NH);
    return hipGetLastError();
}

int flash_attention_bias_rows(int B, int T) { return B * ((T + QB - 1) / QB); }

hipError_t flash_attention_bwd(bf16* dqkv, const bf16* dout, const bf16* qkv, const bf16* out, const float* lse,
                               float* dbuf, int B, int T, int C, int NH, float* bpart, hipStream_t s) {
    if (C / NH != HS || C % NH || T % KB) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((T + QB - 1) / QB * NH * B);
    const int64_t rows = (int64_t)B * NH * T;
    flash_bwd_dq_kernel<<<grid, 256, 0, s>>>(dqkv, dbuf, dbuf + rows, dout, qkv, out, lse, T, C, NH, bpart);
    flash_bwd_dkdv_kernel<<<grid, 256, 0, s>>>(dqkv, dbuf, dbuf + rows, dout, qkv, T, C, NH, bpart);
    return hipGetLastError();
}
