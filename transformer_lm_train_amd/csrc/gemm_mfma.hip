// bf16 matrix products on the gfx950 matrix cores.
//
// One kernel for the three operand forms of a training step (X W^T forward,
// dY W backward-data, dY^T X backward-weight): operands go global -> LDS by
// direct loads in the layout they have in memory (k-contiguous rows, or
// rows contiguous along m / n for the transposed operands, read back with
// transposing LDS reads), NS stages deep; 32x32x16 bf16 MFMAs with fp32
// accumulators; a fused epilogue (bias, residual, GELU and its derivative,
// fp32 gradient accumulation) that leaves through LDS so that global
// accesses are whole row segments.  The weight gradients of a training step,
// whose outputs are small next to their reduction over all tokens, run as
// one grouped launch over the tiles of every product, each tile over the
// whole reduction; a single weight-gradient product may instead split the
// reduction over workgroups and add the partial tiles in a fixed order
// (deterministic).  Block ids are remapped so that the tiles one XCD (one
// L2) runs are neighbours sharing operand panels.  Wide single products with a
// plain store (the classifier's logits) instead run a persistent schedule
// whose k-contiguous operands move through registers in 64-deep k-steps.
#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace {

constexpr int KALIGN = 64;  // K, and every split-K chunk, is a multiple of this

// LDS stages and schedule of the tile shapes in use (256x256 for the forward
// and backward-data products and the grouped weight gradients, 128x128 for
// split weight gradients).
#ifndef GEMM_BIG_NS
#define GEMM_BIG_NS 4
#endif
#ifndef GEMM_BIG_XPF
#define GEMM_BIG_XPF false
#endif
#ifndef GEMM_GROUP_NS
#define GEMM_GROUP_NS 4
#endif
#ifndef GEMM_GROUP_XPF
#define GEMM_GROUP_XPF false
#endif
#ifndef GEMM_PERS_BIAS
#define GEMM_PERS_BIAS 1
#endif
#ifndef GEMM_PERS_GELU
#define GEMM_PERS_GELU 1
#endif
#ifndef GEMM_SPLIT_NS
#define GEMM_SPLIT_NS 5
#endif
#ifndef GEMM_SPLIT_XPF
#define GEMM_SPLIT_XPF true
#endif

constexpr int EPI_PARTIAL = 100;  // split-K partial tile into g.ws[split][M][N]

// The products run the MFMA with the operands swapped, acc = B A^T: register
// r of lane l of the 32x32 block (i, j) then holds row i*32 + l % 32 and
// column j*32 + 8*(r/4) + 4*(l/32) + r%4, so each group of 4 registers is 4
// consecutive columns of one row.
//
// Row-major epilogue through LDS: the wave writes RH rows (32, or 16 when
// its region is small) of one 32-row accumulator block into its own LDS
// region (pitch TN + 4 floats, so the 16 rows a 16-byte access group touches
// fall in distinct bank groups), reads them back so that each lane owns 8
// consecutive outputs of one row, and finishes them with 16-byte bf16 /
// 32-byte fp32 global accesses: LPR lanes cover a whole row segment, so
// every access instruction moves full cache lines instead of 32 scattered
// 16-byte pieces.  LDS order within one wave is
// program order, so the region needs no synchronisation between the blocks.
template <int RH, int TN> constexpr int red_bytes() { return RH * (TN + 4) * 4; }

// Bias values of the 8 columns each lane finishes, per column group: the
// epilogue's layout (lane % LPR covers 8 columns of each CG-wide group).
template <int EPI, int FN>
DEVI void epilogue_bias(const GemmArgs& g, float* b8, int ncol0, int lane) {
    constexpr int TN = FN * 32;
    constexpr int CG = TN % 64 == 0 ? 64 : 32;
    constexpr int NCG = TN / CG, LPR = CG / 8;
    constexpr bool BIAS = EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_D;
#pragma unroll
    for (int cg = 0; cg < NCG; cg++) {
        const int n = ncol0 + cg * CG + (lane % LPR) * 8;
#pragma unroll
        for (int e = 0; e < 8; e++) b8[cg * 8 + e] = 0.f;
        if (BIAS && g.bias && n < g.N) {
            const float4 u = *reinterpret_cast<const float4*>(g.bias + n);
            const float4 v = *reinterpret_cast<const float4*>(g.bias + n + 4);
            b8[cg * 8 + 0] = u.x; b8[cg * 8 + 1] = u.y; b8[cg * 8 + 2] = u.z; b8[cg * 8 + 3] = u.w;
            b8[cg * 8 + 4] = v.x; b8[cg * 8 + 5] = v.y; b8[cg * 8 + 6] = v.z; b8[cg * 8 + 7] = v.w;
        }
    }
}

// PRE: the bias values were loaded beforehand (epilogue_bias) into bpre.
template <int EPI, int RH, int FM, int FN, bool PRE = false>
DEVI void epilogue_rows(const GemmArgs& g, const f32x16 (&acc)[FM][FN], float* red, int mrow0, int ncol0, int split,
                        int prow, int lane, const float* bpre = nullptr) {
    constexpr int TN = FN * 32, P = TN + 4;
    constexpr int CG = TN % 64 == 0 ? 64 : 32;  // columns read back per group
    constexpr int NCG = TN / CG;
    constexpr int LPR = CG / 8;    // lanes per output row segment
    constexpr int RPI = 64 / LPR;  // rows per access instruction
    constexpr int NR = RH / RPI;   // row groups per pass
    static_assert(RH == 32 || RH == 16, "rows per pass");
    constexpr bool BIAS = EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_GELU_D;
    typedef bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    const int hi = lane >> 5, l32 = lane & 31;
    constexpr bool CSUM = EPI == EPI_GELU_BWD || EPI == EPI_MUL_AUX;  // column sums of the outputs, if g.colsum_ws
    float cs[NCG][8];
#pragma unroll
    for (int cg = 0; cg < NCG; cg++)
#pragma unroll
        for (int e = 0; e < 8; e++) cs[cg][e] = 0.f;
    float b8[NCG][8];
    if constexpr (PRE) {
#pragma unroll
        for (int cg = 0; cg < NCG; cg++)
#pragma unroll
            for (int e = 0; e < 8; e++) b8[cg][e] = bpre[cg * 8 + e];
    } else {
        epilogue_bias<EPI, FN>(g, &b8[0][0], ncol0, lane);
    }
#pragma unroll
    for (int pass = 0; pass < FM * (32 / RH); pass++) {
        const int i = pass / (32 / RH), h = pass % (32 / RH);  // rows h*RH .. of block i
        // operands of this pass's outputs, requested before the LDS round trip
        bf16x8_t r16[NCG][NR];
        float4 r32[NCG][NR][2];
#pragma unroll
        for (int cg = 0; cg < NCG; cg++)
#pragma unroll
            for (int rr = 0; rr < NR; rr++) {
                const int m = mrow0 + i * 32 + h * RH + rr * RPI + lane / LPR;
                const int n = ncol0 + cg * CG + (lane % LPR) * 8;
                const bool ok = m < g.M && n < g.N;
                const int64_t o = (int64_t)m * g.ldo + n;
                if constexpr (EPI == EPI_BIAS_RESID)
                    r16[cg][rr] = ok ? *reinterpret_cast<const bf16x8_t*>((const bf16*)g.resid + o) : bf16x8_t{};
                if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_MUL_AUX)
                    r16[cg][rr] = ok ? *reinterpret_cast<const bf16x8_t*>((const bf16*)g.aux + o) : bf16x8_t{};
                if constexpr (EPI == EPI_ACC_F32) {
                    const bool rd = ok && !g.acc_overwrite;
                    r32[cg][rr][0] = rd ? *reinterpret_cast<const float4*>((const float*)g.out + o)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
                    r32[cg][rr][1] = rd ? *reinterpret_cast<const float4*>((const float*)g.out + o + 4)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        if (RH == 32 || (l32 >> 4) == h) {
            const int wr = l32 % RH;
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    *reinterpret_cast<float4*>(red + wr * P + j * 32 + q * 8 + hi * 4) =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
#pragma unroll
        for (int cg = 0; cg < NCG; cg++)
#pragma unroll
            for (int rr = 0; rr < NR; rr++) {
                const int row = rr * RPI + lane / LPR;
                const int cl = cg * CG + (lane % LPR) * 8;
                const int m = mrow0 + i * 32 + h * RH + row;
                const int n = ncol0 + cl;
                const float4 u = *reinterpret_cast<const float4*>(red + row * P + cl);
                const float4 v = *reinterpret_cast<const float4*>(red + row * P + cl + 4);
                float y[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
                if constexpr (EPI == EPI_CE_STATS) {
                    // the LPR lanes of a row segment hold its CG columns: their
                    // max (log2 units) and sum of 2^(z log2 e - max) over the
                    // columns of the real vocabulary, combined in a fixed
                    // butterfly order; every lane takes part in the shuffles
                    constexpr float L2E = 1.4426950408889634f;
                    float mx = -INFINITY;
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        if (n + e < g.ce_V) mx = fmaxf(mx, y[e] * L2E);
#pragma unroll
                    for (int off = 1; off < LPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
                    float se = 0.f;
                    if (mx != -INFINITY) {
#pragma unroll
                        for (int e = 0; e < 8; e++)
                            if (n + e < g.ce_V) se += __builtin_amdgcn_exp2f(fmaf(y[e], L2E, -mx));
                    }
#pragma unroll
                    for (int off = 1; off < LPR; off <<= 1) se += __shfl_xor(se, off, 64);
                    if (m < g.M) {
                        // (the last tile column's waves past N hold no group)
                        if (lane % LPR == 0 && ncol0 + cg * CG < g.N)
                            g.ce_stats[(int64_t)m * g.ce_ld + (ncol0 + cg * CG) / CG] = make_float2(mx, se);
                        const int t = g.ce_targets[m];
#pragma unroll
                        for (int e = 0; e < 8; e++)
                            if (n + e == t) g.ce_zt[m] = y[e];
                    }
                    continue;
                }
                if (m >= g.M || n >= g.N) continue;
                if constexpr (EPI == EPI_CE_GRAD) {
                    constexpr float L2E = 1.4426950408889634f;
                    const int t = g.ce_targets[m];
                    const float l2 = g.ce_lse2[m];
                    bf16x8_t d;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        float x = n + e < g.ce_V ? __builtin_amdgcn_exp2f(fmaf(y[e], L2E, -l2)) * g.ce_scale : 0.f;
                        if (n + e == t) x -= g.ce_scale;
                        d[e] = (bf16)x;
                    }
                    *reinterpret_cast<bf16x8_t*>((bf16*)g.out + (int64_t)m * g.ldo + n) = d;
                    continue;
                }
                const int64_t o = (int64_t)m * g.ldo + n;
                if constexpr (EPI == EPI_PARTIAL) {
                    float* w = g.ws + ((int64_t)split * g.M + m) * g.N + n;
                    *reinterpret_cast<float4*>(w) = u;
                    *reinterpret_cast<float4*>(w + 4) = v;
                    continue;
                }
                if constexpr (EPI == EPI_ACC_F32) {
                    const float4 a0 = r32[cg][rr][0], a1 = r32[cg][rr][1];
                    float* w = (float*)g.out + o;
                    *reinterpret_cast<float4*>(w) = make_float4(a0.x + y[0], a0.y + y[1], a0.z + y[2], a0.w + y[3]);
                    *reinterpret_cast<float4*>(w + 4) = make_float4(a1.x + y[4], a1.y + y[5], a1.z + y[6], a1.w + y[7]);
                    continue;
                }
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    if constexpr (BIAS) y[e] += b8[cg][e];
                    if constexpr (EPI == EPI_BIAS_RESID) y[e] += (float)r16[cg][rr][e];
                    if constexpr (EPI == EPI_GELU_BWD) y[e] *= gelu_grad_f((float)r16[cg][rr][e]);
                    if constexpr (EPI == EPI_MUL_AUX) y[e] *= (float)r16[cg][rr][e];
                }
                bf16x8_t out;
                if constexpr (EPI == EPI_BIAS_GELU_D) {
                    // GELU' (read by the backward, long after: non-temporal, as
                    // the pre-activation below) and GELU (the next product's input)
                    bf16x8_t act;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        float a, d;
                        gelu_and_grad(y[e], a, d);
                        act[e] = (bf16)a;
                        out[e] = (bf16)d;
                    }
                    __builtin_nontemporal_store(out, reinterpret_cast<bf16x8_t*>((bf16*)g.out + o));
                    *reinterpret_cast<bf16x8_t*>((bf16*)g.out2 + o) = act;
                    continue;
                }
#pragma unroll
                for (int e = 0; e < 8; e++) out[e] = (bf16)y[e];
                if constexpr (EPI == EPI_BIAS_GELU)
                    // the pre-activation is read only by the backward, long
                    // after: a non-temporal store keeps it from displacing
                    // the GELU output the next product reads (fc forward
                    // ~7% faster)
                    __builtin_nontemporal_store(out, reinterpret_cast<bf16x8_t*>((bf16*)g.out + o));
                else
                    *reinterpret_cast<bf16x8_t*>((bf16*)g.out + o) = out;
                if constexpr (CSUM) {
#pragma unroll
                    for (int e = 0; e < 8; e++) cs[cg][e] += (float)out[e];
                }
                if constexpr (EPI == EPI_BIAS_GELU) {
                    // GELU of the stored (bf16) pre-activation, which a backward
                    // that recomputes this output starts from as well
#pragma unroll
                    for (int e = 0; e < 8; e++) out[e] = (bf16)gelu_f((float)out[e]);
                    *reinterpret_cast<bf16x8_t*>((bf16*)g.out2 + o) = out;
                }
            }
    }
    if constexpr (CSUM) {
        if (g.colsum_ws) {
            // lanes l, l + LPR, l + 2 LPR, ... hold the same columns: combine
            // them (fixed butterfly order), then lanes 0 .. LPR-1 write the
            // wave's partial row
#pragma unroll
            for (int cg = 0; cg < NCG; cg++)
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    float t = cs[cg][e];
#pragma unroll
                    for (int off = LPR; off < 64; off <<= 1) t += __shfl_xor(t, off, 64);
                    cs[cg][e] = t;
                }
            if (lane < LPR) {
#pragma unroll
                for (int cg = 0; cg < NCG; cg++) {
                    const int n = ncol0 + cg * CG + lane * 8;
                    if (n < g.N) {
                        float* w = g.colsum_ws + (int64_t)prow * g.N + n;
                        *reinterpret_cast<float4*>(w) = make_float4(cs[cg][0], cs[cg][1], cs[cg][2], cs[cg][3]);
                        *reinterpret_cast<float4*>(w + 4) = make_float4(cs[cg][4], cs[cg][5], cs[cg][6], cs[cg][7]);
                    }
                }
            }
        }
    }
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
// Direct-to-LDS kernel: every operand goes global -> LDS by
// global_load_lds_dwordx4, in the layout it has in memory, NS stages deep with
// explicit vmcnt waits and raw barriers, k-step KB (32 or 64).
// LDS has 64 banks of 4 bytes, so a conflict-free read instruction must spread
// each group of lanes served together over all 256 bytes of a bank window:
//  - k-contiguous operand: LDS [row][KB]; the 16-byte chunk c of row r sits in
//    slot c ^ kswz(r), which puts the 16 rows read by 16 lanes (one chunk
//    each) in 16 distinct 16-byte bank groups.  Fragment = one ds_read_b128.
//  - mn-contiguous operand: LDS [k][R] (R = tile rows); chunk c of k-row k sits
//    in slot mn_slot<R>(c, k), which puts the four k-rows a transposing read
//    touches at once in four distinct 64-byte quarters.  Fragment = two
//    ds_read_b64_tr_b16: within each 16-lane group that instruction hands
//    lane i element (i % 4) of the 8-byte read of lane 4e + i/4 as its element
//    e; so when lane j reads X[k0 + j/4][m0 + 4(j%4) .. +3], lane i receives
//    X[k0..k0+3][m0+i], four consecutive k of one row: the MFMA fragment.
// WAVES_M x (NW / WAVES_M) waves, each owning a TM x TN block of 32x32
// accumulators.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int KB> DEVI int kswz(int r) {
    if constexpr (KB == 64) return (r >> 1) & 7;  // 2 rows of 128 B per bank window
    else return (r >> 2) & 3;                     // 4 rows of 64 B per bank window
}
DEVI int mnswz(int k) { return (k & 3) << 2; }
// Slot of 16-byte chunk c of k-row k in an mn-contiguous tile R elements wide.
// R a multiple of 128 (rows a multiple of 256 bytes): c ^ ((k & 3) << 2), the
// four k-rows a transposing read touches at once in four distinct 64-byte
// quarters.
// R = 192 (24 chunks, 384-byte rows, which already put k-rows k and k+1 128
// bytes apart in the 256-byte bank window): chunks rotated by 4 when bit 1 of
// k is set, which moves k-rows k+2, k+3 by another 64 bytes; the four rows
// land at 0, 128, 64, 192 (or, past the wrap, 0, 128, 192, 64) bytes.
template <int R> DEVI int mn_slot(int c, int k) {
    static_assert(R % 128 == 0 || R == 192, "mn-contiguous tile width");
    if constexpr (R != 192) return c ^ mnswz(k);
    else {
        const int s = c + ((k & 2) << 1);
        return s >= 24 ? s - 24 : s;
    }
}
template <int R> DEVI int mn_chunk(int s, int k) {  // inverse of mn_slot
    if constexpr (R != 192) return s ^ mnswz(k);
    else {
        const int c = s - ((k & 2) << 1);
        return c < 0 ? c + 24 : c;
    }
}

// One 16-byte direct load per lane through a buffer resource over the
// operand (base: the operand at the stage's k offset; byte_off: the lane's
// offset).  The k offset then lives in the resource's scalar base and the
// lanes carry 32-bit offsets instead of 64-bit addresses.  dword3 0x00020000:
// raw 32-bit data format, no swizzle; num_records at its maximum (every
// offset here is in bounds).  The builtins exist only in the device pass.
DEVI void buffer_load_lds16(const bf16* base, uint32_t byte_off, uint16_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, -1, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds, 16, byte_off, 0, 0, 0);
#endif
}

// Per-lane element offsets of the direct loads one wave issues per stage for
// tile rows [r0, r0+ROWS) of X; the k-step only adds a uniform offset.  A
// k-contiguous tile is [row][KB] (R rows staged, ROWS <= R loaded); an
// mn-contiguous one [k][R] (ROWS == R: its k-rows are R wide in LDS).  A
// stage takes NIT wave instructions of 1 KB.  When they split evenly over the
// waves, wave w issues instructions w*NIW .. w*NIW+NIW-1; otherwise (the
// 192-wide tiles' B) instruction q goes to wave q % NW, so the first NIT % NW
// waves issue one more (count()).  Rows past the end re-read the last row (in
// bounds); they only feed accumulators the epilogue never stores.
// BUF: buffer loads (buffer_load_lds16) instead of global ones; measured per
// operand form in the training step: faster for both operands of the forward
// products and for every mn-contiguous operand, slower for the k-contiguous
// A of the backward-data products, which keeps global loads.
template <int R, int NW, int KB, bool KCONTIG, int ROWS = R, bool BUF = false>
struct Dma {
    static constexpr int NIT = ROWS * KB / 512;
    static_assert(NIT >= 1 && NIT * 512 == ROWS * KB && ROWS <= R && (KCONTIG || ROWS == R), "tile vs waves");
    static constexpr bool EVEN = NIT % NW == 0;

    static constexpr int NIW = (NIT + NW - 1) / NW;  // most instructions one wave issues
    static DEVI int slot(int wave, int i) { return EVEN ? wave * NIW + i : wave + NW * i; }
    // instructions wave issues (uniform value)
    static DEVI int count(int wave) { return EVEN ? NIW : (wave < NIT % NW ? NIW : NIW - 1); }
    uint32_t off[NIW];
    DEVI void init(int ld, int r0, int rows, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NIW; i++) {
            const int p = min(slot(wave, i), NIT - 1) * 64 + lane;  // 16-byte chunk position in the tile
            if constexpr (KCONTIG) {
                constexpr int CPR = KB / 8;
                const int r = p / CPR;
                const int c = (p % CPR) ^ kswz<KB>(r);
                off[i] = (uint32_t)(min(r0 + r, rows - 1) * ld + c * 8);
            } else {
                constexpr int CPR = R / 8;
                const int k = p / CPR;
                const int c = mn_chunk<R>(p % CPR, k);
                off[i] = (uint32_t)(k * ld + min(r0 + c * 8, rows - 8));
            }
        }
    }
    // kofs: k0 (k-contiguous) or k0 * ld (mn-contiguous).  CNT = count(wave),
    // known at compile time in the caller's copy of the loop, so that no load
    // sits under a branch (the compiler then keeps track of which stage array
    // each direct load writes, and LDS reads of the others need not wait).
    template <int CNT> DEVI void issue(uint16_t* tile, const bf16* X, int64_t kofs, int wave) const {
        static_assert(CNT == NIW || (!EVEN && CNT == NIW - 1), "load count");
        const bf16* base = X + kofs;
#pragma unroll
        for (int i = 0; i < CNT; i++) {
            if constexpr (BUF)
                buffer_load_lds16(base, off[i] * 2u, tile + slot(wave, i) * 512);
            else
                __builtin_amdgcn_global_load_lds((glb_void_t*)(base + off[i]),
                                                 (lds_void_t*)(tile + slot(wave, i) * 512), 16, 0, 0);
        }
    }
};

// Register-staged loads of a k-contiguous operand, k-step 64: each wave
// instruction reads 8 rows x 128 bytes (8 lanes per row, one whole L2 line
// per row) into registers; store() then writes them into the stage tile
// [row][64] with chunk c of row r in slot c ^ kswz<64>(r).  ROWS rows of the
// stage are loaded; instruction i of wave w covers tile rows
// 8 (w NIW + i) .. +7.  The loads go through a buffer resource over the
// operand's rows, so rows past its end read as zero (they only feed
// accumulators the epilogue never stores); each lane keeps one byte offset,
// and the instruction and k offsets are uniform.
template <int NW, int ROWS>
struct RegDma {
    static constexpr int KB = 64;
    static constexpr int NIT = ROWS * KB / 512;
    static_assert(NIT % NW == 0, "register loads split evenly over the waves");
    static constexpr int NIW = NIT / NW;
#if defined(__HIP_DEVICE_COMPILE__)
    __amdgpu_buffer_rsrc_t rs;
#endif
    uint32_t goff;      // lane byte offset in the wave's first instruction
    uint32_t rstep;     // bytes between instructions (8 rows)
    uint32_t loff[2];   // lane LDS element offset in an even / odd instruction
    int q0;             // the wave's first instruction index
    bf16x8 v[NIW];
    DEVI void init(const bf16* X, int64_t ld, int r0, int rows, int wave, int lane) {
        const int l = lane >> 3, c = lane & 7;
        q0 = wave * NIW;
#if defined(__HIP_DEVICE_COMPILE__)
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(X), (short)0, (int)(rows * ld * 2), 0x00020000);
#endif
        goff = (uint32_t)(((int64_t)(r0 + q0 * 8 + l) * ld + c * 8) * 2);
        rstep = (uint32_t)(8 * ld * 2);
        // kswz<64>(8q + l) = ((8q + l) >> 1) & 7 = 4 (q & 1) + (l >> 1)
        loff[0] = (uint32_t)(l * KB + ((c ^ (l >> 1)) << 3));
        loff[1] = (uint32_t)(l * KB + ((c ^ (4 + (l >> 1))) << 3));
    }
    DEVI void load(int k0) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int i = 0; i < NIW; i++) {
            typedef int i32x4 __attribute__((ext_vector_type(4)));
            const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, goff, (int)(i * rstep + k0 * 2), 0);
            v[i] = *reinterpret_cast<const bf16x8*>(&x);
        }
#endif
    }
    DEVI void store(uint16_t* tile) const {
#pragma unroll
        for (int i = 0; i < NIW; i++) {
            const int q = q0 + i;
            *reinterpret_cast<bf16x8*>(tile + q * 512 + loff[q & 1]) = v[i];
        }
    }
};

// MFMA fragment: rows row0 + (lane & 31), k = kk + (lane >> 5) * 8 + 0..7
template <int R, int KB, bool KCONTIG>
DEVI bf16x8 frag_any(const uint16_t* tile, int row0, int kk, int lane) {
    if constexpr (KCONTIG) {
        const int r = row0 + (lane & 31);
        const int c = (kk >> 3) + (lane >> 5);
        return *reinterpret_cast<const bf16x8*>(tile + r * KB + ((c ^ kswz<KB>(r)) << 3));
    } else {
        const int j = lane & 15, g = lane >> 4;
        const int m = row0 + 16 * (g & 1) + 4 * (j & 3);
        const int k = kk + (g >> 1) * 8 + (j >> 2);
        const int o0 = k * R + ((mn_slot<R>(m >> 3, k) << 3) | (m & 7));
        const int o1 = (k + 4) * R + ((mn_slot<R>(m >> 3, k + 4) << 3) | (m & 7));
        i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o0));
        i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + o1));
        i16x4 xy[2] = {x, y};
        return *reinterpret_cast<bf16x8*>(xy);
    }
}

// Scheduling order of one sub-step: its NM MFMAs alternate with the NR LDS
// reads of the next sub-step (mask 0x008: MFMA, 0x100: DS read), so reads
// trickle out while the matrix core is busy and few are outstanding at once.
template <int NM, int NR, int Q = 0> DEVI void interleave_mfma_reads() {
    if constexpr (Q < NM || Q < NR) {
        if constexpr (Q < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (Q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        interleave_mfma_reads<NM, NR, Q + 1>();
    }
}

// One k-step of the wave's FM x FN block of 32x32 accumulators.  The
// fragments of sub-step s+1 are read while the MFMAs of sub-step s run.
// XPF: fa / fb hold the fragments of sub-step 0 on entry, and the last
// sub-step reads sub-step 0 of the next stage (nA / nB) into them, so the next
// k-step can start its MFMAs right after its barrier.  Otherwise sub-step 0
// is read here, after the barrier.
template <int BM, int BN, int KB, int FM, int FN, int TM, int TN, bool AK, bool BKC, bool XPF>
DEVI void mfma_step(f32x16 (&acc)[FM][FN], bf16x8 (&fa)[FM], bf16x8 (&fb)[FN], const uint16_t* As,
                    const uint16_t* Bs, const uint16_t* nA, const uint16_t* nB, int wm, int wn, int lane) {
    constexpr int KS = KB / 16;
    static_assert(KS % 2 == 0, "sub-steps come in pairs");
    constexpr int NRD = FM * (AK ? 1 : 2) + FN * (BKC ? 1 : 2);  // LDS read instructions per sub-step
    bf16x8 a[2][FM], b[2][FN];
    // fragment reads in the order of first use by the i-major MFMA loop
    // (a0, b0 .. b[FN-1], a1 .. a[FM-1]), so the next sub-step's first MFMAs
    // wait only for reads issued several MFMAs earlier
    auto read_frags = [&](bf16x8 (&ra)[FM], bf16x8 (&rb)[FN], const uint16_t* ta, const uint16_t* tb, int kk) {
        ra[0] = frag_any<BM, KB, AK>(ta, wm * TM, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; j++) rb[j] = frag_any<BN, KB, BKC>(tb, wn * TN + j * 32, kk, lane);
#pragma unroll
        for (int i = 1; i < FM; i++) ra[i] = frag_any<BM, KB, AK>(ta, wm * TM + i * 32, kk, lane);
    };
    if constexpr (XPF) {
#pragma unroll
        for (int i = 0; i < FM; i++) a[0][i] = fa[i];
#pragma unroll
        for (int j = 0; j < FN; j++) b[0][j] = fb[j];
    } else {
        read_frags(a[0], b[0], As, Bs, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const uint16_t* ta = ks + 1 < KS ? As : nA;
        const uint16_t* tb = ks + 1 < KS ? Bs : nB;
        const int kk = ks + 1 < KS ? (ks + 1) * 16 : 0;
        if (XPF || ks + 1 < KS) read_frags(a[(ks + 1) & 1], b[(ks + 1) & 1], ta, tb, kk);
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[ks & 1][j], a[ks & 1][i], acc[i][j], 0, 0, 0);
        if (XPF || ks + 1 < KS) interleave_mfma_reads<FM * FN, NRD>();
        else __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
    }
    if constexpr (XPF) {
#pragma unroll
        for (int i = 0; i < FM; i++) fa[i] = a[0][i];
#pragma unroll
        for (int j = 0; j < FN; j++) fb[j] = b[0][j];
    }
}

// OCC: waves per SIMD the register allocation targets (2: up to 256
// registers; 1: up to 512, accumulators in AGPRs).  BNV: output columns per
// tile when fewer than BN; the B operand is still staged BN rows wide (same
// load geometry, every wave issues the same loads), the rows past BNV land in
// LDS that no fragment reads.
// GROUPED: one launch over the tiles of several problems (see GroupSched).
template <int BM, int BN, int NW, int WAVES_M, int KB, int NS, bool XPF, bool AK, bool BKC, int EPI, int OCC = 2,
          int BNV = BN, bool GROUPED = false, bool RL = false, bool PERS = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void gemm_big_kernel(
    GemmArgs garg, int kchunk, GroupSched gs) {
    constexpr int WAVES_N = NW / WAVES_M;
    constexpr int TM = BM / WAVES_M, TN = BNV / WAVES_N, FM = TM / 32, FN = TN / 32;
    static_assert(BNV <= BN && TN % 32 == 0, "tile width");
    static_assert(RL ? (NS == 2 && KB == 64 && AK && BKC && !XPF && !GROUPED) : (NS >= 3 && NS <= 5), "stages");
    constexpr int SA = BM * KB, SB = BN * KB;
    // one array per stage (alias analysis then keeps the reads of one stage
    // independent of the loads in flight into another)
    __shared__ __attribute__((aligned(1024))) uint16_t sa0[SA], sa1[SA], sa2[NS > 2 ? SA : 8], sa3[NS > 3 ? SA : 8],
        sa4[NS > 4 ? SA : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t sb0[SB], sb1[SB], sb2[NS > 2 ? SB : 8], sb3[NS > 3 ? SB : 8],
        sb4[NS > 4 ? SB : 8];
    auto stA = [&](auto J) -> uint16_t* {
        constexpr int j = decltype(J)::value % NS;
        if constexpr (j == 0) return sa0;
        else if constexpr (j == 1) return sa1;
        else if constexpr (j == 2) return sa2;
        else if constexpr (j == 3) return sa3;
        else return sa4;
    };
    auto stB = [&](auto J) -> uint16_t* {
        constexpr int j = decltype(J)::value % NS;
        if constexpr (j == 0) return sb0;
        else if constexpr (j == 1) return sb1;
        else if constexpr (j == 2) return sb2;
        else if constexpr (j == 3) return sb3;
        else return sb4;
    };
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: per-wave load counts branch on it
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // Workgroup L (linear id, x fastest) runs on XCD L % 8.  Give each XCD a
    // contiguous range of the work list (split-major (split, tile) pairs, or
    // the grouped tile list), so that the tiles sharing operand panels (same
    // split, neighbouring tiles) share one L2.
    GemmArgs g;
    int m0, n0, split;
    int half_slot = -1;  // grouped: workspace slot of a half-reduction tile
    if constexpr (GROUPED) {
        const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
        const uint32_t t = gs.tiles[xcd * (gs.full + 2 * gs.split) + pos];
        if (t == ~0u) return;
        g = gs.probs[t >> 22];
        g.acc_overwrite = gs.overwrite != 0;
        m0 = (int)((t >> 11) & 0x7FF) * BM;
        n0 = (int)(t & 0x7FF) * BNV;
        split = 0;
        kchunk = g.K;
        if (pos >= gs.full) {  // the XCD's last round: each tile in two halves of the reduction
            const int q = pos - gs.full;
            split = q & 1;
            kchunk = g.K / 2;
            half_slot = 2 * (xcd * gs.split + (q >> 1)) + split;
        }
    } else if constexpr (PERS) {
        g = garg;
        split = 0;
        m0 = n0 = 0;
    } else {
        g = garg;
        const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BNV - 1) / BNV;
        const int tiles = gridDim.x;
        int work = blockIdx.x + blockIdx.y * tiles;
        const int total = tiles * gridDim.y;
        if ((total & 7) == 0) work = (work & 7) * (total >> 3) + (work >> 3);
        split = work / tiles;
        const int bid = work % tiles;
        constexpr int GM = 8;
        const int gi = bid / (GM * tiles_n);
        const int first_m = gi * GM;
        const int gsz = min(tiles_m - first_m, GM);
        const int in = bid % (GM * tiles_n);
        m0 = (first_m + in % gsz) * BM;
        n0 = (in / gsz) * BNV;
    }
    const bf16* A = (const bf16*)g.a;
    const bf16* B = (const bf16*)g.b;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    const int kbeg = split * kchunk;
    const int nk = (min(g.K, kbeg + kchunk) - kbeg) / KB;
    const int klast = kbeg + (nk - 1) * KB;
    // B is loaded for the BNV rows (columns) the tile uses: k-contiguous into
    // the [BN][KB] stage, mn-contiguous as [KB][BNV] (pitch BPITCH)
    constexpr int BPITCH = BKC ? BN : BNV;
    typedef Dma<BM, NW, KB, AK, BM, !(AK && !BKC)> DmaA;  // global loads for the A of dY W only
    typedef Dma<BPITCH, NW, KB, BKC, BNV, true> DmaB;
    DmaA da;
    DmaB db;
    if constexpr (!RL) {
        da.init(g.lda, m0, g.M, wave, lane);
        db.init(g.ldb, n0, g.N, wave, lane);
    }
    // The main loop, for a wave that issues CB loads of B per stage (all
    // waves issue DmaA::NIW of A).  Where the waves' B counts differ, each
    // count gets its own copy of the loop (same barriers in both).
    bf16x8 fa[FM], fb[FN];
    auto main_loop = [&](auto CB_) {
        constexpr int CB = decltype(CB_)::value;
        constexpr int LPS = DmaA::NIW + CB;  // this wave's loads per stage
        auto dma = [&](uint16_t* ta, uint16_t* tb, int k0) {
            da.template issue<DmaA::NIW>(ta, A, AK ? (int64_t)k0 : (int64_t)k0 * g.lda, wave);
            db.template issue<CB>(tb, B, BKC ? (int64_t)k0 : (int64_t)k0 * g.ldb, wave);
        };
        // Step kt (stage kt % NS): wait for this wave's loads of k-step kt + 1
        // (XPF) or kt, barrier (that k-step is then in LDS for every wave, and
        // every wave is done with k-step kt - 1), load k-step kt + NS - 1 over
        // k-step kt - 1, then the MFMAs of k-step kt.  XPF starts them from
        // fragments already in registers and reads the first fragments of k-step
        // kt + 1 at the end, at the price of one k-step less of load latency cover.
        static_assert(!XPF || NS >= 3, "cross-barrier prefetch needs 3 stages");
        auto step = [&](auto J, int kt) {
            constexpr int j = decltype(J)::value;
            __builtin_amdgcn_s_waitcnt(vmcnt_imm<(XPF ? NS - 3 : NS - 2) * LPS>());
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            dma(stA(std::integral_constant<int, j + NS - 1>{}), stB(std::integral_constant<int, j + NS - 1>{}),
                min(kbeg + (kt + NS - 1) * KB, klast));
            mfma_step<BM, BPITCH, KB, FM, FN, TM, TN, AK, BKC, XPF>(acc, fa, fb, stA(J), stB(J),
                                                           stA(std::integral_constant<int, j + 1>{}),
                                                           stB(std::integral_constant<int, j + 1>{}), wm, wn, lane);
        };
        typedef std::integral_constant<int, 0> I0;
        typedef std::integral_constant<int, 1> I1;
        typedef std::integral_constant<int, 2> I2;
        typedef std::integral_constant<int, 3> I3;
        typedef std::integral_constant<int, 4> I4;

        dma(sa0, sb0, kbeg);
        dma(sa1, sb1, min(kbeg + KB, klast));
        if constexpr (NS > 3) dma(sa2, sb2, min(kbeg + 2 * KB, klast));
        if constexpr (NS > 4) dma(sa3, sb3, min(kbeg + 3 * KB, klast));
        if constexpr (XPF) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm<(NS - 2) * LPS>());  // k-step 0
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < FM; i++) fa[i] = frag_any<BM, KB, AK>(sa0, wm * TM + i * 32, 0, lane);
#pragma unroll
            for (int jj = 0; jj < FN; jj++) fb[jj] = frag_any<BPITCH, KB, BKC>(sb0, wn * TN + jj * 32, 0, lane);
        }
        int kt = 0;
        for (; kt + NS <= nk; kt += NS) {
            step(I0{}, kt);
            step(I1{}, kt + 1);
            step(I2{}, kt + 2);
            if constexpr (NS > 3) step(I3{}, kt + 3);
            if constexpr (NS > 4) step(I4{}, kt + 4);
        }
        if (kt < nk) { step(I0{}, kt); kt++; }
        if (kt < nk) { step(I1{}, kt); kt++; }
        if constexpr (NS > 3) if (kt < nk) { step(I2{}, kt); kt++; }
        if constexpr (NS > 4) if (kt < nk) { step(I3{}, kt); kt++; }
    };
    // The stage buffers become the epilogue's per-wave regions once every
    // wave is past its last LDS read.
    // (two stages: two regions in each stage array)
    constexpr int RBYTES = 2 * (BN < BM ? BN : BM) * KB / (NS == 2 ? 2 : 1);  // smallest region
    constexpr int RH = red_bytes<32, TN>() <= RBYTES ? 32 : 16;
    static_assert(NW <= 8 && NW <= 2 * NS * (NS == 2 ? 2 : 1) && red_bytes<RH, TN>() <= RBYTES,
                  "epilogue regions must fit the stage buffers");
    // persistent: the bias goes to registers before the next tile's loads,
    // behind which it would otherwise wait (loads complete in order)
    constexpr bool PREB = PERS && (EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU ||
                                   EPI == EPI_BIAS_GELU_D);
    constexpr int ENCG = TN % 64 == 0 ? TN / 64 : TN / 32;
    auto epilogue = [&](int m0, int n0, const float* bpre) {
        __syncthreads();
        uint16_t* region;
        if constexpr (NS == 2) {
            uint16_t* arr = (wave >> 1) == 0 ? sa0 : (wave >> 1) == 1 ? sb0 : (wave >> 1) == 2 ? sa1 : sb1;
            region = arr + (wave & 1) * (RBYTES / 2);
        } else switch (wave) {
            case 0: region = sa0; break;
            case 1: region = sb0; break;
            case 2: region = sa1; break;
            case 3: region = sb1; break;
            case 4: region = sa2; break;
            case 5: region = sb2; break;
            case 6: region = sa3; break;
            default: region = sb3; break;
        }
        if (GROUPED && half_slot >= 0) {
            // a half-reduction tile leaves its fp32 partial in its own slot
            GemmArgs h = g;
            h.out = gs.ws + (int64_t)half_slot * (BM * BNV);
            h.ldo = BNV;
            h.M = min(BM, g.M - m0);
            h.N = min(BNV, g.N - n0);
            h.acc_overwrite = true;
            epilogue_rows<EPI, RH>(h, acc, reinterpret_cast<float*>(region), wm * TM, wn * TN, 0, 0, lane);
        } else {
            epilogue_rows<EPI, RH, FM, FN, PREB>(g, acc, reinterpret_cast<float*>(region), m0 + wm * TM,
                                                 n0 + wn * TN, split, (m0 / BM) * WAVES_M + wm, lane, bpre);
        }
    };

    if constexpr (RL) {
        // Register-staged k-steps of 64 over two LDS stages: the registers
        // hold k-step kt + 1 while k-step kt runs out of LDS; at the start of
        // step kt they go to the other stage (free since the last barrier)
        // and k-step kt + 2 is requested into them.
        // PERS: one workgroup per CU slot takes, in turn, the tiles of its
        // XCD's contiguous range that the lock-step launch would give that
        // slot; the next tile's first k-step is requested before the current
        // tile's epilogue.
        const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BNV - 1) / BNV;
        auto tile_of = [&](int bid, int& tm0, int& tn0) {
            constexpr int GM = 8;
            const int gi = bid / (GM * tiles_n);
            const int first_m = gi * GM;
            const int gsz = min(tiles_m - first_m, GM);
            const int in = bid % (GM * tiles_n);
            tm0 = (first_m + in % gsz) * BM;
            tn0 = (in / gsz) * BNV;
        };
        int p_first = 0, p_count = 1, p_stride = 0;
        if constexpr (PERS) {
            const int total = tiles_m * tiles_n;
            const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, slots = gridDim.x >> 3;
            const int lo = (int)((int64_t)total * xcd / 8), hi = (int)((int64_t)total * (xcd + 1) / 8);
            if (lo + slot >= hi) return;
            p_first = lo + slot;
            p_stride = slots;
            p_count = (hi - p_first + slots - 1) / slots;
            tile_of(p_first, m0, n0);
        }
        RegDma<NW, BM> ra;
        RegDma<NW, BNV> rb;
        ra.init(A, g.lda, m0, g.M, wave, lane);
        rb.init(B, g.ldb, n0, g.N, wave, lane);
        ra.load(kbeg);
        rb.load(kbeg);
        constexpr int LGKM0 = 0xC07F;  // lgkmcnt = 0, vmcnt and expcnt unconstrained
        auto bar = [&]() {
            __builtin_amdgcn_s_waitcnt(LGKM0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        auto rstep = [&](uint16_t* cA, uint16_t* cB, uint16_t* oA, uint16_t* oB, int kt) {
            if (kt + 1 < nk) {
                ra.store(oA);
                rb.store(oB);
                if (kt + 2 < nk) {
                    ra.load(kbeg + (kt + 2) * KB);
                    rb.load(kbeg + (kt + 2) * KB);
                }
            }
            mfma_step<BM, BN, KB, FM, FN, TM, TN, true, true, false>(acc, fa, fb, cA, cB, oA, oB, wm, wn, lane);
            bar();
        };
        for (int it = 0; it < p_count; it++) {
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
            ra.store(sa0);
            rb.store(sb0);
            if (nk > 1) {
                ra.load(kbeg + KB);
                rb.load(kbeg + KB);
            }
            bar();
            for (int kt = 0; kt < nk; kt += 2) {
                rstep(sa0, sb0, sa1, sb1, kt);
                if (kt + 1 < nk) rstep(sa1, sb1, sa0, sb0, kt + 1);
            }
            const int cm0 = m0, cn0 = n0;
            float bpre[8 * ENCG];
            if constexpr (PREB) epilogue_bias<EPI, FN>(g, bpre, cn0 + wn * TN, lane);
            if (PERS && it + 1 < p_count) {
                tile_of(p_first + (it + 1) * p_stride, m0, n0);
                ra.init(A, g.lda, m0, g.M, wave, lane);
                rb.init(B, g.ldb, n0, g.N, wave, lane);
                ra.load(kbeg);
                rb.load(kbeg);
            }
            epilogue(cm0, cn0, bpre);
            if (PERS && it + 1 < p_count) __syncthreads();  // epilogue regions read before stage 0 is refilled
        }
        return;
    } else if constexpr (DmaB::EVEN) {
        main_loop(std::integral_constant<int, DmaB::NIW>{});
    } else {
        if (DmaB::count(wave) == DmaB::NIW) main_loop(std::integral_constant<int, DmaB::NIW>{});
        else main_loop(std::integral_constant<int, DmaB::NIW - 1>{});
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());  // no load may still be writing LDS at exit

    epilogue(m0, n0, nullptr);
}

// CUs of the current device (cached per device), rounded down to a multiple of 8.
int device_slots() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
        cache[dev] = cus / 8 * 8;
    }
    return cache[dev];
}

// The register-staged kernel (both operands k-contiguous, k-step 64, two LDS
// stages), one tile per workgroup.
template <int BM, int BN, int NW, int WAVES_M, int EPI, int BNV = BN>
hipError_t launch_rl(const GemmArgs& g, hipStream_t s) {
    gemm_big_kernel<BM, BN, NW, WAVES_M, 64, 2, false, true, true, EPI, 2, BNV, false, true, false>
        <<<(unsigned)(cdiv(g.M, BM) * cdiv(g.N, BNV)), NW * 64, 0, s>>>(g, g.K, GroupSched{});
    return hipGetLastError();
}

// The same kernel, persistent over wgs workgroups when the tiles outnumber them.
template <int BM, int BN, int NW, int WAVES_M, int EPI, int BNV = BN>
hipError_t launch_pers(const GemmArgs& g, hipStream_t s, int wgs) {
    const int tiles = (int)(cdiv(g.M, BM) * cdiv(g.N, BNV));
    if (tiles <= wgs)
        gemm_big_kernel<BM, BN, NW, WAVES_M, 64, 2, false, true, true, EPI, 2, BNV, false, true, false>
            <<<tiles, NW * 64, 0, s>>>(g, g.K, GroupSched{});
    else
        gemm_big_kernel<BM, BN, NW, WAVES_M, 64, 2, false, true, true, EPI, 2, BNV, false, true, true>
            <<<wgs, NW * 64, 0, s>>>(g, g.K, GroupSched{});
    return hipGetLastError();
}

template <int BM, int BN, int NW, int WAVES_M, int KB, int NS, bool XPF, bool AK, bool BKC, int EPI, int OCC = 2,
          int BNV = BN, bool RL = false>
hipError_t launch_big(const GemmArgs& g, hipStream_t s, int splits = 1, int kchunk = 0) {
    dim3 grid(cdiv(g.M, BM) * cdiv(g.N, BNV), splits);
    gemm_big_kernel<BM, BN, NW, WAVES_M, KB, NS, XPF, AK, BKC, EPI, OCC, BNV, false, RL>
        <<<grid, NW * 64, 0, s>>>(g, kchunk ? kchunk : g.K, GroupSched{});
    return hipGetLastError();
}

// Split of the reduction for the weight-gradient products, whose outputs are
// small (C x C .. 4C x C) next to their reduction over all B*T tokens:
// enough splits to give ~512 workgroups, each at least 4 k-steps long.
constexpr int SK_TM = 128, SK_TN = 128;  // tile of the split weight-gradient products
void splitk_plan(int M, int N, int K, int tm, int tn, int* splits, int* kchunk) {
    int tiles = (int)(cdiv(M, tm) * cdiv(N, tn));
    int S = (512 + tiles - 1) / tiles;
    int smax = K / 256;
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    // a grid that is a multiple of 8 lets the kernel keep each split on one XCD
    for (int t = S; t <= smax && t < 2 * S; t++)
        if ((tiles * t) % 8 == 0) { S = t; break; }
    int kc = (int)cdiv(K / KALIGN, S) * KALIGN;
    *kchunk = kc;
    *splits = (K + kc - 1) / kc;
}

__global__ void splitk_reduce_kernel(float* out, int64_t ldo, const float* ws, int S, int M, int N, int overwrite) {
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
        if (!overwrite) {
            const float4 cur = *o;
            acc.x += cur.x; acc.y += cur.y; acc.z += cur.z; acc.w += cur.w;
        }
        *o = acc;
    }
}

// bf16 out = sum over the S fp32 partial tiles ws[s][M][N], in split order
__global__ void splitk_reduce_bf16_kernel(bf16* out, int64_t ldo, const float* ws, int S, int M, int N) {
    const int64_t n4 = (int64_t)M * N / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i * 4;
        const int m = (int)(e / N), n = (int)(e % N);
        float4 acc = reinterpret_cast<const float4*>(ws)[i];
        for (int sp = 1; sp < S; sp++) {
            const float4 v = reinterpret_cast<const float4*>(ws + (int64_t)sp * M * N)[i];
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        typedef bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        *reinterpret_cast<bf16x4_t*>(out + (int64_t)m * ldo + n) = bf16x4_t{(bf16)acc.x, (bf16)acc.y, (bf16)acc.z, (bf16)acc.w};
    }
}

// Split of the reduction for a backward-data product with a plain store whose
// 192-wide tiles fill under one round of the 256 CUs (the fused classifier's
// chunks: 4096 rows x C outputs over a K of Vp): the split count S <= 8 that
// minimises rounds(tiles * S) / S, the fewest on a tie, each split at least
// 16 k-steps long.
void nn_split_plan(int M, int N, int K, int* splits, int* kchunk) {
    constexpr int CUS = 256;
    const int tiles = (int)(cdiv(M, 256) * cdiv(N, 192));
    int S = 1;
    if (tiles < CUS) {
        const int smax = std::min(8, std::max(1, K / (16 * 32)));
        double best = 1.0;
        for (int t = 2; t <= smax; t++) {
            const double cost = (double)((tiles * t + CUS - 1) / CUS) / t;
            if (cost < best - 1e-9) { best = cost; S = t; }
        }
    }
    const int kc = (int)cdiv(K / KALIGN, S) * KALIGN;
    *kchunk = kc;
    *splits = (K + kc - 1) / kc;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Whether 192-wide tiles finish in fewer (tile-size weighted) rounds of one
// workgroup per CU than 256-wide ones, by at least 10%.
bool use_192(int M, int N) {
    constexpr int CUS = 256;
    const int64_t tm = cdiv(M, 256);
    const int64_t r256 = (tm * cdiv(N, 256) + CUS - 1) / CUS;
    const int64_t r192 = (tm * cdiv(N, 192) + CUS - 1) / CUS;
    return 10 * 3 * r192 <= 9 * 4 * r256;
}

// Shapes and operands the direct-to-LDS kernel takes.
bool shape_ok(const GemmArgs& g) {
    if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % KALIGN || g.M % 8 || g.N % 8 || g.lda % 8 || g.ldb % 8)
        return false;
    if (!aligned16(g.a) || !aligned16(g.b)) return false;
    // per-lane operand offsets are 32-bit element counts
    const int64_t amax = g.a_kcontig ? (int64_t)(g.M - 1) * g.lda + g.K : (int64_t)(g.K - 1) * g.lda + g.M;
    const int64_t bmax = g.b_kcontig ? (int64_t)(g.N - 1) * g.ldb + g.K : (int64_t)(g.K - 1) * g.ldb + g.N;
    return amax < (int64_t)1 << 31 && bmax < (int64_t)1 << 31;
}

// The grouped weight-gradient products: 256 x 256 tiles, the whole reduction
// in each workgroup, out (fp32) += acc.
#define GROUPED_DW_KERNEL \
    gemm_big_kernel<256, 256, 8, 2, 32, GEMM_GROUP_NS, GEMM_GROUP_XPF, false, false, EPI_ACC_F32, 2, 256, true>
constexpr int GROUP_TILE = 256;

}  // namespace

int gemm_grouped_tiles(const GemmArgs* probs, int n, uint32_t* tiles, int cap) {
    if (n <= 0 || n > 1024) return -1;
    int cnt = 0;
    for (int p = 0; p < n; p++) {
        const GemmArgs& g = probs[p];
        if (!shape_ok(g) || g.a_kcontig || g.b_kcontig || g.epi != EPI_ACC_F32 || g.ldo % 4 ||
            ((uintptr_t)g.out & 15))
            return -1;
        const int tm = (int)cdiv(g.M, GROUP_TILE), tn = (int)cdiv(g.N, GROUP_TILE);
        if (tm > 2047 || tn > 2047) return -1;
        // row groups of 8 tiles, column by column within a group (as the
        // single-problem launch orders its tiles)
        constexpr int GM = 8;
        for (int bid = 0; bid < tm * tn; bid++) {
            const int first_m = bid / (GM * tn) * GM, gsz = std::min(tm - first_m, GM), in = bid % (GM * tn);
            if (tiles && cnt >= cap) return -1;
            if (tiles) tiles[cnt] = (uint32_t)p << 22 | (uint32_t)(first_m + in % gsz) << 11 | (uint32_t)(in / gsz);
            cnt++;
        }
    }
    for (; cnt % 8; cnt++) {
        if (tiles && cnt >= cap) return -1;
        if (tiles) tiles[cnt] = ~0u;
    }
    return cnt;
}

int gemm_grouped_schedule(const uint32_t* tiles, int n, int cus_per_xcd, uint32_t* sched, int cap,
                          uint32_t* split_tiles, int* full, int* split) {
    if (n <= 0 || n % 8) return -1;
    const int chunk = n / 8;
    int t = cus_per_xcd > 0 ? chunk % cus_per_xcd : 0;  // no CU count: no split
    if (2 * t > cus_per_xcd || t > GROUP_SPLIT_MAX) t = 0;
    const int F = chunk - t, len = 8 * (F + 2 * t);
    if (len > cap) return -1;
    for (int x = 0; x < 8; x++) {
        uint32_t* o = sched + x * (F + 2 * t);
        for (int i = 0; i < F; i++) o[i] = tiles[x * chunk + i];
        for (int q = 0; q < t; q++) {
            const uint32_t e = tiles[x * chunk + F + q];
            o[F + 2 * q] = o[F + 2 * q + 1] = e;
            split_tiles[x * t + q] = e;
        }
    }
    *full = F;
    *split = t;
    return len;
}

namespace {
// out[tile] (+)= P0 + P1 for each half-reduced tile j: block (j, 16-row group)
__global__ __launch_bounds__(256) void grouped_fixup_kernel(const GemmArgs* __restrict__ probs,
                                                            const uint32_t* __restrict__ split_tiles,
                                                            const float* __restrict__ ws, int overwrite) {
    constexpr int TS = GROUP_TILE;
    const int j = blockIdx.x;
    const uint32_t e = split_tiles[j];
    if (e == ~0u) return;
    const GemmArgs& g = probs[e >> 22];
    const int m0 = (int)((e >> 11) & 0x7FF) * TS, n0 = (int)(e & 0x7FF) * TS;
    const int mv = min(TS, g.M - m0), nv = min(TS, g.N - n0);
    const float* p0 = ws + (int64_t)(2 * j) * TS * TS;
    const float* p1 = p0 + TS * TS;
    float* out = (float*)g.out;
    for (int i = threadIdx.x; i < 16 * (TS / 4); i += 256) {
        const int r = blockIdx.y * 16 + i / (TS / 4), c = (i % (TS / 4)) * 4;
        if (r >= mv || c >= nv) continue;
        const float4 a = *reinterpret_cast<const float4*>(p0 + r * TS + c);
        const float4 b = *reinterpret_cast<const float4*>(p1 + r * TS + c);
        float4* o = reinterpret_cast<float4*>(out + (int64_t)(m0 + r) * g.ldo + n0 + c);
        float4 v = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        if (!overwrite) {
            const float4 cur = *o;
            v = make_float4(cur.x + v.x, cur.y + v.y, cur.z + v.z, cur.w + v.w);
        }
        *o = v;
    }
}
}  // namespace

hipError_t gemm_grouped_bf16(const GemmArgs* d_probs, const uint32_t* d_sched, int nsched, int full, int split,
                             const uint32_t* d_split_tiles, float* ws, bool overwrite, hipStream_t s) {
    if (nsched <= 0 || nsched % 8 || !d_probs || !d_sched || full < 0 || split < 0 ||
        nsched != 8 * (full + 2 * split) || (split > 0 && (!ws || !d_split_tiles)))
        return hipErrorInvalidValue;
    GroupSched gs{d_probs, d_sched, ws, full, split, overwrite ? 1 : 0};
    GROUPED_DW_KERNEL<<<nsched, 512, 0, s>>>(GemmArgs{}, 0, gs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || split == 0) return e;
    grouped_fixup_kernel<<<dim3(8 * split, GROUP_TILE / 16), 256, 0, s>>>(d_probs, d_split_tiles, ws, overwrite);
    return hipGetLastError();
}

hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s) {
    if (!shape_ok(g)) return hipErrorInvalidValue;
    // Tile choice from timings at the GPT-2 shapes on gfx950: the 256 x 256
    // tile (8 waves of 128 x 64, k-step 32, 4 LDS stages) leads or ties in
    // every forward and backward-data product.
#define BIG256(AKC, BKCC, E) launch_big<256, 256, 8, 2, 32, GEMM_BIG_NS, GEMM_BIG_XPF, AKC, BKCC, E>(g, s)
    // 192 output columns per tile (8 waves of 64 x 96) when that saves whole
    // rounds of workgroups: N = 768 gives 256 tiles instead of 192 for 256
    // CUs, N = 2304 three full rounds instead of 2.25.
#define BIG192(AKC, BKCC, E) launch_big<256, 256, 8, 4, 32, GEMM_BIG_NS, GEMM_BIG_XPF, AKC, BKCC, E, 2, 192>(g, s)
    const bool w192 = use_192(g.M, g.N);
    if (g.a_kcontig && g.b_kcontig) {
        // 256-wide tiles take the register-staged kernel (its buffer
        // resources span each operand's rows, whose byte extent must fit the
        // 31-bit record count): persistent for a plain store over at least
        // two rounds of tiles (the classifier's logits: 49 rounds at B*T =
        // 16384), for the fused classifier's statistics (as many rounds) and
        // for bias (+ GELU/GELU') over two rounds or more (the fc forward: 3
        // rounds at 124M, 104 -> 99.5 us per launch; the qkv forward at the
        // 350M width), whose bias is read before the next tile's loads are
        // requested; one tile per workgroup for the residual epilogue (its
        // persistent form spills).
        const bool rl = !w192 && (int64_t)g.M * g.lda * 2 < ((int64_t)1 << 31) &&
                        (int64_t)g.N * g.ldb * 2 < ((int64_t)1 << 31);
        const int wgs = device_slots();
        if (rl && g.epi == EPI_STORE && cdiv(g.M, 256) * cdiv(g.N, 256) >= 2 * wgs)
            return launch_pers<256, 256, 8, 2, EPI_STORE>(g, s, wgs);
#define RL256(E) launch_rl<256, 256, 8, 2, E>(g, s)
        switch (g.epi) {
            case EPI_STORE: return w192 ? BIG192(true, true, EPI_STORE) : BIG256(true, true, EPI_STORE);
            case EPI_BIAS:
                if (GEMM_PERS_BIAS && rl && cdiv(g.M, 256) * cdiv(g.N, 256) >= 2 * wgs)
                    return launch_pers<256, 256, 8, 2, EPI_BIAS>(g, s, wgs);
                return w192 ? BIG192(true, true, EPI_BIAS) : rl ? RL256(EPI_BIAS) : BIG256(true, true, EPI_BIAS);
            case EPI_BIAS_RESID:
                return w192 ? BIG192(true, true, EPI_BIAS_RESID)
                            : rl ? RL256(EPI_BIAS_RESID) : BIG256(true, true, EPI_BIAS_RESID);
            case EPI_BIAS_GELU:
                if (GEMM_PERS_GELU && rl && cdiv(g.M, 256) * cdiv(g.N, 256) >= 2 * wgs)
                    return launch_pers<256, 256, 8, 2, EPI_BIAS_GELU>(g, s, wgs);
                return w192 ? BIG192(true, true, EPI_BIAS_GELU)
                            : rl ? RL256(EPI_BIAS_GELU) : BIG256(true, true, EPI_BIAS_GELU);
            case EPI_BIAS_GELU_D:
                if (GEMM_PERS_GELU && rl && cdiv(g.M, 256) * cdiv(g.N, 256) >= 2 * wgs)
                    return launch_pers<256, 256, 8, 2, EPI_BIAS_GELU_D>(g, s, wgs);
                return w192 ? BIG192(true, true, EPI_BIAS_GELU_D)
                            : rl ? RL256(EPI_BIAS_GELU_D) : BIG256(true, true, EPI_BIAS_GELU_D);
            case EPI_MUL_AUX:
                return w192 ? BIG192(true, true, EPI_MUL_AUX) : rl ? RL256(EPI_MUL_AUX) : BIG256(true, true, EPI_MUL_AUX);
            // the fused classifier: 256-wide tiles, whose waves' 64-column
            // groups are the statistics' column groups
            case EPI_CE_STATS:
                if (!g.ce_targets || !g.ce_stats || !g.ce_zt || g.ce_ld != (int)cdiv(g.N, 64)) return hipErrorInvalidValue;
                // persistent: 1.52 -> 1.47 ms at B*T = 16384 over the 50304 columns
                return rl ? launch_pers<256, 256, 8, 2, EPI_CE_STATS>(g, s, wgs) : BIG256(true, true, EPI_CE_STATS);
            case EPI_CE_GRAD:
                if (!g.ce_targets || !g.ce_lse2 || !g.out) return hipErrorInvalidValue;
                return rl ? RL256(EPI_CE_GRAD) : BIG256(true, true, EPI_CE_GRAD);
            default: return hipErrorInvalidValue;
        }
#undef RL256
    }
    if (g.a_kcontig && !g.b_kcontig) {
        if (g.epi == EPI_STORE && g.ws && g.N % 4 == 0 && g.ldo % 4 == 0) {
            int S, kc;
            nn_split_plan(g.M, g.N, g.K, &S, &kc);
            if (S > 1 && (size_t)S * g.M * g.N * 4 <= g.ws_bytes) {
                hipError_t e =
                    launch_big<256, 256, 8, 4, 32, GEMM_BIG_NS, GEMM_BIG_XPF, true, false, EPI_PARTIAL, 2, 192>(g, s, S, kc);
                if (e != hipSuccess) return e;
                const int64_t n4 = (int64_t)g.M * g.N / 4;
                const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
                splitk_reduce_bf16_kernel<<<blocks, 256, 0, s>>>((bf16*)g.out, g.ldo, g.ws, S, g.M, g.N);
                return hipGetLastError();
            }
        }
        switch (g.epi) {
            case EPI_STORE: return w192 ? BIG192(true, false, EPI_STORE) : BIG256(true, false, EPI_STORE);
            case EPI_GELU_BWD: return w192 ? BIG192(true, false, EPI_GELU_BWD) : BIG256(true, false, EPI_GELU_BWD);
            case EPI_MUL_AUX: return w192 ? BIG192(true, false, EPI_MUL_AUX) : BIG256(true, false, EPI_MUL_AUX);
            case EPI_BIAS: return w192 ? BIG192(true, false, EPI_BIAS) : BIG256(true, false, EPI_BIAS);
            case EPI_BIAS_RESID: return w192 ? BIG192(true, false, EPI_BIAS_RESID) : BIG256(true, false, EPI_BIAS_RESID);
            case EPI_BIAS_GELU_D:
                return w192 ? BIG192(true, false, EPI_BIAS_GELU_D) : BIG256(true, false, EPI_BIAS_GELU_D);
            default: return hipErrorInvalidValue;
        }
    }
#undef BIG192
    if (!g.a_kcontig && !g.b_kcontig && g.epi == EPI_ACC_F32) {
        if (cdiv(g.M, 256) * cdiv(g.N, 256) >= 256)  // wide output (the classifier): no split needed
            return BIG256(false, false, EPI_ACC_F32);
        int S, kc;
        splitk_plan(g.M, g.N, g.K, SK_TM, SK_TN, &S, &kc);
        if (S > 1 && g.ws && (size_t)S * g.M * g.N * 4 <= g.ws_bytes && g.N % 4 == 0 && g.ldo % 4 == 0) {
            hipError_t e =
                launch_big<128, 128, 4, 2, 32, GEMM_SPLIT_NS, GEMM_SPLIT_XPF, false, false, EPI_PARTIAL>(g, s, S, kc);
            if (e != hipSuccess) return e;
            int64_t n4 = (int64_t)g.M * g.N / 4;
            unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4096);
            splitk_reduce_kernel<<<blocks, 256, 0, s>>>((float*)g.out, g.ldo, g.ws, S, g.M, g.N, g.acc_overwrite);
            return hipGetLastError();
        }
        return launch_big<128, 128, 4, 2, 32, GEMM_SPLIT_NS, GEMM_SPLIT_XPF, false, false, EPI_ACC_F32>(g, s);
    }
#undef BIG256
    return hipErrorInvalidValue;
}

// one partial row per wave row block: 4 per 256-row tile (192-wide tiles), else 2
int gemm_colsum_rows(int M, int N) { return (int)cdiv(M, 256) * (use_192(M, N) ? 4 : 2); }

size_t gemm_nn_splitk_ws_bytes(int M, int N, int K) {
    int S, kc;
    nn_split_plan(M, N, K, &S, &kc);
    return S > 1 ? (size_t)S * M * N * 4 : 0;
}

size_t gemm_splitk_ws_bytes(int M, int N, int K) {
    int S, kc;
    splitk_plan(M, N, K, SK_TM, SK_TN, &S, &kc);
    return S > 1 ? (size_t)S * M * N * 4 : 0;
}
