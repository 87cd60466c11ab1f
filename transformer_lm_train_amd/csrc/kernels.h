// Internal launch interface of the GPT-2 step kernels.  Every launcher queues
// work on the given stream and returns hipSuccess or the launch error.
#pragma once
#include "common.h"

// Sets the calling thread's gpt2_last_error() message and returns code.
int gpt2_report_error(int code, const char* msg);

// ---- matrix products --------------------------------------------------------
// acc[m][n] = sum_k A(m,k) * B(n,k); an operand is "k-contiguous" when
// A(m,k) = a[m*lda + k] and "mn-contiguous" when A(m,k) = a[k*lda + m]
// (likewise B with n).  The epilogue then writes, for m < M and n < N:
enum GemmEpi {
    EPI_STORE = 0,       // out = acc
    EPI_BIAS = 1,        // out = acc + bias[n]
    EPI_BIAS_RESID = 2,  // out = resid[m][n] + acc + bias[n]
    EPI_BIAS_GELU = 3,   // out = acc + bias[n] (pre-activation); out2 = GELU(that) (bf16: GELU of the stored out)
    EPI_GELU_BWD = 4,    // out = acc * GELU'(aux[m][n])
    EPI_ACC_F32 = 5,     // out (fp32) += acc
    // The classifier fused with the softmax cross-entropy (acc = logits z of
    // row m, column n; columns n >= ce_V are padding):
    EPI_CE_STATS = 6,    // nothing stored as output: for each row m and each 64-column group q of the
                         // tile, ce_stats[m][q] = (max z over the group's columns n < ce_V, in log2
                         // units, and sum of 2^(z log2 e - that max)); ce_zt[m] = z at n = targets[m]
    EPI_CE_GRAD = 7,     // out (bf16) = (softmax - onehot(targets[m])) * ce_scale, i.e.
                         // (2^(z log2 e - ce_lse2[m]) - [n == targets[m]]) * ce_scale, 0 for n >= ce_V
    // The GELU pair of the bf16 MFMA path: the forward keeps the derivative
    // instead of the pre-activation, so that the backward's product only scales.
    EPI_BIAS_GELU_D = 8,  // u = acc + bias[n]: out = GELU'(u), out2 = GELU(u)
    EPI_MUL_AUX = 9,      // out = acc * aux[m][n] (column sums as EPI_GELU_BWD)
};
// EPI_ACC_F32 may split the reduction over several workgroups: each writes
// its fp32 partial tile to ws[split][M][N] and a second kernel adds the
// partials, in split order, into out.  gemm_splitk_ws_bytes gives the
// workspace that split choice needs.

struct GemmArgs {
    int M, N, K;
    const void* a;
    int64_t lda;
    bool a_kcontig;
    const void* b;
    int64_t ldb;
    bool b_kcontig;
    void* out;  // activation dtype, or fp32 for EPI_ACC_F32
    int64_t ldo;
    const float* bias;   // may be NULL (treated as zeros)
    const void* resid;   // activation dtype, leading dim ldo
    const void* aux;     // activation dtype, leading dim ldo
    void* out2;          // activation dtype, leading dim ldo
    int epi;
    float* ws;           // split-K workspace (EPI_ACC_F32), may be NULL
    size_t ws_bytes;
    bool acc_overwrite;  // EPI_ACC_F32: out = acc (out's old contents are not read)
    // EPI_GELU_BWD and EPI_MUL_AUX, bf16 MFMA path: partial column sums of out (the bias
    // gradient of the layer whose output gradient this product produces),
    // one row per wave row block: colsum_ws [gemm_colsum_rows(M, N)][N].
    // The caller sums them (sum_partials_batch).  NULL: off.
    float* colsum_ws;
    // EPI_CE_STATS / EPI_CE_GRAD: row targets (row m of this product), the
    // real vocabulary, the per-row statistics [M][ce_ld] (float2), the target
    // logits [M], the rows' log-sum-exp in log2 units [M] and the gradient scale
    const int* ce_targets;
    int ce_V;
    int ce_ld;
    float2* ce_stats;
    float* ce_zt;
    const float* ce_lse2;
    float ce_scale;
};
size_t gemm_splitk_ws_bytes(int M, int N, int K);
// A backward-data product (dY W, plain store) that fills under half the CUs
// splits its reduction when GemmArgs.ws holds this many bytes: fp32 partial
// tiles summed in split order into the bf16 output.
size_t gemm_nn_splitk_ws_bytes(int M, int N, int K);
int gemm_colsum_rows(int M, int N);
// Grouped weight-gradient products (bf16): one launch over the 256 x 256
// tiles of n problems, each mn-contiguous x mn-contiguous with EPI_ACC_F32.
// gemm_grouped_tiles validates the problems and writes their tile list
// (problem << 22 | tile row << 11 | tile column, padded with ~0 to a multiple
// of 8; tiles may be NULL to count), returning its length, or -1 when a
// problem does not fit or cap is too small.
int gemm_grouped_tiles(const GemmArgs* probs, int n, uint32_t* tiles, int cap);
// Workgroup L runs on XCD L % 8 and takes, in order, the entries of its
// eighth of the list; each XCD's 32 CUs (cus_per_xcd) run them in rounds of
// one workgroup per CU.  gemm_grouped_schedule gives each XCD's last, partial
// round (up to GROUP_SPLIT_MAX tiles, at most half the CUs) to twice as many
// workgroups, each taking half of a tile's reduction: per XCD, `full` whole
// tiles, then `split` tiles listed twice (halves 0 and 1), also collected in
// split_tiles [8 * split] (cus_per_xcd <= 0: no split).  Returns the
// schedule's length (8 * (full + 2 * split)) or -1.
constexpr int GROUP_SPLIT_MAX = 16;
int gemm_grouped_schedule(const uint32_t* tiles, int n, int cus_per_xcd, uint32_t* sched, int cap,
                          uint32_t* split_tiles, int* full, int* split);
// Runs a schedule against the device copies of the problems, the schedule
// and split_tiles; the half tiles leave fp32 partials in ws [8 * split][2]
// [256 x 256] that a second kernel adds, in a fixed order, to their outputs.
// overwrite: out = acc for every problem (instead of out += acc).
hipError_t gemm_grouped_bf16(const GemmArgs* d_probs, const uint32_t* d_sched, int nsched, int full, int split,
                             const uint32_t* d_split_tiles, float* ws, bool overwrite, hipStream_t s);
// What a grouped launch's workgroups read: the problems, the schedule, the
// partial-tile workspace and the schedule's shape.
struct GroupSched {
    const GemmArgs* probs;
    const uint32_t* tiles;
    float* ws;
    int full, split, overwrite;
};

// fp32-accumulating SIMT kernel for any shapes (activation dtype T).
template <typename T> hipError_t gemm_simt(const GemmArgs& g, hipStream_t s);
// bf16 MFMA kernel (gfx950 v_mfma_f32_32x32x16_bf16), fp32 accumulation.
// Needs K % 64 == 0, M % 8 == 0, N % 8 == 0, leading dims % 8 == 0 and
// 16-byte aligned operands; returns hipErrorInvalidValue otherwise.
hipError_t gemm_mfma_bf16(const GemmArgs& g, hipStream_t s);

// ---- element-wise and row kernels ------------------------------------------
// W: the type of the wte / wpe tables (fp32 masters, or the bf16 parameters
// of the stochastic-rounding mode)
// The ids are read from tok_src (and tgt_src, when targets is not NULL) and
// copied into tokens (targets), ids outside [0, V) replaced by 0 and flagged
// in err_flag (1: a token, 2: a target); the sources may be those arrays.
template <typename T, typename W>
hipError_t encoder_fwd(T* out, int* tokens, int* targets, const int* tok_src, const int* tgt_src, const W* wte,
                       const W* wpe, int B, int T_, int C, int V, int* err_flag, hipStream_t s);
// dwte[tokens[i]] += dx[i] for every position (sorted by token and summed in
// position order: deterministic), dwpe[t] (+)= sum_b dx[b][t] (overwrite:
// =, all maxT positions).  ws: encoder_bwd_ws_bytes(B*T, V, C) bytes.
size_t encoder_bwd_ws_bytes(int BT, int V, int C);
template <typename T>
hipError_t encoder_bwd(float* dwte, float* dwpe, const T* dx, const int* tokens, int B, int T_, int maxT, int C,
                       int V, void* ws, bool overwrite, hipStream_t s);
// out[i] = GELU(u[i]) for n bf16 values (the epilogue's GELU of the same
// bf16 pre-activation, so the same results); n % 8 == 0, 16-byte aligned
hipError_t gelu_recompute(bf16* out, const bf16* u, size_t n, hipStream_t s);
template <typename T>
hipError_t layernorm_fwd(T* out, float* mean, float* rstd, const T* x, const float* w, const float* b,
                         int N, int C, hipStream_t s);
// dout = din + LN backward of dy (din NULL: dout = the LN backward alone;
// din may equal dout).  Per-block partial sums go to partial[NP][G][C] with
// G = layernorm_bwd_blocks(N, C, T is bf16) <= 512: dw, db and, if dsum
// (NP = 3), the column sums of dout.  The caller adds them to their outputs
// with sum_partials_batch ({dw, db, dsum-target}, partial, G, C).
int layernorm_bwd_blocks(int N, int C, bool bf16);
template <typename T>
hipError_t layernorm_bwd(T* dout, const T* din, const T* dy, const T* x, const float* w, const float* mean,
                         const float* rstd, float* partial, int N, int C, bool dsum, hipStream_t s);
// A fixed-order column sum of partial rows: out[k][c] += sum_g partial[k*G + g][c]
// for each non-null out[k], k < 3 (out[0] required).
struct SumJob {
    float* out[3];
    const float* partial;
    int G, C;
};
constexpr int SUM_JOBS_MAX = 64;
// Runs n jobs, up to SUM_JOBS_MAX per launch; overwrite: out[k][c] = the sum.
hipError_t sum_partials_batch(const SumJob* jobs, int n, bool overwrite, hipStream_t s);
hipError_t sum_partials(float* out0, float* out1, float* out2, const float* partial, int G, int C, hipStream_t s);
// dbias[n] += sum_m dy[m][n] (deterministic two-stage sum via partial).
template <typename T>
hipError_t colsum_accum(float* dbias, const T* dy, int M, int N, float* partial, hipStream_t s);
// Fused softmax + cross-entropy + dlogits, in place over logits [BT, Vp]:
// losses[r] = logsumexp_{v<V} z - z[target]; z <- (softmax - onehot) * dscale
// for v < V and 0 for v >= V.
template <typename T>
hipError_t softmax_ce(T* logits, float* losses, const int* targets, int BT, int V, int Vp, float dscale,
                      int* err_flag, hipStream_t s);
hipError_t loss_mean(float* out, const float* losses, int n, hipStream_t s);
// The fused classifier's loss: per row, the G partial (max, sum) pairs of
// stats [BT][G] (log2 units) combined into the log-sum-exp (lse2, log2
// units) and loss = lse - z_target.
hipError_t ce_combine(float* losses, float* lse2, const float2* stats, const float* zt, int BT, int G,
                      hipStream_t s);
// norm_scale[0] = ||g||, norm_scale[1] = clip factor (1 if no clip; NaN if
// the norm is not finite).  adamw multiplies g by norm_scale[1], or by 1 when
// norm_scale is NULL; on a non-finite factor it writes nothing and sets
// refused[0] = 1 (refused is required with norm_scale).
hipError_t grad_norm(float* partial, float* norm_scale, const float* g, size_t n, float max_norm,
                     hipStream_t s);
hipError_t adamw(float* p, const float* g, float* m, float* v, bf16* shadow, size_t n, float lr, float b1,
                 float b2, float eps, float wd, float c1, float c2, const float* norm_scale, int* refused,
                 hipStream_t s);
// Flat parameter ranges [lo, hi) whose fp32 copy the stochastic-rounding
// AdamW keeps (as float of the new bf16 value), at p32[dst + (i - lo)].
constexpr int SR_RANGES_MAX = 16;
struct SrRanges {
    uint64_t lo[SR_RANGES_MAX], hi[SR_RANGES_MAX], dst[SR_RANGES_MAX];
    int n;
};
// AdamW over bf16 parameters w[0..n) with stochastic rounding of each fp32
// result (draw: top 16 bits of SplitMix64's output function at state
// key + (i+1) * 0x9E3779B97F4A7C15); p32[dst + i - lo] = float(w[i]) inside
// the ranges.  n, every range boundary and every dst must be multiples of 4.
hipError_t adamw_sr(bf16* w, float* p32, const float* g, float* m, float* v, size_t n, float lr, float b1, float b2,
                    float eps, float wd, float c1, float c2, const float* norm_scale, uint64_t key,
                    const SrRanges& mirror, int* refused, hipStream_t s);
hipError_t cast_bf16(bf16* dst, const float* src, size_t n, hipStream_t s);
template <typename T> hipError_t widen_f32(float* dst, const T* src, size_t n, hipStream_t s);

// ---- attention ---------------------------------------------------------------
// Causal multi-head attention over qkv [B,T,3C] (q|k|v, head h owns
// channels [h*hs,(h+1)*hs) of each); out [B,T,C]; lse [B,NH,T] fp32.
template <typename T>
hipError_t attention_fwd(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s);
template <typename T>
hipError_t attention_bwd(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse, float* dbuf,
                         int B, int T_, int C, int NH, hipStream_t s);
// head size 64, bf16, MFMA flash kernels, T % 64 == 0; dbuf holds 2*B*NH*T
// floats: -D = -rowsum(dO o O), then -lse*log2(e), one per (b, h, t).  With
// bpart, the backward also writes partial column sums of dqkv (the qkv bias
// gradient) to bpart [flash_attention_bias_rows(B, T)][3C], one row per
// (batch, 128-query block); the caller sums them (sum_partials_batch).
int flash_attention_bias_rows(int B, int T_);

hipError_t flash_attention_fwd(bf16* out, float* lse, const bf16* qkv, int B, int T_, int C, int NH, hipStream_t s);
hipError_t flash_attention_bwd(bf16* dqkv, const bf16* dout, const bf16* qkv, const bf16* out, const float* lse,
                               float* dbuf, int B, int T_, int C, int NH, float* bpart, hipStream_t s);
// floats of dbuf the backward needs
inline size_t flash_attention_bwd_ws_floats(int B, int T_, int NH) { return 2 * (size_t)B * NH * T_; }
