// Host side of the GPT-2 step library: buffer planner, parameter init, step
// orchestration and the C ABI declared in include/gpt2.h.
//
// The step follows the llm.c lesson ("llm.c: GPT-2 training in plain C, with
// every gradient written by hand", section 2 "How the code works"):
// gpt2_forward calls each layer in order, gpt2_backward the matching
// backward functions in reverse, gpt2_update applies AdamW, and everything
// lives in one allocation made up front.  Here that allocation is the
// caller's device buffer, carved by the planner below.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

}  // namespace

// The error message of the calling thread, for the other sources of the
// library (their C entry points report through gpt2_last_error too).
int gpt2_report_error(int code, const char* msg) { return fail(code, "%s", msg); }

namespace {

#define HIPCHK(expr)                                                                                     \
    do {                                                                                                 \
        hipError_t e_ = (expr);                                                                          \
        if (e_ != hipSuccess) return fail(GPT2_EIO, "%s failed: %s", #expr, hipGetErrorString(e_));      \
    } while (0)

enum { P_WTE, P_WPE, P_LN1W, P_LN1B, P_QKVW, P_QKVB, P_ATTPROJW, P_ATTPROJB, P_LN2W, P_LN2B, P_FCW, P_FCB,
       P_FCPROJW, P_FCPROJB, P_LNFW, P_LNFB, NPARAM };

void param_sizes(const gpt2_config& c, size_t s[NPARAM]) {
    size_t L = c.num_layers, C = c.channels;
    s[P_WTE] = (size_t)c.padded_vocab_size * C;
    s[P_WPE] = (size_t)c.max_seq_len * C;
    s[P_LN1W] = s[P_LN1B] = L * C;
    s[P_QKVW] = L * 3 * C * C;
    s[P_QKVB] = L * 3 * C;
    s[P_ATTPROJW] = L * C * C;
    s[P_ATTPROJB] = L * C;
    s[P_LN2W] = s[P_LN2B] = L * C;
    s[P_FCW] = L * 4 * C * C;
    s[P_FCB] = L * 4 * C;
    s[P_FCPROJW] = L * C * 4 * C;
    s[P_FCPROJB] = L * C;
    s[P_LNFW] = s[P_LNFB] = C;
}

// Byte offsets of every region of the single device buffer.
struct Layout {
    size_t N, poff[NPARAM];
    // fp32 parameter copy: the full layout (poff32 == poff, N32 == N), or in
    // the stochastic-rounding mode only the tensors the kernels read in fp32
    // (LayerNorm gains and biases, linear biases), packed in tensor order;
    // poff32 is SIZE_MAX for the others
    size_t N32, poff32[NPARAM];
    size_t params, grads, m, v, shadow;
    size_t encoded, ln1, qkv, atty, res2, ln2, fch, fchg, res3, lnf, logits;
    size_t ce_stats, ce_zt, ce_lse2;  // fused classifier: per-row softmax statistics
    int ce_rows;                      // fused classifier: rows of the logits region (one backward chunk)
    size_t ln1_mean, ln1_rstd, ln2_mean, ln2_rstd, lnf_mean, lnf_rstd, lse, losses;
    size_t gres3, gres2, gfch, gqkv, dmid, attD, part_fin, part_ln2, part_ln1, part_fc, part_qkv, norm_partial,
        scalars, err, tokens, targets, splitk, dw_probs, dw_tiles, dw_split_tiles, dw_ws, encws;
    size_t splitk_bytes;
    size_t part_stride_ln, part_stride_fc, part_stride_qkv;  // floats between blocks' partial sets
    int dw_n, dw_ntiles;  // weight-gradient products and their grouped tile list (before scheduling)
    size_t total;
};

// bf16 activations and MFMA products (with fp32 masters, or bf16 parameters
// updated by stochastic rounding)
inline bool is_bf16(int precision) { return precision == GPT2_BF16_MIXED || precision == GPT2_BF16_SR; }

// The parameter tensors every kernel reads in fp32 (LayerNorm gains and
// biases, linear biases); the matrices are read from the bf16 copy in the
// bf16 modes.
inline bool fp32_read(int i) {
    return !(i == P_WTE || i == P_WPE || i == P_QKVW || i == P_ATTPROJW || i == P_FCW || i == P_FCPROJW);
}

int validate(const gpt2_config* c) {
    if (!c) return fail(GPT2_EINVAL, "config is NULL");
    if (c->num_layers <= 0 || c->channels <= 0 || c->num_heads <= 0 || c->max_seq_len <= 0 || c->vocab_size <= 0 ||
        c->padded_vocab_size <= 0 || c->batch_size <= 0 || c->seq_len <= 0)
        return fail(GPT2_EINVAL, "every config size must be positive");
    if (c->channels % c->num_heads) return fail(GPT2_EINVAL, "channels %% num_heads != 0");
    if (c->seq_len > c->max_seq_len) return fail(GPT2_EINVAL, "seq_len > max_seq_len");
    if (c->vocab_size > c->padded_vocab_size) return fail(GPT2_EINVAL, "vocab_size > padded_vocab_size");
    if (c->precision != GPT2_FP32 && c->precision != GPT2_BF16_MIXED && c->precision != GPT2_BF16_SR)
        return fail(GPT2_EINVAL, "unknown precision");
    if (c->channels % 8 || c->padded_vocab_size % 8)
        return fail(GPT2_EINVAL, "channels and padded_vocab_size must be multiples of 8");
    int hs = c->channels / c->num_heads;
    if (c->seq_len > 1024 || hs > 128) return fail(GPT2_EINVAL, "seq_len <= 1024 and head size <= 128 required");
    if (c->channels > 4096) return fail(GPT2_EINVAL, "channels <= 4096 required");
    if (c->vocab_size >= 256 * 1024 - 1) return fail(GPT2_EINVAL, "vocab_size < 262143 required");
    if (c->fused_classifier != 0 && c->fused_classifier != 1) return fail(GPT2_EINVAL, "fused_classifier must be 0 or 1");
    if (c->fused_classifier && !is_bf16(c->precision))
        return fail(GPT2_EINVAL, "the fused classifier needs a bf16 mode");
    if (c->recompute_gelu != 0 && c->recompute_gelu != 1) return fail(GPT2_EINVAL, "recompute_gelu must be 0 or 1");
    if (c->recompute_gelu && !is_bf16(c->precision))
        return fail(GPT2_EINVAL, "recompute_gelu needs a bf16 mode");
    if (c->recompute_layernorm != 0 && c->recompute_layernorm != 1)
        return fail(GPT2_EINVAL, "recompute_layernorm must be 0 or 1");
    if (c->recompute_layernorm && !is_bf16(c->precision))
        return fail(GPT2_EINVAL, "recompute_layernorm needs a bf16 mode");
    if (is_bf16(c->precision)) {
        if (hs != 64) return fail(GPT2_EINVAL, "the bf16 modes need head size 64");
        if (c->channels % 64 || c->padded_vocab_size % 64 || c->seq_len % 64)
            return fail(GPT2_EINVAL, "the bf16 modes need C, Vp and T to be multiples of 64");
    }
    return GPT2_OK;
}

void dw_problems(const gpt2_config& c, const Layout& L, char* base, GemmArgs* out);

Layout make_layout(const gpt2_config& c) {
    Layout L{};
    size_t s[NPARAM];
    param_sizes(c, s);
    L.N = 0;
    for (int i = 0; i < NPARAM; i++) { L.poff[i] = L.N; L.N += s[i]; }
    L.N32 = 0;
    for (int i = 0; i < NPARAM; i++) {
        if (c.precision == GPT2_BF16_SR && !fp32_read(i)) {
            L.poff32[i] = SIZE_MAX;
            continue;
        }
        L.poff32[i] = L.N32;
        L.N32 += s[i];
    }
    size_t total = 0;
    auto add = [&](size_t bytes) {
        size_t off = (total + 255) & ~(size_t)255;
        total = off + bytes;
        return off;
    };
    const size_t A = is_bf16(c.precision) ? 2 : 4;  // activation bytes
    const size_t Ly = c.num_layers, C = c.channels, BT = (size_t)c.batch_size * c.seq_len;
    L.params = add(4 * L.N32);
    L.grads = add(4 * L.N);
    L.m = add(4 * L.N);
    L.v = add(4 * L.N);
    L.shadow = is_bf16(c.precision) ? add(2 * L.N) : 0;
    L.encoded = add(A * BT * C);
    // LayerNorm outputs: every layer's, or with recompute_layernorm one layer's
    // (formed again by the backward for that layer's weight gradients)
    const size_t Lln = c.recompute_layernorm ? 1 : Ly;
    L.ln1 = add(A * Lln * BT * C);
    L.qkv = add(A * Ly * BT * 3 * C);
    L.atty = add(A * Ly * BT * C);
    L.res2 = add(A * Ly * BT * C);
    L.ln2 = add(A * Lln * BT * C);
    L.fch = add(A * Ly * BT * 4 * C);
    // GELU outputs: every layer's, or with recompute_gelu the one layer the
    // next product (forward) or the fcproj weight gradient (backward) reads
    L.fchg = add(A * (c.recompute_gelu ? 1 : Ly) * BT * 4 * C);
    L.res3 = add(A * Ly * BT * C);
    L.lnf = add(A * BT * C);
    if (c.fused_classifier) {
        // no logits are kept: the region holds one backward chunk of dlogits,
        // and the forward leaves (max, sum) per row and 64-column group
        L.ce_rows = (int)std::min<size_t>(BT, 4096);
        L.logits = add(A * (size_t)L.ce_rows * c.padded_vocab_size);
        L.ce_stats = add(8 * BT * cdiv(c.padded_vocab_size, 64));
        L.ce_zt = add(4 * BT);
        L.ce_lse2 = add(4 * BT);
    } else {
        L.ce_rows = 0;
        L.logits = add(A * BT * c.padded_vocab_size);
    }
    L.ln1_mean = add(4 * Ly * BT);
    L.ln1_rstd = add(4 * Ly * BT);
    L.ln2_mean = add(4 * Ly * BT);
    L.ln2_rstd = add(4 * Ly * BT);
    L.lnf_mean = add(4 * BT);
    L.lnf_rstd = add(4 * BT);
    L.lse = add(4 * Ly * BT * c.num_heads);
    L.losses = add(4 * BT);
    // Output gradients of every layer, kept until the weight-gradient
    // products at the end of the backward: d res3 (index l + 1 for block l,
    // index 0 the gradient of the embedding output), d res2, d fch, d qkv.
    L.gres3 = add(A * (Ly + 1) * BT * C);
    L.gres2 = add(A * Ly * BT * C);
    L.gfch = add(A * Ly * BT * 4 * C);
    L.gqkv = add(A * Ly * BT * 3 * C);
    L.dmid = add(A * BT * C);
    L.attD = add(2 * 4 * BT * c.num_heads);  // D and the base-2 lse of every attention row
    {
        // Partial rows of the fixed-order column sums of the backward pass,
        // one region per producer and block, so that every block's sums run
        // in one batch after the block loop: the final LN and the two LNs of a block (3 sums
        // per channel, up to 512 rows), the fc bias (the GELU' product's 4
        // rows per 256 tokens, 4C wide, or the stand-alone column sums' 256
        // rows in fp32 mode) and the qkv bias (attention's row per
        // 128-token block, 3C wide, or the stand-alone column sums).
        const size_t ln = 3 * (size_t)layernorm_bwd_blocks((int)BT, (int)C, is_bf16(c.precision)) * C;
        const size_t fc = std::max<size_t>(cdiv(BT, 256) * 4, 256) * 4 * C;
        const size_t qk = std::max<size_t>((size_t)c.batch_size * cdiv(c.seq_len, 128), 256) * 3 * C;
        L.part_fin = add(4 * ln);
        L.part_ln2 = add(4 * ln * Ly);
        L.part_ln1 = add(4 * ln * Ly);
        L.part_fc = add(4 * fc * Ly);
        L.part_qkv = add(4 * qk * Ly);
        L.part_stride_ln = ln;
        L.part_stride_fc = fc;
        L.part_stride_qkv = qk;
    }
    L.norm_partial = add(4 * 1024);
    L.scalars = add(64);
    L.err = add(64);
    L.tokens = add(4 * BT);
    L.targets = add(4 * BT);
    L.splitk_bytes = 0;
    if (is_bf16(c.precision)) {
        const int dims[5][2] = {{3 * (int)C, (int)C}, {(int)C, (int)C}, {4 * (int)C, (int)C}, {(int)C, 4 * (int)C},
                                {c.padded_vocab_size, (int)C}};
        for (auto& d : dims) L.splitk_bytes = std::max(L.splitk_bytes, gemm_splitk_ws_bytes(d[0], d[1], (int)BT));
        if (c.fused_classifier)  // the chunks' backward-data product
            L.splitk_bytes = std::max(L.splitk_bytes, gemm_nn_splitk_ws_bytes(L.ce_rows, (int)C, c.padded_vocab_size));
    }
    L.splitk = add(L.splitk_bytes);
    // the token-sorted embedding backward: per-block counts, ranks, offsets,
    // the sorted positions and one fp32 partial row per sorted position
    L.encws = add(encoder_bwd_ws_bytes((int)BT, c.vocab_size, (int)C));
    // the fused classifier's run in its chunks; with recompute_gelu the fcproj
    // products run in the block loop, each after its layer's GELU output is recomputed
    // (and with recompute_layernorm the qkv and fc products, after their layer's LayerNorms)
    L.dw_n = (4 - (c.recompute_gelu ? 1 : 0) - (c.recompute_layernorm ? 2 : 0)) * c.num_layers +
             (c.fused_classifier ? 0 : 1);
    L.dw_probs = add(sizeof(GemmArgs) * L.dw_n);
    L.dw_ntiles = 0;
    if (is_bf16(c.precision)) {
        // tile count of the grouped launch, from the problems placed at a
        // stand-in base address with the buffer's alignment
        std::vector<GemmArgs> pr(L.dw_n);
        dw_problems(c, L, reinterpret_cast<char*>((uintptr_t)1 << 20), pr.data());
        L.dw_ntiles = std::max(0, gemm_grouped_tiles(pr.data(), L.dw_n, nullptr, 0));
    }
    // the schedule (the tile list with up to GROUP_SPLIT_MAX tiles per XCD
    // listed twice), the split tiles and their fp32 half-reduction partials
    L.dw_tiles = add(4 * ((size_t)L.dw_ntiles + 8 * GROUP_SPLIT_MAX));
    L.dw_split_tiles = add(4 * 8 * GROUP_SPLIT_MAX);
    L.dw_ws = L.dw_ntiles > 0 ? add(4 * (size_t)8 * GROUP_SPLIT_MAX * 2 * 256 * 256) : 0;
    L.total = add(0);
    return L;
}

// The weight-gradient products of one step, dW[N, K] += dY[BT, N]^T X[BT, K]:
// the tied classifier, then fcproj, fc, attproj and qkv of each block, from
// the output gradients kept by the backward and the forward's activations.
void dw_problems(const gpt2_config& c, const Layout& L, char* base, GemmArgs* out) {
    const size_t A = is_bf16(c.precision) ? 2 : 4;
    const size_t C = c.channels, BT = (size_t)c.batch_size * c.seq_len, BTC = BT * C;
    float* g = reinterpret_cast<float*>(base + L.grads);
    auto act = [&](size_t off, size_t idx) { return base + off + A * idx; };
    auto prob = [&](float* dW, const char* dY, const char* X, size_t N, size_t K) {
        GemmArgs a{};
        a.M = (int)N; a.N = (int)K; a.K = (int)BT;
        a.a = dY; a.lda = (int64_t)N; a.a_kcontig = false;
        a.b = X; a.ldb = (int64_t)K; a.b_kcontig = false;
        a.out = dW; a.ldo = (int64_t)K; a.epi = EPI_ACC_F32;
        a.ws = reinterpret_cast<float*>(base + L.splitk);
        a.ws_bytes = L.splitk_bytes;
        return a;
    };
    int n = 0;
    if (!c.fused_classifier) out[n++] = prob(g + L.poff[P_WTE], act(L.logits, 0), act(L.lnf, 0), c.padded_vocab_size, C);
    for (int l = c.num_layers - 1; l >= 0; l--) {
        const size_t lC = (size_t)l * C;
        if (!c.recompute_gelu)
            out[n++] = prob(g + L.poff[P_FCPROJW] + lC * 4 * C, act(L.gres3, (l + 1) * BTC), act(L.fchg, l * BTC * 4),
                            C, 4 * C);
        if (!c.recompute_layernorm)
            out[n++] = prob(g + L.poff[P_FCW] + lC * 4 * C, act(L.gfch, l * BTC * 4), act(L.ln2, l * BTC), 4 * C, C);
        out[n++] = prob(g + L.poff[P_ATTPROJW] + lC * C, act(L.gres2, l * BTC), act(L.atty, l * BTC), C, C);
        if (!c.recompute_layernorm)
            out[n++] = prob(g + L.poff[P_QKVW] + lC * 3 * C, act(L.gqkv, l * BTC * 3), act(L.ln1, l * BTC), 3 * C, C);
    }
}

// ---- init: SplitMix64 (Steele, Lea & Flood 2014) + Box-Muller -------------
inline uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
    uint64_t z = seed + n * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
inline double gaussian_at(uint64_t seed, uint64_t idx) {
    const double two_pow_m53 = 1.0 / 9007199254740992.0;
    double u1 = ((double)(splitmix64_at(seed, 2 * idx + 1) >> 11) + 0.5) * two_pow_m53;
    double u2 = (double)(splitmix64_at(seed, 2 * idx + 2) >> 11) * two_pow_m53;
    double radius = sqrt(-2.0 * log(u1));
    return radius * cos(6.283185307179586 * u2);
}

void init_params_host(const gpt2_config& c, const Layout& L, uint64_t seed, float* p) {
    size_t s[NPARAM];
    param_sizes(c, s);
    const double sd = 0.02, sd_res = 0.02 / sqrt(2.0 * (double)c.num_layers);
    struct Job { size_t off, n, live; double std; };
    std::vector<Job> jobs;
    for (int i = 0; i < NPARAM; i++) {
        size_t off = L.poff[i];
        switch (i) {
            case P_WTE: jobs.push_back({off, s[i], (size_t)c.vocab_size * c.channels, sd}); break;
            case P_WPE: case P_QKVW: case P_FCW: jobs.push_back({off, s[i], s[i], sd}); break;
            case P_ATTPROJW: case P_FCPROJW: jobs.push_back({off, s[i], s[i], sd_res}); break;
            case P_LN1W: case P_LN2W: case P_LNFW:
                for (size_t j = 0; j < s[i]; j++) p[off + j] = 1.f;
                break;
            default:
                for (size_t j = 0; j < s[i]; j++) p[off + j] = 0.f;
        }
    }
    unsigned nt = std::thread::hardware_concurrency();
    if (nt == 0) nt = 4;
    if (nt > 64) nt = 64;
    std::vector<std::thread> th;
    for (unsigned w = 0; w < nt; w++) {
        th.emplace_back([&, w]() {
            for (const Job& j : jobs) {
                size_t lo = j.n * w / nt, hi = j.n * (w + 1) / nt;
                for (size_t k = lo; k < hi; k++)
                    p[j.off + k] = k < j.live ? (float)(j.std * gaussian_at(seed, j.off + k)) : 0.f;
            }
        });
    }
    for (auto& t : th) t.join();
}

}  // namespace

// ============================================================================
struct gpt2_model {
    gpt2_config cfg;
    Layout L;
    hipStream_t stream;
    char* base;
    size_t bytes;
    int32_t* h_tok;      // pinned staging for host token arrays
    float* h_scalars;    // pinned readback
    hipEvent_t staged;   // last H2D from the staging buffer
    bool have_targets = false;
    const int32_t* src_tokens = nullptr;   // ids of the forward being queued, when the caller's
    const int32_t* src_targets = nullptr;  // device arrays (else the model's own arrays)
    bool logits_valid = false;
    bool norm_bad = false;
    bool clip_pending = false;  // gpt2_clip_grad_norm ran since the last update
    std::vector<GemmArgs> dw;   // the weight-gradient products (device copy at L.dw_probs)
    int dw_nsched = 0, dw_full = 0, dw_split = 0;  // their grouped schedule
    // bf16 mode: gpt2_zero_grad only sets this; the next backward then
    // writes every gradient element instead of adding to it (each element
    // has exactly one first writer), and any earlier reader of the gradient
    // gets it cleared first (materialize_zero_grad).
    bool grads_zero = false;
    std::vector<SumJob> sum_jobs;  // the backward's batched partial sums (kept: no allocation per step)
    // kernel timing
    std::string t_cls;
    bool t_on = false;
    std::vector<hipEvent_t> t_ev;
    size_t t_used = 0;

    template <typename T> T* P(size_t off) { return reinterpret_cast<T*>(base + off); }
    float* params() { return P<float>(L.params); }
    float* grads() { return P<float>(L.grads); }
    bool bf16mode() const { return is_bf16(cfg.precision); }
    // stochastic-rounding mode: the bf16 weights are the parameters
    bool srmode() const { return cfg.precision == GPT2_BF16_SR; }
    uint64_t seed = 0;  // build seed (keys the stochastic-rounding draws)
};

namespace {

// Markers around the launches of one kernel class.  Recorded with the default
// flags, each marker ends in a system-scope release that writes back the L2 and
// stalls the queue: with two markers around each of the 48 forward products of a
// 12-layer step that cost ~0.3 ms per step.  The timing events are only read
// after a stream synchronisation, so they need no fence of their own; without
// it the markers cost ~0.1 ms per step and the spans they bracket hold no cache
// write-back.
constexpr unsigned kTimingEventFlags = hipEventDisableSystemFence;

struct TimeScope {
    gpt2_t* m;
    bool on;
    TimeScope(gpt2_t* m_, const char* cls) : m(m_), on(m_->t_on && m_->t_cls == cls) {
        if (on) rec();
    }
    ~TimeScope() {
        if (on) rec();
    }
    void rec() {
        if (m->t_used >= m->t_ev.size()) {
            hipEvent_t e;
            if (hipEventCreateWithFlags(&e, kTimingEventFlags) != hipSuccess) return;
            m->t_ev.push_back(e);
        }
        (void)hipEventRecord(m->t_ev[m->t_used++], m->stream);
    }
};

#define RUN(cls, expr)                                                                          \
    do {                                                                                        \
        TimeScope ts_(M, cls);                                                                  \
        hipError_t e_ = (expr);                                                                 \
        if (e_ != hipSuccess) return fail(GPT2_EIO, "%s: %s", #expr, hipGetErrorString(e_));   \
    } while (0)

// The GELU pair.  fp32: the forward keeps the pre-activation u and the
// backward's product evaluates GELU'(u).  bf16 modes: the forward's epilogue
// has the sigmoid of u at hand and keeps GELU'(u) itself (the same bytes), so
// the backward's product only multiplies: its epilogue runs once per output
// tile with no overlap, and the derivative there cost ~15 us per layer at
// B*T = 16384, C = 768, against ~3 us more in the forward.
template <typename T> constexpr int kGeluFwdEpi = std::is_same<T, bf16>::value ? EPI_BIAS_GELU_D : EPI_BIAS_GELU;
template <typename T> constexpr int kGeluBwdEpi = std::is_same<T, bf16>::value ? EPI_MUL_AUX : EPI_GELU_BWD;

template <typename T> hipError_t gemm(gpt2_t* M, const GemmArgs& g) {
    if constexpr (std::is_same<T, bf16>::value) return gemm_mfma_bf16(g, M->stream);
    else return gemm_simt<float>(g, M->stream);
}

// out[M,N] = X[M,K] W[N,K]^T + epilogue
template <typename T>
hipError_t lin_fwd(gpt2_t* Mo, T* out, const T* X, const T* W, const float* bias, int M, int N, int K, int epi,
                   const T* resid = nullptr, T* out2 = nullptr) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K;
    g.a = X; g.lda = K; g.a_kcontig = true;
    g.b = W; g.ldb = K; g.b_kcontig = true;
    g.out = out; g.ldo = N; g.bias = bias; g.resid = resid; g.out2 = out2; g.epi = epi;
    return gemm<T>(Mo, g);
}
// dX[M,K] = dY[M,N] W[N,K]  (+ GELU' epilogue with aux)
// With colsum_ws (bf16 GELU' path only), partial column sums of dX as well:
// gemm_colsum_rows(M, K) rows of K.
template <typename T>
hipError_t lin_dx(gpt2_t* Mo, T* dX, const T* dY, const T* W, int M, int N, int K, int epi, const T* aux = nullptr,
                  float* colsum_ws = nullptr) {
    GemmArgs g{};
    g.M = M; g.N = K; g.K = N;
    g.a = dY; g.lda = N; g.a_kcontig = true;
    g.b = W; g.ldb = K; g.b_kcontig = false;
    g.out = dX; g.ldo = K; g.aux = aux; g.epi = epi;
    g.colsum_ws = colsum_ws;
    return gemm<T>(Mo, g);
}
// dW[N,K] += dY[M,N]^T X[M,K]
template <typename T>
hipError_t lin_dw(gpt2_t* Mo, float* dW, const T* dY, const T* X, int M, int N, int K) {
    GemmArgs g{};
    g.M = N; g.N = K; g.K = M;
    g.a = dY; g.lda = N; g.a_kcontig = false;
    g.b = X; g.ldb = K; g.b_kcontig = false;
    g.out = dW; g.ldo = K; g.epi = EPI_ACC_F32;
    g.ws = Mo->P<float>(Mo->L.splitk);
    g.ws_bytes = Mo->L.splitk_bytes;
    return gemm<T>(Mo, g);
}

template <typename T>
hipError_t attn_fwd(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s) {
    if constexpr (std::is_same<T, bf16>::value) return flash_attention_fwd(out, lse, qkv, B, T_, C, NH, s);
    else return attention_fwd<float>(out, lse, qkv, B, T_, C, NH, s);
}
// bpart (bf16 path): partial column sums of dqkv, the qkv bias gradient
template <typename T>
hipError_t attn_bwd(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse, float* dbuf, int B, int T_,
                    int C, int NH, float* bpart, hipStream_t s) {
    if constexpr (std::is_same<T, bf16>::value)
        return flash_attention_bwd(dqkv, dout, qkv, out, lse, dbuf, B, T_, C, NH, bpart, s);
    else return attention_bwd<float>(dqkv, dout, qkv, out, lse, dbuf, B, T_, C, NH, s);
}

template <typename T> struct Acts {
    // per-layer activation pointers
    T *encoded, *ln1, *qkv, *atty, *res2, *ln2, *fch, *fchg, *res3, *lnf, *logits, *gres3, *gres2, *gfch, *gqkv, *dmid;
    float *ln1m, *ln1r, *ln2m, *ln2r, *lnfm, *lnfr, *lse, *losses;
    size_t BTC;
    Acts(gpt2_t* m) {
        const Layout& L = m->L;
        encoded = m->P<T>(L.encoded); ln1 = m->P<T>(L.ln1); qkv = m->P<T>(L.qkv); atty = m->P<T>(L.atty);
        res2 = m->P<T>(L.res2); ln2 = m->P<T>(L.ln2); fch = m->P<T>(L.fch); fchg = m->P<T>(L.fchg);
        res3 = m->P<T>(L.res3); lnf = m->P<T>(L.lnf); logits = m->P<T>(L.logits);
        gres3 = m->P<T>(L.gres3); gres2 = m->P<T>(L.gres2); gfch = m->P<T>(L.gfch); gqkv = m->P<T>(L.gqkv);
        dmid = m->P<T>(L.dmid);
        ln1m = m->P<float>(L.ln1_mean); ln1r = m->P<float>(L.ln1_rstd);
        ln2m = m->P<float>(L.ln2_mean); ln2r = m->P<float>(L.ln2_rstd);
        lnfm = m->P<float>(L.lnf_mean); lnfr = m->P<float>(L.lnf_rstd);
        lse = m->P<float>(L.lse); losses = m->P<float>(L.losses);
        BTC = (size_t)m->cfg.batch_size * m->cfg.seq_len * m->cfg.channels;
    }
};

// matmul weights: the bf16 shadow in mixed mode, the fp32 master otherwise
template <typename T> const T* weights(gpt2_t* m) {
    if constexpr (std::is_same<T, bf16>::value) return m->P<bf16>(m->L.shadow);
    else return m->params();
}

// The tied classifier's product over rows of the final LayerNorm output:
// out[rows, Vp] = X[rows, C] wte[Vp, C]^T with the fused softmax epilogues.
template <typename T>
GemmArgs classifier_args(gpt2_t* Mo, const T* X, const T* wte, int rows, int epi) {
    const gpt2_config& c = Mo->cfg;
    GemmArgs g{};
    g.M = rows; g.N = c.padded_vocab_size; g.K = c.channels;
    g.a = X; g.lda = c.channels; g.a_kcontig = true;
    g.b = wte; g.ldb = c.channels; g.b_kcontig = true;
    g.ldo = c.padded_vocab_size;
    g.epi = epi;
    g.ce_V = c.vocab_size;
    return g;
}

template <typename T> int forward_impl(gpt2_t* M, bool with_targets) {
    const gpt2_config& c = M->cfg;
    const int B = c.batch_size, T_ = c.seq_len, C = c.channels, NH = c.num_heads, Ly = c.num_layers;
    const int BT = B * T_, Vp = c.padded_vocab_size, V = c.vocab_size;
    hipStream_t s = M->stream;
    Acts<T> a(M);
    const float* p = M->params();
    const T* w = weights<T>(M);
    const size_t* po = M->L.poff;    // parameter offsets (gradients, bf16 copy)
    const size_t* pf = M->L.poff32;  // offsets of the fp32 copy
    const size_t BTC = a.BTC;
    int* err = M->P<int>(M->L.err);
    int* tok = M->P<int>(M->L.tokens);
    int* tgt = with_targets ? M->P<int>(M->L.targets) : nullptr;
    // the ids come from the caller's device arrays (gpt2_forward_device) or
    // from the model's own, filled from the host (gpt2_forward)
    const int* tsrc = M->src_tokens ? M->src_tokens : tok;
    const int* ysrc = M->src_targets ? M->src_targets : tgt;

    if constexpr (std::is_same<T, bf16>::value) {
        if (M->srmode()) {  // the bf16 tables are the parameters
            RUN("encoder_fwd", encoder_fwd<T>(a.encoded, tok, tgt, tsrc, ysrc, w + po[P_WTE], w + po[P_WPE], B, T_, C, V,
                                              err, s));
        } else {
            RUN("encoder_fwd", encoder_fwd<T>(a.encoded, tok, tgt, tsrc, ysrc, p + pf[P_WTE], p + pf[P_WPE], B, T_, C, V,
                                              err, s));
        }
    } else {
        RUN("encoder_fwd", encoder_fwd<T>(a.encoded, tok, tgt, tsrc, ysrc, p + pf[P_WTE], p + pf[P_WPE], B, T_, C, V,
                                              err, s));
    }
    const T* x = a.encoded;
    for (int l = 0; l < Ly; l++) {
        T* ln1 = a.ln1 + (c.recompute_layernorm ? 0 : l * BTC);
        T* qkv = a.qkv + l * BTC * 3;
        T* atty = a.atty + l * BTC;
        T* res2 = a.res2 + l * BTC;
        T* ln2 = a.ln2 + (c.recompute_layernorm ? 0 : l * BTC);
        T* fch = a.fch + l * BTC * 4;
        T* fchg = a.fchg + (c.recompute_gelu ? 0 : l * BTC * 4);
        T* res3 = a.res3 + l * BTC;
        const size_t lC = (size_t)l * C;
        RUN("layernorm_fwd", layernorm_fwd<T>(ln1, a.ln1m + (size_t)l * BT, a.ln1r + (size_t)l * BT, x,
                                              p + pf[P_LN1W] + lC, p + pf[P_LN1B] + lC, BT, C, s));
        RUN("gemm_fwd", lin_fwd<T>(M, qkv, ln1, w + po[P_QKVW] + lC * 3 * C, p + pf[P_QKVB] + lC * 3, BT, 3 * C, C,
                                   EPI_BIAS));
        RUN("attention_fwd", attn_fwd<T>(atty, a.lse + (size_t)l * BT * NH, qkv, B, T_, C, NH, s));
        RUN("gemm_fwd", lin_fwd<T>(M, res2, atty, w + po[P_ATTPROJW] + lC * C, p + pf[P_ATTPROJB] + lC, BT, C, C,
                                   EPI_BIAS_RESID, x));
        RUN("layernorm_fwd", layernorm_fwd<T>(ln2, a.ln2m + (size_t)l * BT, a.ln2r + (size_t)l * BT, res2,
                                              p + pf[P_LN2W] + lC, p + pf[P_LN2B] + lC, BT, C, s));
        // fch: the pre-activation (fp32), or in the bf16 modes GELU' of it, so
        // that the backward's product only scales by it; with recompute_gelu
        // the bf16 pre-activation, whose GELU the backward forms again
        RUN("gemm_fwd", lin_fwd<T>(M, fch, ln2, w + po[P_FCW] + lC * 4 * C, p + pf[P_FCB] + lC * 4, BT, 4 * C, C,
                                   c.recompute_gelu ? EPI_BIAS_GELU : kGeluFwdEpi<T>, nullptr, fchg));
        RUN("gemm_fwd", lin_fwd<T>(M, res3, fchg, w + po[P_FCPROJW] + lC * 4 * C, p + pf[P_FCPROJB] + lC, BT, C,
                                   4 * C, EPI_BIAS_RESID, res2));
        x = res3;
    }
    RUN("layernorm_fwd", layernorm_fwd<T>(a.lnf, a.lnfm, a.lnfr, x, p + pf[P_LNFW], p + pf[P_LNFB], BT, C, s));
    if (c.fused_classifier) {
        if constexpr (std::is_same<T, bf16>::value) {
            if (!with_targets) return GPT2_OK;  // no logits are kept: nothing more to compute
            // logits = lnf wte^T, each row's softmax statistics taken in the
            // product's epilogue, then combined into the loss
            GemmArgs g = classifier_args<T>(M, a.lnf, w + po[P_WTE], BT, EPI_CE_STATS);
            g.ce_targets = tgt;
            g.ce_ld = (int)cdiv(Vp, 64);
            g.ce_stats = M->P<float2>(M->L.ce_stats);
            g.ce_zt = M->P<float>(M->L.ce_zt);
            RUN("gemm_classifier_fwd", gemm<T>(M, g));
            RUN("softmax_ce", ce_combine(a.losses, M->P<float>(M->L.ce_lse2), g.ce_stats, g.ce_zt, BT, g.ce_ld, s));
            RUN("loss_mean", loss_mean(M->P<float>(M->L.scalars), a.losses, BT, s));
            return GPT2_OK;
        }
    }
    RUN("gemm_classifier_fwd", lin_fwd<T>(M, a.logits, a.lnf, w + po[P_WTE], nullptr, BT, Vp, C, EPI_STORE));
    if (with_targets) {
        RUN("softmax_ce", softmax_ce<T>(a.logits, a.losses, M->P<int>(M->L.targets), BT, V, Vp, 1.0f / BT, err, s));
        RUN("loss_mean", loss_mean(M->P<float>(M->L.scalars), a.losses, BT, s));
    }
    return GPT2_OK;
}

// All weight gradients of the step: in bf16 mode one grouped launch over the
// tiles of every product (each workgroup takes a whole 256 x 256 tile over
// all B*T tokens, so no split of the reduction is needed), else one product
// at a time.
template <typename T> hipError_t weight_grads(gpt2_t* M, bool overwrite) {
    if constexpr (std::is_same<T, bf16>::value) {
        if (M->L.dw_ntiles > 0)
            return gemm_grouped_bf16(M->P<GemmArgs>(M->L.dw_probs), M->P<uint32_t>(M->L.dw_tiles), M->dw_nsched,
                                     M->dw_full, M->dw_split, M->P<uint32_t>(M->L.dw_split_tiles),
                                     M->P<float>(M->L.dw_ws),
                                     overwrite, M->stream);
    }
    for (GemmArgs g : M->dw) {
        g.acc_overwrite = overwrite;
        hipError_t e = gemm<T>(M, g);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T> int backward_impl(gpt2_t* M) {
    const gpt2_config& c = M->cfg;
    const int B = c.batch_size, T_ = c.seq_len, C = c.channels, NH = c.num_heads, Ly = c.num_layers;
    const int BT = B * T_, Vp = c.padded_vocab_size;
    hipStream_t s = M->stream;
    Acts<T> a(M);
    const float* p = M->params();
    float* g = M->grads();
    const T* w = weights<T>(M);
    const size_t* po = M->L.poff;    // parameter offsets (gradients, bf16 copy)
    const size_t* pf = M->L.poff32;  // offsets of the fp32 copy
    const size_t BTC = a.BTC;
    float* pfin = M->P<float>(M->L.part_fin);
    float* pln2_all = M->P<float>(M->L.part_ln2);
    float* pln1_all = M->P<float>(M->L.part_ln1);
    float* pfc_all = M->P<float>(M->L.part_fc);
    float* pqkv_all = M->P<float>(M->L.part_qkv);
    float* attD = M->P<float>(M->L.attD);
    const int Gln = layernorm_bwd_blocks(BT, C, M->bf16mode());
    // output gradients kept for the weight-gradient products
    auto G3 = [&](int l) { return a.gres3 + (size_t)(l + 1) * BTC; };  // d res3 of block l (l = -1: d encoded)
    auto G2 = [&](int l) { return a.gres2 + (size_t)l * BTC; };        // d res2
    auto GF = [&](int l) { return a.gfch + (size_t)l * BTC * 4; };     // d fch
    auto GQ = [&](int l) { return a.gqkv + (size_t)l * BTC * 3; };     // d qkv

    // first backward since gpt2_zero_grad: every gradient's one first writer stores
    const bool ow = M->grads_zero;
    // one weight gradient outside the grouped launch (the recompute modes):
    // dW[N, K] (+)= dY[BT, N]^T X[BT, K], its reduction split over the workspace
    auto dw_now = [&](float* dW, const T* dY, int N_, const T* X, int K_) {
        GemmArgs d{};
        d.M = N_; d.N = K_; d.K = BT;
        d.a = dY; d.lda = N_; d.a_kcontig = false;
        d.b = X; d.ldb = K_; d.b_kcontig = false;
        d.out = dW; d.ldo = K_; d.epi = EPI_ACC_F32;
        d.ws = M->P<float>(M->L.splitk);
        d.ws_bytes = M->L.splitk_bytes;
        d.acc_overwrite = ow;
        return gemm<T>(M, d);
    };
    if (c.fused_classifier) {
        if constexpr (std::is_same<T, bf16>::value) {
            // the logits were never stored: per chunk of rows, recompute them
            // and leave the product as dlogits, then the chunk's dX rows and its
            // share of dwte (the first chunk stores after gpt2_zero_grad)
            const int R = M->L.ce_rows;
            for (int r0 = 0, ck = 0; r0 < BT; r0 += R, ck++) {
                const int rows = std::min(R, BT - r0);
                GemmArgs cr = classifier_args<T>(M, a.lnf + (size_t)r0 * C, w + po[P_WTE], rows, EPI_CE_GRAD);
                cr.out = a.logits;
                cr.ce_targets = M->P<int>(M->L.targets) + r0;
                cr.ce_lse2 = M->P<float>(M->L.ce_lse2) + r0;
                cr.ce_scale = 1.0f / BT;
                RUN("gemm_classifier_recompute", gemm<T>(M, cr));
                {
                    // dX rows of the chunk (4096 x C outputs over K = Vp: split reduction)
                    GemmArgs dx{};
                    dx.M = rows; dx.N = C; dx.K = Vp;
                    dx.a = a.logits; dx.lda = Vp; dx.a_kcontig = true;
                    dx.b = w + po[P_WTE]; dx.ldb = C; dx.b_kcontig = false;
                    dx.out = a.dmid + (size_t)r0 * C; dx.ldo = C; dx.epi = EPI_STORE;
                    dx.ws = M->P<float>(M->L.splitk);
                    dx.ws_bytes = M->L.splitk_bytes;
                    RUN("gemm_classifier_dx", gemm<T>(M, dx));
                }
                GemmArgs d{};
                d.M = Vp; d.N = C; d.K = rows;
                d.a = a.logits; d.lda = Vp; d.a_kcontig = false;
                d.b = a.lnf + (size_t)r0 * C; d.ldb = C; d.b_kcontig = false;
                d.out = g + po[P_WTE]; d.ldo = C; d.epi = EPI_ACC_F32;
                d.acc_overwrite = ow && ck == 0;
                RUN("gemm_classifier_dw", gemm<T>(M, d));
            }
        }
    } else {
        // classifier (tied to wte): logits now hold dlogits
        RUN("gemm_classifier_dx", lin_dx<T>(M, a.dmid, a.logits, w + po[P_WTE], BT, Vp, C, EPI_STORE));
    }
    const T* xlast = a.res3 + (size_t)(Ly - 1) * BTC;
    // Bias gradients are column sums of the output gradients, taken as
    // partial rows by the kernel that produces each gradient and summed in a
    // fixed order, in one batch after the block loop: attproj and fcproj from the
    // LN backward that writes the residual-stream gradient they see (LN2 of
    // the block, and the final LN or LN1 of the block above); in bf16 mode fc
    // from the GELU' product and qkv from the attention backward (fp32 mode:
    // a column-sum pass each).  The weight gradients, which nothing in the
    // backward reads, are all taken at its end from the kept gradients.
    constexpr bool fused = std::is_same<T, bf16>::value;
    std::vector<SumJob>& jobs = M->sum_jobs;  // every block's sums, run in one batch after the block loop
    jobs.clear();
    jobs.reserve(4 * (size_t)Ly + 1);
    RUN("layernorm_bwd", layernorm_bwd<T>(G3(Ly - 1), nullptr, a.dmid, xlast, p + pf[P_LNFW], a.lnfm, a.lnfr, pfin,
                                          BT, C, true, s));
    for (int l = Ly - 1; l >= 0; l--) {
        const T* xin = l == 0 ? a.encoded : a.res3 + (size_t)(l - 1) * BTC;
        const T* qkv = a.qkv + l * BTC * 3;
        const T* atty = a.atty + l * BTC;
        const T* res2 = a.res2 + l * BTC;
        const T* fch = a.fch + l * BTC * 4;
        const size_t lC = (size_t)l * C;
        float* pln2 = pln2_all + l * M->L.part_stride_ln;
        float* pln1 = pln1_all + l * M->L.part_stride_ln;
        float* pfc = pfc_all + l * M->L.part_stride_fc;
        float* pqkv = pqkv_all + l * M->L.part_stride_qkv;
        if (l == Ly - 1) jobs.push_back(SumJob{{g + po[P_LNFW], g + po[P_LNFB], g + po[P_FCPROJB] + lC}, pfin, Gln, C});
        // fcproj: res3 = res2 + fchg Wfp^T + b  ->  d fch = (d res3 Wfp) * GELU'(pre-activation)
        RUN("gemm_dx", lin_dx<T>(M, GF(l), G3(l), w + po[P_FCPROJW] + lC * 4 * C, BT, C, 4 * C,
                                 c.recompute_gelu ? EPI_GELU_BWD : kGeluBwdEpi<T>, fch, fused ? pfc : nullptr));
        if constexpr (std::is_same<T, bf16>::value) {
            if (c.recompute_gelu) {
                // this layer's GELU output again, from the kept bf16 pre-activation
                // (the values the forward's fcproj product read), then its weight gradient
                RUN("gelu_recompute", gelu_recompute(a.fchg, fch, BTC * 4, s));
                RUN("gemm_dw", dw_now(g + po[P_FCPROJW] + lC * 4 * C, G3(l), C, a.fchg, 4 * C));
            }
        }
        if (fused) jobs.push_back(SumJob{{g + po[P_FCB] + lC * 4}, pfc, gemm_colsum_rows(BT, 4 * C), 4 * C});
        // fc: fch = ln2 Wfc^T + b  ->  d ln2
        RUN("gemm_dx", lin_dx<T>(M, a.dmid, GF(l), w + po[P_FCW] + lC * 4 * C, BT, 4 * C, C, EPI_STORE));
        if (!fused) RUN("colsum", colsum_accum<T>(g + po[P_FCB] + lC * 4, GF(l), BT, 4 * C, pfc, s));
        if (c.recompute_layernorm) {
            // this layer's LN2 output again (the forward's kernel on the same inputs:
            // the same values, mean and rstd rewritten unchanged), then the fc weight gradient
            RUN("layernorm_recompute", layernorm_fwd<T>(a.ln2, a.ln2m + (size_t)l * BT, a.ln2r + (size_t)l * BT, res2,
                                                        p + pf[P_LN2W] + lC, p + pf[P_LN2B] + lC, BT, C, s));
            RUN("gemm_dw", dw_now(g + po[P_FCW] + lC * 4 * C, GF(l), 4 * C, a.ln2, C));
        }
        // ln2: d res2 = d res3 + LN2'(d ln2)
        RUN("layernorm_bwd", layernorm_bwd<T>(G2(l), G3(l), a.dmid, res2, p + pf[P_LN2W] + lC, a.ln2m + (size_t)l * BT,
                                              a.ln2r + (size_t)l * BT, pln2, BT, C, true, s));
        jobs.push_back(SumJob{{g + po[P_LN2W] + lC, g + po[P_LN2B] + lC, g + po[P_ATTPROJB] + lC}, pln2, Gln, C});
        // attproj: res2 = xin + atty Wap^T + b  ->  d atty
        RUN("gemm_dx", lin_dx<T>(M, a.dmid, G2(l), w + po[P_ATTPROJW] + lC * C, BT, C, C, EPI_STORE));
        // attention: d atty -> d qkv
        RUN("attention_bwd", attn_bwd<T>(GQ(l), a.dmid, qkv, atty, a.lse + (size_t)l * BT * NH, attD, B, T_, C, NH,
                                         fused ? pqkv : nullptr, s));
        if (fused) jobs.push_back(SumJob{{g + po[P_QKVB] + lC * 3}, pqkv, flash_attention_bias_rows(B, T_), 3 * C});
        // qkv: qkv = ln1 Wqkv^T + b  ->  d ln1
        RUN("gemm_dx", lin_dx<T>(M, a.dmid, GQ(l), w + po[P_QKVW] + lC * 3 * C, BT, 3 * C, C, EPI_STORE));
        if (!fused) RUN("colsum", colsum_accum<T>(g + po[P_QKVB] + lC * 3, GQ(l), BT, 3 * C, pqkv, s));
        if (c.recompute_layernorm) {  // as LN2 above: this layer's LN1 output, then the qkv weight gradient
            RUN("layernorm_recompute", layernorm_fwd<T>(a.ln1, a.ln1m + (size_t)l * BT, a.ln1r + (size_t)l * BT, xin,
                                                        p + pf[P_LN1W] + lC, p + pf[P_LN1B] + lC, BT, C, s));
            RUN("gemm_dw", dw_now(g + po[P_QKVW] + lC * 3 * C, GQ(l), 3 * C, a.ln1, C));
        }
        // ln1: d xin = d res2 + LN1'(d ln1), whose column sums are the fcproj
        // bias gradient of the block below
        RUN("layernorm_bwd", layernorm_bwd<T>(G3(l - 1), G2(l), a.dmid, xin, p + pf[P_LN1W] + lC,
                                              a.ln1m + (size_t)l * BT, a.ln1r + (size_t)l * BT, pln1, BT, C, l > 0, s));
        jobs.push_back(SumJob{{g + po[P_LN1W] + lC, g + po[P_LN1B] + lC, l > 0 ? g + po[P_FCPROJB] + lC - C : nullptr},
                              pln1, Gln, C});
    }
    RUN("bias_sums", sum_partials_batch(jobs.data(), (int)jobs.size(), ow, s));
    RUN("gemm_dw", weight_grads<T>(M, ow));  // the classifier's product (or chunks) wrote every wte row first
    RUN("encoder_bwd", encoder_bwd<T>(g + po[P_WTE], g + po[P_WPE], G3(-1), M->P<int>(M->L.tokens), B, T_,
                                      c.max_seq_len, C, c.vocab_size, M->base + M->L.encws, ow, s));
    M->grads_zero = false;
    return GPT2_OK;
}

// Device-side conditions, in the err region: [0] a token or target id was
// out of range (replaced by 0), [1] an AdamW update was refused because the
// gradient norm was not finite.  Both are reported, and cleared, by the next
// call that reads a value back.
int report_flags(gpt2_t* M, const int flags[2]) {
    if (flags[0]) {
        HIPCHK(hipMemsetAsync(M->P<int>(M->L.err), 0, 4, M->stream));
        return fail(GPT2_EINVAL, "token or target id outside [0, vocab_size) (flag %d); it was replaced by 0",
                    flags[0]);
    }
    if (flags[1]) {
        HIPCHK(hipMemsetAsync(M->P<int>(M->L.err) + 1, 0, 4, M->stream));
        return fail(GPT2_ERANGE, "an AdamW update was refused on the device: the gradient norm was not finite "
                                 "(parameters and optimizer state were left unchanged)");
    }
    return GPT2_OK;
}

// Loss (and the other small scalars) plus the device flags, one sync.
int read_scalars(gpt2_t* M) {
    HIPCHK(hipMemcpyAsync(M->h_scalars, M->P<float>(M->L.scalars), 16, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipMemcpyAsync(M->h_scalars + 4, M->P<int>(M->L.err), 8, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    int flags[2];
    memcpy(flags, M->h_scalars + 4, 8);
    return report_flags(M, flags);
}

int forward_common(gpt2_t* M, bool with_targets, float* mean_loss) {
    int rc = M->bf16mode() ? forward_impl<bf16>(M, with_targets) : forward_impl<float>(M, with_targets);
    if (rc) return rc;
    M->have_targets = with_targets;
    M->logits_valid = !with_targets;
    if (mean_loss) {
        if (!with_targets) {
            *mean_loss = NAN;
            return GPT2_OK;
        }
        rc = read_scalars(M);
        if (rc && rc != GPT2_ERANGE) {
            M->have_targets = false;
            return rc;
        }
        *mean_loss = M->h_scalars[0];  // valid: an earlier refused update is reported alongside
        if (rc) return rc;
    }
    return GPT2_OK;
}

// The deferred clear of gpt2_zero_grad, for a reader that comes before the
// next backward.
int materialize_zero_grad(gpt2_t* M) {
    if (M->grads_zero) {
        HIPCHK(hipMemsetAsync(M->grads(), 0, 4 * M->L.N, M->stream));
        M->grads_zero = false;
    }
    return GPT2_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

const char* gpt2_last_error(void) { return g_last_error.c_str(); }

int gpt2_plan(const gpt2_config* cfg, size_t* device_bytes) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!device_bytes) return fail(GPT2_EINVAL, "device_bytes is NULL");
    *device_bytes = make_layout(*cfg).total;
    return GPT2_OK;
}

namespace {
// Staging for parameter copies in chunks: the d fch region of the kept output
// gradients (only used inside gpt2_backward), whose first block alone holds
// B*T*4C activations = B*T*2C floats or more.
size_t staging_chunk(const gpt2_t* M) {
    return (size_t)M->cfg.batch_size * M->cfg.seq_len * M->cfg.channels * 2;
}

// Set the parameters from N host floats: fp32 copy (and its bf16 rounding in
// bf16 mixed mode); in the stochastic-rounding mode the bf16 parameters are
// the nearest-even rounding (staged in chunks) and the packed fp32 copy their
// widened values.  Synchronises the stream (the host array may go away).
hipError_t upload_params(gpt2_t* M, const float* host) {
    const Layout& L = M->L;
    hipStream_t s = M->stream;
    hipError_t e = hipSuccess;
    if (!M->srmode()) {
        e = hipMemcpyAsync(M->params(), host, 4 * L.N, hipMemcpyHostToDevice, s);
        if (e == hipSuccess && M->bf16mode()) e = cast_bf16(M->P<bf16>(L.shadow), M->params(), L.N, s);
    } else {
        float* tmp = M->P<float>(L.gfch);
        bf16* w = M->P<bf16>(L.shadow);
        const size_t chunk = staging_chunk(M);
        for (size_t o = 0; o < L.N && e == hipSuccess; o += chunk) {
            const size_t k = std::min(chunk, L.N - o);
            e = hipMemcpyAsync(tmp, host + o, 4 * k, hipMemcpyHostToDevice, s);
            if (e == hipSuccess) e = cast_bf16(w + o, tmp, k, s);
        }
        size_t sz[NPARAM];
        param_sizes(M->cfg, sz);
        for (int i = 0; i < NPARAM && e == hipSuccess; i++)
            if (fp32_read(i)) e = widen_f32<bf16>(M->params() + L.poff32[i], w + L.poff[i], sz[i], s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e;
}

}  // namespace

int gpt2_build(const gpt2_config* cfg, uint64_t seed, void* device_buf, size_t bytes, void* hip_stream,
               gpt2_t** out) {
    int rc = validate(cfg);
    if (rc) return rc;
    if (!out) return fail(GPT2_EINVAL, "out is NULL");
    *out = nullptr;
    Layout L = make_layout(*cfg);
    if (!device_buf) return fail(GPT2_EINVAL, "device_buf is NULL");
    if ((uintptr_t)device_buf & 255) return fail(GPT2_EINVAL, "device_buf must be 256-byte aligned");
    if (bytes < L.total) return fail(GPT2_ENOMEM, "device buffer has %zu bytes, the plan needs %zu", bytes, L.total);
    gpt2_t* M = new gpt2_model();
    M->cfg = *cfg;
    M->L = L;
    M->stream = (hipStream_t)hip_stream;
    M->base = (char*)device_buf;
    M->bytes = bytes;
    size_t BT = (size_t)cfg->batch_size * cfg->seq_len;
    if (hipHostMalloc((void**)&M->h_tok, 8 * BT, 0) != hipSuccess ||
        hipHostMalloc((void**)&M->h_scalars, 64, 0) != hipSuccess || hipEventCreate(&M->staged) != hipSuccess) {
        delete M;
        return fail(GPT2_EIO, "pinned host staging allocation failed");
    }
    std::vector<float> host(L.N);
    init_params_host(*cfg, L, seed, host.data());
    hipStream_t s = M->stream;
    hipError_t e = hipMemsetAsync(M->grads(), 0, 4 * L.N, s);
    if (e == hipSuccess) e = hipMemsetAsync(M->P<float>(L.m), 0, 4 * L.N, s);
    if (e == hipSuccess) e = hipMemsetAsync(M->P<float>(L.v), 0, 4 * L.N, s);
    if (e == hipSuccess) e = hipMemsetAsync(M->P<int>(L.err), 0, 64, s);
    if (e == hipSuccess) e = hipMemsetAsync(M->P<float>(L.scalars), 0, 64, s);
    if (e == hipSuccess) e = upload_params(M, host.data());
    M->seed = seed;
    M->dw.resize(L.dw_n);
    dw_problems(*cfg, L, M->base, M->dw.data());
    std::vector<uint32_t> tiles(L.dw_ntiles), sched(L.dw_ntiles + 8 * GROUP_SPLIT_MAX),
        split_tiles(8 * GROUP_SPLIT_MAX, ~0u);
    if (L.dw_ntiles > 0) {
        // each XCD's last round of tiles in halves, for this device's CUs per XCD
        int dev = 0, cus = 0;
        if (e == hipSuccess) e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (gemm_grouped_tiles(M->dw.data(), L.dw_n, tiles.data(), L.dw_ntiles) != L.dw_ntiles) e = hipErrorInvalidValue;
        if (e == hipSuccess) {
            M->dw_nsched = gemm_grouped_schedule(tiles.data(), L.dw_ntiles, cus % 8 ? 0 : cus / 8, sched.data(),
                                                 (int)sched.size(), split_tiles.data(), &M->dw_full, &M->dw_split);
            if (M->dw_nsched <= 0) e = hipErrorInvalidValue;
        }
    }
    if (e == hipSuccess)
        e = hipMemcpyAsync(M->P<GemmArgs>(L.dw_probs), M->dw.data(), sizeof(GemmArgs) * L.dw_n, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && L.dw_ntiles > 0)
        e = hipMemcpyAsync(M->P<uint32_t>(L.dw_tiles), sched.data(), 4 * (size_t)M->dw_nsched, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && L.dw_ntiles > 0)
        e = hipMemcpyAsync(M->P<uint32_t>(L.dw_split_tiles), split_tiles.data(), 4 * split_tiles.size(),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        gpt2_destroy(M);
        return fail(GPT2_EIO, "gpt2_build: %s", hipGetErrorString(e));
    }
    *out = M;
    return GPT2_OK;
}

int gpt2_destroy(gpt2_t* M) {
    if (!M) return GPT2_OK;
    (void)hipStreamSynchronize(M->stream);
    if (M->h_tok) (void)hipHostFree(M->h_tok);
    if (M->h_scalars) (void)hipHostFree(M->h_scalars);
    if (M->staged) (void)hipEventDestroy(M->staged);
    for (auto e : M->t_ev) (void)hipEventDestroy(e);
    delete M;
    return GPT2_OK;
}

int gpt2_forward(gpt2_t* M, const int32_t* tokens, const int32_t* targets, float* mean_loss) {
    if (!M || !tokens) return fail(GPT2_EINVAL, "NULL model or tokens");
    const gpt2_config& c = M->cfg;
    size_t BT = (size_t)c.batch_size * c.seq_len;
    for (size_t i = 0; i < BT; i++) {
        if (tokens[i] < 0 || tokens[i] >= c.vocab_size) return fail(GPT2_EINVAL, "token %zu = %d out of range", i, tokens[i]);
        if (targets && (targets[i] < 0 || targets[i] >= c.vocab_size))
            return fail(GPT2_EINVAL, "target %zu = %d out of range", i, targets[i]);
    }
    HIPCHK(hipEventSynchronize(M->staged));  // the previous upload has left the staging buffer
    memcpy(M->h_tok, tokens, 4 * BT);
    if (targets) memcpy(M->h_tok + BT, targets, 4 * BT);
    HIPCHK(hipMemcpyAsync(M->P<int>(M->L.tokens), M->h_tok, 4 * BT, hipMemcpyHostToDevice, M->stream));
    if (targets)
        HIPCHK(hipMemcpyAsync(M->P<int>(M->L.targets), M->h_tok + BT, 4 * BT, hipMemcpyHostToDevice, M->stream));
    HIPCHK(hipEventRecord(M->staged, M->stream));
    return forward_common(M, targets != nullptr, mean_loss);
}

int gpt2_forward_device(gpt2_t* M, const int32_t* d_tokens, const int32_t* d_targets, float* mean_loss) {
    if (!M || !d_tokens) return fail(GPT2_EINVAL, "NULL model or tokens");
    // the embedding kernel reads the caller's arrays and writes the model's copies
    M->src_tokens = d_tokens;
    M->src_targets = d_targets;
    const int rc = forward_common(M, d_targets != nullptr, mean_loss);
    M->src_tokens = M->src_targets = nullptr;
    return rc;
}

int gpt2_read_loss(gpt2_t* M, float* mean_loss) {
    if (!M || !mean_loss) return fail(GPT2_EINVAL, "NULL argument");
    if (!M->have_targets) return fail(GPT2_EPERM, "no forward with targets since the last update");
    int rc = read_scalars(M);
    if (rc && rc != GPT2_ERANGE) return rc;
    *mean_loss = M->h_scalars[0];
    return rc;
}

int gpt2_sync(gpt2_t* M) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    HIPCHK(hipMemcpyAsync(M->h_scalars + 4, M->P<int>(M->L.err), 8, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    int flags[2];
    memcpy(flags, M->h_scalars + 4, 8);
    return report_flags(M, flags);
}

int gpt2_zero_grad(gpt2_t* M) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    if (M->bf16mode()) M->grads_zero = true;
    else HIPCHK(hipMemsetAsync(M->grads(), 0, 4 * M->L.N, M->stream));
    return GPT2_OK;
}

int gpt2_backward(gpt2_t* M) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    if (!M->have_targets) return fail(GPT2_EPERM, "gpt2_backward needs a forward with targets first");
    int rc = M->bf16mode() ? backward_impl<bf16>(M) : backward_impl<float>(M);
    M->have_targets = false;  // dlogits were consumed
    return rc;
}

int gpt2_clip_grad_norm(gpt2_t* M, float max_norm, float* norm) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    if (int rc = materialize_zero_grad(M)) return rc;
    float* ns = M->P<float>(M->L.scalars) + 4;
    RUN("grad_norm", grad_norm(M->P<float>(M->L.norm_partial), ns, M->grads(), M->L.N, max_norm, M->stream));
    M->norm_bad = false;
    M->clip_pending = true;
    if (norm) {
        HIPCHK(hipMemcpyAsync(M->h_scalars, ns, 8, hipMemcpyDeviceToHost, M->stream));
        HIPCHK(hipStreamSynchronize(M->stream));
        *norm = M->h_scalars[0];
        if (!isfinite(*norm)) {
            M->norm_bad = true;
            return fail(GPT2_ERANGE, "gradient norm is not finite");
        }
    }
    return GPT2_OK;
}

namespace {
// The parameter tensors the kernels read in fp32: in the stochastic-rounding
// mode their packed fp32 copy mirrors the bf16 parameters (flat range
// [lo, hi) to packed offset dst; adjacent tensors are merged).
SrRanges mirror_ranges(const gpt2_t* M) {
    size_t s[NPARAM];
    param_sizes(M->cfg, s);
    SrRanges r{};
    for (int i = 0; i < NPARAM; i++) {
        if (!fp32_read(i)) continue;
        const uint64_t lo = M->L.poff[i], hi = lo + s[i], dst = M->L.poff32[i];
        if (r.n > 0 && r.hi[r.n - 1] == lo && r.dst[r.n - 1] + (lo - r.lo[r.n - 1]) == dst) r.hi[r.n - 1] = hi;
        else if (r.n < SR_RANGES_MAX) { r.lo[r.n] = lo; r.hi[r.n] = hi; r.dst[r.n] = dst; r.n++; }
    }
    return r;
}
}  // namespace

int gpt2_adamw_step(gpt2_t* M, float lr, float beta1, float beta2, float eps, float weight_decay, int t) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    if (t < 1) return fail(GPT2_EINVAL, "AdamW step t must be >= 1 (got %d)", t);
    if (M->norm_bad) return fail(GPT2_ERANGE, "refusing the update: the last gradient norm was not finite");
    if (int rc = materialize_zero_grad(M)) return rc;
    float c1 = (float)(1.0 - pow((double)beta1, t)), c2 = (float)(1.0 - pow((double)beta2, t));
    float* ns = M->clip_pending ? M->P<float>(M->L.scalars) + 4 : nullptr;
    bf16* sh = M->bf16mode() ? M->P<bf16>(M->L.shadow) : nullptr;
    int* refused = M->P<int>(M->L.err) + 1;  // set by the kernel if the clip factor is not finite
    if (M->srmode()) {
        // the draws of step t: SplitMix64 keyed by the build seed (state 2^62 + t)
        const uint64_t key = splitmix64_at(M->seed, ((uint64_t)1 << 62) + (uint64_t)t);
        RUN("adamw", adamw_sr(sh, M->params(), M->grads(), M->P<float>(M->L.m), M->P<float>(M->L.v), M->L.N, lr,
                              beta1, beta2, eps, weight_decay, c1, c2, ns, key, mirror_ranges(M), refused,
                              M->stream));
    } else {
        RUN("adamw", adamw(M->params(), M->grads(), M->P<float>(M->L.m), M->P<float>(M->L.v), sh, M->L.N, lr, beta1,
                           beta2, eps, weight_decay, c1, c2, ns, refused, M->stream));
    }
    M->clip_pending = false;  // a clip factor applies to one update only
    M->have_targets = false;
    return GPT2_OK;
}

size_t gpt2_num_params(const gpt2_t* M) { return M ? M->L.N : 0; }

int gpt2_param_offsets(const gpt2_t* M, size_t offsets[16]) {
    if (!M || !offsets) return fail(GPT2_EINVAL, "NULL argument");
    for (int i = 0; i < NPARAM; i++) offsets[i] = M->L.poff[i];
    return GPT2_OK;
}

int gpt2_copy_params(gpt2_t* M, float* dst) {
    if (!M || !dst) return fail(GPT2_EINVAL, "NULL argument");
    if (M->srmode()) {
        // the bf16 parameters widened, staged in chunks
        float* tmp = M->P<float>(M->L.gfch);
        const bf16* w = M->P<bf16>(M->L.shadow);
        const size_t chunk = staging_chunk(M);
        for (size_t o = 0; o < M->L.N; o += chunk) {
            const size_t k = std::min(chunk, M->L.N - o);
            HIPCHK(widen_f32<bf16>(tmp, w + o, k, M->stream));
            HIPCHK(hipMemcpyAsync(dst + o, tmp, 4 * k, hipMemcpyDeviceToHost, M->stream));
            HIPCHK(hipStreamSynchronize(M->stream));
        }
        return GPT2_OK;
    }
    HIPCHK(hipMemcpyAsync(dst, M->params(), 4 * M->L.N, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    return GPT2_OK;
}

int gpt2_copy_grads(gpt2_t* M, float* dst) {
    if (!M || !dst) return fail(GPT2_EINVAL, "NULL argument");
    if (int rc = materialize_zero_grad(M)) return rc;
    HIPCHK(hipMemcpyAsync(dst, M->grads(), 4 * M->L.N, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    return GPT2_OK;
}

int gpt2_copy_opt_state(gpt2_t* M, float* mdst, float* vdst) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    if (mdst) HIPCHK(hipMemcpyAsync(mdst, M->P<float>(M->L.m), 4 * M->L.N, hipMemcpyDeviceToHost, M->stream));
    if (vdst) HIPCHK(hipMemcpyAsync(vdst, M->P<float>(M->L.v), 4 * M->L.N, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    return GPT2_OK;
}

int gpt2_copy_logits(gpt2_t* M, float* dst) {
    if (!M || !dst) return fail(GPT2_EINVAL, "NULL argument");
    if (M->cfg.fused_classifier) return fail(GPT2_EPERM, "the fused classifier keeps no logits");
    if (!M->logits_valid) return fail(GPT2_EPERM, "logits are only kept by a forward without targets");
    size_t n = (size_t)M->cfg.batch_size * M->cfg.seq_len * M->cfg.padded_vocab_size;
    if (M->bf16mode()) {
        // widen in chunks through the d fch region of the kept gradients (its
        // first block alone holds B*T*4C bf16 = B*T*2C floats)
        const bf16* src = M->P<bf16>(M->L.logits);
        float* tmp = M->P<float>(M->L.gfch);
        size_t chunk = (size_t)M->cfg.batch_size * M->cfg.seq_len * M->cfg.channels * 2;
        for (size_t o = 0; o < n; o += chunk) {
            size_t k = n - o < chunk ? n - o : chunk;
            HIPCHK(widen_f32<bf16>(tmp, src + o, k, M->stream));
            HIPCHK(hipMemcpyAsync(dst + o, tmp, 4 * k, hipMemcpyDeviceToHost, M->stream));
            HIPCHK(hipStreamSynchronize(M->stream));
        }
    } else {
        HIPCHK(hipMemcpyAsync(dst, M->P<float>(M->L.logits), 4 * n, hipMemcpyDeviceToHost, M->stream));
        HIPCHK(hipStreamSynchronize(M->stream));
    }
    return GPT2_OK;
}

int gpt2_copy_losses(gpt2_t* M, float* dst) {
    if (!M || !dst) return fail(GPT2_EINVAL, "NULL argument");
    size_t n = (size_t)M->cfg.batch_size * M->cfg.seq_len;
    HIPCHK(hipMemcpyAsync(dst, M->P<float>(M->L.losses), 4 * n, hipMemcpyDeviceToHost, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    return GPT2_OK;
}

int gpt2_set_grads(gpt2_t* M, const float* src) {
    if (!M || !src) return fail(GPT2_EINVAL, "NULL argument");
    HIPCHK(hipMemcpyAsync(M->grads(), src, 4 * M->L.N, hipMemcpyHostToDevice, M->stream));
    HIPCHK(hipStreamSynchronize(M->stream));
    M->grads_zero = false;  // the values just set replace any pending clear
    return GPT2_OK;
}

int gpt2_set_params(gpt2_t* M, const float* src) {
    if (!M || !src) return fail(GPT2_EINVAL, "NULL argument");
    HIPCHK(upload_params(M, src));
    return GPT2_OK;
}

void* gpt2_device_params(gpt2_t* M) { return M ? M->params() : nullptr; }
void* gpt2_device_grads(gpt2_t* M) {
    if (!M || materialize_zero_grad(M)) return nullptr;
    return M->grads();
}
void* gpt2_device_shadow(gpt2_t* M) { return (M && M->bf16mode()) ? M->base + M->L.shadow : nullptr; }

int gpt2_kernel_timing_enable(gpt2_t* M, const char* cls, int enable) {
    if (!M) return fail(GPT2_EINVAL, "NULL model");
    HIPCHK(hipStreamSynchronize(M->stream));
    M->t_on = enable != 0;
    M->t_cls = cls ? cls : "";
    M->t_used = 0;
    // pre-create events so that none is created inside a timed region
    while (M->t_ev.size() < 4096) {
        hipEvent_t e;
        HIPCHK(hipEventCreateWithFlags(&e, kTimingEventFlags));
        M->t_ev.push_back(e);
    }
    return GPT2_OK;
}

int gpt2_kernel_timing_read(gpt2_t* M, int* launches, double* total_ms) {
    if (!M || !launches || !total_ms) return fail(GPT2_EINVAL, "NULL argument");
    HIPCHK(hipStreamSynchronize(M->stream));
    double tot = 0;
    size_t n = M->t_used / 2;
    for (size_t i = 0; i < n; i++) {
        float ms = 0;
        HIPCHK(hipEventElapsedTime(&ms, M->t_ev[2 * i], M->t_ev[2 * i + 1]));
        tot += ms;
    }
    *launches = (int)n;
    *total_ms = tot;
    return GPT2_OK;
}

int gpt2_test_gemm_nt(gpt2_t* M, void* out, const void* a, const void* w, const float* bias, int m, int n, int k) {
    if (!M || !out || !a || !w) return fail(GPT2_EINVAL, "NULL argument");
    int epi = bias ? EPI_BIAS : EPI_STORE;
    if (M->bf16mode())
        RUN("gemm_test", lin_fwd<bf16>(M, (bf16*)out, (const bf16*)a, (const bf16*)w, bias, m, n, k, epi));
    else
        RUN("gemm_test", lin_fwd<float>(M, (float*)out, (const float*)a, (const float*)w, bias, m, n, k, epi));
    return GPT2_OK;
}

int gpt2_test_gemm_nn(gpt2_t* M, void* dx, const void* dy, const void* w, int m, int n, int k) {
    if (!M || !dx || !dy || !w) return fail(GPT2_EINVAL, "NULL argument");
    if (M->bf16mode())
        RUN("gemm_test", lin_dx<bf16>(M, (bf16*)dx, (const bf16*)dy, (const bf16*)w, m, n, k, EPI_STORE));
    else
        RUN("gemm_test", lin_dx<float>(M, (float*)dx, (const float*)dy, (const float*)w, m, n, k, EPI_STORE));
    return GPT2_OK;
}

int gpt2_test_gemm_tn(gpt2_t* M, float* dw, const void* dy, const void* x, int m, int n, int k) {
    if (!M || !dw || !dy || !x) return fail(GPT2_EINVAL, "NULL argument");
    if (M->bf16mode())
        RUN("gemm_test", lin_dw<bf16>(M, dw, (const bf16*)dy, (const bf16*)x, m, n, k));
    else
        RUN("gemm_test", lin_dw<float>(M, dw, (const float*)dy, (const float*)x, m, n, k));
    return GPT2_OK;
}

int gpt2_test_attention_fwd(gpt2_t* M, void* out, float* lse, const void* qkv, int B, int T_, int C, int NH) {
    if (!M || !out || !lse || !qkv || B <= 0 || T_ <= 0 || NH <= 0 || C % NH) return fail(GPT2_EINVAL, "bad argument");
    if (M->bf16mode())
        RUN("attention_test", attn_fwd<bf16>((bf16*)out, lse, (const bf16*)qkv, B, T_, C, NH, M->stream));
    else
        RUN("attention_test", attn_fwd<float>((float*)out, lse, (const float*)qkv, B, T_, C, NH, M->stream));
    return GPT2_OK;
}

int gpt2_test_attention_bwd(gpt2_t* M, void* dqkv, const void* dout, const void* qkv, const void* out,
                            const float* lse, int B, int T_, int C, int NH) {
    if (!M || !dqkv || !dout || !qkv || !out || !lse || B <= 0 || T_ <= 0 || NH <= 0 || C % NH)
        return fail(GPT2_EINVAL, "bad argument");
    const gpt2_config& c = M->cfg;
    if ((int64_t)B * NH * T_ > (int64_t)c.batch_size * c.num_heads * c.seq_len)
        return fail(GPT2_EINVAL, "B*NH*T exceeds the model's attention row buffer");
    float* D = M->P<float>(M->L.attD);
    if (M->bf16mode())
        RUN("attention_test", attn_bwd<bf16>((bf16*)dqkv, (const bf16*)dout, (const bf16*)qkv, (const bf16*)out, lse,
                                             D, B, T_, C, NH, nullptr, M->stream));
    else
        RUN("attention_test", attn_bwd<float>((float*)dqkv, (const float*)dout, (const float*)qkv,
                                              (const float*)out, lse, D, B, T_, C, NH, nullptr, M->stream));
    return GPT2_OK;
}

}  // extern "C"
