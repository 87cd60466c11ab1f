/*
 * GPT-2 training-step ORACLE.  Test infrastructure only.
 *
 * This file is the plain, slow, obviously-correct CPU definition of one GPT-2
 * training step: token+position embedding, L pre-LN transformer blocks,
 * tied classifier, softmax cross-entropy, a hand-derived backward pass,
 * global-norm gradient clipping and AdamW.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it; the product library
 * shares no code, header, table or helper with it.
 *
 * It is compiled twice from this one source: REAL=float (the fp32 oracle the
 * GPU path is compared against) and REAL=double (used for central finite
 * difference checks of every backward function).  Every reduction accumulates
 * in double and runs in one fixed order, and OpenMP only splits loops over
 * independent outputs, so results do not depend on the thread count.
 *
 * Sources (the pages describing llm.c):
 *  [P5]  "llm.c: GPT-2 training in plain C, with every gradient written by
 *        hand" (fernfant learning-robotics lesson): section 2 "How the code
 *        works" lists the layer pairs (encoder, layernorm, matmul, attention,
 *        gelu, residual, softmax, crossentropy), the per-layer forward call
 *        sequence, the attention-backward accumulation rule, the causal
 *        t2 <= t loop, the saved mean/rstd and attention weights, and the
 *        single-block memory layout; section 3 "Run it, tested" prints the
 *        model config (V=50257 padded to 50304, L=12, NH=12, C=768,
 *        maxT=1024) and the counts N=124,475,904 and 73,347,840 activations.
 *  [P4]  pyshine.com tour of llm.c: the fused classifier (output projection
 *        merged with the softmax loss), the AdamW and global-norm headers.
 *  [P1]  "llm.c's Origin and the Future of LLM Compilers" transcript,
 *        section "Pure C": m and v buffers of AdamW, mean/rstd saved for the
 *        layernorm backward, one up-front allocation.
 *
 * Readings where the pages are silent (GELU form, LN epsilon, weight tying,
 * init RNG, AdamW details) are the plain ones: tanh-approximation GELU,
 * eps=1e-5 with biased variance, classifier tied to wte (pinned by N),
 * SplitMix64 + Box-Muller init, bias-corrected decoupled AdamW.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef REAL
#define REAL float
#endif
typedef double ACC;

typedef struct {
    int L, C, NH, maxT, V, Vp;
} orc_config;

enum { NPARAM = 16, NACT = 23 };

/* ------------------------------------------------------------------------ */
/* sizes and layout                                                          */
/* ------------------------------------------------------------------------ */

/* Parameter tensors, in this fixed order (names from [P5] section 2):
 * wte (Vp,C), wpe (maxT,C), ln1w (L,C), ln1b (L,C), qkvw (L,3C,C),
 * qkvb (L,3C), attprojw (L,C,C), attprojb (L,C), ln2w (L,C), ln2b (L,C),
 * fcw (L,4C,C), fcb (L,4C), fcprojw (L,C,4C), fcprojb (L,C), lnfw (C),
 * lnfb (C).  Weight matrices are (out, in) row-major; the classifier
 * reuses wte (tied), which is what makes N come out at 124,475,904. */
void orc_param_sizes(const orc_config* g, size_t* s) {
    size_t L = g->L, C = g->C;
    s[0] = (size_t)g->Vp * C;
    s[1] = (size_t)g->maxT * C;
    s[2] = L * C;
    s[3] = L * C;
    s[4] = L * 3 * C * C;
    s[5] = L * 3 * C;
    s[6] = L * C * C;
    s[7] = L * C;
    s[8] = L * C;
    s[9] = L * C;
    s[10] = L * 4 * C * C;
    s[11] = L * 4 * C;
    s[12] = L * C * 4 * C;
    s[13] = L * C;
    s[14] = C;
    s[15] = C;
}

size_t orc_num_params(const orc_config* g) {
    size_t s[NPARAM], n = 0;
    orc_param_sizes(g, s);
    for (int i = 0; i < NPARAM; i++) n += s[i];
    return n;
}

/* Activation tensors of the CPU layout ([P5] section 2: the forward pass
 * keeps att, the layernorm mean and rstd, ... for the backward pass):
 * encoded, ln1, ln1_mean, ln1_rstd, qkv, atty, preatt, att, attproj,
 * residual2, ln2, ln2_mean, ln2_rstd, fch, fch_gelu, fcproj, residual3,
 * lnf, lnf_mean, lnf_rstd, logits, probs, losses. */
void orc_act_sizes(const orc_config* g, int B, int T, size_t* s) {
    size_t L = g->L, C = g->C, NH = g->NH, BT = (size_t)B * T, Vp = g->Vp;
    s[0] = BT * C;
    s[1] = L * BT * C;
    s[2] = L * BT;
    s[3] = L * BT;
    s[4] = L * BT * 3 * C;
    s[5] = L * BT * C;
    s[6] = L * B * NH * (size_t)T * T;
    s[7] = L * B * NH * (size_t)T * T;
    s[8] = L * BT * C;
    s[9] = L * BT * C;
    s[10] = L * BT * C;
    s[11] = L * BT;
    s[12] = L * BT;
    s[13] = L * BT * 4 * C;
    s[14] = L * BT * 4 * C;
    s[15] = L * BT * C;
    s[16] = L * BT * C;
    s[17] = BT * C;
    s[18] = BT;
    s[19] = BT;
    s[20] = BT * Vp;
    s[21] = BT * Vp;
    s[22] = BT;
}

size_t orc_num_acts(const orc_config* g, int B, int T) {
    size_t s[NACT], n = 0;
    orc_act_sizes(g, B, T, s);
    for (int i = 0; i < NACT; i++) n += s[i];
    return n;
}

/* ------------------------------------------------------------------------ */
/* initialisation: SplitMix64 (Steele, Lea & Flood 2014) + Box-Muller        */
/* ------------------------------------------------------------------------ */

/* SplitMix64 output function applied to the state seed + n*golden_gamma. */
static uint64_t sm64_draw(uint64_t seed, uint64_t n) {
    uint64_t z = seed + n * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Standard normal for flat parameter index gidx: draws 2*gidx+1 and
 * 2*gidx+2 of the SplitMix64 stream, Box-Muller cosine branch, in double. */
static double normal_at(uint64_t seed, uint64_t gidx) {
    uint64_t w0 = sm64_draw(seed, 2 * gidx + 1);
    uint64_t w1 = sm64_draw(seed, 2 * gidx + 2);
    double u1 = ((double)(w0 >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    double u2 = (double)(w1 >> 11) * (1.0 / 9007199254740992.0);
    double r = sqrt(-2.0 * log(u1));
    return r * cos(6.283185307179586 * u2);
}

/* GPT-2 init as fixed for the workloads: wte rows [0,V), wpe, qkvw, fcw ~
 * N(0, 0.02); the residual projections attprojw, fcprojw ~ N(0, 0.02 /
 * sqrt(2L)); biases 0, LN gains 1, LN biases 0, padded wte rows 0.
 * Each value is (float)(std * z) with z from normal_at(seed, flat index). */
void orc_init_params(const orc_config* g, uint64_t seed, REAL* params) {
    size_t s[NPARAM], off[NPARAM], o = 0;
    orc_param_sizes(g, s);
    for (int i = 0; i < NPARAM; i++) { off[i] = o; o += s[i]; }
    double std_main = 0.02;
    double std_res = 0.02 / sqrt(2.0 * (double)g->L);
    for (int i = 0; i < NPARAM; i++) {
        REAL* p = params + off[i];
        size_t n = s[i];
        if (i == 0 || i == 1 || i == 4 || i == 10 || i == 6 || i == 12) {
            double sd = (i == 6 || i == 12) ? std_res : std_main;
            size_t nlive = (i == 0) ? (size_t)g->V * g->C : n;
            #pragma omp parallel for schedule(static)
            for (size_t j = 0; j < n; j++) {
                if (j < nlive) p[j] = (REAL)(float)(sd * normal_at(seed, off[i] + j));
                else p[j] = 0;
            }
        } else if (i == 2 || i == 8 || i == 14) {
            for (size_t j = 0; j < n; j++) p[j] = 1;
        } else {
            for (size_t j = 0; j < n; j++) p[j] = 0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* layer functions (forward / backward pairs of [P5] section 2)             */
/* ------------------------------------------------------------------------ */

/* Token plus position embedding: x[b,t,:] = wte[tok[b,t],:] + wpe[t,:]. */
void orc_embed_fwd(const int* tok, const REAL* wte, const REAL* wpe, int B, int T, int C, REAL* x) {
    #pragma omp parallel for collapse(2)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            REAL* o = x + ((size_t)b * T + t) * C;
            const REAL* we = wte + (size_t)tok[b * T + t] * C;
            const REAL* pe = wpe + (size_t)t * C;
            for (int c = 0; c < C; c++) o[c] = we[c] + pe[c];
        }
}

/* Its gradient: dwte[tok[b,t],:] += dx[b,t,:]; dwpe[t,:] += dx[b,t,:].
 * Parallel over channels only, each channel summed over (b,t) in order. */
void orc_embed_bwd(const REAL* dx, const int* tok, int B, int T, int C, REAL* dwte, REAL* dwpe) {
    #pragma omp parallel for
    for (int c = 0; c < C; c++) {
        for (int b = 0; b < B; b++)
            for (int t = 0; t < T; t++) {
                REAL d = dx[((size_t)b * T + t) * C + c];
                dwte[(size_t)tok[b * T + t] * C + c] += d;
                dwpe[(size_t)t * C + c] += d;
            }
    }
}

/* Layer normalisation of each of `rows` rows of width C: biased variance,
 * eps = 1e-5, y = (x - mu) * rs * gain + shift with rs = 1/sqrt(var+eps);
 * mu and rs are kept for the backward ([P1] "Pure C"). */
void orc_norm_fwd(const REAL* xin, const REAL* gain, const REAL* shift, int rows, int C,
                  REAL* y, REAL* mu, REAL* rs) {
    #pragma omp parallel for
    for (int n = 0; n < rows; n++) {
        const REAL* x = xin + (size_t)n * C;
        ACC m = 0;
        for (int c = 0; c < C; c++) m += x[c];
        m /= C;
        ACC v = 0;
        for (int c = 0; c < C; c++) { ACC d = x[c] - m; v += d * d; }
        v /= C;
        ACC r = 1.0 / sqrt(v + 1e-5);
        REAL* o = y + (size_t)n * C;
        for (int c = 0; c < C; c++) o[c] = (REAL)(((x[c] - m) * r) * gain[c] + shift[c]);
        mu[n] = (REAL)m;
        rs[n] = (REAL)r;
    }
}

/* Its gradient, with xhat = (x-mu)*rs and g = dy*gain:
 *   dx     += rs * (g - mean_c(g) - xhat * mean_c(g*xhat))
 *   dgain  += sum_rows dy*xhat,   dshift += sum_rows dy. */
void orc_norm_bwd(const REAL* dyin, const REAL* xin, const REAL* gain, const REAL* mu, const REAL* rs,
                  int rows, int C, REAL* dxout, REAL* dgain, REAL* dshift) {
    #pragma omp parallel for
    for (int n = 0; n < rows; n++) {
        const REAL* x = xin + (size_t)n * C;
        const REAL* dy = dyin + (size_t)n * C;
        ACC m = mu[n], r = rs[n];
        ACC sg = 0, sgx = 0;
        for (int c = 0; c < C; c++) {
            ACC xh = (x[c] - m) * r;
            ACC gg = (ACC)dy[c] * gain[c];
            sg += gg;
            sgx += gg * xh;
        }
        sg /= C;
        sgx /= C;
        REAL* dx = dxout + (size_t)n * C;
        for (int c = 0; c < C; c++) {
            ACC xh = (x[c] - m) * r;
            ACC gg = (ACC)dy[c] * gain[c];
            dx[c] = (REAL)(dx[c] + r * (gg - sg - xh * sgx));
        }
    }
    #pragma omp parallel for
    for (int c = 0; c < C; c++) {
        ACC aw = 0, ab = 0;
        for (int n = 0; n < rows; n++) {
            ACC xh = (xin[(size_t)n * C + c] - (ACC)mu[n]) * rs[n];
            ACC d = dyin[(size_t)n * C + c];
            aw += d * xh;
            ab += d;
        }
        dgain[c] = (REAL)(dgain[c] + aw);
        dshift[c] = (REAL)(dshift[c] + ab);
    }
}

/* Affine map y = x W^T + bias on `rows` rows: x (rows,in), W (out,in)
 * row-major, bias (out) or NULL, y (rows,out). */
void orc_linear_fwd(const REAL* xin, const REAL* W, const REAL* bias, int rows, int in, int out, REAL* y) {
    #pragma omp parallel for
    for (int n = 0; n < rows; n++) {
        const REAL* x = xin + (size_t)n * in;
        for (int o = 0; o < out; o++) {
            const REAL* wr = W + (size_t)o * in;
            ACC acc = bias ? (ACC)bias[o] : 0.0;
            #pragma omp simd reduction(+:acc)
            for (int c = 0; c < in; c++) acc += (ACC)x[c] * wr[c];
            y[(size_t)n * out + o] = (REAL)acc;
        }
    }
}

/* Its gradient, every product of the forward taken in reverse:
 *   dx += dy W,  dW += dy^T x,  dbias += sum_rows dy  (dbias may be NULL). */
void orc_linear_bwd(const REAL* dy, const REAL* xin, const REAL* W, int rows, int in, int out,
                    REAL* dx, REAL* dW, REAL* dbias) {
    #pragma omp parallel
    {
        ACC* acc = (ACC*)malloc(sizeof(ACC) * (size_t)in);
        #pragma omp for
        for (int n = 0; n < rows; n++) {
            for (int c = 0; c < in; c++) acc[c] = 0;
            for (int o = 0; o < out; o++) {
                ACC d = dy[(size_t)n * out + o];
                const REAL* wr = W + (size_t)o * in;
                #pragma omp simd
                for (int c = 0; c < in; c++) acc[c] += d * wr[c];
            }
            REAL* dxr = dx + (size_t)n * in;
            for (int c = 0; c < in; c++) dxr[c] = (REAL)(dxr[c] + acc[c]);
        }
        #pragma omp for
        for (int o = 0; o < out; o++) {
            for (int c = 0; c < in; c++) acc[c] = 0;
            ACC ab = 0;
            for (int n = 0; n < rows; n++) {
                ACC d = dy[(size_t)n * out + o];
                const REAL* x = xin + (size_t)n * in;
                ab += d;
                #pragma omp simd
                for (int c = 0; c < in; c++) acc[c] += d * x[c];
            }
            REAL* dwr = dW + (size_t)o * in;
            for (int c = 0; c < in; c++) dwr[c] = (REAL)(dwr[c] + acc[c]);
            if (dbias) dbias[o] = (REAL)(dbias[o] + ab);
        }
        free(acc);
    }
}

/* Causal multi-head self-attention on qkv (B,T,3C) packed q|k|v, head h
 * owning channels [h*hs, (h+1)*hs) of each third.  For keys t2 <= t:
 * score = q_t . k_t2 / sqrt(hs); weight = softmax of the scores over t2 <= t
 * (the row maximum subtracted first); y_t = sum_t2 weight * v_t2.  The
 * scores go to pre and the weights to att, both (B,NH,T,T), with 0 where
 * t2 > t. */
void orc_attn_fwd(const REAL* qkv, int B, int T, int C, int NH, REAL* y, REAL* preatt, REAL* att) {
    int hs = C / NH;
    ACC scale = 1.0 / sqrt((ACC)hs);
    size_t C3 = 3 * (size_t)C;
    #pragma omp parallel for collapse(3)
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++)
            for (int h = 0; h < NH; h++) {
                const REAL* q = qkv + ((size_t)b * T + t) * C3 + (size_t)h * hs;
                REAL* pre = preatt + (((size_t)b * NH + h) * T + t) * T;
                REAL* a = att + (((size_t)b * NH + h) * T + t) * T;
                ACC mx = -INFINITY;
                for (int t2 = 0; t2 <= t; t2++) {
                    const REAL* k = qkv + ((size_t)b * T + t2) * C3 + C + (size_t)h * hs;
                    ACC s = 0;
                    for (int i = 0; i < hs; i++) s += (ACC)q[i] * k[i];
                    s *= scale;
                    pre[t2] = (REAL)s;
                    if (s > mx) mx = s;
                }
                ACC den = 0;
                for (int t2 = 0; t2 <= t; t2++) den += exp((ACC)pre[t2] - mx);
                for (int t2 = 0; t2 < T; t2++) {
                    if (t2 <= t) a[t2] = (REAL)(exp((ACC)pre[t2] - mx) / den);
                    else { a[t2] = 0; pre[t2] = 0; }
                }
                REAL* o = y + ((size_t)b * T + t) * C + (size_t)h * hs;
                for (int i = 0; i < hs; i++) {
                    ACC acc = 0;
                    for (int t2 = 0; t2 <= t; t2++) {
                        const REAL* v = qkv + ((size_t)b * T + t2) * C3 + 2 * (size_t)C + (size_t)h * hs;
                        acc += (ACC)a[t2] * v[i];
                    }
                    o[i] = (REAL)acc;
                }
            }
}

/* Its gradient ([P5] section 2: each product of the forward sends gradient
 * to both of its factors), accumulated into dqkv:
 *   datt_t2 = v_t2 . dy_t;  dv_t2 += att_t2 dy_t;
 *   dpre_t2 = att_t2 (datt_t2 - sum_t3 att_t3 datt_t3);
 *   dq_t += dpre_t2 k_t2 / sqrt(hs);  dk_t2 += dpre_t2 q_t / sqrt(hs).
 * One (b,h) pair owns every row it writes, so (b,h) is the parallel loop. */
void orc_attn_bwd(const REAL* dyin, const REAL* qkv, const REAL* att, int B, int T, int C, int NH, REAL* dqkv) {
    int hs = C / NH;
    ACC scale = 1.0 / sqrt((ACC)hs);
    size_t C3 = 3 * (size_t)C;
    #pragma omp parallel
    {
        ACC* datt = (ACC*)malloc(sizeof(ACC) * (size_t)T);
        ACC* dpre = (ACC*)malloc(sizeof(ACC) * (size_t)T);
        #pragma omp for collapse(2)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < NH; h++) {
                for (int t = 0; t < T; t++) {
                    const REAL* a = att + (((size_t)b * NH + h) * T + t) * T;
                    const REAL* dy = dyin + ((size_t)b * T + t) * C + (size_t)h * hs;
                    const REAL* q = qkv + ((size_t)b * T + t) * C3 + (size_t)h * hs;
                    REAL* dq = dqkv + ((size_t)b * T + t) * C3 + (size_t)h * hs;
                    for (int t2 = 0; t2 <= t; t2++) {
                        const REAL* v = qkv + ((size_t)b * T + t2) * C3 + 2 * (size_t)C + (size_t)h * hs;
                        REAL* dv = dqkv + ((size_t)b * T + t2) * C3 + 2 * (size_t)C + (size_t)h * hs;
                        ACC s = 0;
                        for (int i = 0; i < hs; i++) {
                            s += (ACC)v[i] * dy[i];
                            dv[i] = (REAL)(dv[i] + (ACC)a[t2] * dy[i]);
                        }
                        datt[t2] = s;
                    }
                    ACC inner = 0;
                    for (int t3 = 0; t3 <= t; t3++) inner += (ACC)a[t3] * datt[t3];
                    for (int t2 = 0; t2 <= t; t2++) dpre[t2] = (ACC)a[t2] * (datt[t2] - inner);
                    for (int t2 = 0; t2 <= t; t2++) {
                        const REAL* k = qkv + ((size_t)b * T + t2) * C3 + C + (size_t)h * hs;
                        REAL* dk = dqkv + ((size_t)b * T + t2) * C3 + C + (size_t)h * hs;
                        ACC g = dpre[t2] * scale;
                        for (int i = 0; i < hs; i++) {
                            dq[i] = (REAL)(dq[i] + g * k[i]);
                            dk[i] = (REAL)(dk[i] + g * q[i]);
                        }
                    }
                }
            }
        free(datt);
        free(dpre);
    }
}

/* GELU, tanh approximation: 0.5 u (1 + tanh(k (u + 0.044715 u^3))),
 * k = sqrt(2/pi). */
static ACC gelu_k(void) { return sqrt(2.0 / 3.14159265358979323846); }

void orc_gelu_fwd(const REAL* uin, size_t n, REAL* y) {
    ACC k = gelu_k();
    #pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        ACC u = uin[i];
        y[i] = (REAL)(0.5 * u * (1.0 + tanh(k * (u + 0.044715 * u * u * u))));
    }
}

/* Its gradient, accumulated into du: with tau = tanh(k (u + 0.044715 u^3)),
 * d/du = 0.5(1+tau) + 0.5 u (1-tau^2) k (1 + 3*0.044715 u^2). */
void orc_gelu_bwd(const REAL* dy, const REAL* uin, size_t n, REAL* du) {
    ACC k = gelu_k();
    #pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        ACC u = uin[i];
        ACC tau = tanh(k * (u + 0.044715 * u * u * u));
        ACC d = 0.5 * (1.0 + tau) + 0.5 * u * (1.0 - tau * tau) * k * (1.0 + 3.0 * 0.044715 * u * u);
        du[i] = (REAL)(du[i] + d * dy[i]);
    }
}

/* Softmax over the real vocabulary v < V of each of `rows` rows of width Vp
 * (padded columns excluded, their probability set to 0), and the
 * cross-entropy loss_n = logsumexp - logit[target] when targets is given. */
void orc_xent_fwd(const REAL* logits, const int* targets, int rows, int V, int Vp, REAL* probs, REAL* losses) {
    #pragma omp parallel for
    for (int n = 0; n < rows; n++) {
        const REAL* z = logits + (size_t)n * Vp;
        REAL* p = probs + (size_t)n * Vp;
        ACC mx = -INFINITY;
        for (int v = 0; v < V; v++) if (z[v] > mx) mx = z[v];
        ACC s = 0;
        for (int v = 0; v < V; v++) s += exp((ACC)z[v] - mx);
        for (int v = 0; v < Vp; v++) p[v] = (v < V) ? (REAL)(exp((ACC)z[v] - mx) / s) : 0;
        if (targets) losses[n] = (REAL)(mx + log(s) - (ACC)z[targets[n]]);
    }
}

/* Its gradient, accumulated into dlogits: (probs[n,v] - [v == target]) *
 * dloss[n] for v < V; the padded columns receive nothing. */
void orc_xent_bwd(const REAL* dlosses, const REAL* probs, const int* targets, int rows, int V, int Vp,
                  REAL* dlogits) {
    #pragma omp parallel for
    for (int n = 0; n < rows; n++) {
        REAL* d = dlogits + (size_t)n * Vp;
        const REAL* p = probs + (size_t)n * Vp;
        for (int v = 0; v < Vp; v++) {
            if (v < V) d[v] = (REAL)(d[v] + ((ACC)p[v] - (v == targets[n] ? 1.0 : 0.0)) * dlosses[n]);
        }
    }
}

/* sqrt(sum g^2) over n values, summed in index order in double. */
double orc_global_norm(const REAL* g, size_t n) {
    ACC s = 0;
    for (size_t i = 0; i < n; i++) s += (ACC)g[i] * g[i];
    return sqrt(s);
}

/* Decoupled, bias-corrected AdamW for step t >= 1:
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   mhat = m/(1-b1^t);  vhat = v/(1-b2^t);
 *   theta -= lr (mhat/(sqrt(vhat)+eps) + wd theta).
 * grad_scale multiplies g first (the global-norm clip factor, 1 if none). */
void orc_adamw_update(REAL* params, const REAL* grads, REAL* m, REAL* v, size_t n,
                      double lr, double b1, double b2, double eps, double wd, int t,
                      double grad_scale) {
    ACC c1 = 1.0 - pow(b1, t), c2 = 1.0 - pow(b2, t);
    #pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        ACC g = (ACC)grads[i] * grad_scale;
        ACC mi = b1 * (ACC)m[i] + (1.0 - b1) * g;
        ACC vi = b2 * (ACC)v[i] + (1.0 - b2) * g * g;
        ACC mh = mi / c1, vh = vi / c2;
        ACC th = params[i];
        params[i] = (REAL)(th - lr * (mh / (sqrt(vh) + eps) + wd * th));
        m[i] = (REAL)mi;
        v[i] = (REAL)vi;
    }
}

/* ------------------------------------------------------------------------ */
/* bf16 parameters with stochastic rounding ("llm.c's Origin and the Future */
/* of LLM Compilers", section "Avengers": stochastic rounding)               */
/* ------------------------------------------------------------------------ */

/* The 16-bit draw of flat parameter index i at AdamW step t: the top 16 bits
 * of SplitMix64 drawn at (k, i + 1), where k is SplitMix64 drawn at
 * (seed, 2^62 + t).  A counter-based stream: every (t, i) has its own draw. */
uint32_t orc_sr_draw(uint64_t seed, int t, uint64_t i) {
    uint64_t k = sm64_draw(seed, ((uint64_t)1 << 62) + (uint64_t)t);
    return (uint32_t)(sm64_draw(k, i + 1) >> 48);
}

/* Stochastic rounding of the fp32 value x to bf16 with the draw u in
 * [0, 65536).  bf16 keeps the top 16 bits of the fp32 pattern, so the two
 * bf16 neighbours of x are lo (its pattern with the low 16 bits cleared, x
 * truncated toward zero) and hi (the next bf16 value away from zero), and
 * f = (low 16 bits of x) / 65536 is where x sits between them.  The result
 * is hi when u >= 65536 - f*65536 (probability f), else lo, so its
 * expectation over u is x.  Exact values (f = 0) and non-finite x are
 * returned unchanged.  The result is returned widened to float. */
float orc_sr_bf16(float x, uint32_t u) {
    uint32_t b;
    memcpy(&b, &x, 4);
    if ((b & 0x7F800000u) == 0x7F800000u) return x;  /* inf, NaN */
    uint32_t frac = b & 0xFFFFu;
    if (frac == 0) return x;
    uint32_t lo = b & 0xFFFF0000u;
    uint32_t hi = lo + 0x10000u; /* next magnitude (the exponent carries at a binade end) */
    uint32_t r = (u >= 65536u - frac) ? hi : lo;
    float y;
    memcpy(&y, &r, 4);
    return y;
}

/* Array forms of the two functions above (for the tests). */
void orc_sr_draws(uint64_t seed, int t, uint64_t i0, size_t n, uint32_t* out) {
    for (size_t j = 0; j < n; j++) out[j] = orc_sr_draw(seed, t, i0 + j);
}
void orc_sr_bf16_array(const float* x, const uint32_t* u, size_t n, float* out) {
    for (size_t j = 0; j < n; j++) out[j] = orc_sr_bf16(x[j], u[j]);
}

/* AdamW as orc_adamw_update on parameters that are bf16 values (stored as
 * float): the updated value is computed in double, rounded to fp32, then
 * rounded to bf16 by orc_sr_bf16 with the draw orc_sr_draw(seed, t, i). */
void orc_adamw_sr_update(float* params, const float* grads, float* m, float* v, size_t n,
                         double lr, double b1, double b2, double eps, double wd, int t,
                         double grad_scale, uint64_t seed) {
    ACC c1 = 1.0 - pow(b1, t), c2 = 1.0 - pow(b2, t);
    #pragma omp parallel for
    for (size_t i = 0; i < n; i++) {
        ACC g = (ACC)grads[i] * grad_scale;
        ACC mi = b1 * (ACC)m[i] + (1.0 - b1) * g;
        ACC vi = b2 * (ACC)v[i] + (1.0 - b2) * g * g;
        ACC mh = mi / c1, vh = vi / c2;
        ACC th = params[i];
        float x = (float)(th - lr * (mh / (sqrt(vh) + eps) + wd * th));
        params[i] = orc_sr_bf16(x, orc_sr_draw(seed, t, i));
        m[i] = (float)mi;
        v[i] = (float)vi;
    }
}

/* ------------------------------------------------------------------------ */
/* the model: one allocation for params, grads, m, v, acts, act grads       */
/* ------------------------------------------------------------------------ */

typedef struct {
    orc_config cfg;
    int B, T;
    size_t psz[NPARAM], np;
    size_t asz[NACT], na;
    REAL *params, *grads, *m, *v, *acts, *gacts;
    REAL *P[NPARAM], *G[NPARAM], *A[NACT], *GA[NACT];
    int *inputs, *targets;
    int have_targets;
    double grad_scale;
} orc_model;

orc_model* orc_create(const orc_config* cfg, int B, int T) {
    if (cfg->C % cfg->NH != 0 || T > cfg->maxT || cfg->V > cfg->Vp) return NULL;
    orc_model* M = (orc_model*)calloc(1, sizeof(orc_model));
    M->cfg = *cfg;
    M->B = B;
    M->T = T;
    orc_param_sizes(cfg, M->psz);
    orc_act_sizes(cfg, B, T, M->asz);
    M->np = orc_num_params(cfg);
    M->na = orc_num_acts(cfg, B, T);
    M->params = (REAL*)calloc(M->np, sizeof(REAL));
    M->grads = (REAL*)calloc(M->np, sizeof(REAL));
    M->m = (REAL*)calloc(M->np, sizeof(REAL));
    M->v = (REAL*)calloc(M->np, sizeof(REAL));
    M->acts = (REAL*)calloc(M->na, sizeof(REAL));
    M->gacts = (REAL*)calloc(M->na, sizeof(REAL));
    M->inputs = (int*)calloc((size_t)B * T, sizeof(int));
    M->targets = (int*)calloc((size_t)B * T, sizeof(int));
    if (!M->params || !M->grads || !M->m || !M->v || !M->acts || !M->gacts) return NULL;
    size_t o = 0;
    for (int i = 0; i < NPARAM; i++) { M->P[i] = M->params + o; M->G[i] = M->grads + o; o += M->psz[i]; }
    o = 0;
    for (int i = 0; i < NACT; i++) { M->A[i] = M->acts + o; M->GA[i] = M->gacts + o; o += M->asz[i]; }
    M->grad_scale = 1.0;
    return M;
}

void orc_free(orc_model* M) {
    if (!M) return;
    free(M->params); free(M->grads); free(M->m); free(M->v);
    free(M->acts); free(M->gacts); free(M->inputs); free(M->targets);
    free(M);
}

REAL* orc_params(orc_model* M) { return M->params; }
REAL* orc_grads(orc_model* M) { return M->grads; }
REAL* orc_mbuf(orc_model* M) { return M->m; }
REAL* orc_vbuf(orc_model* M) { return M->v; }
REAL* orc_acts(orc_model* M) { return M->acts; }
REAL* orc_act_grads(orc_model* M) { return M->gacts; }
size_t orc_model_num_params(orc_model* M) { return M->np; }
size_t orc_model_num_acts(orc_model* M) { return M->na; }

/* Views of block l's slices of the flat buffers: its parameters (or their
 * gradients), and below its saved activations (or their gradients). */
typedef struct {
    REAL *norm1_gain, *norm1_shift, *Wqkv, *bqkv, *Wo, *bo;
    REAL *norm2_gain, *norm2_shift, *Wup, *bup, *Wdown, *bdown;
} orc_block_params;

/* The two normalisations read the block input and mid; out is the block's
 * output and the next block's input. */
typedef struct {
    REAL *n1, *n1_mu, *n1_rs, *qkv, *heads, *scores, *weights, *attn_out, *mid;
    REAL *n2, *n2_mu, *n2_rs, *up, *up_act, *down, *out;
} orc_block_acts;

static orc_block_params block_params(REAL** T, size_t l, size_t C) {
    orc_block_params w;
    w.norm1_gain = T[2] + l * C;
    w.norm1_shift = T[3] + l * C;
    w.Wqkv = T[4] + l * 3 * C * C;
    w.bqkv = T[5] + l * 3 * C;
    w.Wo = T[6] + l * C * C;
    w.bo = T[7] + l * C;
    w.norm2_gain = T[8] + l * C;
    w.norm2_shift = T[9] + l * C;
    w.Wup = T[10] + l * 4 * C * C;
    w.bup = T[11] + l * 4 * C;
    w.Wdown = T[12] + l * 4 * C * C;
    w.bdown = T[13] + l * C;
    return w;
}

static orc_block_acts block_acts(REAL** X, size_t l, size_t BT, size_t C, size_t BHTT) {
    size_t n = BT * C;
    orc_block_acts a;
    a.n1 = X[1] + l * n;
    a.n1_mu = X[2] + l * BT;
    a.n1_rs = X[3] + l * BT;
    a.qkv = X[4] + l * 3 * n;
    a.heads = X[5] + l * n;
    a.scores = X[6] + l * BHTT;
    a.weights = X[7] + l * BHTT;
    a.attn_out = X[8] + l * n;
    a.mid = X[9] + l * n;
    a.n2 = X[10] + l * n;
    a.n2_mu = X[11] + l * BT;
    a.n2_rs = X[12] + l * BT;
    a.up = X[13] + l * 4 * n;
    a.up_act = X[14] + l * 4 * n;
    a.down = X[15] + l * n;
    a.out = X[16] + l * n;
    return a;
}

/* Residual join out = a + b, and its gradient: d(out) reaches both terms. */
static void residual_fwd(const REAL* a, const REAL* b, size_t n, REAL* out) {
    for (size_t i = 0; i < n; i++) out[i] = a[i] + b[i];
}
static void residual_bwd(const REAL* dout, size_t n, REAL* da, REAL* db) {
    for (size_t i = 0; i < n; i++) { da[i] += dout[i]; db[i] += dout[i]; }
}

/* A pre-norm block ([P5] section 2 gives the layer order):
 *   mid = x + Wo attn(Wqkv norm1(x))
 *   out = mid + Wdown gelu(Wup norm2(mid)). */
static void block_fwd(const REAL* x, const orc_block_params* w, int B, int T, int C, int NH,
                      const orc_block_acts* a) {
    int BT = B * T;
    size_t n = (size_t)BT * C;
    orc_norm_fwd(x, w->norm1_gain, w->norm1_shift, BT, C, a->n1, a->n1_mu, a->n1_rs);
    orc_linear_fwd(a->n1, w->Wqkv, w->bqkv, BT, C, 3 * C, a->qkv);
    orc_attn_fwd(a->qkv, B, T, C, NH, a->heads, a->scores, a->weights);
    orc_linear_fwd(a->heads, w->Wo, w->bo, BT, C, C, a->attn_out);
    residual_fwd(x, a->attn_out, n, a->mid);
    orc_norm_fwd(a->mid, w->norm2_gain, w->norm2_shift, BT, C, a->n2, a->n2_mu, a->n2_rs);
    orc_linear_fwd(a->n2, w->Wup, w->bup, BT, C, 4 * C, a->up);
    orc_gelu_fwd(a->up, n * 4, a->up_act);
    orc_linear_fwd(a->up_act, w->Wdown, w->bdown, BT, 4 * C, C, a->down);
    residual_fwd(a->mid, a->down, n, a->out);
}

/* Its gradient, from d(out) already in da->out: every step of block_fwd in
 * reverse.  Parameter gradients accumulate into dw; the gradient of the
 * block input accumulates into dx. */
static void block_bwd(const REAL* x, const orc_block_params* w, const orc_block_acts* a, int B, int T, int C,
                      int NH, const orc_block_params* dw, const orc_block_acts* da, REAL* dx) {
    int BT = B * T;
    size_t n = (size_t)BT * C;
    residual_bwd(da->out, n, da->mid, da->down);
    orc_linear_bwd(da->down, a->up_act, w->Wdown, BT, 4 * C, C, da->up_act, dw->Wdown, dw->bdown);
    orc_gelu_bwd(da->up_act, a->up, n * 4, da->up);
    orc_linear_bwd(da->up, a->n2, w->Wup, BT, C, 4 * C, da->n2, dw->Wup, dw->bup);
    orc_norm_bwd(da->n2, a->mid, w->norm2_gain, a->n2_mu, a->n2_rs, BT, C, da->mid, dw->norm2_gain,
                 dw->norm2_shift);
    residual_bwd(da->mid, n, dx, da->attn_out);
    orc_linear_bwd(da->attn_out, a->heads, w->Wo, BT, C, C, da->heads, dw->Wo, dw->bo);
    orc_attn_bwd(da->heads, a->qkv, a->weights, B, T, C, NH, da->qkv);
    orc_linear_bwd(da->qkv, a->n1, w->Wqkv, BT, C, 3 * C, da->n1, dw->Wqkv, dw->bqkv);
    orc_norm_bwd(da->n1, x, w->norm1_gain, a->n1_mu, a->n1_rs, BT, C, dx, dw->norm1_gain, dw->norm1_shift);
}

/* Forward pass: embedding, the L blocks, the final normalisation, the tied
 * classifier (logits = lnf wte^T) and softmax cross-entropy.  Returns the
 * mean loss over the B*T positions, or NaN when targets is NULL (then only
 * logits and probs are produced). */
double orc_forward(orc_model* M, const int* inputs, const int* targets) {
    const orc_config* g = &M->cfg;
    int B = M->B, T = M->T, C = g->C, L = g->L, NH = g->NH, V = g->V, Vp = g->Vp;
    int BT = B * T;
    memcpy(M->inputs, inputs, sizeof(int) * (size_t)BT);
    M->have_targets = targets != NULL;
    if (targets) memcpy(M->targets, targets, sizeof(int) * (size_t)BT);
    REAL** P = M->P;
    REAL** A = M->A;
    size_t BHTT = (size_t)B * NH * T * T;
    orc_embed_fwd(M->inputs, P[0], P[1], B, T, C, A[0]);
    const REAL* x = A[0];
    for (int l = 0; l < L; l++) {
        orc_block_params w = block_params(P, l, C);
        orc_block_acts a = block_acts(A, l, BT, C, BHTT);
        block_fwd(x, &w, B, T, C, NH, &a);
        x = a.out;
    }
    orc_norm_fwd(x, P[14], P[15], BT, C, A[17], A[18], A[19]);
    orc_linear_fwd(A[17], P[0], NULL, BT, C, Vp, A[20]);
    orc_xent_fwd(A[20], targets ? M->targets : NULL, BT, V, Vp, A[21], A[22]);
    if (!targets) return NAN;
    ACC s = 0;
    for (int i = 0; i < BT; i++) s += A[22][i];
    return s / BT;
}

void orc_zero_grad(orc_model* M) {
    memset(M->grads, 0, sizeof(REAL) * M->np);
    M->grad_scale = 1.0;
}

/* Backward pass: the forward in reverse, seeded with d(loss_n) = 1/(B*T) for
 * every position (the loss is their mean).  Parameter gradients accumulate
 * (+=); activation gradients start from zero on every call. */
int orc_backward(orc_model* M) {
    if (!M->have_targets) return -1;
    const orc_config* g = &M->cfg;
    int B = M->B, T = M->T, C = g->C, L = g->L, NH = g->NH, V = g->V, Vp = g->Vp;
    int BT = B * T;
    size_t BHTT = (size_t)B * NH * T * T;
    REAL** P = M->P;
    REAL** G = M->G;
    REAL** A = M->A;
    REAL** D = M->GA;
    memset(M->gacts, 0, sizeof(REAL) * M->na);
    for (int i = 0; i < BT; i++) D[22][i] = (REAL)(1.0 / BT);
    orc_xent_bwd(D[22], A[21], M->targets, BT, V, Vp, D[20]);
    orc_linear_bwd(D[20], A[17], P[0], BT, C, Vp, D[17], G[0], NULL);
    orc_block_acts top = block_acts(A, L - 1, BT, C, BHTT);
    orc_block_acts dtop = block_acts(D, L - 1, BT, C, BHTT);
    orc_norm_bwd(D[17], top.out, P[14], A[18], A[19], BT, C, dtop.out, G[14], G[15]);
    for (int l = L - 1; l >= 0; l--) {
        orc_block_params w = block_params(P, l, C), dw = block_params(G, l, C);
        orc_block_acts a = block_acts(A, l, BT, C, BHTT), da = block_acts(D, l, BT, C, BHTT);
        const REAL* x = l == 0 ? A[0] : block_acts(A, l - 1, BT, C, BHTT).out;
        REAL* dx = l == 0 ? D[0] : block_acts(D, l - 1, BT, C, BHTT).out;
        block_bwd(x, &w, &a, B, T, C, NH, &dw, &da, dx);
    }
    orc_embed_bwd(D[0], M->inputs, B, T, C, G[0], G[1]);
    return 0;
}

/* Global-norm clipping: n = ||g||_2 over all parameters; with n > max_norm
 * the gradients are scaled by max_norm / n.  max_norm <= 0 disables the
 * clip.  Returns n (before clipping). */
double orc_clip_grad_norm(orc_model* M, double max_norm) {
    double n = orc_global_norm(M->grads, M->np);
    if (max_norm > 0 && n > max_norm) {
        double s = max_norm / n;
        for (size_t i = 0; i < M->np; i++) M->grads[i] = (REAL)((ACC)M->grads[i] * s);
    }
    return n;
}

int orc_adamw(orc_model* M, double lr, double b1, double b2, double eps, double wd, int t) {
    if (t < 1) return -1;
    orc_adamw_update(M->params, M->grads, M->m, M->v, M->np, lr, b1, b2, eps, wd, t, 1.0);
    return 0;
}

/* The stochastic-rounding update on the model (fp32 build only: the
 * parameters are bf16 values held in float). */
int orc_adamw_sr(orc_model* M, double lr, double b1, double b2, double eps, double wd, int t, uint64_t seed) {
    if (t < 1 || sizeof(REAL) != sizeof(float)) return -1;
    orc_adamw_sr_update((float*)M->params, (const float*)M->grads, (float*)M->m, (float*)M->v, M->np, lr, b1, b2,
                        eps, wd, t, 1.0, seed);
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}
