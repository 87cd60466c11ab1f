// Memory-bound kernels of the GPT-2 step: embedding, LayerNorm fwd/bwd,
// bias-gradient column sums, fused softmax cross-entropy, loss mean, global
// gradient norm and AdamW.  Rows are processed one wavefront (64 lanes) per
// row with 16-byte loads; reductions are wavefront butterflies and
// fixed-order block partials, so results do not depend on scheduling.
#include <type_traits>

#include "kernels.h"

#define LAUNCH_CHECK() hipGetLastError()

// ============================================================================
// encoder: x[b,t,:] = wte[tok[b,t],:] + wpe[t,:]   (llm.c lesson, section 2:
// encoder_forward, token + position embedding)
// ============================================================================
template <typename T, typename W>
__global__ void encoder_fwd_kernel(T* out, int* tokens, int* targets, const int* tok_src, const int* tgt_src,
                                   const W* wte, const W* wpe, int T_, int C, int V, int BT, int* err) {
    constexpr int VN = Vec16<T>::N;
    int chunks = C / VN;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)BT * chunks) return;
    int row = (int)(i / chunks), ch = (int)(i % chunks);
    int t = row % T_;
    if (targets && ch == 0) {
        // targets (when given) are checked here as well, before any reader,
        // and copied into the model's own array
        const int y = tgt_src[row];
        const bool ok = y >= 0 && y < V;
        if (!ok) atomicOr(err, 2);
        targets[row] = ok ? y : 0;
    }
    int tok = tok_src[row];
    if (tok < 0 || tok >= V) {
        // flagged, and 0 in the model's own token copy, so that the
        // backward's scatter into dwte stays in bounds
        if (ch == 0) atomicOr(err, 1);
        tok = 0;
    }
    // (tok_src may be the model's array itself: the other lanes of the row
    // then read either the original id or the 0 that replaces an invalid one)
    if (ch == 0) tokens[row] = tok;
    const W* we = wte + (int64_t)tok * C + ch * VN;
    const W* pe = wpe + (int64_t)t * C + ch * VN;
    Vec16<T> o;
    if constexpr (std::is_same<W, float>::value) {
#pragma unroll
        for (int j = 0; j < VN; j += 4) {
            float4 a = *reinterpret_cast<const float4*>(we + j);
            float4 b = *reinterpret_cast<const float4*>(pe + j);
            o.v[j + 0] = from_f32<T>(a.x + b.x);
            o.v[j + 1] = from_f32<T>(a.y + b.y);
            o.v[j + 2] = from_f32<T>(a.z + b.z);
            o.v[j + 3] = from_f32<T>(a.w + b.w);
        }
    } else {  // bf16 tables: 8 values per 16-byte load
        static_assert(VN == 8, "bf16 tables feed bf16 activations");
        const Vec16<bf16> a = ld16(we), b = ld16(pe);
#pragma unroll
        for (int j = 0; j < 8; j++) o.v[j] = from_f32<T>((float)a.v[j] + (float)b.v[j]);
    }
    st16(out + (int64_t)row * C + ch * VN, o);
}

template <typename T, typename W>
hipError_t encoder_fwd(T* out, int* tokens, int* targets, const int* tok_src, const int* tgt_src, const W* wte,
                       const W* wpe, int B, int T_, int C, int V, int* err, hipStream_t s) {
    if (!tok_src || (targets && !tgt_src)) return hipErrorInvalidValue;
    int BT = B * T_;
    int64_t n = (int64_t)BT * (C / Vec16<T>::N);
    encoder_fwd_kernel<T, W><<<cdiv(n, 256), 256, 0, s>>>(out, tokens, targets, tok_src, tgt_src, wte, wpe, T_, C, V,
                                                          BT, err);
    return LAUNCH_CHECK();
}

// dwte[tok] += dx, deterministically (no float atomics; a token may repeat
// within the batch, Zipf-hot ones thousands of times): the positions are
// sorted by token id, stably, by a counting sort, and each id's rows are
// summed in position order.
//   rank:    per block of ENC_B positions, each position's rank among the
//            earlier positions of its block with the same id, and the
//            block's count of each id (written by the id's first position).
//   offsets: the total count of every id and its exclusive prefix sum, in
//            two levels (within groups of 1024 ids, then over the groups),
//            and, in place of the block counts, each block's exclusive
//            prefix of them (the count of the id in the earlier blocks).
//   scatter: position i goes to sorted slot base[id] + (count of id in the
//            earlier blocks) + rank.
//   chunks:  per ENC_S consecutive sorted slots, one partial row per run of
//            equal ids, summed in slot order, stored at the run's first slot.
//   segments: at each id's first slot, its pieces (that slot, then every
//            chunk start inside the id's range) are added in order into dwte.
// Ids outside [0, V) (already flagged by the forward) go to a last bin, V,
// which is dropped.
constexpr int ENC_B = 256, ENC_S = 32, ENC_G = 1024;

struct EncWs {
    int *H, *R, *tot, *lbase, *goff, *perm, *sid;
    float* Q;
};
// carve the workspace: H [NB][V+1], R [BT], tot, lbase [V+1], goff [groups],
// perm, sid [BT], Q [BT][C]
static size_t enc_ws_layout(int BT, int V, int C, char* p, EncWs* w) {
    const size_t NB = cdiv(BT, ENC_B), NG = cdiv(V + 1, ENC_G);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return p ? p + o : nullptr;
    };
    EncWs e;
    e.H = (int*)take(4 * NB * (V + 1));
    e.R = (int*)take(4 * (size_t)BT);
    e.tot = (int*)take(4 * (size_t)(V + 1));
    e.lbase = (int*)take(4 * (size_t)(V + 1));
    e.goff = (int*)take(4 * NG);
    e.perm = (int*)take(4 * (size_t)BT);
    e.sid = (int*)take(4 * (size_t)BT);
    e.Q = (float*)take(4 * (size_t)BT * C);
    if (w) *w = e;
    return off;
}
size_t encoder_bwd_ws_bytes(int BT, int V, int C) { return enc_ws_layout(BT, V, C, nullptr, nullptr); }

__global__ void fill_i32_kernel(int* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

DEVI int enc_bin(int t, int V) { return t >= 0 && t < V ? t : V; }

__global__ __launch_bounds__(ENC_B) void enc_rank_kernel(const int* tokens, int BT, int V, int* H, int* R) {
    __shared__ int tk[ENC_B];
    const int i = blockIdx.x * ENC_B + threadIdx.x;
    const int id = i < BT ? enc_bin(tokens[i], V) : -1;
    tk[threadIdx.x] = id;
    __syncthreads();
    if (i >= BT) return;
    int r = 0, cnt = 0;
    for (int j = 0; j < ENC_B; j++) {
        const bool eq = tk[j] == id;
        cnt += eq;
        r += eq && j < (int)threadIdx.x;
    }
    R[i] = r;
    if (r == 0) H[(int64_t)blockIdx.x * (V + 1) + id] = cnt;
}

// per group of ENC_G ids: totals over the NB blocks (the block counts are
// replaced by their exclusive prefix over the blocks), the totals'
// exclusive scan within the group (lbase) and the group's sum (gsum)
__global__ __launch_bounds__(ENC_G) void enc_group_kernel(int* H, int NB, int V, int* tot, int* lbase, int* gsum) {
    __shared__ int sc[ENC_G];
    const int id = blockIdx.x * ENC_G + threadIdx.x;
    int t = 0;
    if (id <= V) {
        constexpr int U = 16;
        for (int b0 = 0; b0 < NB; b0 += U) {
            int h[U];
#pragma unroll
            for (int u = 0; u < U; u++) h[u] = b0 + u < NB ? H[(int64_t)(b0 + u) * (V + 1) + id] : 0;
#pragma unroll
            for (int u = 0; u < U; u++)
                if (b0 + u < NB) {
                    H[(int64_t)(b0 + u) * (V + 1) + id] = t;
                    t += h[u];
                }
        }
    }
    sc[threadIdx.x] = t;
    __syncthreads();
    for (int o = 1; o < ENC_G; o <<= 1) {  // inclusive scan (Hillis-Steele)
        const int v = (int)threadIdx.x >= o ? sc[threadIdx.x - o] : 0;
        __syncthreads();
        sc[threadIdx.x] += v;
        __syncthreads();
    }
    if (id <= V) {
        tot[id] = t;
        lbase[id] = sc[threadIdx.x] - t;
    }
    if (threadIdx.x == ENC_G - 1) gsum[blockIdx.x] = sc[ENC_G - 1];
}

// each block first scans the NG group sums in LDS (NG <= ENC_B)
__global__ __launch_bounds__(ENC_B) void enc_scatter_kernel(const int* tokens, int BT, int V, const int* Hpre,
                                                           const int* R, const int* lbase, const int* gsum, int NG,
                                                           int* perm, int* sid) {
    __shared__ int go[ENC_B];
    go[threadIdx.x] = (int)threadIdx.x < NG ? gsum[threadIdx.x] : 0;
    __syncthreads();
    for (int o = 1; o < ENC_B; o <<= 1) {
        const int v = (int)threadIdx.x >= o ? go[threadIdx.x - o] : 0;
        __syncthreads();
        go[threadIdx.x] += v;
        __syncthreads();
    }
    const int i = blockIdx.x * ENC_B + threadIdx.x;
    if (i >= BT) return;
    const int id = enc_bin(tokens[i], V);
    const int g = id / ENC_G;
    const int dst = (g > 0 ? go[g - 1] : 0) + lbase[id] + Hpre[(int64_t)blockIdx.x * (V + 1) + id] + R[i];
    perm[dst] = i;
    sid[dst] = id;
}

// one block per ENC_S sorted slots, one thread per 4 channels; the slots'
// rows are all requested before the runs are summed
template <typename T>
__global__ __launch_bounds__(1024) void enc_chunk_kernel(const T* dx, const int* perm, const int* sid, int BT, int C,
                                                         float* Q) {
    __shared__ int sp[ENC_S], si[ENC_S];
    const int k0 = blockIdx.x * ENC_S, n = min(BT - k0, ENC_S);
    if ((int)threadIdx.x < n) {
        sp[threadIdx.x] = perm[k0 + threadIdx.x];
        si[threadIdx.x] = sid[k0 + threadIdx.x];
    }
    __syncthreads();
    const int c = threadIdx.x * 4;
    if (c >= C) return;
    float v[ENC_S][4];
    if (n == ENC_S) {  // every chunk but the last: all loads unconditional
#pragma unroll
        for (int k = 0; k < ENC_S; k++) {
            const T* r = dx + (int64_t)sp[k] * C + c;
#pragma unroll
            for (int e = 0; e < 4; e++) v[k][e] = to_f32(r[e]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < ENC_S; k++)
            if (k < n) {
                const T* r = dx + (int64_t)sp[k] * C + c;
#pragma unroll
                for (int e = 0; e < 4; e++) v[k][e] = to_f32(r[e]);
            }
    }
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int run = 0;
#pragma unroll
    for (int k = 0; k < ENC_S; k++) {
        if (k >= n) break;
        if (k > 0 && si[k] != si[k - 1]) {
            *reinterpret_cast<float4*>(Q + (int64_t)(k0 + run) * C + c) = make_float4(a0, a1, a2, a3);
            a0 = a1 = a2 = a3 = 0.f;
            run = k;
        }
        a0 += v[k][0];
        a1 += v[k][1];
        a2 += v[k][2];
        a3 += v[k][3];
    }
    *reinterpret_cast<float4*>(Q + (int64_t)(k0 + run) * C + c) = make_float4(a0, a1, a2, a3);
}

// one wave per sorted slot; at an id's first slot, its pieces go into dwte
__global__ __launch_bounds__(256) void enc_segment_kernel(const int* sid, const int* tot, const float* Q, int BT,
                                                          int V, int C, float* dwte) {
    const int k = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (k >= BT) return;
    const int id = sid[k];
    if (id >= V || (k > 0 && sid[k - 1] == id)) return;
    const int end = k + tot[id];
    // up to 4 float4 columns per lane at a time (C <= 1024 in one pass): the
    // first piece and the current gradient rows are requested together
    constexpr int NCH = 4;
    for (int c0 = lane * 4; c0 < C; c0 += 256 * NCH) {
        float4 a[NCH], cur[NCH];
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int c = c0 + j * 256;
            if (c < C) {
                a[j] = *reinterpret_cast<const float4*>(Q + (int64_t)k * C + c);
                cur[j] = *reinterpret_cast<const float4*>(dwte + (int64_t)id * C + c);
            }
        }
        // the further pieces in order (ids whose range crosses a chunk), U at
        // a time
        constexpr int U = 4;
        for (int m0 = (k / ENC_S + 1) * ENC_S; m0 < end; m0 += U * ENC_S) {
            float4 q[U][NCH];
#pragma unroll
            for (int u = 0; u < U; u++)
#pragma unroll
                for (int j = 0; j < NCH; j++) {
                    const int m = m0 + u * ENC_S, c = c0 + j * 256;
                    q[u][j] = m < end && c < C ? *reinterpret_cast<const float4*>(Q + (int64_t)m * C + c)
                                               : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
            for (int u = 0; u < U; u++)
                if (m0 + u * ENC_S < end) {
#pragma unroll
                    for (int j = 0; j < NCH; j++) {
                        a[j].x += q[u][j].x; a[j].y += q[u][j].y; a[j].z += q[u][j].z; a[j].w += q[u][j].w;
                    }
                }
        }
#pragma unroll
        for (int j = 0; j < NCH; j++) {
            const int c = c0 + j * 256;
            if (c < C)
                *reinterpret_cast<float4*>(dwte + (int64_t)id * C + c) =
                    make_float4(cur[j].x + a[j].x, cur[j].y + a[j].y, cur[j].z + a[j].z, cur[j].w + a[j].w);
        }
    }
}

// dwpe[t][c] (+)= sum_b dx[b][t][c] over all maxT positions (0 for t >= T_,
// so that overwrite also clears the positions the batch does not reach);
// each thread takes one 16-byte chunk of channels, summed over b in order.
template <typename T>
__global__ void encoder_bwd_wpe_kernel(float* dwpe, const T* dx, int B, int T_, int maxT, int C, int overwrite) {
    constexpr int VN = Vec16<T>::N;
    const int chunks = C / VN;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= maxT * chunks) return;
    const int t = i / chunks, c = (i - t * chunks) * VN;
    float acc[VN];
#pragma unroll
    for (int j = 0; j < VN; j++) acc[j] = 0.f;
    if (t < T_)
        for (int b = 0; b < B; b++) {
            const Vec16<T> v = ld16(dx + ((int64_t)b * T_ + t) * C + c);
#pragma unroll
            for (int j = 0; j < VN; j++) acc[j] += to_f32(v.v[j]);
        }
    float* o = dwpe + (int64_t)t * C + c;
#pragma unroll
    for (int j = 0; j < VN; j++) o[j] = overwrite ? acc[j] : o[j] + acc[j];
}

template <typename T>
hipError_t encoder_bwd(float* dwte, float* dwpe, const T* dx, const int* tokens, int B, int T_, int maxT, int C,
                       int V, void* ws, bool overwrite, hipStream_t s) {
    const int BT = B * T_;
    if (T_ > maxT || BT <= 0 || C % Vec16<T>::N || C > 4096 || V <= 0 || !ws) return hipErrorInvalidValue;
    EncWs w;
    enc_ws_layout(BT, V, C, (char*)ws, &w);
    const int NB = (int)cdiv(BT, ENC_B), NG = (int)cdiv(V + 1, ENC_G);
    if (NG > ENC_B) return hipErrorInvalidValue;  // V < 256 * 1024
    const int64_t nh = (int64_t)NB * (V + 1);
    fill_i32_kernel<<<(unsigned)std::min<int64_t>(cdiv(nh, 256), 4096), 256, 0, s>>>(w.H, nh);
    enc_rank_kernel<<<NB, ENC_B, 0, s>>>(tokens, BT, V, w.H, w.R);
    enc_group_kernel<<<NG, ENC_G, 0, s>>>(w.H, NB, V, w.tot, w.lbase, w.goff);
    enc_scatter_kernel<<<NB, ENC_B, 0, s>>>(tokens, BT, V, w.H, w.R, w.lbase, w.goff, NG, w.perm, w.sid);
    const int nt = (int)cdiv(C / 4, 64) * 64;
    enc_chunk_kernel<T><<<(unsigned)cdiv(BT, ENC_S), nt, 0, s>>>(dx, w.perm, w.sid, BT, C, w.Q);
    enc_segment_kernel<<<(unsigned)cdiv(BT, 4), 256, 0, s>>>(w.sid, w.tot, w.Q, BT, V, C, dwte);
    encoder_bwd_wpe_kernel<T><<<cdiv((int64_t)maxT * (C / Vec16<T>::N), 256), 256, 0, s>>>(dwpe, dx, B, T_, maxT, C,
                                                                                            overwrite);
    return LAUNCH_CHECK();
}

// ============================================================================
// LayerNorm forward: mean, biased variance, rstd = 1/sqrt(var + 1e-5);
// y = (x - mean) * rstd * w + b; mean and rstd saved for the backward
// (origin-of-llm.c transcript, "Pure C").  One wavefront per row, the row
// held in registers (up to MAXV 16-byte chunks per lane); each wave takes R
// rows (stride 4 rows apart) and requests all of them before any arithmetic.
// ============================================================================
constexpr int LN_MAXV = 8;

template <typename T, int MAXV, int R>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(T* out, float* mean, float* rstd, const T* x,
                                                            const float* w, const float* b, int N, int C) {
    constexpr int VN = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    // the wave index read into a scalar register: row addresses are then a
    // scalar base plus small lane offsets
    const int row0 = blockIdx.x * 4 * R + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunks = C / VN;
    Vec16<T> q[R][MAXV];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = row0 + 4 * r;
#pragma unroll
        for (int i = 0; i < MAXV; i++) {
            const int ch = lane + i * 64;
            if (row < N && ch < chunks) q[r][i] = ld16(x + (int64_t)row * C + ch * VN);
        }
    }
    float mu[R], rs[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < MAXV; i++)
            if (lane + i * 64 < chunks)
#pragma unroll
                for (int j = 0; j < VN; j++) s += to_f32(q[r][i].v[j]);
        mu[r] = wave_sum(s) / C;
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < MAXV; i++)
            if (lane + i * 64 < chunks)
#pragma unroll
                for (int j = 0; j < VN; j++) {
                    const float d = to_f32(q[r][i].v[j]) - mu[r];
                    ss += d * d;
                }
        rs[r] = rsqrtf(wave_sum(ss) / C + 1e-5f);
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = row0 + 4 * r;
        if (row >= N) break;
        T* orow = out + (int64_t)row * C;
#pragma unroll
        for (int i = 0; i < MAXV; i++) {
            const int ch = lane + i * 64;
            if (ch < chunks) {
                Vec16<T> o;
#pragma unroll
                for (int j = 0; j < VN; j++) {
                    const int c = ch * VN + j;
                    o.v[j] = from_f32<T>((to_f32(q[r][i].v[j]) - mu[r]) * rs[r] * w[c] + b[c]);
                }
                st16(orow + ch * VN, o);
            }
        }
        if (lane == 0) {
            mean[row] = mu[r];
            rstd[row] = rs[r];
        }
    }
}

// The same LayerNorm with each wave taking rows row0, row0 + step, ...
// (step = 4 x the grid): the lane's gains and biases are read once into
// registers, and the next row's chunks are requested before the current row
// is worked.  Per-lane sums run over the chunks in the same order as above,
// so the results are the same bit for bit.
template <typename T, int MAXV>
__global__ __launch_bounds__(256) void layernorm_fwd_rows_kernel(T* out, float* mean, float* rstd, const T* x,
                                                                 const float* w, const float* b, int N, int C) {
    constexpr int VN = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int step = gridDim.x * 4;
    int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunks = C / VN;
    float wr[MAXV][VN], br[MAXV][VN];
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int ch = lane + i * 64;
#pragma unroll
        for (int j = 0; j < VN; j += 4) {
            float4 u = make_float4(0.f, 0.f, 0.f, 0.f), v = u;
            if (ch < chunks) {
                u = *reinterpret_cast<const float4*>(w + ch * VN + j);
                v = *reinterpret_cast<const float4*>(b + ch * VN + j);
            }
            wr[i][j] = u.x; wr[i][j + 1] = u.y; wr[i][j + 2] = u.z; wr[i][j + 3] = u.w;
            br[i][j] = v.x; br[i][j + 1] = v.y; br[i][j + 2] = v.z; br[i][j + 3] = v.w;
        }
    }
    Vec16<T> q[MAXV], qn[MAXV];
    auto load = [&](Vec16<T>(&dst)[MAXV], int r) {
#pragma unroll
        for (int i = 0; i < MAXV; i++) {
            const int ch = lane + i * 64;
            if (ch < chunks) dst[i] = ld16(x + (int64_t)r * C + ch * VN);
        }
    };
    if (row < N) load(q, row);
    for (; row < N; row += step) {
        if (row + step < N) load(qn, row + step);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < MAXV; i++)
            if (lane + i * 64 < chunks)
#pragma unroll
                for (int j = 0; j < VN; j++) s += to_f32(q[i].v[j]);
        const float mu = wave_sum(s) / C;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < MAXV; i++)
            if (lane + i * 64 < chunks)
#pragma unroll
                for (int j = 0; j < VN; j++) {
                    const float d = to_f32(q[i].v[j]) - mu;
                    ss += d * d;
                }
        const float rs = rsqrtf(wave_sum(ss) / C + 1e-5f);
        T* orow = out + (int64_t)row * C;
#pragma unroll
        for (int i = 0; i < MAXV; i++) {
            const int ch = lane + i * 64;
            if (ch < chunks) {
                Vec16<T> o;
#pragma unroll
                for (int j = 0; j < VN; j++) o.v[j] = from_f32<T>((to_f32(q[i].v[j]) - mu) * rs * wr[i][j] + br[i][j]);
                st16(orow + ch * VN, o);
            }
        }
        if (lane == 0) {
            mean[row] = mu;
            rstd[row] = rs;
        }
#pragma unroll
        for (int i = 0; i < MAXV; i++) q[i] = qn[i];
    }
}

// Sums over each half-wave of x, for the half h the lane is in: row-wise DPP
// adds leave the sum of the 16-lane row r in lane 16r, and half h adds rows
// 2h and 2h + 1.
DEVI void half_sums(float x, int h, float& s) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x124>(x);
    x += dpp_mov<0x128>(x);
    const float s0 = lane_value(x, 0) + lane_value(x, 16), s1 = lane_value(x, 32) + lane_value(x, 48);
    s = h ? s1 : s0;
}

// Rows of 32*CPL 16-byte chunks with CPL odd (C = 768 in bf16): one row per
// half-wave, lane l of the half holding the chunks l, l + 32, ... (every lane
// CPL chunks, where the whole-wave kernel leaves half the lanes idle in its
// last chunk); the wave works rows r + h, r + step + h, ... two at a time,
// the next two requested first.  Row sums as in the LayerNorm backward's
// half-wave kernel.
template <typename T, int CPL>
__global__ __launch_bounds__(256) void layernorm_fwd_half_kernel(T* out, float* mean, float* rstd, const T* x,
                                                                 const float* w, const float* b, int N, int C) {
    constexpr int VN = Vec16<T>::N;
    const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int step = gridDim.x * 8;
    const int r0 = (blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 2;
    float wr[CPL][VN], br[CPL][VN];
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int ch = l32 + i * 32;
#pragma unroll
        for (int j = 0; j < VN; j += 4) {
            const float4 u = *reinterpret_cast<const float4*>(w + ch * VN + j);
            const float4 v = *reinterpret_cast<const float4*>(b + ch * VN + j);
            wr[i][j] = u.x; wr[i][j + 1] = u.y; wr[i][j + 2] = u.z; wr[i][j + 3] = u.w;
            br[i][j] = v.x; br[i][j + 1] = v.y; br[i][j + 2] = v.z; br[i][j + 3] = v.w;
        }
    }
    Vec16<T> q[CPL], qn[CPL];
    auto load = [&](Vec16<T>(&dst)[CPL], int row) {
        if (row >= N) return;
#pragma unroll
        for (int i = 0; i < CPL; i++) dst[i] = ld16(x + (int64_t)row * C + (l32 + i * 32) * VN);
    };
    load(q, r0 + h);
    // both halves run every pair (they share the row sums' lane reads)
    for (int r = r0; r < N; r += step) {
        const int row = r + h;
        load(qn, row + step);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; i++)
#pragma unroll
            for (int j = 0; j < VN; j++) s += to_f32(q[i].v[j]);
        half_sums(s, h, s);
        const float mu = s / C;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; i++)
#pragma unroll
            for (int j = 0; j < VN; j++) {
                const float d = to_f32(q[i].v[j]) - mu;
                ss += d * d;
            }
        half_sums(ss, h, ss);
        const float rs = rsqrtf(ss / C + 1e-5f);
        if (row < N) {
            T* orow = out + (int64_t)row * C;
#pragma unroll
            for (int i = 0; i < CPL; i++) {
                const int ch = l32 + i * 32;
                Vec16<T> o;
#pragma unroll
                for (int j = 0; j < VN; j++) o.v[j] = from_f32<T>((to_f32(q[i].v[j]) - mu) * rs * wr[i][j] + br[i][j]);
                st16(orow + ch * VN, o);
            }
            if (l32 == 0) {
                mean[row] = mu;
                rstd[row] = rs;
            }
        }
#pragma unroll
        for (int i = 0; i < CPL; i++) q[i] = qn[i];
    }
}

#ifndef LN_FWD_ROWS_PER_WAVE
#define LN_FWD_ROWS_PER_WAVE 4
#endif

template <typename T>
hipError_t layernorm_fwd(T* out, float* mean, float* rstd, const T* x, const float* w, const float* b, int N,
                         int C, hipStream_t s) {
    if (C % Vec16<T>::N || C / Vec16<T>::N > LN_MAXV * 64) return hipErrorInvalidValue;
    const int per_lane = (int)cdiv(C / Vec16<T>::N, 64);
    // rows per wave: 4 for rows of one chunk per lane; one at two chunks per
    // lane (C = 768 in bf16: more, shorter waves overlap one block's stores
    // with another's loads, ~3% faster than 4 rows per wave), two beyond
#define LN_FWD(V, R) layernorm_fwd_kernel<T, V, R><<<cdiv(N, 4 * R), 256, 0, s>>>(out, mean, rstd, x, w, b, N, C)
#define LN_FWD_ROWS(V)                                                                                            \
    layernorm_fwd_rows_kernel<T, V><<<cdiv(N, 4 * LN_FWD_ROWS_PER_WAVE), 256, 0, s>>>(out, mean, rstd, x, w, b, N, C)
    if (per_lane <= 1) LN_FWD(1, 4);
    else if (std::is_same<T, bf16>::value && C == 768)  // a row per half-wave, 4 rows per wave
        layernorm_fwd_half_kernel<T, 3><<<cdiv(N, 16), 256, 0, s>>>(out, mean, rstd, x, w, b, N, C);
    else if (per_lane <= 2) LN_FWD_ROWS(2);
    else if (per_lane <= 4) LN_FWD_ROWS(4);
    else LN_FWD(8, 1);
#undef LN_FWD
#undef LN_FWD_ROWS
    return LAUNCH_CHECK();
}

// ============================================================================
// LayerNorm backward.  With xhat = (x-mean)*rstd and g = dy*w:
//   dx = rstd * (g - mean_c(g) - xhat * mean_c(g*xhat)),  dout = din + dx
//   (the residual-stream gradient, written out of place),
//   dw += sum_rows dy*xhat,  db += sum_rows dy,
// and, with NP = 3, the column sums of dout as well: that is the gradient of
// the bias of the projection whose output joined the residual stream at this
// point.  Each block handles rows blk*4+wave, stepping by 4*G, R rows at a
// time (the next R rows' operands are requested before the current ones are
// worked), keeps its per-channel sums in registers, reduces its 4 waves in
// LDS and writes one partial row per sum; sum_partials_batch adds the G
// partials in block order.
// ============================================================================
constexpr int LN_BWD_G = 512;

// bf16 rows of 768 (the half-wave kernel): blocks of 8 waves, so half as many
// partial rows for the same waves (the partial sums read them back from HBM)
int layernorm_bwd_blocks(int N, int C, bool bf16) {
    if (bf16 && C == 768) return (int)std::min<int64_t>(cdiv(N, 16), LN_BWD_G / 2);
    return (int)std::min<int64_t>(cdiv(N, 4), LN_BWD_G);
}

// Register budget: two waves per SIMD (256 VGPRs) up to 2 chunks per lane;
// wider rows (C > 1024 in bf16) hold 4 or 8 chunks of three operands plus
// NP x chunks accumulators per lane and take one wave per SIMD (512 VGPRs)
// rather than spilling.
template <int MAXV> constexpr int ln_bwd_occupancy() { return MAXV <= 2 ? 2 : 1; }

template <typename T, int MAXV, int NP, int R>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ln_bwd_occupancy<MAXV>(),
                                                                      ln_bwd_occupancy<MAXV>())))
void layernorm_bwd_kernel(T* dout, const T* din, const T* dy, const T* x, const float* w, const float* mean,
                          const float* rstd, float* partial, int N, int C) {
    constexpr int VN = Vec16<T>::N;
    extern __shared__ float smem[];  // [4][NP][C]
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
    const int chunks = C / VN;
    const int step = gridDim.x * 4;  // a wave's rows: row0, row0 + step, ...
    const int row0 = blockIdx.x * 4 + wv;
    float acc[NP][MAXV][VN];
    float wr[MAXV][VN];
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int ch = lane + i * 64;
#pragma unroll
        for (int j = 0; j < VN; j++) {
            wr[i][j] = ch < chunks ? w[ch * VN + j] : 0.f;
#pragma unroll
            for (int k = 0; k < NP; k++) acc[k][i][j] = 0.f;
        }
    }
    // operands of the R rows being worked (c) and of the next R (n)
    Vec16<T> xc[R][MAXV], dc[R][MAXV], oc[R][MAXV], xn[R][MAXV], dn[R][MAXV], on[R][MAXV];
    float mun[R], rsn[R];
    auto load = [&](int k0) {
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int row = row0 + (k0 + r) * step;
            if (row < N) {
                const int64_t o = (int64_t)row * C;
#pragma unroll
                for (int i = 0; i < MAXV; i++) {
                    const int ch = lane + i * 64;
                    if (ch < chunks) {
                        xn[r][i] = ld16(x + o + ch * VN);
                        dn[r][i] = ld16(dy + o + ch * VN);
                        if (din) on[r][i] = ld16(din + o + ch * VN);
                    }
                }
                mun[r] = mean[row];
                rsn[r] = rstd[row];
            }
        }
    };
    load(0);
    for (int k0 = 0; row0 + k0 * step < N; k0 += R) {
        float mu[R], rs[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            mu[r] = mun[r];
            rs[r] = rsn[r];
#pragma unroll
            for (int i = 0; i < MAXV; i++) { xc[r][i] = xn[r][i]; dc[r][i] = dn[r][i]; oc[r][i] = on[r][i]; }
        }
        if (row0 + (k0 + R) * step < N) load(k0 + R);
        float sg[R], sgx[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            sg[r] = 0.f;
            sgx[r] = 0.f;
            if (row0 + (k0 + r) * step >= N) continue;
#pragma unroll
            for (int i = 0; i < MAXV; i++) {
                if (lane + i * 64 < chunks) {
#pragma unroll
                    for (int j = 0; j < VN; j++) {
                        const float d = to_f32(dc[r][i].v[j]);
                        const float xh = (to_f32(xc[r][i].v[j]) - mu[r]) * rs[r];
                        const float gg = d * wr[i][j];
                        sg[r] += gg;
                        sgx[r] += gg * xh;
                        acc[0][i][j] += d * xh;
                        acc[1][i][j] += d;
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            sg[r] = wave_sum(sg[r]) / C;
            sgx[r] = wave_sum(sgx[r]) / C;
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int row = row0 + (k0 + r) * step;
            if (row >= N) continue;
            T* orow = dout + (int64_t)row * C;
#pragma unroll
            for (int i = 0; i < MAXV; i++) {
                const int ch = lane + i * 64;
                if (ch < chunks) {
                    Vec16<T> o;
#pragma unroll
                    for (int j = 0; j < VN; j++) {
                        const float xh = (to_f32(xc[r][i].v[j]) - mu[r]) * rs[r];
                        const float gg = to_f32(dc[r][i].v[j]) * wr[i][j];
                        const float dx = rs[r] * (gg - sg[r] - xh * sgx[r]);
                        const T v = from_f32<T>(din ? to_f32(oc[r][i].v[j]) + dx : dx);
                        o.v[j] = v;
                        if constexpr (NP == 3) acc[2][i][j] += to_f32(v);
                    }
                    st16(orow + ch * VN, o);
                }
            }
        }
    }
    // block reduction of the per-channel sums over the 4 waves
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int ch = lane + i * 64;
        if (ch < chunks) {
#pragma unroll
            for (int k = 0; k < NP; k++)
#pragma unroll
                for (int j = 0; j < VN; j++) smem[(wv * NP + k) * C + ch * VN + j] = acc[k][i][j];
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += 256) {
#pragma unroll
        for (int k = 0; k < NP; k++) {
            float t = 0.f;
            for (int q = 0; q < 4; q++) t += smem[(q * NP + k) * C + c];
            partial[((int64_t)k * gridDim.x + blockIdx.x) * C + c] = t;
        }
    }
}

// Rows of 32*CPL 16-byte chunks with CPL odd (C = 768 in bf16: CPL = 3),
// which the whole-wave kernel spreads unevenly (lanes 0-31 two chunks, lanes
// 32-63 one): each half-wave takes a row of its own, lane l of the half the
// chunks l, l + 32, ...; the wave works two rows at a time (its next two
// requested first), with the same per-row arithmetic.  The halves' row sums
// come out of one pass of row-wise DPP adds (lanes 16r hold the sums of the
// 16-lane rows r; the half h adds rows 2h and 2h + 1).  Channel sums as in the
// whole-wave kernel, the two halves added (half 0 first), then the block's 8
// waves: partial[k][block][c], the same layout.
constexpr int LN_HALF_NW = 8;  // waves per block

template <typename T, int CPL, int NP>
__global__ __launch_bounds__(LN_HALF_NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void layernorm_bwd_half_kernel(T* dout, const T* din, const T* dy, const T* x, const float* w, const float* mean,
                               const float* rstd, float* partial, int N, int C) {
    constexpr int VN = Vec16<T>::N;
    extern __shared__ float smem[];  // [LN_HALF_NW][NP][C]
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
    const int h = lane >> 5, l32 = lane & 31;
    const int step = gridDim.x * LN_HALF_NW * 2;               // rows between a wave's consecutive pairs
    const int row0 = (blockIdx.x * LN_HALF_NW + wv) * 2 + h;  // this half's first row
    float acc[NP][CPL][VN];
    float wr[CPL][VN];
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int ch = l32 + i * 32;
#pragma unroll
        for (int j = 0; j < VN; j++) {
            wr[i][j] = w[ch * VN + j];
#pragma unroll
            for (int k = 0; k < NP; k++) acc[k][i][j] = 0.f;
        }
    }
    Vec16<T> xc[CPL], dc[CPL], oc[CPL], xn[CPL], dn[CPL], on[CPL];
    float mun = 0.f, rsn = 0.f;
    auto load = [&](int row) {
        if (row >= N) return;
        const int64_t o = (int64_t)row * C;
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            const int ch = l32 + i * 32;
            xn[i] = ld16(x + o + ch * VN);
            dn[i] = ld16(dy + o + ch * VN);
            if (din) on[i] = ld16(din + o + ch * VN);
        }
        mun = mean[row];
        rsn = rstd[row];
    };
    load(row0);
    // every wave runs while either of its halves has a row (both halves take
    // part in the row sums' lane reads)
    for (int r = row0 - h; r < N; r += step) {
        const int row = r + h;
        const bool ok = row < N;
        const float mu = mun, rs = rsn;
#pragma unroll
        for (int i = 0; i < CPL; i++) { xc[i] = xn[i]; dc[i] = dn[i]; oc[i] = on[i]; }
        load(row + step);
        float sg = 0.f, sgx = 0.f;
        if (ok) {
#pragma unroll
            for (int i = 0; i < CPL; i++)
#pragma unroll
                for (int j = 0; j < VN; j++) {
                    const float d = to_f32(dc[i].v[j]);
                    const float xh = (to_f32(xc[i].v[j]) - mu) * rs;
                    const float gg = d * wr[i][j];
                    sg += gg;
                    sgx += gg * xh;
                    acc[0][i][j] += d * xh;
                    acc[1][i][j] += d;
                }
        }
        half_sums(sg, h, sg);
        half_sums(sgx, h, sgx);
        sg /= C;
        sgx /= C;
        if (!ok) continue;
        T* orow = dout + (int64_t)row * C;
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            const int ch = l32 + i * 32;
            Vec16<T> o;
#pragma unroll
            for (int j = 0; j < VN; j++) {
                const float xh = (to_f32(xc[i].v[j]) - mu) * rs;
                const float gg = to_f32(dc[i].v[j]) * wr[i][j];
                const float dx = rs * (gg - sg - xh * sgx);
                const T v = from_f32<T>(din ? to_f32(oc[i].v[j]) + dx : dx);
                o.v[j] = v;
                if constexpr (NP == 3) acc[2][i][j] += to_f32(v);
            }
            st16(orow + ch * VN, o);
        }
    }
    // the halves' channel sums (half 0 first), then the block's waves
#pragma unroll
    for (int k = 0; k < NP; k++)
#pragma unroll
        for (int i = 0; i < CPL; i++)
#pragma unroll
            for (int j = 0; j < VN; j++) {
                const float other = __shfl_xor(acc[k][i][j], 32, 64);
                acc[k][i][j] = h ? other + acc[k][i][j] : acc[k][i][j] + other;
            }
    if (h == 0) {
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            const int ch = l32 + i * 32;
#pragma unroll
            for (int k = 0; k < NP; k++)
#pragma unroll
                for (int j = 0; j < VN; j++) smem[(wv * NP + k) * C + ch * VN + j] = acc[k][i][j];
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += LN_HALF_NW * 64) {
#pragma unroll
        for (int k = 0; k < NP; k++) {
            float t = 0.f;
            for (int q = 0; q < LN_HALF_NW; q++) t += smem[(q * NP + k) * C + c];
            partial[((int64_t)k * gridDim.x + blockIdx.x) * C + c] = t;
        }
    }
}

// Rows of 129-256 16-byte chunks (C = 1032 ... 2048 in bf16): each row is
// split over a pair of waves, wave h of the pair taking half h of its chunks,
// so a lane holds at most two chunks of each operand and the kernel keeps two
// waves per SIMD (the whole-row kernel needs one wave per SIMD there).  The
// block's two pairs work rows rbase and rbase + 1 of each step; the pair adds
// its two halves of the row sums (half 0 first) through a double-buffered LDS
// slot, one barrier per step, and every wave runs the same steps, so all of
// them reach every barrier.  Channel sums as above, per pair, then the two
// pairs added: partial[k][block][c], the same layout.
template <typename T, int NP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void layernorm_bwd_split_kernel(T* dout, const T* din, const T* dy, const T* x, const float* w, const float* mean,
                                const float* rstd, float* partial, int N, int C) {
    constexpr int VN = Vec16<T>::N, MAXV = 2;
    extern __shared__ float smem[];  // [2 pairs][NP][C]
    __shared__ float rsum[2][2][2][2];  // [buffer][pair][half][sum g, sum g*xhat]
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform
    const int pair = wv >> 1, half = wv & 1;
    const int chunks = C / VN, H = (chunks + 1) / 2;
    const int cbeg = half * H, cend = min(chunks, cbeg + H);
    const int step = gridDim.x * 2;
    float acc[NP][MAXV][VN];
    float wr[MAXV][VN];
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int ch = cbeg + lane + i * 64;
#pragma unroll
        for (int j = 0; j < VN; j++) {
            wr[i][j] = ch < cend ? w[ch * VN + j] : 0.f;
#pragma unroll
            for (int k = 0; k < NP; k++) acc[k][i][j] = 0.f;
        }
    }
    Vec16<T> xc[MAXV], dc[MAXV], oc[MAXV], xn[MAXV], dn[MAXV], on[MAXV];
    float mun = 0.f, rsn = 0.f;
    auto load = [&](int row) {
        if (row >= N) return;
        const int64_t o = (int64_t)row * C;
#pragma unroll
        for (int i = 0; i < MAXV; i++) {
            const int ch = cbeg + lane + i * 64;
            if (ch < cend) {
                xn[i] = ld16(x + o + ch * VN);
                dn[i] = ld16(dy + o + ch * VN);
                if (din) on[i] = ld16(din + o + ch * VN);
            }
        }
        mun = mean[row];
        rsn = rstd[row];
    };
    int buf = 0;
    load(blockIdx.x * 2 + pair);
    for (int rbase = blockIdx.x * 2; rbase < N; rbase += step, buf ^= 1) {
        const int row = rbase + pair;
        const float mu = mun, rs = rsn;
#pragma unroll
        for (int i = 0; i < MAXV; i++) { xc[i] = xn[i]; dc[i] = dn[i]; oc[i] = on[i]; }
        load(rbase + step + pair);
        float sg = 0.f, sgx = 0.f;
        if (row < N) {
#pragma unroll
            for (int i = 0; i < MAXV; i++) {
                if (cbeg + lane + i * 64 < cend) {
#pragma unroll
                    for (int j = 0; j < VN; j++) {
                        const float d = to_f32(dc[i].v[j]);
                        const float xh = (to_f32(xc[i].v[j]) - mu) * rs;
                        const float gg = d * wr[i][j];
                        sg += gg;
                        sgx += gg * xh;
                        acc[0][i][j] += d * xh;
                        acc[1][i][j] += d;
                    }
                }
            }
        }
        sg = wave_sum(sg);
        sgx = wave_sum(sgx);
        if (lane == 0) {
            rsum[buf][pair][half][0] = sg;
            rsum[buf][pair][half][1] = sgx;
        }
        __syncthreads();
        const float SG = (rsum[buf][pair][0][0] + rsum[buf][pair][1][0]) / C;
        const float SGX = (rsum[buf][pair][0][1] + rsum[buf][pair][1][1]) / C;
        if (row < N) {
            T* orow = dout + (int64_t)row * C;
#pragma unroll
            for (int i = 0; i < MAXV; i++) {
                const int ch = cbeg + lane + i * 64;
                if (ch < cend) {
                    Vec16<T> o;
#pragma unroll
                    for (int j = 0; j < VN; j++) {
                        const float xh = (to_f32(xc[i].v[j]) - mu) * rs;
                        const float gg = to_f32(dc[i].v[j]) * wr[i][j];
                        const float dx = rs * (gg - SG - xh * SGX);
                        const T v = from_f32<T>(din ? to_f32(oc[i].v[j]) + dx : dx);
                        o.v[j] = v;
                        if constexpr (NP == 3) acc[2][i][j] += to_f32(v);
                    }
                    st16(orow + ch * VN, o);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MAXV; i++) {
        const int ch = cbeg + lane + i * 64;
        if (ch < cend) {
#pragma unroll
            for (int k = 0; k < NP; k++)
#pragma unroll
                for (int j = 0; j < VN; j++) smem[(pair * NP + k) * C + ch * VN + j] = acc[k][i][j];
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += 256) {
#pragma unroll
        for (int k = 0; k < NP; k++)
            partial[((int64_t)k * gridDim.x + blockIdx.x) * C + c] = smem[k * C + c] + smem[(NP + k) * C + c];
    }
}

// For each job, out_k[c] += sum_g partial[k*G + g][c] for its non-null out_k
// (k < 3).  Block: 64 columns x 64 row lanes of one job (the jobs' blocks are
// laid end to end); each lane holds 4 consecutive columns (16 lanes read 256
// contiguous bytes of a partial row), row lane r sums partial rows r, r+64,
// ... in that order, U rows' loads issued before their adds, then the 64
// row-lane sums of a column are combined in a fixed order.
struct SumBatch {
    SumJob job[SUM_JOBS_MAX];
    int start[SUM_JOBS_MAX + 1];  // first block of each job
    int n;
    int overwrite;  // out = sum instead of out += sum
};

// Each partial row is read once, long after it was written: non-temporal
// loads (the step's batch, ~146 MB from cold caches: 71.6 -> 34.8 us).
DEVI float4 ld_f4_stream(const float* p) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__global__ __launch_bounds__(1024) void sum_partials_kernel(SumBatch bt) {
    __shared__ __attribute__((aligned(16))) float red[3][64][68];  // read and written as float4
    // the job whose block range holds this block: the last k with start[k] <= blockIdx.x
    int k = 0;
    for (int w = SUM_JOBS_MAX / 2; w >= 1; w >>= 1)
        if (k + w < bt.n && (int)blockIdx.x >= bt.start[k + w]) k += w;
    const SumJob& jb = bt.job[k];
    const int G = jb.G, C = jb.C;  // C % 4 == 0 (checked by the caller)
    const float* partial = jb.partial;
    // a block takes 64 columns: lane cx of row lane ry holds columns
    // c0 .. c0 + 3, so 16 lanes read 256 contiguous bytes of a partial row
    const int cx = threadIdx.x & 15, ry = threadIdx.x >> 4;
    const int cb = ((int)blockIdx.x - bt.start[k]) * 64;
    const int c0 = cb + cx * 4;
    const int nk = jb.out[2] ? 3 : jb.out[1] ? 2 : 1;  // out[0] is always given
    // rows ry, ry + 64, ... in that order, U rows' loads issued before their
    // adds (U = 4: three operands of 4 x float4 fit 128 registers)
    constexpr int U = 4;
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 t0 = z4, t1 = z4, t2 = z4;
    auto add4 = [](float4& t, const float4& v) { t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w; };
    if (c0 < C)
        for (int g0 = ry; g0 < G; g0 += 64 * U) {
            float4 v0[U], v1[U], v2[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int g = g0 + 64 * u;
                const float* pr = partial + (int64_t)g * C + c0;
                v0[u] = g < G ? ld_f4_stream(pr) : z4;
                v1[u] = nk > 1 && g < G ? ld_f4_stream(pr + (int64_t)G * C) : z4;
                v2[u] = nk > 2 && g < G ? ld_f4_stream(pr + 2 * (int64_t)G * C) : z4;
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                add4(t0, v0[u]);
                add4(t1, v1[u]);
                add4(t2, v2[u]);
            }
        }
    *reinterpret_cast<float4*>(&red[0][ry][cx * 4]) = t0;
    *reinterpret_cast<float4*>(&red[1][ry][cx * 4]) = t1;
    *reinterpret_cast<float4*>(&red[2][ry][cx * 4]) = t2;
    __syncthreads();
    if (threadIdx.x < 192) {
        const int q = threadIdx.x >> 6, col = threadIdx.x & 63, c = cb + col;
        float* out = q == 0 ? jb.out[0] : q == 1 ? jb.out[1] : jb.out[2];
        if (c < C && out) {
            float t = 0.f;
            for (int i = 0; i < 64; i++) t += red[q][i][col];
            out[c] = bt.overwrite ? t : out[c] + t;
        }
    }
}

hipError_t sum_partials_batch(const SumJob* jobs, int n, bool overwrite, hipStream_t s) {
    if (n < 0) return hipErrorInvalidValue;
    for (int i = 0; i < n; i++)  // whole float4 groups of columns: C % 4 == 0, 16-byte aligned partial rows
        if (!jobs[i].out[0] || !jobs[i].partial || jobs[i].G <= 0 || jobs[i].C <= 0 || jobs[i].C % 4 ||
            (uintptr_t)jobs[i].partial % 16)
            return hipErrorInvalidValue;
    for (int j0 = 0; j0 < n; j0 += SUM_JOBS_MAX) {
        const int m = std::min(n - j0, SUM_JOBS_MAX);
        SumBatch bt{};
        bt.n = m;
        bt.overwrite = overwrite ? 1 : 0;
        bt.start[0] = 0;
        for (int i = 0; i < m; i++) {
            bt.job[i] = jobs[j0 + i];
            bt.start[i + 1] = bt.start[i] + (int)cdiv(jobs[j0 + i].C, 64);
        }
        sum_partials_kernel<<<bt.start[m], 1024, 0, s>>>(bt);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t sum_partials(float* out0, float* out1, float* out2, const float* partial, int G, int C, hipStream_t s) {
    const SumJob j{{out0, out1, out2}, partial, G, C};
    return sum_partials_batch(&j, 1, false, s);
}

template <typename T>
hipError_t layernorm_bwd(T* dout, const T* din, const T* dy, const T* x, const float* w, const float* mean,
                         const float* rstd, float* partial, int N, int C, bool dsum, hipStream_t s) {
    if (C % Vec16<T>::N || C / Vec16<T>::N > LN_MAXV * 64 || N <= 0) return hipErrorInvalidValue;
    const int G = layernorm_bwd_blocks(N, C, std::is_same<T, bf16>::value);
    const int NP = dsum ? 3 : 2;
    const size_t lds = sizeof(float) * 4 * NP * C;
    const int per_lane = (int)cdiv(C / Vec16<T>::N, 64);
#define LN_BWD(V, R)                                                                                               \
    (dsum ? layernorm_bwd_kernel<T, V, 3, R><<<G, 256, lds, s>>>(dout, din, dy, x, w, mean, rstd, partial, N, C)  \
          : layernorm_bwd_kernel<T, V, 2, R><<<G, 256, lds, s>>>(dout, din, dy, x, w, mean, rstd, partial, N, C))
    // two chunks per lane (C = 768 in bf16): one row at a time, its successor
    // requested first, measured ~5% faster than two (more waves per SIMD or a
    // larger grid gain nothing and add partial rows)
    if (per_lane <= 1) LN_BWD(1, 2);
    else if (std::is_same<T, bf16>::value && C == 768) {
        // rows per half-wave
        const size_t ldsh = sizeof(float) * LN_HALF_NW * NP * C;
        if (dsum)
            layernorm_bwd_half_kernel<T, 3, 3><<<G, LN_HALF_NW * 64, ldsh, s>>>(dout, din, dy, x, w, mean, rstd, partial, N, C);
        else
            layernorm_bwd_half_kernel<T, 3, 2><<<G, LN_HALF_NW * 64, ldsh, s>>>(dout, din, dy, x, w, mean, rstd, partial, N, C);
    } else if (per_lane <= 2) LN_BWD(2, 1);
    else if (per_lane <= 4 && (C / Vec16<T>::N + 1) / 2 <= 128) {
        // rows split over two waves (C = 1600 in bf16, 8192 rows: 37.8 -> 25.5 us per
        // launch against the whole-row kernel at one wave per SIMD)
        const size_t lds2 = sizeof(float) * 2 * NP * C;
        if (dsum) layernorm_bwd_split_kernel<T, 3><<<G, 256, lds2, s>>>(dout, din, dy, x, w, mean, rstd, partial, N, C);
        else layernorm_bwd_split_kernel<T, 2><<<G, 256, lds2, s>>>(dout, din, dy, x, w, mean, rstd, partial, N, C);
    } else if (per_lane <= 4) LN_BWD(4, 2);
    else LN_BWD(8, 1);
#undef LN_BWD
    return LAUNCH_CHECK();
}

// ============================================================================
// bias gradient: dbias[n] += sum_m dy[m][n]
// Block: 64 column chunks x 4 row lanes; grid.y = G row groups.
// ============================================================================
constexpr int COLSUM_G = 256;

template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(float* partial, const T* dy, int M, int N) {
    constexpr int VN = Vec16<T>::N;
    __shared__ float red[4][64][VN];
    int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
    int ch = blockIdx.x * 64 + cx;
    int chunks = N / VN;
    float acc[VN];
#pragma unroll
    for (int j = 0; j < VN; j++) acc[j] = 0.f;
    if (ch < chunks) {
        for (int m = blockIdx.y * 4 + ry; m < M; m += gridDim.y * 4) {
            Vec16<T> q = ld16(dy + (int64_t)m * N + ch * VN);
#pragma unroll
            for (int j = 0; j < VN; j++) acc[j] += to_f32(q.v[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < VN; j++) red[ry][cx][j] = acc[j];
    __syncthreads();
    if (ry == 0 && ch < chunks) {
#pragma unroll
        for (int j = 0; j < VN; j++) {
            float s = red[0][cx][j] + red[1][cx][j] + red[2][cx][j] + red[3][cx][j];
            partial[(int64_t)blockIdx.y * N + ch * VN + j] = s;
        }
    }
}

template <typename T>
hipError_t colsum_accum(float* dbias, const T* dy, int M, int N, float* partial, hipStream_t s) {
    constexpr int VN = Vec16<T>::N;
    if (N % VN) return hipErrorInvalidValue;
    int G = COLSUM_G;
    dim3 grid(cdiv(N / VN, 64), G);
    colsum_kernel<T><<<grid, 256, 0, s>>>(partial, dy, M, N);
    hipError_t e = LAUNCH_CHECK();
    return e != hipSuccess ? e : sum_partials(dbias, nullptr, nullptr, partial, G, N, s);
}

// ============================================================================
// Fused softmax + cross-entropy + dlogits (the pyshine tour's "fused
// classifier": the softmax loss merged with the output projection's
// backward seed).  One block per row; pass 1 keeps an online (max, sum) per
// thread over the real columns v < V, pass 2 rewrites the row in place as
// (softmax - onehot(target)) * dscale and zeros the padded columns.
// ============================================================================
// block-wide max / sum over NT threads (fixed combine order)
template <int NT> DEVI float block_max(float x, float* sh) {
    x = wave_max(x);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < NT / 64; i++) r = fmaxf(r, sh[i]);
    __syncthreads();  // sh is reused by the next reduction
    return r;
}
template <int NT> DEVI float block_sum(float x, float* sh) {
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; i++) r += sh[i];
    return r;
}

// Makes the packed chunk opaque to the compiler, so that each pass widens it
// again instead of keeping every widened value live across passes.
template <typename T> DEVI void keep_packed(Vec16<T>& q) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    u32x4_t r;
    __builtin_memcpy(&r, &q, 16);
    asm volatile("" : "+v"(r));
    __builtin_memcpy(&q, &r, 16);
}

// One block of NT threads per row.  The row is read once into registers
// (MAXC 16-byte chunks per thread), reduced, and written back once as
// dlogits.  NT is small (4 waves for bf16) so that several rows are in flight
// per CU and the block reductions are short.  Rows are streamed with
// non-temporal loads and stores (3.3 GB per step at 124M, far above the
// caches: 0.66 -> 0.63 ms per step against plain accesses).
//
// The three passes over the registers (max, sum of exponentials, gradient)
// are vector-ALU bound, so the per-element work is kept to the widening, one
// FMA and one exp2 (plus the max, the add or the scale and the packing):
// only the chunk that holds the vocabulary's end tests columns against V,
// the target logit is read separately by one thread, and the -1 of the
// target is applied by the one thread whose chunk holds it.
template <typename T, int NT, int MAXC>
__global__ __launch_bounds__(NT) void softmax_ce_kernel(T* logits, float* losses, const int* targets, int V, int Vp,
                                                        float dscale, int* err) {
    constexpr int VN = Vec16<T>::N;
    constexpr float L2E = 1.4426950408889634f;
    __shared__ float sh[NT / 64];
    __shared__ float s_zt;
    const int row = blockIdx.x;
    T* z = logits + (int64_t)row * Vp;
    const int chunks = Vp / VN;
    const int full = V / VN;  // chunks whose columns are all below V
    int tgt = targets[row];
    if (tgt < 0 || tgt >= V) {
        if (threadIdx.x == 0) atomicOr(err, 2);
        tgt = 0;
    }
    const int tch = tgt / VN, tj = tgt - tch * VN;
    Vec16<T> q[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
        const int ch = threadIdx.x + i * NT;
        if (ch < chunks) q[i] = ld16_stream(z + ch * VN);
    }
    // read before any thread of the block overwrites the row (the stores
    // follow the two block reductions and their barriers)
    if (threadIdx.x == 0) s_zt = to_f32(z[tgt]);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
        const int ch = threadIdx.x + i * NT;
        if (ch < full) {
#pragma unroll
            for (int j = 0; j < VN; j++) mx = fmaxf(mx, to_f32(q[i].v[j]));
        } else if (ch < chunks) {
#pragma unroll
            for (int j = 0; j < VN; j++)
                if (ch * VN + j < V) mx = fmaxf(mx, to_f32(q[i].v[j]));
        }
    }
    const float M2 = block_max<NT>(mx, sh) * L2E;  // row max, log2 units
#pragma unroll
    for (int i = 0; i < MAXC; i++) keep_packed(q[i]);
    float se = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
        const int ch = threadIdx.x + i * NT;
        if (ch < full) {
#pragma unroll
            for (int j = 0; j < VN; j++) se += __builtin_amdgcn_exp2f(fmaf(to_f32(q[i].v[j]), L2E, -M2));
        } else if (ch < chunks) {
#pragma unroll
            for (int j = 0; j < VN; j++)
                if (ch * VN + j < V) se += __builtin_amdgcn_exp2f(fmaf(to_f32(q[i].v[j]), L2E, -M2));
        }
    }
    const float S = block_sum<NT>(se, sh);  // its barrier also publishes s_zt
    if (threadIdx.x == 0) losses[row] = (M2 + __log2f(S)) * 0.6931471805599453f - s_zt;
    const float ps = dscale / S;  // softmax scale folded with the loss-mean factor
#pragma unroll
    for (int i = 0; i < MAXC; i++) keep_packed(q[i]);
#pragma unroll
    for (int i = 0; i < MAXC; i++) {
        const int ch = threadIdx.x + i * NT;
        if (ch < chunks) {
            float d[VN];
            if (ch < full) {
#pragma unroll
                for (int j = 0; j < VN; j++) d[j] = __builtin_amdgcn_exp2f(fmaf(to_f32(q[i].v[j]), L2E, -M2)) * ps;
            } else {
#pragma unroll
                for (int j = 0; j < VN; j++)
                    d[j] = ch * VN + j < V ? __builtin_amdgcn_exp2f(fmaf(to_f32(q[i].v[j]), L2E, -M2)) * ps : 0.f;
            }
            if (ch == tch) {
#pragma unroll
                for (int j = 0; j < VN; j++)
                    if (j == tj) d[j] -= dscale;
            }
            Vec16<T> o;
#pragma unroll
            for (int j = 0; j < VN; j++) o.v[j] = from_f32<T>(d[j]);
            st16_stream(z + ch * VN, o);
        }
    }
}

template <typename T, int NT>
hipError_t softmax_ce_nt(T* logits, float* losses, const int* targets, int BT, int V, int Vp, float dscale, int* err,
                         hipStream_t s) {
    constexpr int VN = Vec16<T>::N;
    const int per = (int)cdiv(Vp / VN, NT);
    if (per <= 4) softmax_ce_kernel<T, NT, 4><<<BT, NT, 0, s>>>(logits, losses, targets, V, Vp, dscale, err);
    else if (per <= 8) softmax_ce_kernel<T, NT, 8><<<BT, NT, 0, s>>>(logits, losses, targets, V, Vp, dscale, err);
    else if (per <= 16) softmax_ce_kernel<T, NT, 16><<<BT, NT, 0, s>>>(logits, losses, targets, V, Vp, dscale, err);
    else if (per <= 25) softmax_ce_kernel<T, NT, 25><<<BT, NT, 0, s>>>(logits, losses, targets, V, Vp, dscale, err);
    else if (per <= 32) softmax_ce_kernel<T, NT, 32><<<BT, NT, 0, s>>>(logits, losses, targets, V, Vp, dscale, err);
    else return hipErrorInvalidValue;
    return LAUNCH_CHECK();
}

template <typename T>
hipError_t softmax_ce(T* logits, float* losses, const int* targets, int BT, int V, int Vp, float dscale, int* err,
                      hipStream_t s) {
    if (Vp % Vec16<T>::N) return hipErrorInvalidValue;
    // 256 threads per bf16 row, 512 per fp32 row: rows up to 65536 (bf16) or 65536 (fp32) columns
    if constexpr (std::is_same<T, bf16>::value) return softmax_ce_nt<T, 256>(logits, losses, targets, BT, V, Vp, dscale, err, s);
    else return softmax_ce_nt<T, 512>(logits, losses, targets, BT, V, Vp, dscale, err, s);
}

// mean of n losses, summed in a fixed order in double by one block
// Fixed-order fp64 sum of x[0 .. n) by one block of 1024 threads: thread t
// adds x[t], x[t + 1024], ... (its loads issued 4 at a time, independent of
// one another), then a pairwise tree over the 1024 thread sums.
DEVI double block_sum_f64(const float* x, int n, double* red) {
    double s = 0.0;
    for (int i0 = threadIdx.x; i0 < n; i0 += 4 * 1024) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) v[u] = i0 + u * 1024 < n ? x[i0 + u * 1024] : 0.f;
#pragma unroll
        for (int u = 0; u < 4; u++) s += v[u];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 512; o >= 1; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    return red[0];
}

// The fused classifier's loss, one wave per row: the row's G partial (max,
// sum) pairs (log2 units; a group with no real column has max -inf and sum 0)
// combined as M = max of the maxima, S = sum of sum_q 2^(max_q - M), each lane
// taking groups lane, lane + 64, ... in order and the lanes combined by the
// fixed-order wave reductions; lse2 = M + log2 S, loss = lse2 ln 2 - z_target.
__global__ __launch_bounds__(256) void ce_combine_kernel(float* losses, float* lse2, const float2* stats,
                                                         const float* zt, int BT, int G) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= BT) return;  // uniform over the wave
    const float2* st = stats + (int64_t)row * G;
    float mx = -INFINITY;
    for (int q = lane; q < G; q += 64) mx = fmaxf(mx, st[q].x);
    const float M = wave_max(mx);
    float se = 0.f;
    for (int q = lane; q < G; q += 64) {
        const float2 p = st[q];
        if (p.x != -INFINITY) se += p.y * __builtin_amdgcn_exp2f(p.x - M);
    }
    const float S = wave_sum(se);
    if (lane == 0) {
        const float l2 = M + __log2f(S);
        lse2[row] = l2;
        losses[row] = l2 * 0.6931471805599453f - zt[row];
    }
}

hipError_t ce_combine(float* losses, float* lse2, const float2* stats, const float* zt, int BT, int G,
                      hipStream_t s) {
    if (BT <= 0 || G <= 0) return hipErrorInvalidValue;
    ce_combine_kernel<<<cdiv(BT, 4), 256, 0, s>>>(losses, lse2, stats, zt, BT, G);
    return LAUNCH_CHECK();
}

__global__ __launch_bounds__(1024) void loss_mean_kernel(float* out, const float* losses, int n) {
    __shared__ double red[1024];
    const double s = block_sum_f64(losses, n, red);
    if (threadIdx.x == 0) out[0] = (float)(s / n);
}

hipError_t loss_mean(float* out, const float* losses, int n, hipStream_t s) {
    loss_mean_kernel<<<1, 1024, 0, s>>>(out, losses, n);
    return LAUNCH_CHECK();
}

// ============================================================================
// global gradient norm (pyshine tour: global-norm header) and clip factor
// ============================================================================
constexpr int NORM_G = 1024;

// Each pass of a block reads NORM_U x 256 float4 groups (group u at
// (block * NORM_U + u) * 256 + thread), all requested before any is used,
// with non-temporal loads: 0.5 GB of gradients at 124M, 122 -> 73 us from
// cold caches against plain loads one group at a time (6.8 TB/s).
constexpr int NORM_U = 4;
__global__ __launch_bounds__(256) void sumsq_kernel(float* partial, const float* g, size_t n) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    __shared__ float red[4];
    float s = 0.f;
    const size_t n4 = n / 4;
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    const size_t stride = (size_t)gridDim.x * NORM_U * 256;
    for (size_t base = (size_t)blockIdx.x * NORM_U * 256 + threadIdx.x; base < n4; base += stride) {
        f32x4 q[NORM_U];
#pragma unroll
        for (int u = 0; u < NORM_U; u++) {
            const size_t i = base + (size_t)u * 256;
            q[u] = i < n4 ? __builtin_nontemporal_load(g4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < NORM_U; u++) s += q[u].x * q[u].x + q[u].y * q[u].y + q[u].z * q[u].z + q[u].w * q[u].w;
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        float q = g[n4 * 4 + threadIdx.x];
        s += q * q;
    }
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(1024) void norm_final_kernel(float* norm_scale, const float* partial, int G,
                                                          float max_norm) {
    __shared__ double red[1024];
    const double s = block_sum_f64(partial, G, red);
    if (threadIdx.x == 0) {
        const float n = (float)sqrt(s);
        norm_scale[0] = n;
        // a non-finite norm (a NaN or inf gradient, or a sum of squares past
        // the float range) leaves a NaN factor: the AdamW kernels refuse to
        // update on it
        norm_scale[1] = !isfinite(n) ? __builtin_nanf("") : (max_norm > 0.f && n > max_norm) ? max_norm / n : 1.f;
    }
}

hipError_t grad_norm(float* partial, float* norm_scale, const float* g, size_t n, float max_norm, hipStream_t s) {
    sumsq_kernel<<<NORM_G, 256, 0, s>>>(partial, g, n);
    norm_final_kernel<<<1, 1024, 0, s>>>(norm_scale, partial, NORM_G, max_norm);
    return LAUNCH_CHECK();
}

// ============================================================================
// AdamW (decoupled weight decay, bias-corrected; c1 = 1-b1^t, c2 = 1-b2^t),
// gradient times the clip factor norm_scale[1]; refreshes the bf16 shadow.
// ============================================================================
// ic1 = 1 / (1 - b1^t), ic2 = 1 / (1 - b2^t)
DEVI void adamw_one(float& p, float g, float& m, float& v, float lr, float b1, float b2, float eps, float wd,
                    float ic1, float ic2) {
    m = fmaf(b1, m, (1.f - b1) * g);
    v = fmaf(b2, v, (1.f - b2) * g * g);
    const float mh = m * ic1, vh = v * ic2;
    p = p - lr * (mh * __builtin_amdgcn_rcpf(sqrtf(vh) + eps) + wd * p);
}

// Each block updates ADAM_U x 256 float4 groups; group u of a block sits at
// (block * ADAM_U + u) * 256 + thread, so every load and store instruction
// covers 4 KB contiguously.  All loads of a thread are issued first.  The
// arrays are streamed with non-temporal accesses (3.7 GB per step at 124M:
// 0.674 -> 0.618 ms against plain loads and stores).  Two groups per thread
// measured ~1.5% faster than four, eight slower.
constexpr int ADAM_U = 2;
__global__ __launch_bounds__(256) void adamw_kernel(float* p, const float* g, float* m, float* v, bf16* shadow,
                                                    size_t n, float lr, float b1, float b2, float eps, float wd,
                                                    float ic1, float ic2, const float* norm_scale, int* refused) {
    const float sc = norm_scale ? norm_scale[1] : 1.f;
    if (!isfinite(sc)) {  // the same for every workgroup: nothing is written
        if (blockIdx.x == 0 && threadIdx.x == 0) refused[0] = 1;
        return;
    }
    const size_t n4 = n / 4;
    float4 pp[ADAM_U], gg[ADAM_U], mm[ADAM_U], vv[ADAM_U];
#pragma unroll
    for (int u = 0; u < ADAM_U; u++) {
        const size_t i = ((size_t)blockIdx.x * ADAM_U + u) * 256 + threadIdx.x;
        if (i < n4) {
            pp[u] = ld_stream(p, i);
            gg[u] = ld_stream(g, i);
            mm[u] = ld_stream(m, i);
            vv[u] = ld_stream(v, i);
        }
    }
#pragma unroll
    for (int u = 0; u < ADAM_U; u++) {
        const size_t i = ((size_t)blockIdx.x * ADAM_U + u) * 256 + threadIdx.x;
        if (i < n4) {
            adamw_one(pp[u].x, gg[u].x * sc, mm[u].x, vv[u].x, lr, b1, b2, eps, wd, ic1, ic2);
            adamw_one(pp[u].y, gg[u].y * sc, mm[u].y, vv[u].y, lr, b1, b2, eps, wd, ic1, ic2);
            adamw_one(pp[u].z, gg[u].z * sc, mm[u].z, vv[u].z, lr, b1, b2, eps, wd, ic1, ic2);
            adamw_one(pp[u].w, gg[u].w * sc, mm[u].w, vv[u].w, lr, b1, b2, eps, wd, ic1, ic2);
            st_stream(p, i, pp[u]);
            st_stream(m, i, mm[u]);
            st_stream(v, i, vv[u]);
            if (shadow) st_stream(shadow, i, bf16x4_nt{(bf16)pp[u].x, (bf16)pp[u].y, (bf16)pp[u].z, (bf16)pp[u].w});
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const size_t i = n4 * 4 + threadIdx.x;
        float a = p[i], b = m[i], c = v[i];
        adamw_one(a, g[i] * sc, b, c, lr, b1, b2, eps, wd, ic1, ic2);
        p[i] = a;
        m[i] = b;
        v[i] = c;
        if (shadow) shadow[i] = (bf16)a;
    }
}

hipError_t adamw(float* p, const float* g, float* m, float* v, bf16* shadow, size_t n, float lr, float b1, float b2,
                 float eps, float wd, float c1, float c2, const float* norm_scale, int* refused, hipStream_t s) {
    if (norm_scale && !refused) return hipErrorInvalidValue;
    const size_t blocks = cdiv(n / 4, 256 * ADAM_U) + 1;
    adamw_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, g, m, v, shadow, n, lr, b1, b2, eps, wd, 1.f / c1, 1.f / c2,
                                                  norm_scale, refused);
    return LAUNCH_CHECK();
}

// ---- AdamW over bf16 parameters with stochastic rounding -------------------
// ("llm.c's Origin and the Future of LLM Compilers", section "Avengers":
// stochastic rounding).  The bf16 values are the parameters: theta =
// float(w[i]), the update runs in fp32 exactly as adamw_one, and the result x
// is rounded to bf16 by adding a uniform 16-bit integer u to its bit pattern
// and keeping the top half: the magnitude moves up to the next bf16 value
// iff u + (low 16 bits of x) carries, i.e. with probability equal to the
// discarded fraction, so the rounding is unbiased.  u is the top 16 bits of
// SplitMix64's output function (Steele, Lea & Flood 2014) at state
// key + (i+1) * gamma: a counter-based draw per (step, flat index).
// Non-finite results are kept as they are (NaN stays NaN).

DEVI uint32_t sr_draw16(uint64_t key, uint64_t i) {
    uint64_t z = key + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (uint32_t)(z >> 48);
}

DEVI bf16 sr_round_bf16(float x, uint32_t u) {
    uint32_t b = __float_as_uint(x);
    if ((b & 0x7F800000u) != 0x7F800000u) b += u;  // finite: carry into the kept half with P = fraction
    else if (b & 0x007FFFFFu) b |= 0x00400000u;     // NaN: keep it a (quiet) NaN after truncation
    return __builtin_bit_cast(bf16, (uint16_t)(b >> 16));
}

// Each thread updates ADAM_U groups of 4 parameters, laid out as in
// adamw_kernel; every range boundary is a multiple of 4, so a group is
// wholly inside or outside each mirrored range.
__global__ __launch_bounds__(256) void adamw_sr_kernel(bf16* w, float* p32, const float* g, float* m, float* v,
                                                       size_t n, float lr, float b1, float b2, float eps, float wd,
                                                       float ic1, float ic2, const float* norm_scale, uint64_t key,
                                                       SrRanges mr, int* refused) {
    typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const float sc = norm_scale ? norm_scale[1] : 1.f;
    if (!isfinite(sc)) {  // the same for every workgroup: nothing is written
        if (blockIdx.x == 0 && threadIdx.x == 0) refused[0] = 1;
        return;
    }
    const size_t n4 = n / 4;
    bf16x4 ww[ADAM_U];
    float4 gg[ADAM_U], mm[ADAM_U], vv[ADAM_U];
#pragma unroll
    for (int u = 0; u < ADAM_U; u++) {
        const size_t i = ((size_t)blockIdx.x * ADAM_U + u) * 256 + threadIdx.x;
        if (i < n4) {
            ww[u] = ld_stream(w, i);
            gg[u] = ld_stream(g, i);
            mm[u] = ld_stream(m, i);
            vv[u] = ld_stream(v, i);
        }
    }
#pragma unroll
    for (int u = 0; u < ADAM_U; u++) {
        const size_t i = ((size_t)blockIdx.x * ADAM_U + u) * 256 + threadIdx.x;
        if (i < n4) {
            float x[4] = {(float)ww[u][0], (float)ww[u][1], (float)ww[u][2], (float)ww[u][3]};
            adamw_one(x[0], gg[u].x * sc, mm[u].x, vv[u].x, lr, b1, b2, eps, wd, ic1, ic2);
            adamw_one(x[1], gg[u].y * sc, mm[u].y, vv[u].y, lr, b1, b2, eps, wd, ic1, ic2);
            adamw_one(x[2], gg[u].z * sc, mm[u].z, vv[u].z, lr, b1, b2, eps, wd, ic1, ic2);
            adamw_one(x[3], gg[u].w * sc, mm[u].w, vv[u].w, lr, b1, b2, eps, wd, ic1, ic2);
            bf16x4 o;
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = sr_round_bf16(x[e], sr_draw16(key, 4 * i + e));
            st_stream(w, i, o);
            st_stream(m, i, mm[u]);
            st_stream(v, i, vv[u]);
            for (int r = 0; r < mr.n; r++)
                if (4 * i >= mr.lo[r] && 4 * i < mr.hi[r])
                    *reinterpret_cast<float4*>(p32 + mr.dst[r] + (4 * i - mr.lo[r])) =
                        make_float4((float)o[0], (float)o[1], (float)o[2], (float)o[3]);
        }
    }
}

hipError_t adamw_sr(bf16* w, float* p32, const float* g, float* m, float* v, size_t n, float lr, float b1, float b2,
                    float eps, float wd, float c1, float c2, const float* norm_scale, uint64_t key,
                    const SrRanges& mirror, int* refused, hipStream_t s) {
    if (n % 4 || mirror.n < 0 || mirror.n > SR_RANGES_MAX) return hipErrorInvalidValue;
    if (norm_scale && !refused) return hipErrorInvalidValue;
    for (int r = 0; r < mirror.n; r++)
        if (mirror.lo[r] % 4 || mirror.hi[r] % 4 || mirror.dst[r] % 4 || mirror.lo[r] > mirror.hi[r] ||
            mirror.hi[r] > n)
            return hipErrorInvalidValue;
    const size_t blocks = cdiv(n / 4, 256 * ADAM_U);
    adamw_sr_kernel<<<(unsigned)blocks, 256, 0, s>>>(w, p32, g, m, v, n, lr, b1, b2, eps, wd, 1.f / c1, 1.f / c2,
                                                     norm_scale, key, mirror, refused);
    return LAUNCH_CHECK();
}

__global__ void cast_bf16_kernel(bf16* dst, const float* src, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = (bf16)src[i];
}
// GELU of the kept bf16 pre-activation, 8 values per thread and step; the
// pre-activation is read once (non-temporal), the output is read next by
// the weight-gradient product
__global__ __launch_bounds__(256) void gelu_recompute_kernel(bf16* out, const bf16* u, size_t n8) {
    typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (size_t)gridDim.x * blockDim.x) {
        const bf16x8_t x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(u) + i);
        bf16x8_t y;
#pragma unroll
        for (int e = 0; e < 8; e++) y[e] = (bf16)gelu_f((float)x[e]);
        reinterpret_cast<bf16x8_t*>(out)[i] = y;
    }
}
hipError_t gelu_recompute(bf16* out, const bf16* u, size_t n, hipStream_t s) {
    if (n % 8 || (reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(u)) % 16) return hipErrorInvalidValue;
    const size_t n8 = n / 8;
    size_t blocks = cdiv(n8, 256);
    if (blocks > 8192) blocks = 8192;
    gelu_recompute_kernel<<<(unsigned)blocks, 256, 0, s>>>(out, u, n8);
    return LAUNCH_CHECK();
}

hipError_t cast_bf16(bf16* dst, const float* src, size_t n, hipStream_t s) {
    size_t blocks = cdiv(n, 256);
    if (blocks > 8192) blocks = 8192;
    cast_bf16_kernel<<<(unsigned)blocks, 256, 0, s>>>(dst, src, n);
    return LAUNCH_CHECK();
}

template <typename T> __global__ void widen_kernel(float* dst, const T* src, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        dst[i] = to_f32(src[i]);
}
template <typename T> hipError_t widen_f32(float* dst, const T* src, size_t n, hipStream_t s) {
    size_t blocks = cdiv(n, 256);
    if (blocks > 8192) blocks = 8192;
    widen_kernel<T><<<(unsigned)blocks, 256, 0, s>>>(dst, src, n);
    return LAUNCH_CHECK();
}

// ---- explicit instantiations ------------------------------------------------
#define INST(T)                                                                                              \
    template hipError_t encoder_fwd<T, float>(T*, int*, int*, const int*, const int*, const float*, const float*,  \
                                              int, int, int, int, int*, hipStream_t);                            \
    template hipError_t encoder_bwd<T>(float*, float*, const T*, const int*, int, int, int, int, int, void*,  \
                                        bool, hipStream_t);                                                  \
    template hipError_t layernorm_fwd<T>(T*, float*, float*, const T*, const float*, const float*, int, int, \
                                         hipStream_t);                                                       \
    template hipError_t layernorm_bwd<T>(T*, const T*, const T*, const T*, const float*, const float*,      \
                                         const float*, float*, int, int, bool, hipStream_t);                 \
    template hipError_t colsum_accum<T>(float*, const T*, int, int, float*, hipStream_t);                    \
    template hipError_t softmax_ce<T>(T*, float*, const int*, int, int, int, float, int*, hipStream_t);      \
    template hipError_t widen_f32<T>(float*, const T*, size_t, hipStream_t);
INST(float)
INST(bf16)
template hipError_t encoder_fwd<bf16, bf16>(bf16*, int*, int*, const int*, const int*, const bf16*, const bf16*, int,
                                            int, int, int, int*, hipStream_t);
