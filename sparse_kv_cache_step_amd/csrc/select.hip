// Selection half of the decode step (review page, section 三, Algorithm 2
// steps 1-2, and the Telegram write-up's set-difference cache):
//   score   P = q . L^T / sqrt(d) for every chunk, with per-tile softmax
//           partials over the selectable chunks;
//   select  one workgroup per (sequence, KV head): the group score
//           S2 = per-head softmax over selectable chunks averaged over the
//           query heads of the KV group, ArgTopK(S2, k) by radix selection,
//           and the set difference against the previous step's resident
//           chunks (miss list, hit counts).
// The same radix selection picks the prefill's outlier chunks.
#include "skv_device.h"

namespace skv {

// ---------------------------------------------------------------------------
// Landmark scoring, bfloat16, on MFMA.  For one (sequence, KV head) the
// contraction P[g, j] = sum_i q[g, i] L[j, i] has M = the G query heads of the
// group (padded to 16), N = chunks, K = d.  One v_mfma_f32_16x16x32_bf16 takes
// 16 chunks x 32 dims: lane l feeds head (l & 15) of q and chunk (l & 15) of
// L with dims 32*ks + 8*(l >> 4) .. +8, so the four lane groups of one load
// instruction read 64 contiguous bytes of each landmark row.  Each wave
// scores a tile of 64 chunks (4 rounds of 16, all loads issued up front).
//
// Softmax bookkeeping per tile and head: M = max of the tile's selectable
// scores, u[j] = exp(P[j] - M) (0 for non-selectable chunks) written as
// U (b, h_kv, n, G), and S = sum of u.  The group score then needs no
// further exponentials: with m = max over tiles and Z = sum_t S_t exp(M_t-m),
// S2[j] = sum_g u_g[j] exp(M_t,g - m_g) / (Z_g G).
// For G <= 4 the MFMA result (heads in lanes 0-15) is first transposed so
// every lane holds one (head, chunk) value.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sel_max16(float v) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float sel_sum16(float v) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int D, bool SMALLG>
__global__ __launch_bounds__(256) void score_mfma_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ L,
                                                         const uint32_t *__restrict__ cand, int mask_words,
                                                         float *__restrict__ U, float2 *__restrict__ stats,
                                                         int hkv, int G, int n, int wtiles, float scale) {
    constexpr int KS = D / 32;
    constexpr int ROUNDS = 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, quad = lane >> 4;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    const int wt = blockIdx.x * 4 + wave;  // 64-chunk tile of this wave
    if (wt >= wtiles) return;              // no barrier in this kernel

    bf16x8 qa[KS];
    {
        const uint16_t *qrow = q + (static_cast<size_t>(b) * hq + h * G + row) * D + quad * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = row < G ? *reinterpret_cast<const u32x4 *>(qrow + ks * 32) : u32x4{0u, 0u, 0u, 0u};
            qa[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    const int wbase = wt * 64;
    const uint16_t *Lbh = L + static_cast<size_t>(bh) * n * D;
    u32x4 lb[ROUNDS][KS];
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        const int j = wbase + rd * 16 + row;
        const uint16_t *lrow = Lbh + static_cast<size_t>(j < n ? j : 0) * D + quad * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            lb[rd][ks] = j < n ? *reinterpret_cast<const u32x4 *>(lrow + ks * 32) : u32x4{0u, 0u, 0u, 0u};
    }
    const uint32_t *cm = cand + static_cast<size_t>(bh) * mask_words;
    float *Ub = U + static_cast<size_t>(bh) * n * G;
    float2 *st = stats + static_cast<size_t>(bh) * G * wtiles;

    if constexpr (SMALLG) {
        // lane (quad, row) <- head quad of chunk row of each round
        float p[ROUNDS];
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8, lb[rd][ks]), acc, 0, 0, 0);
            const float t0 = __shfl(acc[0], row, 64), t1 = __shfl(acc[1], row, 64);
            const float t2 = __shfl(acc[2], row, 64), t3 = __shfl(acc[3], row, 64);
            const float mine = quad == 0 ? t0 : (quad == 1 ? t1 : (quad == 2 ? t2 : t3));
            const int j = wbase + rd * 16 + row;
            const bool valid = quad < G && j < n && mask_bit(cm, j);
            p[rd] = valid ? mine * scale : -INFINITY;
        }
        float M = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
        M = sel_max16(M);
        float S = 0.f;
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            const float u = p[rd] == -INFINITY ? 0.f : expf(p[rd] - M);
            S += u;
            const int j = wbase + rd * 16 + row;
            if (quad < G && j < n) Ub[static_cast<size_t>(j) * G + quad] = u;
        }
        S = sel_sum16(S);
        if (row == 0 && quad < G) st[static_cast<size_t>(quad) * wtiles + wt] = make_float2(M, S);
    } else {
        // lane holds heads 4*quad + e of chunk row; G > 4 keeps that layout
        float p[ROUNDS][4];
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8, lb[rd][ks]), acc, 0, 0, 0);
            const int j = wbase + rd * 16 + row;
            const bool jv = j < n && mask_bit(cm, j);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[rd][e] = (jv && quad * 4 + e < G) ? acc[e] * scale : -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float M = fmaxf(fmaxf(p[0][e], p[1][e]), fmaxf(p[2][e], p[3][e]));
            M = sel_max16(M);
            float S = 0.f;
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd) {
                const float u = p[rd][e] == -INFINITY ? 0.f : expf(p[rd][e] - M);
                p[rd][e] = u;
                S += u;
            }
            S = sel_sum16(S);
            if (row == 0 && quad * 4 + e < G) st[static_cast<size_t>(quad * 4 + e) * wtiles + wt] = make_float2(M, S);
        }
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            const int j = wbase + rd * 16 + row;
            if (j < n && quad * 4 < G) {
                float *dst = Ub + static_cast<size_t>(j) * G + quad * 4;
                if (G % 4 == 0) {
                    *reinterpret_cast<float4 *>(dst) = make_float4(p[rd][0], p[rd][1], p[rd][2], p[rd][3]);
                } else {
                    for (int e = 0; e < 4 && quad * 4 + e < G; ++e) dst[e] = p[rd][e];
                }
            }
        }
    }
}

// Generic scoring (any storage type): thread per chunk, all G heads; same
// outputs as the MFMA kernel (U and per-64-chunk tile statistics).
template <typename T, int D>
__global__ __launch_bounds__(256) void score_generic_kernel(const T *__restrict__ q, const T *__restrict__ L,
                                                            const uint32_t *__restrict__ cand, int mask_words,
                                                            float *__restrict__ U, float2 *__restrict__ stats,
                                                            int hkv, int G, int n, int wtiles, float scale) {
    __shared__ float qs[kMaxGroup][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    for (int i = threadIdx.x; i < G * D; i += 256)
        qs[i / D][i % D] = Elem<T>::ld(q, (static_cast<size_t>(b) * hq + h * G) * D + i);
    __syncthreads();
    const int wt = blockIdx.x * 4 + wave;
    if (wt >= wtiles) return;
    const int j = wt * 64 + lane;
    const bool valid = j < n && mask_bit(cand + static_cast<size_t>(bh) * mask_words, j);
    const T *lrow = L + (static_cast<size_t>(bh) * n + (j < n ? j : 0)) * D;
    for (int g = 0; g < G; ++g) {
        float p = -INFINITY;
        if (valid) {
            float acc = 0.f;
            for (int i = 0; i < D; ++i) acc += qs[g][i] * Elem<T>::ld(lrow, i);
            p = acc * scale;
        }
        const float M = wave_max(p);
        const float u = p == -INFINITY ? 0.f : expf(p - M);
        if (j < n) U[(static_cast<size_t>(bh) * n + j) * G + g] = u;
        const float S = wave_sum(u);
        if (lane == 0) stats[(static_cast<size_t>(bh) * G + g) * wtiles + wt] = make_float2(M, S);
    }
}

// ---------------------------------------------------------------------------
// Block-wide helpers (blockDim.x threads, a multiple of 64, at most 2048).
// ---------------------------------------------------------------------------
struct SelectScratch {
    uint32_t hist[4096];
    int wtmp[2][32];
    uint32_t digit;
    int above;
};

// Inclusive prefix sums of two per-thread counts over the threads of the
// block in one pass (one pair of barriers); totals in *ta, *tb.
__device__ __forceinline__ void block_scan2(int &a, int &b, SelectScratch &sc, int *ta, int *tb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int x = __shfl_up(a, off, 64), y = __shfl_up(b, off, 64);
        if (lane >= off) { a += x; b += y; }
    }
    if (lane == 63) { sc.wtmp[0][wave] = a; sc.wtmp[1][wave] = b; }
    __syncthreads();
    int pa = 0, pb = 0, sa = 0, sb = 0;
    for (int w = 0; w < nw; ++w) {
        const int x = sc.wtmp[0][w], y = sc.wtmp[1][w];
        if (w < wave) { pa += x; pb += y; }
        sa += x;
        sb += y;
    }
    __syncthreads();
    a += pa;
    b += pb;
    *ta = sa;
    *tb = sb;
}

// The k largest of keys[0, n), exact ties to the lower index, written to
// out[0, k) (and to lds_out if given) in ascending index order.  Radix
// selection on 12 + 12 + 8 bits finds the k-th largest key T and how many
// keys equal to T are taken: all threads build a histogram of the current
// digit, one wave scans it from the top to find the digit holding the k-th
// key (and clears it).  An ordered compaction over contiguous per-thread
// segments then writes the indices.  Requires 1 <= k <= n.  Every thread of
// the block must call it; sc.hist must be zero on entry.
__device__ void radix_topk(const uint32_t *keys, int n, int k, int32_t *out, int32_t *lds_out, SelectScratch &sc) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    uint32_t prefix = 0, pmask = 0;
    int krem = k;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
        const int nbins = pass == 2 ? 256 : 4096;
        const uint32_t dmask = static_cast<uint32_t>(nbins - 1);
        for (int j = tid; j < n; j += nt) {
            const uint32_t key = keys[j];
            if ((key & pmask) == prefix) atomicAdd(&sc.hist[(key >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            const int per = nbins / 64;  // lane l owns bins top-l*per .. downwards
            const int top = nbins - 1 - lane * per;
            int local = 0;
            for (int i = 0; i < per; ++i) local += static_cast<int>(sc.hist[top - i]);
            int incl = local;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(incl, off, 64);
                if (lane >= off) incl += t;
            }
            const int excl = incl - local;
            if (excl < krem && krem <= incl) {
                int acc = excl;
                for (int i = 0; i < per; ++i) {
                    const int cnt = static_cast<int>(sc.hist[top - i]);
                    if (acc + cnt >= krem) { sc.digit = static_cast<uint32_t>(top - i); sc.above = acc; break; }
                    acc += cnt;
                }
            }
            for (int i = 0; i < per; ++i) sc.hist[top - i] = 0;  // ready for the next pass
        }
        __syncthreads();
        prefix |= sc.digit << shift;
        pmask |= dmask << shift;
        krem -= sc.above;
    }
    const uint32_t thr = prefix;
    const int need_eq = krem;
    const int seg = (n + nt - 1) / nt;
    const int j0 = min(n, tid * seg), j1 = min(n, j0 + seg);
    int gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t key = keys[j];
        gt += key > thr;
        eq += key == thr;
    }
    int gt_incl = gt, eq_incl = eq, tg, te;
    block_scan2(gt_incl, eq_incl, sc, &tg, &te);
    const int gt_before = gt_incl - gt, eq_before = eq_incl - eq;
    // equal keys are taken in index order until need_eq of them are taken
    const int take_eq = min(max(need_eq - eq_before, 0), eq);
    int pos = gt_before + min(eq_before, need_eq);
    int eq_seen = 0;
    for (int j = j0; j < j1 && pos < k; ++j) {
        const uint32_t key = keys[j];
        bool t = key > thr;
        if (key == thr) t = eq_seen++ < take_eq;
        if (t) {
            out[pos] = j;
            if (lds_out) lds_out[pos] = j;
            ++pos;
        }
    }
}

// Outlier selection for the prefill: the o chunks with the lowest minimum
// cosine among chunks [0, n_valid); keys from -min_cos.
__global__ __launch_bounds__(kSelectThreads) void topo_kernel(const float *__restrict__ min_cos, int n, int n_valid,
                                                              int o, int32_t *__restrict__ out,
                                                              uint32_t *__restrict__ gscratch, int use_lds) {
    extern __shared__ uint32_t dyn[];
    __shared__ SelectScratch sc;
    const int row = blockIdx.x;
    uint32_t *keys = use_lds ? dyn : gscratch + static_cast<size_t>(row) * n;
    for (int j = threadIdx.x; j < n; j += blockDim.x)
        keys[j] = j < n_valid ? float_key(-min_cos[static_cast<size_t>(row) * n + j]) : 0u;
    for (int i = threadIdx.x; i < 4096; i += blockDim.x) sc.hist[i] = 0;
    __syncthreads();
    if (o > 0) radix_topk(keys, n, o, out + static_cast<size_t>(row) * o, nullptr, sc);
}

// ---------------------------------------------------------------------------
// Group score of one (sequence, KV head) row: S2[j] = sum_g U[j, g] w[t, g]
// with t the 64-chunk tile of j and w[t, g] = exp(M_t,g - m_g) / (Z_g G);
// selectable chunks only (0 elsewhere).  Written to S2 and kept as
// order-preserving keys (selectable keys > 0).  Each thread takes 64/GP
// chunks per batch and issues all their loads before any arithmetic.
// ---------------------------------------------------------------------------
template <int GP>
__device__ __forceinline__ void group_scores(const float *Ub, const uint32_t *cm, const float *w, int G, int n,
                                             float *S2b, uint32_t *keys) {
    constexpr int UNR = 64 / GP;
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int j0 = 0; j0 < n; j0 += nt * UNR) {
        float v[UNR][GP];
        uint32_t word[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + tid + nt * u;
            const int jj = j < n ? j : 0;
            word[u] = cm[jj >> 5];
            if (G == GP) {
#pragma unroll
                for (int q4 = 0; q4 < GP / 4; ++q4) {
                    const float4 f = *reinterpret_cast<const float4 *>(Ub + static_cast<size_t>(jj) * GP + 4 * q4);
                    v[u][4 * q4] = f.x; v[u][4 * q4 + 1] = f.y; v[u][4 * q4 + 2] = f.z; v[u][4 * q4 + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int g = 0; g < GP; ++g) v[u][g] = g < G ? Ub[static_cast<size_t>(jj) * G + g] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + tid + nt * u;
            if (j >= n) continue;
            const bool valid = (word[u] >> (j & 31)) & 1u;
            const float *wt = w + (j >> 6) * G;
            float acc = 0.f;
#pragma unroll
            for (int g = 0; g < GP; ++g)
                if (g < G) acc += v[u][g] * wt[g];
            S2b[j] = valid ? acc : 0.f;
            keys[j] = valid ? float_key(acc) : 0u;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode selection, one workgroup per (sequence, KV head):
//  1. (m_g, Z_g) of every query head of the group from the score tiles;
//  2. S2[j] = (1/G) sum_g exp(P[j, g] - m_g) / Z_g over selectable j (0
//     elsewhere), kept as order-preserving keys (selectable keys > 0);
//  3. I = ArgTopK(S2, k), ascending;
//  4. set difference against the resident chunks: a slot keeps its chunk when
//     the chunk is selected again (hit); the m-th missing chunk (ascending)
//     goes to the m-th freed slot (ascending); emit the miss list and count
//     hits and misses.
// ---------------------------------------------------------------------------
template <int GP>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const float *__restrict__ P, const float2 *__restrict__ stats, const uint32_t *__restrict__ cand, int mask_words,
    float *__restrict__ S2, int32_t *__restrict__ sel, int32_t *__restrict__ slot_chunk, int2 *__restrict__ misses,
    int32_t *__restrict__ miss_count, unsigned long long *__restrict__ counters, uint32_t *__restrict__ gscratch,
    int use_lds, int G, int n, int k, int tiles) {
    extern __shared__ uint32_t dyn[];
    __shared__ SelectScratch sc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nt = blockDim.x, nw = nt >> 6;
    const int bh = blockIdx.x;
    int32_t *s_sel = reinterpret_cast<int32_t *>(dyn);  // k selected chunks, ascending
    int32_t *s_keep = s_sel + k;                        // k: chunk kept by each slot, -1 if freed
    int32_t *s_hit = s_keep + k;                        // k: 1 if selected chunk i is resident
    int32_t *s_rank = s_hit + k;                        // k: index in s_sel of the m-th miss
    float *s_w = reinterpret_cast<float *>(s_rank + k);  // tiles * G tile weights
    uint32_t *keys = use_lds ? reinterpret_cast<uint32_t *>(s_w + tiles * G) : gscratch + static_cast<size_t>(bh) * n;

    // per head: m = max_t M_t, Z = sum_t S_t exp(M_t - m); w[t] = exp(M_t - m) / (Z G)
    for (int i = tid; i < 4096; i += nt) sc.hist[i] = 0;
    for (int i = tid; i < k; i += nt) s_hit[i] = 0;
    for (int g = wave; g < G; g += nw) {
        const float2 *st = stats + (static_cast<size_t>(bh) * G + g) * tiles;
        constexpr int TPL = 8;  // tiles held per lane (more are streamed)
        float2 v[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = lane + 64 * i;
            v[i] = t < tiles ? st[t] : make_float2(-INFINITY, 0.f);
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < TPL; ++i) m = fmaxf(m, v[i].x);
        for (int t = lane + 64 * TPL; t < tiles; t += 64) m = fmaxf(m, st[t].x);
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < TPL; ++i) z += v[i].x == -INFINITY ? 0.f : v[i].y * expf(v[i].x - m);
        for (int t = lane + 64 * TPL; t < tiles; t += 64) z += st[t].x == -INFINITY ? 0.f : st[t].y * expf(st[t].x - m);
        z = wave_sum(z);
        const float inv = z > 0.f ? 1.f / (z * static_cast<float>(G)) : 0.f;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = lane + 64 * i;
            if (t < tiles) s_w[t * G + g] = v[i].x == -INFINITY ? 0.f : expf(v[i].x - m) * inv;
        }
        for (int t = lane + 64 * TPL; t < tiles; t += 64) s_w[t * G + g] = st[t].x == -INFINITY ? 0.f : expf(st[t].x - m) * inv;
    }
    __syncthreads();
    group_scores<GP>(P + static_cast<size_t>(bh) * n * G, cand + static_cast<size_t>(bh) * mask_words, s_w, G, n,
                     S2 + static_cast<size_t>(bh) * n, keys);
    __syncthreads();
    if (k <= 0) return;
    radix_topk(keys, n, k, sel + static_cast<size_t>(bh) * k, s_sel, sc);
    __syncthreads();

    // set difference: a slot keeps its chunk if the chunk is selected again
    int32_t *gc = slot_chunk + static_cast<size_t>(bh) * k;
    for (int sl = tid; sl < k; sl += nt) {
        const int32_t c = gc[sl];
        int keep = -1;
        if (c >= 0) {
            int lo = 0, hi = k;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_sel[mid] < c) lo = mid + 1; else hi = mid;
            }
            if (lo < k && s_sel[lo] == c) { keep = c; s_hit[lo] = 1; }
        }
        s_keep[sl] = keep;
    }
    __syncthreads();
    // ascending ranks of the misses (over selection positions) and of the
    // freed slots (over slot indices), one scan for both
    int nmiss = 0, nfree = 0;
    for (int i0 = 0; i0 < k; i0 += nt) {
        const int i = i0 + tid;
        const int miss = (i < k && !s_hit[i]) ? 1 : 0;
        const int fr = (i < k && s_keep[i] < 0) ? 1 : 0;
        int mi = miss, fi = fr, tm, tf;
        block_scan2(mi, fi, sc, &tm, &tf);
        if (miss) s_rank[nmiss + mi - 1] = i;
        if (fr) s_keep[i] = -2 - (nfree + fi - 1);  // freed slot: -2 - its rank
        nmiss += tm;
        nfree += tf;
    }
    __syncthreads();
    // the m-th missing chunk goes to the m-th freed slot
    int2 *ml = misses + static_cast<size_t>(bh) * k;
    for (int sl = tid; sl < k; sl += nt) {
        const int kv = s_keep[sl];
        if (kv <= -2) {
            const int r = -2 - kv;
            if (r < nmiss) {  // freed slots and misses are equal in number
                const int32_t chunk = s_sel[s_rank[r]];
                gc[sl] = chunk;
                ml[r] = make_int2(chunk, sl);
            }
        }
    }
    if (tid == 0) {
        miss_count[bh] = nmiss;
        atomicAdd(&counters[0], static_cast<unsigned long long>(k - nmiss));
        atomicAdd(&counters[1], static_cast<unsigned long long>(nmiss));
        if (bh == 0) atomicAdd(&counters[2], 1ull);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static hipError_t allow_lds(const void *fn, size_t bytes) {
    if (bytes <= 48 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

hipError_t launch_score(const Dims &dm, const void *q, const void *landmarks, const uint32_t *cand, float *P,
                        float2 *stats, hipStream_t st) {
    dim3 grid(dm.score_tiles, dm.b * dm.hkv);
    if (dm.bf16) {
        const uint16_t *qq = static_cast<const uint16_t *>(q), *LL = static_cast<const uint16_t *>(landmarks);
        if (dm.d == 128 && dm.G <= 4)
            hipLaunchKernelGGL((score_mfma_kernel<128, true>), grid, dim3(256), 0, st, qq, LL, cand, dm.mask_words, P,
                               stats, dm.hkv, dm.G, dm.n, dm.wtiles, dm.scale);
        else if (dm.d == 128)
            hipLaunchKernelGGL((score_mfma_kernel<128, false>), grid, dim3(256), 0, st, qq, LL, cand, dm.mask_words, P,
                               stats, dm.hkv, dm.G, dm.n, dm.wtiles, dm.scale);
        else if (dm.G <= 4)
            hipLaunchKernelGGL((score_mfma_kernel<64, true>), grid, dim3(256), 0, st, qq, LL, cand, dm.mask_words, P,
                               stats, dm.hkv, dm.G, dm.n, dm.wtiles, dm.scale);
        else
            hipLaunchKernelGGL((score_mfma_kernel<64, false>), grid, dim3(256), 0, st, qq, LL, cand, dm.mask_words, P,
                               stats, dm.hkv, dm.G, dm.n, dm.wtiles, dm.scale);
    } else {
        if (dm.d == 128)
            hipLaunchKernelGGL((score_generic_kernel<float, 128>), grid, dim3(256), 0, st,
                               static_cast<const float *>(q), static_cast<const float *>(landmarks), cand,
                               dm.mask_words, P, stats, dm.hkv, dm.G, dm.n, dm.wtiles, dm.scale);
        else
            hipLaunchKernelGGL((score_generic_kernel<float, 64>), grid, dim3(256), 0, st,
                               static_cast<const float *>(q), static_cast<const float *>(landmarks), cand,
                               dm.mask_words, P, stats, dm.hkv, dm.G, dm.n, dm.wtiles, dm.scale);
    }
    return hipGetLastError();
}

size_t select_dynamic_lds(const Dims &dm, bool keys_in_lds) {
    return 4ull * dm.k * sizeof(int32_t) + static_cast<size_t>(dm.wtiles) * dm.G * sizeof(float) +
           (keys_in_lds ? static_cast<size_t>(dm.n) * sizeof(uint32_t) : 0);
}

size_t select_static_lds() { return sizeof(SelectScratch); }

template <int GP>
static hipError_t select_t(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                           int32_t *sel, int32_t *slot_chunk, int2 *misses, int32_t *miss_count,
                           unsigned long long *counters, uint32_t *gscratch, int keys_in_lds, hipStream_t st) {
    const size_t lds = select_dynamic_lds(dm, keys_in_lds != 0);
    hipError_t e = allow_lds(reinterpret_cast<const void *>(select_kernel<GP>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_kernel<GP>, dim3(dm.b * dm.hkv), dim3(kSelectThreads), lds, st, P, stats, cand,
                       dm.mask_words, S2, sel, slot_chunk, misses, miss_count, counters, gscratch, keys_in_lds,
                       dm.G, dm.n, dm.k, dm.wtiles);
    return hipGetLastError();
}

hipError_t launch_select(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                         int32_t *sel, int32_t *slot_chunk, int2 *misses, int32_t *miss_count,
                         unsigned long long *counters, uint32_t *gscratch, int keys_in_lds, hipStream_t st) {
    switch (dm.GP) {
        case 4: return select_t<4>(dm, P, stats, cand, S2, sel, slot_chunk, misses, miss_count, counters, gscratch,
                                   keys_in_lds, st);
        case 8: return select_t<8>(dm, P, stats, cand, S2, sel, slot_chunk, misses, miss_count, counters, gscratch,
                                   keys_in_lds, st);
        default: return select_t<16>(dm, P, stats, cand, S2, sel, slot_chunk, misses, miss_count, counters,
                                     gscratch, keys_in_lds, st);
    }
}

hipError_t launch_topo(const Dims &dm, const float *min_cos, int32_t *outliers, uint32_t *gscratch, int keys_in_lds,
                       hipStream_t st) {
    if (dm.o <= 0) return hipSuccess;
    const size_t lds = keys_in_lds ? static_cast<size_t>(dm.n) * sizeof(uint32_t) : 0;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(topo_kernel), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topo_kernel, dim3(dm.b * dm.hkv), dim3(kSelectThreads), lds, st, min_cos, dm.n,
                       dm.n - dm.n_loc, dm.o, outliers, gscratch, keys_in_lds);
    return hipGetLastError();
}

}  // namespace skv
