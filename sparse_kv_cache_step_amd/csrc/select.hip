// Selection half of the decode step (review page, section 三, Algorithm 2
// steps 1-2, and the Telegram write-up's set-difference cache):
//   score   P = q . L^T / sqrt(d) for every chunk, with per-tile softmax
//           partials over the selectable chunks;
//   group   S2 = per-head softmax over selectable chunks, averaged over the
//           query heads of a KV group;
//   topk    (prefill.hip) ArgTopK(S2, k);
//   setdiff hits, evictions and the miss list against the previous step.
#include "skv_device.h"

namespace skv {

// ---------------------------------------------------------------------------
// Landmark scoring, bfloat16, on MFMA.  For one (sequence, KV head) the
// contraction P[g, j] = sum_i q[g, i] L[j, i] has M = the G query heads of the
// group (padded to 16), N = chunks, K = d.  One v_mfma_f32_16x16x32_bf16 takes
// 16 chunks x 32 dims; lane l feeds head (l & 15) of q and chunk (l & 15) of
// L with the same eight dims, so lane group l >> 4 owns a contiguous quarter
// of d and reads 16-byte slices of each 256-byte landmark row.
// Each wave scores 64 chunks (4 rounds), a workgroup 256 chunks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void score_mfma_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ L,
                                                         const uint32_t *__restrict__ cand, int mask_words,
                                                         float *__restrict__ P, float2 *__restrict__ stats,
                                                         int hkv, int G, int n, int tiles, float scale) {
    constexpr int KS = D / 32;      // k-steps over d
    constexpr int QW = D / 4;       // dims owned by one lane group
    constexpr int ROUNDS = 4;
    __shared__ float2 red[4][kMaxGroup];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, quad = lane >> 4;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;

    bf16x8 qa[KS];
    {
        const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
        const uint16_t *qrow = q + (static_cast<size_t>(b) * hq + h * G + row) * D + quad * QW;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = row < G ? *reinterpret_cast<const u32x4 *>(qrow + ks * 8) : zero;
            qa[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const int wbase = blockIdx.x * kScoreTile + wave * 64;
    const uint16_t *Lbh = L + static_cast<size_t>(bh) * n * D;
    u32x4 lb[ROUNDS][KS];
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        const int j = wbase + rd * 16 + row;
        const uint16_t *lrow = Lbh + static_cast<size_t>(j < n ? j : 0) * D + quad * QW;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            lb[rd][ks] = j < n ? *reinterpret_cast<const u32x4 *>(lrow + ks * 8) : u32x4{0u, 0u, 0u, 0u};
    }

    const uint32_t *cm = cand + static_cast<size_t>(bh) * mask_words;
    float mx[4], sm[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { mx[e] = -INFINITY; sm[e] = 0.f; }
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8, lb[rd][ks]), acc, 0, 0, 0);
        // lane holds heads 4*quad + e of chunk wbase + rd*16 + row
        const int j = wbase + rd * 16 + row;
        const bool valid = j < n && mask_bit(cm, j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int g = quad * 4 + e;
            if (g < G && j < n) {
                const float p = valid ? acc[e] * scale : -INFINITY;
                P[(static_cast<size_t>(b) * hq + h * G + g) * n + j] = p;
                if (valid) {
                    if (p > mx[e]) { sm[e] = sm[e] * expf(mx[e] - p) + 1.f; mx[e] = p; }
                    else sm[e] += expf(p - mx[e]);
                }
            }
        }
    }
    // reduce over the 16 chunks (lanes) of each lane group
#pragma unroll
    for (int e = 0; e < 4; ++e) ms_reduce_lanes(mx[e], sm[e], 16);
    if (row == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int g = quad * 4 + e;
            if (g < G) red[wave][g] = make_float2(mx[e], sm[e]);
        }
    }
    __syncthreads();
    if (threadIdx.x < G) {
        const int g = threadIdx.x;
        float m = red[0][g].x, s = red[0][g].y;
        for (int w = 1; w < 4; ++w) ms_merge(m, s, red[w][g].x, red[w][g].y);
        stats[(static_cast<size_t>(b) * hq + h * G + g) * tiles + blockIdx.x] = make_float2(m, s);
    }
}

// Generic scoring (any storage type): thread per chunk, all G heads.
template <typename T, int D>
__global__ __launch_bounds__(256) void score_generic_kernel(const T *__restrict__ q, const T *__restrict__ L,
                                                            const uint32_t *__restrict__ cand, int mask_words,
                                                            float *__restrict__ P, float2 *__restrict__ stats,
                                                            int hkv, int G, int n, int tiles, float scale) {
    __shared__ float qs[kMaxGroup][D];
    __shared__ float2 red[4][kMaxGroup];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    for (int i = threadIdx.x; i < G * D; i += 256)
        qs[i / D][i % D] = Elem<T>::ld(q, (static_cast<size_t>(b) * hq + h * G) * D + i);
    __syncthreads();
    const int j = blockIdx.x * kScoreTile + threadIdx.x;
    const bool valid = j < n && mask_bit(cand + static_cast<size_t>(bh) * mask_words, j);
    const T *lrow = L + (static_cast<size_t>(bh) * n + (j < n ? j : 0)) * D;
    for (int g = 0; g < G; ++g) {
        float p = -INFINITY;
        if (valid) {
            float acc = 0.f;
            for (int i = 0; i < D; ++i) acc += qs[g][i] * Elem<T>::ld(lrow, i);
            p = acc * scale;
        }
        if (j < n) P[(static_cast<size_t>(b) * hq + h * G + g) * n + j] = p;
        float m = p, s = valid ? 1.f : 0.f;
        ms_reduce_lanes(m, s, 64);
        if (lane == 0) red[wave][g] = make_float2(m, s);
    }
    __syncthreads();
    if (threadIdx.x < G) {
        const int g = threadIdx.x;
        float m = red[0][g].x, s = red[0][g].y;
        for (int w = 1; w < 4; ++w) ms_merge(m, s, red[w][g].x, red[w][g].y);
        stats[(static_cast<size_t>(b) * hq + h * G + g) * tiles + blockIdx.x] = make_float2(m, s);
    }
}

// ---------------------------------------------------------------------------
// Group score S2[j] = (1/G) sum_g exp(P[g, j] - m_g) / Z_g over selectable j,
// 0 elsewhere.  (m_g, Z_g) come from the per-tile partials.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void group_kernel(const float *__restrict__ P, const float2 *__restrict__ stats,
                                                    const uint32_t *__restrict__ cand, int mask_words,
                                                    float *__restrict__ S2, int hkv, int G, int n, int tiles) {
    __shared__ float gm[kMaxGroup], ginvz[kMaxGroup];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    for (int g = wave; g < G; g += 4) {
        const float2 *st = stats + (static_cast<size_t>(b) * hq + h * G + g) * tiles;
        float m = -INFINITY, s = 0.f;
        for (int t = lane; t < tiles; t += 64) ms_merge(m, s, st[t].x, st[t].y);
        ms_reduce_lanes(m, s, 64);
        if (lane == 0) { gm[g] = m; ginvz[g] = s > 0.f ? 1.f / s : 0.f; }
    }
    __syncthreads();
    const int j = blockIdx.x * kGroupTile + threadIdx.x;
    if (j >= n) return;
    float v = 0.f;
    if (mask_bit(cand + static_cast<size_t>(bh) * mask_words, j)) {
        for (int g = 0; g < G; ++g)
            v += expf(P[(static_cast<size_t>(b) * hq + h * G + g) * n + j] - gm[g]) * ginvz[g];
        v /= static_cast<float>(G);
    }
    S2[static_cast<size_t>(bh) * n + j] = v;
}

// ---------------------------------------------------------------------------
// Set difference against the resident chunks (one workgroup per sequence and
// KV head).  A slot keeps its chunk when the chunk is selected again (hit);
// the other slots are freed and take the missing chunks: the m-th missing
// chunk (ascending) goes to the m-th free slot (ascending).  Emits the miss
// list (chunk, slot) and counts hits and misses.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void setdiff_kernel(const int32_t *__restrict__ sel,
                                                      int32_t *__restrict__ slot_chunk,
                                                      int2 *__restrict__ misses, int32_t *__restrict__ miss_count,
                                                      unsigned long long *__restrict__ counters, int k) {
    extern __shared__ int32_t smem[];
    __shared__ int wcnt[4];
    int32_t *s_sel = smem;          // selected chunks, ascending
    int32_t *s_keep = smem + k;     // chunk kept by each slot, -1 if the slot is free
    int32_t *s_hit = smem + 2 * k;  // 1 if selected chunk i is already resident
    int32_t *s_rank = smem + 3 * k; // index into s_sel of the m-th miss
    const int bh = blockIdx.x;
    const int32_t *gs = sel + static_cast<size_t>(bh) * k;
    int32_t *gc = slot_chunk + static_cast<size_t>(bh) * k;
    for (int i = threadIdx.x; i < k; i += blockDim.x) { s_sel[i] = gs[i]; s_hit[i] = 0; }
    __syncthreads();
    for (int sl = threadIdx.x; sl < k; sl += blockDim.x) {
        const int32_t c = gc[sl];
        int keep = -1;
        if (c >= 0) {
            int lo = 0, hi = k;
            while (lo < hi) {
                int mid = (lo + hi) >> 1;
                if (s_sel[mid] < c) lo = mid + 1; else hi = mid;
            }
            if (lo < k && s_sel[lo] == c) { keep = c; s_hit[lo] = 1; }
        }
        s_keep[sl] = keep;
    }
    __syncthreads();
    int nmiss = 0;
    for (int i0 = 0; i0 < k; i0 += blockDim.x) {
        const int i = i0 + threadIdx.x;
        const bool miss = i < k && !s_hit[i];
        int tot;
        const int r = block_excl_count(miss, wcnt, &tot);
        if (miss) s_rank[nmiss + r] = i;
        nmiss += tot;
    }
    __syncthreads();
    int nfree = 0;
    int2 *ml = misses + static_cast<size_t>(bh) * k;
    for (int s0 = 0; s0 < k; s0 += blockDim.x) {
        const int sl = s0 + threadIdx.x;
        const bool fr = sl < k && s_keep[sl] < 0;
        int tot;
        const int r = block_excl_count(fr, wcnt, &tot);
        if (fr && nfree + r < nmiss) {  // free slots and misses are equal in number
            const int32_t chunk = s_sel[s_rank[nfree + r]];
            gc[sl] = chunk;
            ml[nfree + r] = make_int2(chunk, sl);
        }
        nfree += tot;
    }
    if (threadIdx.x == 0) {
        miss_count[bh] = nmiss;
        atomicAdd(&counters[0], static_cast<unsigned long long>(k - nmiss));
        atomicAdd(&counters[1], static_cast<unsigned long long>(nmiss));
        if (bh == 0) atomicAdd(&counters[2], 1ull);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_score(const Dims &dm, const void *q, const void *landmarks, const uint32_t *cand, float *P,
                        float2 *stats, hipStream_t st) {
    dim3 grid(dm.score_tiles, dm.b * dm.hkv);
    if (dm.bf16) {
        if (dm.d == 128)
            hipLaunchKernelGGL(score_mfma_kernel<128>, grid, dim3(256), 0, st, static_cast<const uint16_t *>(q),
                               static_cast<const uint16_t *>(landmarks), cand, dm.mask_words, P, stats, dm.hkv,
                               dm.G, dm.n, dm.score_tiles, dm.scale);
        else
            hipLaunchKernelGGL(score_mfma_kernel<64>, grid, dim3(256), 0, st, static_cast<const uint16_t *>(q),
                               static_cast<const uint16_t *>(landmarks), cand, dm.mask_words, P, stats, dm.hkv,
                               dm.G, dm.n, dm.score_tiles, dm.scale);
    } else {
        if (dm.d == 128)
            hipLaunchKernelGGL((score_generic_kernel<float, 128>), grid, dim3(256), 0, st,
                               static_cast<const float *>(q), static_cast<const float *>(landmarks), cand,
                               dm.mask_words, P, stats, dm.hkv, dm.G, dm.n, dm.score_tiles, dm.scale);
        else
            hipLaunchKernelGGL((score_generic_kernel<float, 64>), grid, dim3(256), 0, st,
                               static_cast<const float *>(q), static_cast<const float *>(landmarks), cand,
                               dm.mask_words, P, stats, dm.hkv, dm.G, dm.n, dm.score_tiles, dm.scale);
    }
    return hipGetLastError();
}

hipError_t launch_group(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                        hipStream_t st) {
    dim3 grid((dm.n + kGroupTile - 1) / kGroupTile, dm.b * dm.hkv);
    hipLaunchKernelGGL(group_kernel, grid, dim3(256), 0, st, P, stats, cand, dm.mask_words, S2, dm.hkv, dm.G, dm.n,
                       dm.score_tiles);
    return hipGetLastError();
}

hipError_t launch_setdiff(const Dims &dm, const int32_t *sel, int32_t *slot_chunk, int2 *misses,
                          int32_t *miss_count, unsigned long long *counters, hipStream_t st) {
    if (dm.k <= 0) return hipSuccess;
    const size_t lds = 4ull * dm.k * sizeof(int32_t);
    hipLaunchKernelGGL(setdiff_kernel, dim3(dm.b * dm.hkv), dim3(256), lds, st, sel, slot_chunk, misses, miss_count,
                       counters, dm.k);
    return hipGetLastError();
}

}  // namespace skv
