// Selection half of the decode step (review page, section 三, Algorithm 2
// steps 1-2, and the Telegram write-up's set-difference cache):
//   score   P = q . L^T / sqrt(d) for every chunk, with per-tile softmax
//           partials over the selectable chunks;
//   group   the group score S2 = per-head softmax over selectable chunks
//           averaged over the query heads of the KV group, as selection keys;
//   select  one workgroup per (sequence, KV head): ArgTopK(S2, k) by radix
//           selection, and the set difference against the previous step's
//           resident chunks (miss list, hit counts).
// The same radix selection picks the prefill's outlier chunks.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "skv_device.h"

namespace skv {

// ---------------------------------------------------------------------------
// Landmark scoring, bfloat16, on MFMA.  For one (sequence, KV head) the
// contraction P[g, j] = sum_i q[g, i] L[j, i] has M = the G query heads of the
// group (padded to 16), N = chunks, K = d.  One v_mfma_f32_16x16x32_bf16 takes
// 16 chunks x 32 dims: lane l feeds head (l & 15) of q and chunk (l & 15) of
// L with dims 32*ks + 8*(l >> 4) .. +8, so the four lane groups of one load
// instruction read 64 contiguous bytes of each landmark row.  The kernel is
// persistent: each wave scores a contiguous run of 64-chunk tiles (4 rounds
// of 16 chunks), and as soon as a round's MFMAs have consumed its registers
// the same round of the next tile is loaded into them, so every wave keeps a
// whole tile of landmark loads in flight while it finishes the current one.
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

// MODE 0: G <= 4 (U stored one value per lane); 1: G > 4, G % 4 == 0 (four
// heads per 16-byte store); 2: other G > 4 (four single stores).
template <int D, int MODE>
__global__ __launch_bounds__(256) void score_mfma_kernel(const uint16_t *__restrict__ q,
                                                         const uint16_t *__restrict__ L,
                                                         const uint32_t *__restrict__ cand, int mask_words,
                                                         float *__restrict__ U, float2 *__restrict__ stats,
                                                         int hkv, int Gr, int w_obs, int o_base, int wp,
                                                         int n, int wtiles, int rows, int tiles_per_wave,
                                                         float scale) {
    constexpr int KS = D / 32;
    constexpr int ROUNDS = 4;
    const int G = Gr * wp;  // scored rows (heads) per KV head: see QRows
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row = lane & 15, quad = lane >> 4;
    const int hq = hkv * Gr;
    const int total = rows * wtiles;
    int T = (blockIdx.x * 4 + wave) * tiles_per_wave;  // this wave's run of tiles
    const int t_end = min(total, T + tiles_per_wave);
    if (T >= t_end) return;  // no barrier in this kernel

    // Loads and stores go through buffer resources: the next tile's loads are
    // switched off (not branched around) after the last tile, chunks past n
    // read zeros and their stores are dropped.
    const Rsrc qr = make_rsrc(q, static_cast<uint32_t>(rows) * Gr * w_obs * D * 2);
    const Rsrc cr = make_rsrc(cand, static_cast<uint32_t>(rows) * mask_words * 4);
    const uint32_t lrow_bytes = static_cast<uint32_t>(n) * D * 2;
    auto l_rsrc = [&](int bh) { return make_rsrc(L + static_cast<size_t>(bh) * n * D, lrow_bytes); };
    // query rows of the group: lane row = head; rows past G repeat the last
    // head and their MFMA outputs are ignored
    auto q_off = [&](int bh) {
        const int b = bh / hkv, h = bh % hkv, gv = min(row, G - 1);
        return (((b * hq + h * Gr + gv / wp) * w_obs + o_base + gv % wp) * D + quad * 8) * 2;
    };
    auto load_q = [&](int off, bf16x8 *qa) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = __builtin_bit_cast(bf16x8, buf_ld128(qr, off + ks * 64));
    };
    // round rd (16 chunks) of a tile: lane row takes chunk 64*wt + 16*rd + row
    auto load_round = [&](Rsrc lr, int off, u32x4 *dst) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dst[ks] = buf_ld128(lr, off + ks * 64);
    };
    auto round_off = [&](int wt, int rd) { return ((wt * 64 + rd * 16 + row) * D + quad * 8) * 2; };

    bf16x8 qa[KS];
    u32x4 lb[ROUNDS][KS];
    uint32_t mw0, mw1;
    {
        // the prologue issues its loads in the loop body's order (query,
        // mask, rounds 0-3), so the wait counts at the loop head hold on both
        // paths into it
        const int bh = T / wtiles, wt = T - bh * wtiles;
        load_q(q_off(bh), qa);
        __builtin_amdgcn_sched_barrier(0);
        mw0 = buf_ld32(cr, (bh * mask_words + 2 * wt) * 4);
        mw1 = buf_ld32(cr, 2 * wt + 1 < mask_words ? (bh * mask_words + 2 * wt + 1) * 4 : kOob);
        __builtin_amdgcn_sched_barrier(0);
        const Rsrc lr = l_rsrc(bh);
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
            load_round(lr, round_off(wt, rd), lb[rd]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    for (; T < t_end; ++T) {
        const int bh = T / wtiles, wt = T - bh * wtiles;
        const int wbase = wt * 64;
        const bool more = T + 1 < t_end;
        const int bhn = more ? (T + 1) / wtiles : bh, wtn = more ? T + 1 - bhn * wtiles : wt;
        const bool new_row = bhn != bh;
        bf16x8 qn[KS];
        load_q(new_row ? q_off(bhn) : kOob, qn);
        const uint32_t m0 = mw0, m1 = mw1;
        mw0 = buf_ld32(cr, more ? (bhn * mask_words + 2 * wtn) * 4 : kOob);
        mw1 = buf_ld32(cr, more && 2 * wtn + 1 < mask_words ? (bhn * mask_words + 2 * wtn + 1) * 4 : kOob);
        const Rsrc lrn = l_rsrc(bhn);
        const Rsrc ur = make_rsrc(U + static_cast<size_t>(bh) * n * G, static_cast<uint32_t>(n) * G * 4);
        const Rsrc sr = make_rsrc(stats + static_cast<size_t>(bh) * G * wtiles, static_cast<uint32_t>(G) * wtiles * 8);
        auto valid_chunk = [&](int rd) {
            const int jl = rd * 16 + row;  // chunk within the tile
            const uint32_t word = jl < 32 ? m0 : m1;
            return wbase + jl < n && ((word >> (jl & 31)) & 1u);
        };

        if constexpr (MODE == 0) {
            // lane (quad, row) <- head quad of chunk row of each round
            float p[ROUNDS];
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8, lb[rd][ks]), acc,
                                                                  0, 0, 0);
                load_round(lrn, more ? round_off(wtn, rd) : kOob, lb[rd]);
                const float t0 = __shfl(acc[0], row, 64), t1 = __shfl(acc[1], row, 64);
                const float t2 = __shfl(acc[2], row, 64), t3 = __shfl(acc[3], row, 64);
                const float mine = quad == 0 ? t0 : (quad == 1 ? t1 : (quad == 2 ? t2 : t3));
                p[rd] = (quad < G && valid_chunk(rd)) ? mine * scale : -INFINITY;
            }
            float M = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
            M = sel_max16(M);
            float S = 0.f;
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd) {
                const float u = p[rd] == -INFINITY ? 0.f : expf(p[rd] - M);
                S += u;
                const int j = wbase + rd * 16 + row;
                buf_st32(u, ur, quad < G ? (j * G + quad) * 4 : kOob);
            }
            S = sel_sum16(S);
            buf_st64(make_float2(M, S), sr, row == 0 && quad < G ? (quad * wtiles + wt) * 8 : kOob);
        } else {
            // lane holds heads 4*quad + e of chunk row
            float p[ROUNDS][4];
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8, lb[rd][ks]), acc,
                                                                  0, 0, 0);
                load_round(lrn, more ? round_off(wtn, rd) : kOob, lb[rd]);
                const bool jv = valid_chunk(rd);
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
                buf_st64(make_float2(M, S), sr, row == 0 && quad * 4 + e < G ? ((quad * 4 + e) * wtiles + wt) * 8 : kOob);
            }
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd) {
                const int j = wbase + rd * 16 + row;
                if constexpr (MODE == 1) {
                    buf_st128(make_float4(p[rd][0], p[rd][1], p[rd][2], p[rd][3]), ur,
                              quad * 4 < G ? (j * G + quad * 4) * 4 : kOob);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) buf_st32(p[rd][e], ur, quad * 4 + e < G ? (j * G + quad * 4 + e) * 4 : kOob);
                }
            }
        }
        if (new_row) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[ks] = qn[ks];
        }
    }
}

// Generic scoring (any storage type): thread per chunk, all G heads; same
// outputs as the MFMA kernel (U and per-64-chunk tile statistics).
template <typename T, int D>
__global__ __launch_bounds__(256) void score_generic_kernel(const T *__restrict__ q, const T *__restrict__ L,
                                                            const uint32_t *__restrict__ cand, int mask_words,
                                                            float *__restrict__ U, float2 *__restrict__ stats,
                                                            int hkv, int Gr, int w_obs, int o_base, int wp, int n,
                                                            int wtiles, float scale) {
    __shared__ float qs[kMaxGroup][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * Gr, G = Gr * wp;
    for (int i = threadIdx.x; i < G * D; i += 256) {
        const int gv = i / D;
        qs[gv][i % D] = Elem<T>::ld(q, ((static_cast<size_t>(b) * hq + h * Gr + gv / wp) * w_obs + o_base + gv % wp) * D +
                                           i % D);
    }
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
    alignas(16) uint32_t hist[4096];
    int wtmp[2][32];
    uint32_t digit;
    int above;
};

// The waves' pairs of partials in sc.wtmp (blockDim.x / 64 of each): this
// wave's exclusive prefix of both and their totals.  Lane w of every wave
// loads wave w's pair, a scan across those lanes forms the inclusive sums,
// and lane reads hand each wave the entries it needs, so no thread walks the
// list.  Call between the barrier that publishes wtmp and the next write.
__device__ __forceinline__ void wave_partials_prefix(const SelectScratch &sc, int *pa, int *pb, int *ta, int *tb) {
    const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int x = lane < nw ? sc.wtmp[0][lane] : 0, y = lane < nw ? sc.wtmp[1][lane] : 0;
    x = wave_incl_scan(x);
    y = wave_incl_scan(y);
    const int src = wave > 0 ? wave - 1 : 0;
    const int px = __builtin_amdgcn_readlane(x, src), py = __builtin_amdgcn_readlane(y, src);
    *pa = wave > 0 ? px : 0;
    *pb = wave > 0 ? py : 0;
    *ta = __builtin_amdgcn_readlane(x, nw - 1);
    *tb = __builtin_amdgcn_readlane(y, nw - 1);
}

// Inclusive prefix sums of two per-thread counts over the threads of the
// block in one pass (one pair of barriers); totals in *ta, *tb.
__device__ __forceinline__ void block_scan2(int &a, int &b, SelectScratch &sc, int *ta, int *tb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_incl_scan(a);
    b = wave_incl_scan(b);
    if (lane == 63) { sc.wtmp[0][wave] = a; sc.wtmp[1][wave] = b; }
    __syncthreads();
    int pa, pb;
    wave_partials_prefix(sc, &pa, &pb, ta, tb);
    __syncthreads();
    a += pa;
    b += pb;
}

// Minimum and maximum of per-thread values over the block (one pair of
// barriers); every thread gets both.
__device__ __forceinline__ void block_minmax(uint32_t &mn, uint32_t &mx, SelectScratch &sc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), off, 64)));
        mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), off, 64)));
    }
    if (lane == 0) { sc.wtmp[0][wave] = static_cast<int>(mn); sc.wtmp[1][wave] = static_cast<int>(mx); }
    __syncthreads();
    // lane w < nw takes wave w's pair; lanes past nw hold the identities
    uint32_t a = lane < nw ? static_cast<uint32_t>(sc.wtmp[0][lane]) : 0xffffffffu;
    uint32_t c = lane < nw ? static_cast<uint32_t>(sc.wtmp[1][lane]) : 0u;
    for (int off = 1; off < nw; off <<= 1) {
        a = min(a, static_cast<uint32_t>(__shfl_xor(static_cast<int>(a), off, 64)));
        c = max(c, static_cast<uint32_t>(__shfl_xor(static_cast<int>(c), off, 64)));
    }
    mn = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(a), 0));
    mx = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(c), 0));
    __syncthreads();
}

// The k largest of keys[0, n), exact ties to the lower index, written to
// out[0, k) and/or lds_out[0, k) (each if not null) in ascending index
// order.  The caller
// passes kmin <= kmax bounding the candidate keys: at least k keys lie in
// [kmin, kmax], none above kmax, and keys below kmin are never taken.
// Radix selection runs on the offsets key - kmin, 12 bits per pass from the
// highest bit the range needs, so a tight range takes two passes and spreads
// over many bins.  Each pass: all threads build the histogram of the current
// digit among the keys that match the prefix found so far; every thread then
// takes four bins (highest first), clears them, and a block scan finds the bin
// holding the k-th largest key.  The threshold T and the number of keys equal
// to T to take follow; an ordered compaction over wave-contiguous segments
// (ballots and popcounts) writes the indices.  Requires blockDim.x == 1024
// (four bins per thread) and 1 <= k; every thread of the block must call it;
// sc.hist must be zero on entry and is zero again on return.
struct RadixCut {
    uint32_t thr;  // the k-th largest key
    int need_eq;   // keys equal to thr among the k largest
};

// The threshold passes of radix_topk alone: the k-th largest key and how many
// keys equal to it the k largest take.
__device__ RadixCut radix_cut(const uint32_t *keys, int n, int k, uint32_t kmin, uint32_t kmax, SelectScratch &sc) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const uint32_t range = kmax - kmin;
    int hi = range == 0 ? 0 : 32 - __clz(static_cast<int>(range));  // bits of the offsets
    uint64_t prefix = 0;  // offset bits fixed so far (above hi)
    int krem = k;
    while (hi > 0) {
        const int lo = hi > 12 ? hi - 12 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        const uint64_t want = prefix >> hi;
        for (int j0 = tid; j0 < n; j0 += 4 * nt) {
            uint32_t kk[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) kk[u] = j0 + u * nt < n ? keys[j0 + u * nt] : 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint64_t rel = static_cast<uint64_t>(kk[u] - kmin);
                if (j0 + u * nt < n && kk[u] >= kmin && (rel >> hi) == want)
                    atomicAdd(&sc.hist[(rel >> lo) & dmask], 1u);
            }
        }
        __syncthreads();  // every thread has also read the previous pass's digit
        if (tid == 0) { sc.digit = 0; sc.above = 0; }
        // thread t takes bins nb4 - 4t - 4 .. nb4 - 4t - 1 (highest first)
        const int nb4 = max(4, static_cast<int>(dmask) + 1);
        const int base = nb4 - 4 * (tid + 1);
        u32x4 cnt = {0u, 0u, 0u, 0u};
        if (base >= 0) {
            cnt = *reinterpret_cast<const u32x4 *>(&sc.hist[base]);
            *reinterpret_cast<u32x4 *>(&sc.hist[base]) = u32x4{0u, 0u, 0u, 0u};
        }
        const int local = static_cast<int>(cnt[0] + cnt[1] + cnt[2] + cnt[3]);
        int incl = local, dummy = 0, tot, tot2;
        block_scan2(incl, dummy, sc, &tot, &tot2);
        const int excl = incl - local;
        if (base >= 0 && excl < krem && krem <= incl) {
            int acc = excl;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                const int c = static_cast<int>(cnt[i]);
                if (acc + c >= krem) { sc.digit = static_cast<uint32_t>(base + i); sc.above = acc; break; }
                acc += c;
            }
        }
        __syncthreads();
        prefix |= static_cast<uint64_t>(sc.digit) << lo;
        krem -= sc.above;
        hi = lo;
    }
    return RadixCut{kmin + static_cast<uint32_t>(prefix), krem};
}

__device__ void radix_topk(const uint32_t *keys, int n, int k, uint32_t kmin, uint32_t kmax, int32_t *out,
                           int32_t *lds_out, SelectScratch &sc) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
    const RadixCut cut = radix_cut(keys, n, k, kmin, kmax, sc);
    const uint32_t thr = cut.thr;
    const int need_eq = cut.need_eq;  // keys equal to thr that are taken, lowest index first

    // ordered compaction: wave w owns keys [w * seg, (w + 1) * seg)
    const int seg = ((n + nw - 1) / nw + 63) & ~63;
    const int j0 = min(n, wave * seg), j1 = min(n, j0 + seg);
    int cg = 0, ce = 0;
    for (int jb = j0; jb < j1; jb += 256) {
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kk[u] = jb + u * 64 + lane < j1 ? keys[jb + u * 64 + lane] : 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool in = jb + u * 64 + lane < j1;
            cg += __popcll(__ballot(in && kk[u] > thr));
            ce += __popcll(__ballot(in && kk[u] == thr));
        }
    }
    if (lane == 0) { sc.wtmp[0][wave] = cg; sc.wtmp[1][wave] = ce; }
    __syncthreads();
    int gt_run, eq_run, gt_all, eq_all;
    wave_partials_prefix(sc, &gt_run, &eq_run, &gt_all, &eq_all);
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    for (int jb = j0; jb < j1 && gt_run + min(eq_run, need_eq) < k; jb += 256) {
        uint32_t kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kk[u] = jb + u * 64 + lane < j1 ? keys[jb + u * 64 + lane] : 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = jb + u * 64 + lane;
            const bool g = j < j1 && kk[u] > thr, e = j < j1 && kk[u] == thr;
            const uint64_t bg = __ballot(g), be = __ballot(e);
            const int gb = gt_run + __popcll(bg & below), eb = eq_run + __popcll(be & below);
            if (g || (e && eb < need_eq)) {
                const int pos = gb + min(eb, need_eq);
                if (pos < k) {
                    if (out) out[pos] = j;
                    if (lds_out) lds_out[pos] = j;
                }
            }
            gt_run += __popcll(bg);
            eq_run += __popcll(be);
        }
    }
}

// radix_topk with the keys in registers, for rows of at most blockDim.x * KPT
// keys: thread t holds keys[KPT t .. KPT t + KPT) (LDS, zeros from n to
// blockDim.x * KPT), read once.  Each pass: the threads add their matching
// keys to the histogram; then wave 0 alone finds the bin of the krem-th
// largest offset -- lane L owns the 64 bins of block 63 - L (lane 0 the
// highest), held so that bins 4m .. 4m + 3 of all blocks are 64 consecutive
// 16-byte words (bin 64 j + i at hist_pos), four sums of 16 bins per lane, a
// wave prefix sum, the owner lane's 16 bins -- and clears the histogram: two
// barriers a pass.  The ordered compaction is one prefix sum of the threads'
// counts (their keys are contiguous).  The selection goes to s_sel[0, k),
// ascending; with MARK each selected key keys[j] is replaced by its position
// + 1, which no key takes (selectable keys are at least 2^31, the others 0).
// Requires blockDim.x == 1024 and 1 <= k; sc.hist zero on entry and on
// return.
__device__ __forceinline__ int hist_pos(uint32_t b) {
    return static_cast<int>(((b & 63u) >> 2) * 256u + (b >> 6) * 4u + (b & 3u));
}

template <int KPT, bool MARK>
__device__ __forceinline__ void radix_topk_regs(uint32_t *keys, int n, int k, uint32_t kmin, uint32_t kmax,
                                                int32_t *s_sel, SelectScratch &sc) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t kr[KPT];
#pragma unroll
    for (int v = 0; v < KPT / 4; ++v) {
        const u32x4 x = reinterpret_cast<const u32x4 *>(keys)[tid * (KPT / 4) + v];
        kr[4 * v] = x[0]; kr[4 * v + 1] = x[1]; kr[4 * v + 2] = x[2]; kr[4 * v + 3] = x[3];
    }
    const uint32_t range = kmax - kmin;
    int hi = range == 0 ? 0 : 32 - __clz(static_cast<int>(range));  // bits of the offsets
    uint64_t prefix = 0;  // offset bits fixed so far (above hi)
    int krem = k;
    const int blk = 63 - lane;  // wave 0: this lane's block of 64 bins (lane 0: the highest)
    while (hi > 0) {
        const int lo = hi > 12 ? hi - 12 : 0;
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        // offsets matching the prefix: equal to it in the bits at and above hi
        const uint32_t himask = hi >= 32 ? 0u : ~((1u << hi) - 1u), want = static_cast<uint32_t>(prefix);
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const uint32_t rel = kr[u] - kmin;
            if (kr[u] >= kmin && (rel & himask) == want) atomicAdd(&sc.hist[hist_pos((rel >> lo) & dmask)], 1u);
        }
        __syncthreads();  // the histogram is complete (and the previous digit read by all)
        if (wave == 0) {
            u32x4 *h4 = reinterpret_cast<u32x4 *>(sc.hist);
            int sub[4] = {0, 0, 0, 0};
#pragma unroll 1
            for (int q = 0; q < 4; ++q) {
                u32x4 x[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) x[m] = h4[(4 * q + m) * 64 + blk];
#pragma unroll
                for (int m = 0; m < 4; ++m) sub[q] += static_cast<int>(x[m][0] + x[m][1] + x[m][2] + x[m][3]);
            }
            const int sum = sub[0] + sub[1] + sub[2] + sub[3];
            const int incl = wave_incl_scan(sum), excl = incl - sum;
            const uint64_t owner = __ballot(excl < krem && krem <= incl);
            const int src = owner ? __ffsll(static_cast<long long>(owner)) - 1 : 0;
            if (lane == src) {
                int acc = excl, q = 0;
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    if (acc + sub[i] >= krem) { q = i; break; }
                    acc += sub[i];
                }
                u32x4 x[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) x[m] = h4[(4 * q + m) * 64 + blk];
                int digit = blk * 64 + q * 16, above = acc;
                bool found = false;
#pragma unroll
                for (int i = 15; i >= 0; --i) {
                    const int c = static_cast<int>(x[i >> 2][i & 3]);
                    if (!found && acc + c >= krem) { found = true; digit = blk * 64 + q * 16 + i; above = acc; }
                    acc += c;
                }
                sc.digit = static_cast<uint32_t>(digit);
                sc.above = above;
            }
            // every lane's reads above precede its clears (same lane, in order)
#pragma unroll
            for (int m = 0; m < 16; ++m) h4[m * 64 + blk] = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
        prefix |= static_cast<uint64_t>(sc.digit) << lo;
        krem -= sc.above;
        hi = lo;
    }
    const uint32_t thr = kmin + static_cast<uint32_t>(prefix);  // the k-th largest key
    const int need_eq = krem;  // keys equal to thr that are taken, lowest index first
    int cg = 0, ce = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        cg += kr[u] > thr ? 1 : 0;
        ce += kr[u] == thr ? 1 : 0;
    }
    int ig = cg, ie = ce, tg, te;
    block_scan2(ig, ie, sc, &tg, &te);  // also orders the digit reads above before wtmp's reuse
    int gb = ig - cg, eb = ie - ce;     // keys of lower index: greater, equal
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int j = tid * KPT + u;
        const bool g = kr[u] > thr, e = kr[u] == thr;
        if (g || (e && eb < need_eq)) {
            const int pos = gb + min(eb, need_eq);
            if (pos < k) {
                s_sel[pos] = j;
                if constexpr (MARK) keys[j] = static_cast<uint32_t>(pos + 1);
            }
        }
        gb += g ? 1 : 0;
        eb += e ? 1 : 0;
    }
}

// keys per thread of the register form for a row of n keys (0: rows longer
// than 1024 x 32 keep radix_topk)
__host__ __device__ constexpr int select_kpt(int n) {
    return n <= 4096 ? 4 : (n <= 8192 ? 8 : (n <= 16384 ? 16 : (n <= 32768 ? 32 : 0)));
}

// Outlier selection for the prefill: the o chunks with the lowest minimum
// cosine among chunks [0, n_valid); keys from -min_cos.
__global__ __launch_bounds__(kSelectThreads) void topo_kernel(const float *__restrict__ min_cos, int n, int n_valid,
                                                              int o, int32_t *__restrict__ out,
                                                              uint32_t *__restrict__ gscratch, int use_lds) {
    extern __shared__ uint32_t dyn[];
    __shared__ SelectScratch sc;
    const int row = blockIdx.x;
    // LDS keys through dyn itself, global ones through gk (see select_kernel)
    uint32_t *gk = gscratch + static_cast<size_t>(row) * n;
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    for (int j = threadIdx.x; j < n; j += blockDim.x) {
        const uint32_t key = j < n_valid ? float_key(-min_cos[static_cast<size_t>(row) * n + j]) : 0u;
        if (use_lds) dyn[j] = key;
        else gk[j] = key;
        if (j < n_valid) { kmn = min(kmn, key); kmx = max(kmx, key); }
    }
    for (int i = threadIdx.x; i < 4096; i += blockDim.x) sc.hist[i] = 0;
    block_minmax(kmn, kmx, sc);  // its barriers also publish keys and hist
    if (o > 0 && kmn <= kmx) {
        int32_t *orow = out + static_cast<size_t>(row) * o;
        if (use_lds) radix_topk(dyn, n, o, kmn, kmx, orow, nullptr, sc);
        else radix_topk(gk, n, o, kmn, kmx, orow, nullptr, sc);
    }
}

// ---------------------------------------------------------------------------
// Group score, one workgroup per (slice of kGroupSlice chunks, row):
//  1. per query head g of the group, m_g = max over tiles of M_t,g and
//     Z_g = sum_t S_t,g exp(M_t,g - m_g) (every workgroup of a row repeats
//     this small reduction over the tile statistics);
//  2. tile weights w[t, g] = exp(M_t,g - m_g) / (Z_g G) of the slice's tiles;
//  3. S2[j] = sum_g U[j, g] w[t(j), g] = (1/G) sum_g softmax_g(P)[j] over
//     the selectable chunks j (0 elsewhere), written to S2 and as
//     order-preserving keys (selectable keys > 0), with the slice's smallest
//     and largest selectable key.
// ---------------------------------------------------------------------------
template <int GP>
__global__ __launch_bounds__(256) void group_kernel(const float *__restrict__ U, const float2 *__restrict__ stats,
                                                    const uint32_t *__restrict__ cand, int mask_words,
                                                    float *__restrict__ S2, uint32_t *__restrict__ keys,
                                                    uint2 *__restrict__ kbounds, int G, int n, int tiles,
                                                    int slices) {
    constexpr int TPS = kGroupSlice / 64;  // tiles per slice
    constexpr int UNR = kGroupSlice / 256;  // chunks per thread
    static_assert(TPS <= 64 && 64 % TPS == 0, "a slice's tiles sit in one 64-tile register block");
    __shared__ float s_w[TPS][GP];
    __shared__ uint32_t s_red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sl = blockIdx.x, bh = blockIdx.y;
    const int j0 = sl * kGroupSlice;
    const float *Ub = U + static_cast<size_t>(bh) * n * G;
    const uint32_t *cm = cand + static_cast<size_t>(bh) * mask_words;

    // the slice's U rows and mask words are loaded first, under the reduction
    float v[UNR][GP];
    uint32_t word[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int j = min(j0 + tid + 256 * u, n - 1);
        word[u] = cm[j >> 5];
        if (G == GP) {
#pragma unroll
            for (int q4 = 0; q4 < GP / 4; ++q4) {
                const float4 f = *reinterpret_cast<const float4 *>(Ub + static_cast<size_t>(j) * GP + 4 * q4);
                v[u][4 * q4] = f.x; v[u][4 * q4 + 1] = f.y; v[u][4 * q4 + 2] = f.z; v[u][4 * q4 + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int g = 0; g < GP; ++g) v[u][g] = g < G ? Ub[static_cast<size_t>(j) * G + g] : 0.f;
        }
    }
    // per head (one wave per head): all of the row's tile statistics in
    // flight at once (TPL per lane, more are streamed), the two wave
    // reductions, then the slice's tile weights straight from registers
    const int t0 = j0 / 64;  // first tile of the slice (a multiple of TPS)
    for (int g = wave; g < G; g += 4) {
        const float2 *st = stats + (static_cast<size_t>(bh) * G + g) * tiles;
        constexpr int TPL = 8;
        float2 sv[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = lane + 64 * i;
            sv[i] = t < tiles ? st[t] : make_float2(-INFINITY, 0.f);
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < TPL; ++i) m = fmaxf(m, sv[i].x);
        for (int t = lane + 64 * TPL; t < tiles; t += 64) m = fmaxf(m, st[t].x);
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < TPL; ++i) z += sv[i].x == -INFINITY ? 0.f : sv[i].y * expf(sv[i].x - m);
        for (int t = lane + 64 * TPL; t < tiles; t += 64) {
            const float2 x = st[t];
            z += x.x == -INFINITY ? 0.f : x.y * expf(x.x - m);
        }
        z = wave_sum(z);
        const float inv = z > 0.f ? 1.f / (z * static_cast<float>(G)) : 0.f;
        const int tl = lane - (t0 & 63);  // this lane's tile within the slice
        if (tl >= 0 && tl < TPS) {
            const int t = t0 + tl;
            float2 x = make_float2(-INFINITY, 0.f);
            if (t0 / 64 < TPL) {
#pragma unroll
                for (int i = 0; i < TPL; ++i)
                    if (i == t0 / 64) x = sv[i];
            } else if (t < tiles) {
                x = st[t];
            }
            s_w[tl][g] = x.x == -INFINITY ? 0.f : expf(x.x - m) * inv;
        }
    }
    __syncthreads();
    uint32_t kmn = 0xffffffffu, kmx = 0u;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int j = j0 + tid + 256 * u;
        if (j >= n) continue;
        const bool valid = (word[u] >> (j & 31)) & 1u;
        const float *wt = s_w[(j - j0) >> 6];
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < GP; ++g)
            if (g < G) acc += v[u][g] * wt[g];
        S2[static_cast<size_t>(bh) * n + j] = valid ? acc : 0.f;
        const uint32_t key = float_key(acc);
        keys[static_cast<size_t>(bh) * n + j] = valid ? key : 0u;
        if (valid) { kmn = min(kmn, key); kmx = max(kmx, key); }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kmn = min(kmn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmn), off, 64)));
        kmx = max(kmx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmx), off, 64)));
    }
    if (lane == 0) { s_red[0][wave] = kmn; s_red[1][wave] = kmx; }
    __syncthreads();
    if (tid == 0) {
        uint32_t a = s_red[0][0], c = s_red[1][0];
        for (int w = 1; w < 4; ++w) { a = min(a, s_red[0][w]); c = max(c, s_red[1][w]); }
        kbounds[static_cast<size_t>(bh) * slices + sl] = make_uint2(a, c);
    }
}

// ---------------------------------------------------------------------------
// Group score with a slice-local Top-K, one 1024-thread workgroup per (slice
// of SL chunks, row): the group kernel's S2 and keys for the slice (steps 1-3
// above), kept in LDS, then the slice's k largest keys (ties to the lower
// chunk; every selectable chunk of the slice when it has no more than k),
// written as the slice's candidates (key, chunk) in ascending chunk order.
// The row's ArgTopK is among the union of its slices' candidates: a chunk of
// the row's k largest has fewer than k chunks of the row ahead of it (larger
// key, or equal key and lower index), hence fewer than k of its own slice.
// The select kernel then ranks the union (slices x k keys) instead of all n.
// ---------------------------------------------------------------------------
template <int GP, int KPT>
__global__ __launch_bounds__(kSelectThreads) void group_topk_kernel(
    const float *__restrict__ U, const float2 *__restrict__ stats, const uint32_t *__restrict__ cand,
    int mask_words, float *__restrict__ S2, uint32_t *__restrict__ cand_key, int32_t *__restrict__ cand_idx,
    int32_t *__restrict__ cand_count, int G, int n, int tiles, int SL, int slices, int k) {
    extern __shared__ __align__(16) uint32_t dyn[];
    __shared__ SelectScratch sc;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
    const int sl = blockIdx.x, bh = blockIdx.y;
    const int j0 = sl * SL, cnt = min(SL, n - j0), t0 = j0 / 64, ntl = (cnt + 63) / 64;
    uint32_t *keys = dyn;                                    // SL keys of the slice
    int32_t *s_pos = reinterpret_cast<int32_t *>(keys + SL);  // k positions of the slice's Top-K
    float *s_w = reinterpret_cast<float *>(s_pos + k);       // (SL / 64) x GP tile weights
    for (int i = tid; i < 4096; i += nt) sc.hist[i] = 0;

    // 1-2. per head: m_g, Z_g over all the row's tiles, the slice's tile weights
    for (int g = wave; g < G; g += nw) {
        const float2 *st = stats + (static_cast<size_t>(bh) * G + g) * tiles;
        float m = -INFINITY;
        for (int t = lane; t < tiles; t += 64) m = fmaxf(m, st[t].x);
        m = wave_max(m);
        float z = 0.f;
        for (int t = lane; t < tiles; t += 64) {
            const float2 x = st[t];
            z += x.x == -INFINITY ? 0.f : x.y * expf(x.x - m);
        }
        z = wave_sum(z);
        const float inv = z > 0.f ? 1.f / (z * static_cast<float>(G)) : 0.f;
        for (int tl = lane; tl < ntl; tl += 64) {
            const float2 x = st[t0 + tl];
            s_w[tl * GP + g] = x.x == -INFINITY ? 0.f : expf(x.x - m) * inv;
        }
    }
    __syncthreads();

    // 3. S2 and the keys of the slice, four chunks' U rows in flight per thread
    const float *Ub = U + static_cast<size_t>(bh) * n * G;
    const uint32_t *cm = cand + static_cast<size_t>(bh) * mask_words;
    float *s2row = S2 + static_cast<size_t>(bh) * n;
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    int nvalid = 0;
    constexpr int UNR = 4;
    for (int i0 = tid; i0 < cnt; i0 += UNR * nt) {
        float v[UNR][GP];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = j0 + min(i0 + u * nt, cnt - 1);
            if (G == GP) {
#pragma unroll
                for (int q4 = 0; q4 < GP / 4; ++q4) {
                    const float4 f = *reinterpret_cast<const float4 *>(Ub + static_cast<size_t>(j) * GP + 4 * q4);
                    v[u][4 * q4] = f.x; v[u][4 * q4 + 1] = f.y; v[u][4 * q4 + 2] = f.z; v[u][4 * q4 + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int g = 0; g < GP; ++g) v[u][g] = g < G ? Ub[static_cast<size_t>(j) * G + g] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int i = i0 + u * nt;
            if (i >= cnt) break;
            const int j = j0 + i;
            const bool valid = (cm[j >> 5] >> (j & 31)) & 1u;
            const float *wt = s_w + (i >> 6) * GP;
            float acc = 0.f;
#pragma unroll
            for (int g = 0; g < GP; ++g)
                if (g < G) acc += v[u][g] * wt[g];
            s2row[j] = valid ? acc : 0.f;
            const uint32_t key = float_key(acc);
            keys[i] = valid ? key : 0u;
            if (valid) { kmn = min(kmn, key); kmx = max(kmx, key); ++nvalid; }
        }
    }
    if constexpr (KPT > 0)  // the register form reads 1024 x KPT (= SL) keys
        for (int i = cnt + tid; i < SL; i += nt) keys[i] = 0u;
    int tv, zero = 0, tz;
    block_scan2(nvalid, zero, sc, &tv, &tz);
    block_minmax(kmn, kmx, sc);  // its barriers also publish the keys
    const int kl = min(k, tv);
    int32_t *out = cand_idx + (static_cast<size_t>(bh) * slices + sl) * k;
    if (kl > 0) {
        // 4. the slice's Top-K (radix selection over the slice's keys)
        if constexpr (KPT > 0) radix_topk_regs<KPT, false>(keys, cnt, kl, kmn, kmx, s_pos, sc);
        else radix_topk(keys, cnt, kl, kmn, kmx, nullptr, s_pos, sc);
        __syncthreads();
        uint32_t *ok = cand_key + (static_cast<size_t>(bh) * slices + sl) * k;
        for (int i = tid; i < kl; i += nt) {
            const int p = s_pos[i];
            ok[i] = keys[p];
            out[i] = j0 + p;
        }
    }
    if (tid == 0) cand_count[static_cast<size_t>(bh) * slices + sl] = kl;
}

// ---------------------------------------------------------------------------
// The group score of one row into LDS, by a whole workgroup (group_kernel's
// steps 1-3 with the same arithmetic): the per-head maxima and sums over the
// row's tiles, the tile weights into s_w (tiles x GP), then S2 for every
// chunk, written to S2 and as keys into keys[0, n) (LDS), with the smallest
// and largest selectable key of this thread's chunks.  The first chunks' U
// rows are requested before the reduction, and each batch of chunks while
// the previous one is scored.  Every thread must call it (one barrier).
template <int GP>
__device__ __forceinline__ void group_score_lds(const float *__restrict__ U, const float2 *__restrict__ stats,
                                                const uint32_t *__restrict__ cand, int mask_words,
                                                float *__restrict__ S2, uint32_t *keys, float *s_w, int G, int n,
                                                int tiles, int bh, uint32_t &kmn, uint32_t &kmx) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
    constexpr int UNR = 32 / GP;
    const float *Ub = U + static_cast<size_t>(bh) * n * G;
    const uint32_t *cm = cand + static_cast<size_t>(bh) * mask_words;
    float *s2row = S2 + static_cast<size_t>(bh) * n;
    const int per = UNR * nt, iters = (n + per - 1) / per;
    float v[2][UNR][GP];
    uint32_t word[2][UNR];
    auto load = [&](int buf, int it) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = min(it * per + u * nt + tid, n - 1);
            word[buf][u] = cm[j >> 5];
            if (G == GP) {
#pragma unroll
                for (int q4 = 0; q4 < GP / 4; ++q4) {
                    const float4 f = *reinterpret_cast<const float4 *>(Ub + static_cast<size_t>(j) * GP + 4 * q4);
                    v[buf][u][4 * q4] = f.x; v[buf][u][4 * q4 + 1] = f.y;
                    v[buf][u][4 * q4 + 2] = f.z; v[buf][u][4 * q4 + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int g = 0; g < GP; ++g) v[buf][u][g] = g < G ? Ub[static_cast<size_t>(j) * G + g] : 0.f;
            }
        }
    };
    auto score = [&](int buf, int it) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int j = it * per + u * nt + tid;
            if (j >= n) break;
            const bool valid = (word[buf][u] >> (j & 31)) & 1u;
            const float *wt = s_w + (j >> 6) * GP;
            float acc = 0.f;
#pragma unroll
            for (int g = 0; g < GP; ++g)
                if (g < G) acc += v[buf][u][g] * wt[g];
            s2row[j] = valid ? acc : 0.f;
            const uint32_t key = float_key(acc);
            keys[j] = valid ? key : 0u;
            if (valid) { kmn = min(kmn, key); kmx = max(kmx, key); }
        }
    };
    load(0, 0);
    // per head (a wave each): m_g, Z_g over the row's tiles, the tile weights
    for (int g = wave; g < G; g += nw) {
        const float2 *st = stats + (static_cast<size_t>(bh) * G + g) * tiles;
        constexpr int TPL = 8;
        float2 sv[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = lane + 64 * i;
            sv[i] = t < tiles ? st[t] : make_float2(-INFINITY, 0.f);
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < TPL; ++i) m = fmaxf(m, sv[i].x);
        for (int t = lane + 64 * TPL; t < tiles; t += 64) m = fmaxf(m, st[t].x);
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < TPL; ++i) z += sv[i].x == -INFINITY ? 0.f : sv[i].y * expf(sv[i].x - m);
        for (int t = lane + 64 * TPL; t < tiles; t += 64) {
            const float2 x = st[t];
            z += x.x == -INFINITY ? 0.f : x.y * expf(x.x - m);
        }
        z = wave_sum(z);
        const float inv = z > 0.f ? 1.f / (z * static_cast<float>(G)) : 0.f;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            const int t = lane + 64 * i;
            if (t < tiles) s_w[t * GP + g] = sv[i].x == -INFINITY ? 0.f : expf(sv[i].x - m) * inv;
        }
        for (int t = lane + 64 * TPL; t < tiles; t += 64) {
            const float2 x = st[t];
            s_w[t * GP + g] = x.x == -INFINITY ? 0.f : expf(x.x - m) * inv;
        }
    }
    __syncthreads();
    for (int it = 0; it < iters; it += 2) {
        if (it + 1 < iters) load(1, it + 1);
        score(0, it);
        if (it + 1 < iters) {
            if (it + 2 < iters) load(0, it + 2);
            score(1, it + 1);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode selection, one workgroup per (sequence, KV head) row:
//  1. the row's keys (from the group kernel) into LDS when they fit, and
//     their bounds from the per-slice minima and maxima;
//  2. I = ArgTopK(S2, k) by radix selection, ascending;
//  3. cache update over the row's cap slots: a slot whose chunk is selected
//     again is a hit (its stamp becomes this step's); of the resident chunks
//     not selected, the E oldest (smallest stamp; equal stamps: higher chunk
//     index first) are evicted, E = max(0, misses - empty slots), so that the
//     cache keeps the selection and, in what room is left, the chunks
//     selected most recently -- with cap = k, every unselected chunk;
//  4. the m-th missing chunk (ascending) goes to the m-th free slot
//     (ascending, empty or evicted); emit the miss list, each selected
//     chunk's slot, and count hits and misses.
// ---------------------------------------------------------------------------
// CAND: the keys are the slices' candidates from group_topk_kernel (cslices
// slices of up to k per row, ascending chunk order), ranked here and mapped
// back to chunks.  GP > 0: the keys are the group score, computed in step 1
// from U and the tile statistics (group_score_lds) straight into LDS, which
// saves the group kernel's launch and the keys' round trip through memory
// (it pays where the rows alone fill the CUs: one CU reads a row's U at a
// fraction of the device rate).  Otherwise all n keys of the row with
// per-slice bounds.
template <bool CAND, int GP, int KPT>
__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const float *__restrict__ U, const float2 *__restrict__ stats, const uint32_t *__restrict__ cand,
    int mask_words, float *__restrict__ S2, int G, int tiles,
    const uint32_t *__restrict__ keys_g, const uint2 *__restrict__ kbounds, int slices,
    const uint32_t *__restrict__ cand_key, const int32_t *__restrict__ cand_idx,
    const int32_t *__restrict__ cand_count, int cslices, int32_t *__restrict__ sel,
    int32_t *__restrict__ sel_slot, int32_t *__restrict__ slot_chunk, uint32_t *__restrict__ slot_stamp,
    uint32_t stamp, int2 *__restrict__ misses, int32_t *__restrict__ miss_count,
    unsigned long long *__restrict__ counters, int use_lds, int n, int k, int cap) {
    extern __shared__ __align__(16) uint32_t dyn[];
    __shared__ SelectScratch sc;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int bh = blockIdx.x;
    // dynamic LDS: the keys first (16-byte aligned): the row's n keys when
    // they fit, or the candidates (keys, then their chunks)
    const uint32_t *krow = keys_g + static_cast<size_t>(bh) * n;
    // key entries held in LDS (the register form pads the row with zeros to 1024 x KPT)
    const int kcap = KPT > 0 ? kSelectThreads * KPT : (CAND ? cslices * k : (use_lds ? n : 0));
    // keys in LDS are reached through dyn itself (never through a pointer
    // that may also be global), so their accesses compile to LDS instructions
    const bool lds_keys = CAND || use_lds;
    uint32_t *keys = dyn;
    int32_t *s_ci = reinterpret_cast<int32_t *>(dyn + kcap);  // CAND: the chunk of each of cslices * k candidates
    int32_t *s_sel = s_ci + (CAND ? cslices * k : 0);    // k selected chunks, ascending
    int32_t *s_sslot = s_sel + k;                       // k: slot of selected chunk i (-1: missing)
    int32_t *s_rank = s_sslot + k;                      // k: index in s_sel of the m-th miss
    uint32_t *s_age = reinterpret_cast<uint32_t *>(s_rank + k);  // cap: eviction key (0: not evictable)
    int32_t *s_free = reinterpret_cast<int32_t *>(s_age + cap);  // cap: rank of a free slot, -1 otherwise
    float *s_w = reinterpret_cast<float *>(s_free + cap);        // GP > 0: tiles x GP tile weights

    uint32_t kmn = 0xffffffffu, kmx = 0u;
    int nkeys = n;
    // with no more cache slots than threads, each thread's slot entry is read
    // here, beside the keys, rather than after the Top-K
    const bool one_slot = cap <= nt;
    // (buffer loads: no branch around them, so they and the keys' loads are
    // all in flight together)
    const Rsrc scr = make_rsrc(slot_chunk + static_cast<size_t>(bh) * cap, static_cast<uint32_t>(cap) * 4);
    const Rsrc ssr = make_rsrc(slot_stamp + static_cast<size_t>(bh) * cap, static_cast<uint32_t>(cap) * 4);
    const int32_t my_c = static_cast<int32_t>(buf_ld32(scr, one_slot && tid < cap ? tid * 4 : kOob));
    const uint32_t my_s = buf_ld32(ssr, one_slot && tid < cap ? tid * 4 : kOob);
    if constexpr (CAND) {
        // the slices' candidates, slice after slice (so in ascending chunk order)
        int off = 0;
        for (int c = 0; c < cslices; ++c) {
            const size_t base = (static_cast<size_t>(bh) * cslices + c) * k;
            const int cnt = cand_count[static_cast<size_t>(bh) * cslices + c];
            for (int i = tid; i < cnt; i += nt) {
                const uint32_t key = cand_key[base + i];
                keys[off + i] = key;
                s_ci[off + i] = cand_idx[base + i];
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
            off += cnt;
        }
        nkeys = off;
    } else {
        bool from_global = true;
        if constexpr (GP > 0) {
            // the group score computed here, straight into LDS
            group_score_lds<GP>(U, stats, cand, mask_words, S2, dyn, s_w, G, n, tiles, bh, kmn, kmx);
            from_global = false;
        }
        if (from_global) {
        if (use_lds) {
            // 16-byte buffer loads, four per thread in flight (16384 keys per
            // batch); offsets past the row read zeros and are not stored
            const int nv = (n & 3) == 0 && (reinterpret_cast<uintptr_t>(krow) & 15) == 0 ? n / 4 : 0;
            const Rsrc kr = make_rsrc(krow, static_cast<uint32_t>(n) * 4);
            for (int v0 = 0; v0 < nv; v0 += 4 * nt) {
                u32x4 t[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int v = v0 + tid + u * nt;
                    t[u] = buf_ld128(kr, v < nv ? v * 16 : kOob);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int v = v0 + tid + u * nt;
                    if (v < nv) reinterpret_cast<u32x4 *>(dyn)[v] = t[u];
                }
            }
            for (int j = 4 * nv + tid; j < n; j += nt) dyn[j] = krow[j];
        }
        for (int i = tid; i < slices; i += nt) {
            const uint2 b2 = kbounds[static_cast<size_t>(bh) * slices + i];
            kmn = min(kmn, b2.x);
            kmx = max(kmx, b2.y);
        }
        }
    }
    if constexpr (KPT > 0)  // the register form reads kcap keys: zeros past the row (or the candidates)
        for (int j = nkeys + tid; j < kcap; j += nt) dyn[j] = 0u;
    for (int i = tid; i < 4096; i += nt) sc.hist[i] = 0;
    for (int i = tid; i < k; i += nt) s_sslot[i] = -1;
    block_minmax(kmn, kmx, sc);  // its barriers also publish the keys
    if (k <= 0 || kmn > kmx) {  // nothing to select: the step still counts
        if (tid == 0) {
            miss_count[bh] = 0;
            if (bh == 0) atomicAdd(&counters[2], 1ull);
        }
        return;
    }
    // the selection stays in LDS until the last phase: on this chip a wait
    // for a load also waits for every earlier store, so the kernel's global
    // stores all come after its last global load
    int32_t *srow = sel + static_cast<size_t>(bh) * k;
    if constexpr (KPT > 0) radix_topk_regs<KPT, !CAND>(dyn, nkeys, k, kmn, kmx, s_sel, sc);
    else if (lds_keys) radix_topk(dyn, nkeys, k, kmn, kmx, nullptr, s_sel, sc);
    else radix_topk(krow, nkeys, k, kmn, kmx, nullptr, s_sel, sc);
    __syncthreads();
    if constexpr (CAND) {  // candidate positions to chunks (still ascending)
        for (int i = tid; i < k; i += nt) s_sel[i] = s_ci[s_sel[i]];
        __syncthreads();
    }

    // hits, and the age (stamp distance, >= 1) of every resident chunk that
    // is not selected again
    int32_t *gc = slot_chunk + static_cast<size_t>(bh) * cap;
    uint32_t *gs = slot_stamp + static_cast<size_t>(bh) * cap;
    // slot sl's chunk before this step's update (sl == tid when one_slot)
    auto chunk_of = [&](int sl) { return one_slot ? my_c : gc[sl]; };
    int nres = 0, nhit = 0;
    uint32_t amn = 0xffffffffu, amx = 0u;
    for (int sl = tid; sl < cap; sl += nt) {
        const int32_t c = chunk_of(sl);
        uint32_t age = 0;
        if (c >= 0) {
            ++nres;
            int lo = 0, hi = k;
            if constexpr (KPT > 0 && !CAND) {
                // the selection marked its chunks' keys with position + 1
                const uint32_t mk = c < n ? dyn[c] : 0u;
                lo = mk >= 1u && mk <= static_cast<uint32_t>(k) ? static_cast<int>(mk) - 1 : k;
            } else {
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (s_sel[mid] < c) lo = mid + 1; else hi = mid;
                }
            }
            if (lo < k && s_sel[lo] == c) {
                s_sslot[lo] = sl;  // a hit: its stamp is renewed in the last phase
                ++nhit;
            } else {
                age = stamp - (one_slot ? my_s : gs[sl]);
                amn = min(amn, age);
                amx = max(amx, age);
            }
        }
        s_age[sl] = age;
    }
    int tres, thit;
    block_scan2(nres, nhit, sc, &tres, &thit);  // its barriers also publish s_age and s_sslot
    const int nmiss = k - thit, nempty = cap - tres, ncand = tres - thit;
    const int evict = max(0, nmiss - nempty);
    // the evicted slots: ages above cut1, and of those equal to cut1 the
    // need_eq with the highest chunk index (keys chunk + 1 >= cut2)
    uint32_t cut1 = 1u, cut2 = 0u;
    bool tie_split = false;
    if (evict == 0) {
        cut1 = 0xffffffffu;  // no age exceeds it; equal ages not taken (cut2 above every key)
        cut2 = 0xffffffffu;
        tie_split = true;
    } else if (evict < ncand) {  // only with more slots than k
        block_minmax(amn, amx, sc);
        const RadixCut c1 = radix_cut(s_age, cap, evict, amn, amx, sc);
        cut1 = c1.thr;
        int eq = 0, dummy = 0, teq, td;
        for (int sl = tid; sl < cap; sl += nt) eq += s_age[sl] == cut1 ? 1 : 0;
        block_scan2(eq, dummy, sc, &teq, &td);
        if (c1.need_eq < teq) {
            // equal ages: keys chunk + 1 in s_free, the need_eq largest go
            for (int sl = tid; sl < cap; sl += nt)
                s_free[sl] = s_age[sl] == cut1 ? chunk_of(sl) + 1 : 0;
            __syncthreads();
            cut2 = radix_cut(reinterpret_cast<const uint32_t *>(s_free), cap, c1.need_eq, 1u,
                             static_cast<uint32_t>(n), sc).thr;
            tie_split = true;
        }
        // else every slot of age cut1 goes: cut1 alone decides
    }
    // else every resident unselected chunk goes (cut1 = 1, no tie split)
    __syncthreads();

    // ascending ranks of the misses (over selection positions) and of the
    // free slots (over slot indices), one scan for both
    int rmiss = 0, rfree = 0;
    const int span = max(k, cap);
    for (int i0 = 0; i0 < span; i0 += nt) {
        const int i = i0 + tid;
        const int miss = (i < k && s_sslot[i] < 0) ? 1 : 0;
        bool fr = false;
        if (i < cap) {
            const uint32_t a = s_age[i];
            const int32_t ci = chunk_of(i);  // i == tid when one_slot (i < cap <= nt)
            const bool empty = ci < 0;
            const bool gone = a != 0 && (a > cut1 || (a == cut1 && (!tie_split ||
                                                      static_cast<uint32_t>(ci + 1) >= cut2)));
            fr = empty || gone;
        }
        int mi = miss, fi = fr ? 1 : 0, tm, tf;
        block_scan2(mi, fi, sc, &tm, &tf);
        if (miss) s_rank[rmiss + mi - 1] = i;
        if (i < cap) s_free[i] = fr ? rfree + fi - 1 : -1;
        rmiss += tm;
        rfree += tf;
    }
    __syncthreads();
    // the m-th missing chunk goes to the m-th free slot; hits (resident, age
    // 0) keep theirs with a new stamp
    int2 *ml = misses + static_cast<size_t>(bh) * k;
    for (int sl = tid; sl < cap; sl += nt) {
        const int r = s_free[sl];
        if (r >= 0 && r < nmiss) {  // free slots number at least the misses
            const int i = s_rank[r];
            const int32_t chunk = s_sel[i];
            gc[sl] = chunk;
            gs[sl] = stamp;
            s_sslot[i] = sl;
            ml[r] = make_int2(chunk, sl);
        } else if (r < 0 && s_age[sl] == 0 && chunk_of(sl) >= 0) {
            gs[sl] = stamp;
        }
    }
    __syncthreads();
    for (int i = tid; i < k; i += nt) {
        srow[i] = s_sel[i];
        sel_slot[static_cast<size_t>(bh) * k + i] = s_sslot[i];
    }
    if (tid == 0) {
        miss_count[bh] = nmiss;
        atomicAdd(&counters[0], static_cast<unsigned long long>(k - nmiss));
        atomicAdd(&counters[1], static_cast<unsigned long long>(nmiss));
        if (bh == 0) atomicAdd(&counters[2], 1ull);
    }
}

// ---------------------------------------------------------------------------
// SnapKV-style selection (the SnapKV review page, 核心公式 and 池化策略), at
// chunk level against the landmarks.  The importance of a chunk is the
// attention it receives, summed over the query heads of its KV group and the
// queries of an observation window; each scoring pass covers up to kMaxGroup
// (head, window position) rows, and the group kernel leaves their mean
// softmax in S2.
//   snap_accum: acc (+)= rows_in_pass * S2, the pass's summed attention;
//   snap_pool:  pooled[j] = (1/pool) sum over |i - j| <= pool/2 of acc[i]
//               (zero padding), written to S2 for selectable chunks (0
//               elsewhere) and as selection keys with per-slice bounds,
//               exactly the group kernel's outputs, for the select kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void snap_accum_kernel(const float *__restrict__ S2, float *__restrict__ acc,
                                                         size_t count, float weight, int first) {
    for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < count; i += gridDim.x * 256ull)
        acc[i] = (first ? 0.f : acc[i]) + weight * S2[i];
}

__global__ __launch_bounds__(256) void snap_pool_kernel(const float *__restrict__ acc,
                                                        const uint32_t *__restrict__ cand, int mask_words,
                                                        float *__restrict__ S2, uint32_t *__restrict__ keys,
                                                        uint2 *__restrict__ kbounds, int n, int pool, int slices) {
    __shared__ uint32_t s_red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sl = blockIdx.x, bh = blockIdx.y;
    const int j0 = sl * kGroupSlice, half = pool / 2;
    const float *a = acc + static_cast<size_t>(bh) * n;
    const uint32_t *cm = cand + static_cast<size_t>(bh) * mask_words;
    const float inv = 1.f / static_cast<float>(pool);
    uint32_t kmn = 0xffffffffu, kmx = 0u;
    for (int u = 0; u < kGroupSlice / 256; ++u) {
        const int j = j0 + tid + 256 * u;
        if (j >= n) break;
        float sum = 0.f;
        for (int i = max(0, j - half); i <= min(n - 1, j + half); ++i) sum += a[i];
        const float pooled = sum * inv;
        const bool valid = mask_bit(cm, j);
        S2[static_cast<size_t>(bh) * n + j] = valid ? pooled : 0.f;
        const uint32_t key = float_key(pooled);
        keys[static_cast<size_t>(bh) * n + j] = valid ? key : 0u;
        if (valid) { kmn = min(kmn, key); kmx = max(kmx, key); }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kmn = min(kmn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmn), off, 64)));
        kmx = max(kmx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmx), off, 64)));
    }
    if (lane == 0) { s_red[0][wave] = kmn; s_red[1][wave] = kmx; }
    __syncthreads();
    if (tid == 0) {
        uint32_t lo = s_red[0][0], hi = s_red[1][0];
        for (int w = 1; w < 4; ++w) { lo = min(lo, s_red[0][w]); hi = max(hi, s_red[1][w]); }
        kbounds[static_cast<size_t>(bh) * slices + sl] = make_uint2(lo, hi);
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static hipError_t allow_lds(const void *fn, size_t bytes) {
    if (bytes <= 48 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

static int score_mode(int G) { return G <= 4 ? 0 : (G % 4 == 0 ? 1 : 2); }

hipError_t launch_score(const Dims &dm, const void *q, const void *landmarks, const uint32_t *cand, float *P,
                        float2 *stats, int score_wgs, QRows qr, hipStream_t st) {
    const int Gv = dm.G * qr.wp;  // scored rows per KV head
    if (Gv > kMaxGroup || qr.wp < 1 || qr.o_base + qr.wp > qr.w_obs) return hipErrorInvalidValue;
    if (dm.bf16) {
        const uint16_t *qq = static_cast<const uint16_t *>(q), *LL = static_cast<const uint16_t *>(landmarks);
        const int rows = dm.b * dm.hkv, total = rows * dm.wtiles;
        // default: two tiles per wave (measured best on MI355X at 128K)
        const int want = score_wgs > 0 ? score_wgs : (total + 7) / 8;
        const int wgs = std::max(1, std::min(want, (total + 3) / 4));
        const int tpw = (total + 4 * wgs - 1) / (4 * wgs);
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(wgs), dim3(256), 0, st, qq, LL, cand, dm.mask_words, P, stats, dm.hkv,
                               dm.G, qr.w_obs, qr.o_base, qr.wp, dm.n, dm.wtiles, rows, tpw, dm.scale);
        };
        const int m = score_mode(Gv);
        if (dm.d == 128) {
            if (m == 0) go(score_mfma_kernel<128, 0>);
            else if (m == 1) go(score_mfma_kernel<128, 1>);
            else go(score_mfma_kernel<128, 2>);
        } else {
            if (m == 0) go(score_mfma_kernel<64, 0>);
            else if (m == 1) go(score_mfma_kernel<64, 1>);
            else go(score_mfma_kernel<64, 2>);
        }
    } else {
        dim3 grid(dm.score_tiles, dm.b * dm.hkv);
        if (dm.d == 128)
            hipLaunchKernelGGL((score_generic_kernel<float, 128>), grid, dim3(256), 0, st,
                               static_cast<const float *>(q), static_cast<const float *>(landmarks), cand,
                               dm.mask_words, P, stats, dm.hkv, dm.G, qr.w_obs, qr.o_base, qr.wp, dm.n, dm.wtiles,
                               dm.scale);
        else
            hipLaunchKernelGGL((score_generic_kernel<float, 64>), grid, dim3(256), 0, st,
                               static_cast<const float *>(q), static_cast<const float *>(landmarks), cand,
                               dm.mask_words, P, stats, dm.hkv, dm.G, qr.w_obs, qr.o_base, qr.wp, dm.n, dm.wtiles,
                               dm.scale);
    }
    return hipGetLastError();
}

int select_kpt_of(const Dims &dm) {
    if (const char *e = std::getenv("SKV_SELECT_REGS"))
        if (std::atoi(e) == 0) return 0;
    return select_kpt(dm.n);
}

size_t select_dynamic_lds(const Dims &dm, bool keys_in_lds) {
    const int kpt = keys_in_lds ? select_kpt_of(dm) : 0;
    const size_t kent = kpt > 0 ? static_cast<size_t>(kSelectThreads) * kpt : static_cast<size_t>(dm.n);
    return (3ull * dm.k + 2ull * dm.cap) * sizeof(int32_t) + (keys_in_lds ? kent * sizeof(uint32_t) : 0);
}

int topk_slice(const Dims &dm) { return dm.tslice > 0 ? dm.tslice : dm.k <= 1024 ? 4096 : 16384; }

int topk_slices(const Dims &dm) { return (dm.n + topk_slice(dm) - 1) / topk_slice(dm); }

size_t group_topk_lds(const Dims &dm) {
    const size_t SL = topk_slice(dm);
    return SL * sizeof(uint32_t) + static_cast<size_t>(dm.k) * sizeof(int32_t) + SL / 64 * dm.GP * sizeof(float);
}

static int select_cand_kpt(const Dims &dm) {
    if (const char *e = std::getenv("SKV_SELECT_REGS"))
        if (std::atoi(e) == 0) return 0;
    return select_kpt(topk_slices(dm) * dm.k);
}

size_t select_cand_lds(const Dims &dm) {
    const int kpt = select_cand_kpt(dm);
    const size_t cs = static_cast<size_t>(topk_slices(dm)) * dm.k;
    const size_t kent = kpt > 0 ? static_cast<size_t>(kSelectThreads) * kpt : cs;
    return (kent + cs + 3ull * dm.k + 2ull * dm.cap) * sizeof(int32_t);
}

size_t select_static_lds() { return sizeof(SelectScratch); }

int group_slices(const Dims &dm) { return (dm.n + kGroupSlice - 1) / kGroupSlice; }

hipError_t launch_group(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                        uint32_t *keys, uint2 *kbounds, hipStream_t st) {
    const int slices = group_slices(dm);
    dim3 grid(slices, dm.b * dm.hkv);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, P, stats, cand, dm.mask_words, S2, keys, kbounds, dm.G, dm.n,
                           dm.wtiles, slices);
    };
    switch (dm.GP) {
        case 4: go(group_kernel<4>); break;
        case 8: go(group_kernel<8>); break;
        default: go(group_kernel<16>); break;
    }
    return hipGetLastError();
}

hipError_t launch_select(const Dims &dm, const uint32_t *keys, const uint2 *kbounds, int32_t *sel,
                         int32_t *sel_slot, int32_t *slot_chunk, uint32_t *slot_stamp, uint32_t stamp,
                         int2 *misses, int32_t *miss_count, unsigned long long *counters, int keys_in_lds,
                         hipStream_t st) {
    if (dm.k > 0 && dm.cap < dm.k) return hipErrorInvalidValue;
    const int kpt = keys_in_lds ? select_kpt_of(dm) : 0;
    const size_t lds = select_dynamic_lds(dm, keys_in_lds != 0);
    auto go = [&](auto kern) {
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(dm.b * dm.hkv), dim3(kSelectThreads), lds, st, nullptr, nullptr, nullptr, 0,
                           nullptr, 0, 0, keys, kbounds, group_slices(dm), nullptr, nullptr, nullptr, 0, sel,
                           sel_slot, slot_chunk, slot_stamp, stamp, misses, miss_count, counters, keys_in_lds, dm.n,
                           dm.k, dm.cap);
        return hipGetLastError();
    };
    switch (kpt) {
        case 8: return go(select_kernel<false, 0, 8>);
        case 16: return go(select_kernel<false, 0, 16>);
        case 32: return go(select_kernel<false, 0, 32>);
        default: return go(select_kernel<false, 0, 0>);
    }
}

size_t select_fused_lds(const Dims &dm) {
    return select_dynamic_lds(dm, true) + static_cast<size_t>(dm.wtiles) * dm.GP * sizeof(float);
}

hipError_t launch_select_fused(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                               int32_t *sel, int32_t *sel_slot, int32_t *slot_chunk, uint32_t *slot_stamp,
                               uint32_t stamp, int2 *misses, int32_t *miss_count, unsigned long long *counters,
                               hipStream_t st) {
    if (dm.k > 0 && dm.cap < dm.k) return hipErrorInvalidValue;
    const size_t lds = select_fused_lds(dm);
    auto go = [&](auto kern) {
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(dm.b * dm.hkv), dim3(kSelectThreads), lds, st, P, stats, cand, dm.mask_words,
                           S2, dm.G, dm.wtiles, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, sel, sel_slot,
                           slot_chunk, slot_stamp, stamp, misses, miss_count, counters, 1, dm.n, dm.k, dm.cap);
        return hipGetLastError();
    };
    auto by_kpt = [&](auto gp) {
        constexpr int G4 = decltype(gp)::value;
        switch (select_kpt_of(dm)) {
            case 8: return go(select_kernel<false, G4, 8>);
            case 16: return go(select_kernel<false, G4, 16>);
            case 32: return go(select_kernel<false, G4, 32>);
            default: return go(select_kernel<false, G4, 0>);
        }
    };
    switch (dm.GP) {
        case 4: return by_kpt(std::integral_constant<int, 4>{});
        case 8: return by_kpt(std::integral_constant<int, 8>{});
        default: return by_kpt(std::integral_constant<int, 16>{});
    }
}

hipError_t launch_group_topk(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                             uint32_t *cand_key, int32_t *cand_idx, int32_t *cand_count, hipStream_t st) {
    if (dm.k <= 0) return hipSuccess;
    const int SL = topk_slice(dm), slices = topk_slices(dm);
    const size_t lds = group_topk_lds(dm);
    auto go = [&](auto kern) {
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(slices, dm.b * dm.hkv), dim3(kSelectThreads), lds, st, P, stats, cand,
                           dm.mask_words, S2, cand_key, cand_idx, cand_count, dm.G, dm.n, dm.wtiles, SL, slices,
                           dm.k);
        return hipGetLastError();
    };
    // the register form when a slice is exactly 1024 x KPT keys
    int kpt = select_kpt(SL);
    if (kpt == 0 || SL != kSelectThreads * kpt) kpt = 0;
    if (const char *e = std::getenv("SKV_SELECT_REGS"))
        if (std::atoi(e) == 0) kpt = 0;
    auto by_kpt = [&](auto gp) {
        constexpr int G4 = decltype(gp)::value;
        switch (kpt) {
            case 4: return go(group_topk_kernel<G4, 4>);
            case 8: return go(group_topk_kernel<G4, 8>);
            case 16: return go(group_topk_kernel<G4, 16>);
            default: return go(group_topk_kernel<G4, 0>);
        }
    };
    switch (dm.GP) {
        case 4: return by_kpt(std::integral_constant<int, 4>{});
        case 8: return by_kpt(std::integral_constant<int, 8>{});
        default: return by_kpt(std::integral_constant<int, 16>{});
    }
}

hipError_t launch_select_cand(const Dims &dm, const uint32_t *cand_key, const int32_t *cand_idx,
                              const int32_t *cand_count, int32_t *sel, int32_t *sel_slot, int32_t *slot_chunk,
                              uint32_t *slot_stamp, uint32_t stamp, int2 *misses, int32_t *miss_count,
                              unsigned long long *counters, hipStream_t st) {
    if (dm.k > 0 && dm.cap < dm.k) return hipErrorInvalidValue;
    const size_t lds = select_cand_lds(dm);
    auto kern = select_kernel<true, 0, 0>;
    switch (select_cand_kpt(dm)) {
        case 4: kern = select_kernel<true, 0, 4>; break;
        case 8: kern = select_kernel<true, 0, 8>; break;
        case 16: kern = select_kernel<true, 0, 16>; break;
        case 32: kern = select_kernel<true, 0, 32>; break;
        default: break;
    }
    hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(dm.b * dm.hkv), dim3(kSelectThreads), lds, st, nullptr, nullptr, nullptr, 0,
                       nullptr, 0, 0, nullptr, nullptr, 0, cand_key,
                       cand_idx, cand_count, topk_slices(dm), sel, sel_slot, slot_chunk, slot_stamp, stamp, misses,
                       miss_count, counters, 0, dm.n, dm.k, dm.cap);
    return hipGetLastError();
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

hipError_t launch_snap_accum(const Dims &dm, const float *S2, float *acc, float weight, int first, hipStream_t st) {
    const size_t count = static_cast<size_t>(dm.b) * dm.hkv * dm.n;
    const int grid = static_cast<int>(std::min<size_t>((count + 255) / 256, 4096));
    hipLaunchKernelGGL(snap_accum_kernel, dim3(grid), dim3(256), 0, st, S2, acc, count, weight, first);
    return hipGetLastError();
}

hipError_t launch_snap_pool(const Dims &dm, const float *acc, const uint32_t *cand, float *S2, uint32_t *keys,
                            uint2 *kbounds, int pool, hipStream_t st) {
    const int slices = group_slices(dm);
    hipLaunchKernelGGL(snap_pool_kernel, dim3(slices, dm.b * dm.hkv), dim3(256), 0, st, acc, cand, dm.mask_words,
                       S2, keys, kbounds, dm.n, pool, slices);
    return hipGetLastError();
}

}  // namespace skv
