// Attention half of the decode step (review page, section 三, Algorithm 2
// steps 3-4):
//   fetch     V of the chunks that missed the resident cache, read by the GPU
//             straight from pinned host memory;
//   qk_static logits of the full-rank outlier and local-window keys (MFMA);
//   qk_sparse logits of the rebuilt keys: Gather(A, I) . B on MFMA, RoPE at
//             the chunks' original positions in registers; the rebuilt keys
//             are never written to memory;
//   pv        softmax-weighted values per key split; the last split of each
//             (sequence, KV head) merges the partials into the output.
#include <algorithm>

#include "skv_device.h"

namespace skv {

// ---------------------------------------------------------------------------
// Host-V fetch.  The select kernel leaves, per (sequence, KV head) row, a
// compacted list of the chunks that missed the resident cache and the slots
// freed for them.  Each workgroup first forms the prefix sums of the per-row
// miss counts in LDS; its waves then walk the global miss index (rows one
// after another), find each miss's row by binary search, and copy the missing
// chunk (c * d elements, contiguous on both sides) from pinned host memory
// into its cache slot, every load of the chunk in flight before the stores.
// A chunk stored in a coded form (its code word, see prefill.hip) is read in
// that form and decoded in registers: the 12-bit form's exponents are offsets
// from the chunk's base; the class form's are 2-bit classes below the chunk's
// top plus, for class 3, 3-bit codes from a side stream that the wave stages
// in LDS and each lane reads at its own bit position (a wave prefix sum of
// the lanes' class-3 counts); escapes patch their values' exponents.  Only
// real misses are visited, so the PCIe reads are issued back to back.
// ---------------------------------------------------------------------------
template <int VPL>  // 16-byte vectors per lane and chunk (0: any, looped)
__global__ __launch_bounds__(256) void fetch_kernel(const u32x4 *__restrict__ v_host, u32x4 *__restrict__ vc,
                                                    const int2 *__restrict__ misses,
                                                    const int32_t *__restrict__ miss_count,
                                                    const uint32_t *__restrict__ vcode,
                                                    unsigned long long *__restrict__ counters, int rows, int k,
                                                    int cap, int n, int chunk_vec) {
    extern __shared__ int pre[];  // rows + 1 prefix sums
    __shared__ int wsum[4];
    // per wave: a class-form chunk's side stream (up to 3N/8 bytes, with slack)
    // (rows of whole 16-byte words: 3N/8 bytes is a multiple of 16)
    constexpr int SW = VPL > 0 ? (3 * 512 * VPL / 8) / 4 + 8 : 4;
    __shared__ __align__(16) uint32_t s_side[4][SW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int base = 0; base < rows; base += 256) {
        const int r = base + tid;
        int v = r < rows ? miss_count[r] : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(v, off, 64);
            if (lane >= off) v += t;
        }
        if (lane == 63) wsum[wave] = v;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        if (r < rows) pre[r + 1] = before + v;
        carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (tid == 0) pre[0] = 0;
    __syncthreads();
    const int total = pre[rows];
    const int gw = blockIdx.x * 4 + wave, nw = gridDim.x * 4;
    // the miss with global index g: its row (pre[r] <= g < pre[r + 1]) and
    // its (chunk, slot) entry
    auto locate = [&](int g, int &row) {
        int lo = 0, hi = rows - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= g) lo = mid; else hi = mid - 1;
        }
        row = lo;
        return misses[static_cast<size_t>(lo) * k + (g - pre[lo])];
    };
    unsigned long long wire = 0;  // bytes this wave read over PCIe
    int g = gw, row = 0;
    int2 e = g < total ? locate(g, row) : make_int2(0, 0);
    uint32_t code = g < total && vcode ? vcode[static_cast<size_t>(row) * n + e.x] : 0u;
    for (; g < total; g += nw) {
        const u32x4 *src = v_host + (static_cast<size_t>(row) * n + e.x) * chunk_vec;
        u32x4 *dst = vc + (static_cast<size_t>(row) * cap + e.y) * chunk_vec;
        if constexpr (VPL > 0) {
            constexpr int Q = 8 * VPL;  // values per lane
            const int N = 64 * Q;
            if ((code & 0xC0000000u) == 0xC0000000u) {  // wave-uniform: the class form (see prefill.hip)
                const int top = static_cast<int>(code & 0xffu), nesc = static_cast<int>((code >> 8) & 0xffu);
                const int S = static_cast<int>((code >> 20) & 0xffu) * 4;
                const uint8_t *sb = reinterpret_cast<const uint8_t *>(src);
                uint32_t bw[Q / 4], cw[(Q + 15) / 16];
                if constexpr (Q == 8) {
                    const u32x2 b2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sb) + lane);
                    bw[0] = b2[0]; bw[1] = b2[1];
                    cw[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(sb + N) + lane);
                } else if constexpr (Q == 16) {
                    const u32x4 b4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb) + lane);
                    bw[0] = b4[0]; bw[1] = b4[1]; bw[2] = b4[2]; bw[3] = b4[3];
                    cw[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + N) + lane);
                } else {
                    const u32x4 b4a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb) + 2 * lane);
                    const u32x4 b4b = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb) + 2 * lane + 1);
                    bw[0] = b4a[0]; bw[1] = b4a[1]; bw[2] = b4a[2]; bw[3] = b4a[3];
                    bw[4] = b4b[0]; bw[5] = b4b[1]; bw[6] = b4b[2]; bw[7] = b4b[3];
                    const u32x2 c2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sb + N) + lane);
                    cw[0] = c2[0]; cw[1] = c2[1];
                }
                // the side stream, 16 bytes a lane, and the escapes
                const u32x4 sv = 16 * lane < S ? __builtin_nontemporal_load(
                                                     reinterpret_cast<const u32x4 *>(sb + N + N / 4) + lane)
                                               : u32x4{0u, 0u, 0u, 0u};
                const uint32_t esc = lane < nesc
                    ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + N + N / 4 + S) + lane) : 0u;
                // the next miss is located while this chunk's host reads are in flight
                int row_n = row;
                const int2 e_n = g + nw < total ? locate(g + nw, row_n) : e;
                const uint32_t code_n = g + nw < total && vcode ? vcode[static_cast<size_t>(row_n) * n + e_n.x] : 0u;
                uint32_t *side = s_side[wave];
                if (16 * lane < S) reinterpret_cast<u32x4 *>(side)[lane] = sv;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                // the stream holds the class-3 codes in value order, so this
                // lane's start is the class-3 count of the lanes before it
                int n3l = 0;
#pragma unroll
                for (int h = 0; h < (Q + 15) / 16; ++h) n3l += __popc(cw[h] & (cw[h] >> 1) & 0x55555555u);
                int pos = 3 * (wave_incl_scan(n3l) - n3l);
                uint32_t x[Q];
#pragma unroll
                for (int h = 0; h < (Q + 15) / 16; ++h) {
                    // a 64-bit window of the stream at pos (a group of 16
                    // values takes at most 48 bits)
                    const int w0 = pos >> 5, sh = pos & 31;
                    uint64_t win = (static_cast<uint64_t>(side[w0]) | (static_cast<uint64_t>(side[w0 + 1]) << 32)) >> sh;
                    if (sh) win |= static_cast<uint64_t>(side[w0 + 2]) << (64 - sh);
                    const uint32_t c = cw[h];
                    constexpr int GQ = Q < 16 ? Q : 16;
#pragma unroll
                    for (int q = 0; q < GQ; ++q) {
                        const int cl = static_cast<int>((c >> (2 * q)) & 3u);
                        int ex = top - cl;
                        if (cl == 3) {
                            const int xc = static_cast<int>(win & 7u);
                            win >>= 3;
                            pos += 3;
                            ex = xc == 0 ? top + 1 : top - 2 - xc;  // 7: an escape, patched below
                        }
                        const int qq = 16 * h + q;
                        const uint32_t byte = (bw[qq >> 2] >> (8 * (qq & 3))) & 0xffu;
                        x[qq] = ((byte & 0x80u) << 8) | ((static_cast<uint32_t>(ex) & 0xffu) << 7) | (byte & 0x7fu);
                    }
                }
                // escapes: the exponent itself, for the lane owning the value
                for (int j = 0; j < nesc; ++j) {
                    const uint32_t ej = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(esc), j));
                    const int idx = static_cast<int>(ej >> 8);
                    if (idx / Q == lane) {
#pragma unroll
                        for (int q = 0; q < Q; ++q)
                            if (q == idx % Q) x[q] = (x[q] & 0x807fu) | ((ej & 0xffu) << 7);
                    }
                }
#pragma unroll
                for (int u = 0; u < VPL; ++u)
                    dst[lane * VPL + u] = u32x4{x[8 * u] | (x[8 * u + 1] << 16), x[8 * u + 2] | (x[8 * u + 3] << 16),
                                                x[8 * u + 4] | (x[8 * u + 5] << 16), x[8 * u + 6] | (x[8 * u + 7] << 16)};
                wire += static_cast<unsigned long long>(N + N / 4 + S + 4 * nesc);
                row = row_n;
                e = e_n;
                code = code_n;
            } else if (code & 0x80000000u) {  // wave-uniform: the 12-bit form (see prefill.hip)
                const int base = static_cast<int>(code & 0xffu), nesc = static_cast<int>((code >> 16) & 0xffu);
                const uint8_t *sb = reinterpret_cast<const uint8_t *>(src);
                uint32_t bw[Q / 4], nwd[Q / 8];
                if constexpr (Q == 8) {
                    const u32x2 b2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sb) + lane);
                    bw[0] = b2[0]; bw[1] = b2[1];
                    nwd[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + N) + lane);
                } else if constexpr (Q == 16) {
                    const u32x4 b4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb) + lane);
                    bw[0] = b4[0]; bw[1] = b4[1]; bw[2] = b4[2]; bw[3] = b4[3];
                    const u32x2 n2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(sb + N) + lane);
                    nwd[0] = n2[0]; nwd[1] = n2[1];
                } else {
                    const u32x4 b4a = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb) + 2 * lane);
                    const u32x4 b4b = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb) + 2 * lane + 1);
                    bw[0] = b4a[0]; bw[1] = b4a[1]; bw[2] = b4a[2]; bw[3] = b4a[3];
                    bw[4] = b4b[0]; bw[5] = b4b[1]; bw[6] = b4b[2]; bw[7] = b4b[3];
                    const u32x4 n4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(sb + N) + lane);
                    nwd[0] = n4[0]; nwd[1] = n4[1]; nwd[2] = n4[2]; nwd[3] = n4[3];
                }
                const uint32_t esc = lane < nesc
                    ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(sb + 3 * N / 2) + lane) : 0u;
                // the next miss is located while this chunk's host reads are in flight
                int row_n = row;
                const int2 e_n = g + nw < total ? locate(g + nw, row_n) : e;
                const uint32_t code_n = g + nw < total && vcode ? vcode[static_cast<size_t>(row_n) * n + e_n.x] : 0u;
                uint32_t x[Q];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const uint32_t byte = (bw[q >> 2] >> (8 * (q & 3))) & 0xffu;
                    const uint32_t ex = static_cast<uint32_t>(base) + ((nwd[q >> 3] >> (4 * (q & 7))) & 0xfu);
                    x[q] = ((byte & 0x80u) << 8) | ((ex & 0xffu) << 7) | (byte & 0x7fu);
                }
                // escapes: the exponent itself, for the lane owning the value
                for (int j = 0; j < nesc; ++j) {
                    const uint32_t ej = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(esc), j));
                    const int idx = static_cast<int>(ej >> 8);
                    if (idx / Q == lane) {
#pragma unroll
                        for (int q = 0; q < Q; ++q)
                            if (q == idx % Q) x[q] = (x[q] & 0x807fu) | ((ej & 0xffu) << 7);
                    }
                }
#pragma unroll
                for (int u = 0; u < VPL; ++u)
                    dst[lane * VPL + u] = u32x4{x[8 * u] | (x[8 * u + 1] << 16), x[8 * u + 2] | (x[8 * u + 3] << 16),
                                                x[8 * u + 4] | (x[8 * u + 5] << 16), x[8 * u + 6] | (x[8 * u + 7] << 16)};
                wire += static_cast<unsigned long long>(3 * N / 2 + 4 * nesc);
                row = row_n;
                e = e_n;
                code = code_n;
            } else {
                u32x4 t[VPL];
#pragma unroll
                for (int u = 0; u < VPL; ++u) t[u] = __builtin_nontemporal_load(src + u * 64 + lane);
                // the next miss is located while this chunk's host reads are in flight
                int row_n = row;
                const int2 e_n = g + nw < total ? locate(g + nw, row_n) : e;
                const uint32_t code_n = g + nw < total && vcode ? vcode[static_cast<size_t>(row_n) * n + e_n.x] : 0u;
#pragma unroll
                for (int u = 0; u < VPL; ++u) dst[u * 64 + lane] = t[u];
                wire += static_cast<unsigned long long>(chunk_vec) * 16;
                row = row_n;
                e = e_n;
                code = code_n;
            }
        } else {
            for (int i0 = 0; i0 < chunk_vec; i0 += 256) {
                u32x4 t[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + u * 64 + lane;
                    if (i < chunk_vec) t[u] = __builtin_nontemporal_load(src + i);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + u * 64 + lane;
                    if (i < chunk_vec) dst[i] = t[u];
                }
            }
            wire += static_cast<unsigned long long>(chunk_vec) * 16;
            if (g + nw < total) e = locate(g + nw, row);
        }
    }
    if (counters && lane == 0 && wire) atomicAdd(&counters[3], wire);
}

// ---------------------------------------------------------------------------
// Generic QK (any storage type): 64 keys per workgroup.  Keys of the tile are
// staged in LDS in single precision; rebuilt keys are computed there
// (r multiply-adds each) and rotated in place.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void qk_generic_kernel(const T *__restrict__ q, const T *__restrict__ k_out,
                                                         const T *__restrict__ k_loc, const T *__restrict__ A,
                                                         const T *__restrict__ Bt,
                                                         const int32_t *__restrict__ sel,
                                                         const double *__restrict__ theta,
                                                         float *__restrict__ logits, int hkv, int G, int s, int c,
                                                         int r, int k, int OC, int KC, int w, int wcap, int NK, int t_out,
                                                         int t_sp, float scale) {
    __shared__ float Ks[kQkTile][D + 1];
    __shared__ float qs[kMaxGroup][D];
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    int tile = blockIdx.x, seg, key0, cnt, gbase;
    if (tile < t_out) {
        seg = 0; key0 = tile * kQkTile; cnt = min(kQkTile, OC - key0); gbase = key0;
    } else if (tile < t_out + t_sp) {
        seg = 1; key0 = (tile - t_out) * kQkTile; cnt = min(kQkTile, KC - key0); gbase = OC + key0;
    } else {
        seg = 2; key0 = (tile - t_out - t_sp) * kQkTile; cnt = min(kQkTile, w - key0); gbase = OC + KC + key0;
    }
    for (int i = threadIdx.x; i < G * D; i += 256)
        qs[i / D][i % D] = Elem<T>::ld(q, (static_cast<size_t>(b) * hq + h * G) * D + i) * scale;
    if (seg != 1) {
        const T *src = seg == 0 ? k_out + (static_cast<size_t>(bh) * OC + key0) * D
                                : k_loc + (static_cast<size_t>(bh) * wcap + key0) * D;
        for (int idx = threadIdx.x; idx < cnt * D; idx += 256) Ks[idx / D][idx % D] = Elem<T>::ld(src, idx);
    } else {
        const T *Bh = Bt + static_cast<size_t>(bh) * D * r;
        for (int idx = threadIdx.x; idx < cnt * D; idx += 256) {
            const int rr = idx / D, i = idx % D, key = key0 + rr;
            const int pos = sel[static_cast<size_t>(bh) * k + key / c] * c + key % c;
            const T *arow = A + (static_cast<size_t>(b) * s + pos) * r;
            const T *brow = Bh + static_cast<size_t>(i) * r;
            float acc = 0.f;
            for (int e = 0; e < r; ++e) acc += Elem<T>::ld(arow, e) * Elem<T>::ld(brow, e);
            Ks[rr][i] = acc;
        }
        __syncthreads();
        constexpr int H = D / 2;
        for (int idx = threadIdx.x; idx < cnt * H; idx += 256) {
            const int rr = idx / H, i = idx % H, key = key0 + rr;
            const int pos = sel[static_cast<size_t>(bh) * k + key / c] * c + key % c;
            float sn, cs, y1, y2;
            angle_sincos(static_cast<double>(pos) * theta[i], &sn, &cs);
            rope_rotate(Ks[rr][i], Ks[rr][i + H], sn, cs, y1, y2);
            Ks[rr][i] = y1;
            Ks[rr][i + H] = y2;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < cnt * G; idx += 256) {
        const int rr = idx / G, g = idx % G;
        float dot = 0.f;
        for (int i = 0; i < D; ++i) dot += qs[g][i] * Ks[rr][i];
        logits[(static_cast<size_t>(bh) * G + g) * NK + gbase + rr] = dot;
    }
}

// ---------------------------------------------------------------------------
// Logits of the static keys (outlier chunks, then the local window), bfloat16
// on MFMA: C[key, head] = sum_i K[key, i] q[head, i] with 16 keys per
// v_mfma_f32_16x16x32_bf16 (keys as rows, the group's heads as columns).
// ---------------------------------------------------------------------------
// Workgroup `blk` of `nblk` per (sequence, KV head) row; no barrier.
template <int D>
__device__ __forceinline__ void qk_static_tile(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_out,
                                               const uint16_t *__restrict__ k_loc, float *__restrict__ logits,
                                               int hkv, int G, int OC, int KC, int w, int wcap, int NK, float scale,
                                               int blk, int nblk) {
    constexpr int KS = D / 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = lane & 15, quad = lane >> 4;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    const int nstat = OC + w;
    bf16x8 qb[KS];
    {
        const uint16_t *qrow = q + (static_cast<size_t>(b) * hq + h * G + row) * D + quad * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = __builtin_bit_cast(bf16x8, row < G ? *reinterpret_cast<const u32x4 *>(qrow + ks * 32)
                                                        : u32x4{0u, 0u, 0u, 0u});
    }
    for (int kb0 = (blk * 4 + wave) * 16; kb0 < nstat; kb0 += nblk * 64) {
        const int sk = kb0 + row;
        const uint16_t *src = sk < OC ? k_out + (static_cast<size_t>(bh) * OC + sk) * D
                                      : k_loc + (static_cast<size_t>(bh) * wcap + (sk - OC)) * D;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = sk < nstat ? *reinterpret_cast<const u32x4 *>(src + ks * 32 + quad * 8)
                                       : u32x4{0u, 0u, 0u, 0u};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), qb[ks], acc, 0, 0, 0);
        }
        if (row < G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ks_ = kb0 + quad * 4 + e;
                if (ks_ < nstat) {
                    const int gkey = ks_ < OC ? ks_ : KC + ks_;
                    logits[(static_cast<size_t>(bh) * G + row) * NK + gkey] = acc[e] * scale;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Rebuilt keys on MFMA (bfloat16).  Per (sequence, KV head) the rebuild is
// K[key, :] = A[pos(key), :] . B[h] with pos(key) = sel[key / c] * c + key % c, a
// genuine rank-r x d contraction.  A workgroup takes 256 keys (4 waves x 64);
// B[h] (stored transposed, d x r) is staged once in LDS and shared by the four
// waves; each wave requests the gathered A rows of all four of its 16-key
// blocks at once and then computes the blocks in turn, transposed,
// K^T[dim, key] = sum_r Bt[dim, r] A[key, r]: the staged Bt rows are the MFMA
// A operand and the gathered A rows the B operand.  v_mfma_f32_16x16x32_bf16
// then leaves lane l with key (l & 15) of the block and dims
// 16*nb + 4*(l >> 4) + e (e < 4) of every 16-dim block nb, so the RoPE pair
// (i, i + d/2) sits in one lane and each lane rotates its own key at its own
// position.  The logits are a second contraction on MFMA: in a fixed
// permutation of the head dimension (dims 32p + 4*(l >> 4) + e and
// 32p + 16 + 4*(l >> 4) + e of dim pair p), the rotated keys, split into two
// bfloat16 terms, already sit in the B-operand layout, and the group's
// queries, permuted the same way, are the A operand (query heads as rows).
// ---------------------------------------------------------------------------
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the
// lower 32 lanes of its second, so the sum of the two results holds, in lanes
// 0-31, lo(l) + lo(l + 32) and, in lanes 32-63, hi(l - 32) + hi(l).
__device__ __forceinline__ float swap_sum32(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second: rows 0 and 2 end with lo summed over the row
// pair, rows 1 and 3 with hi summed over it.
__device__ __forceinline__ float swap_sum16(float lo, float hi) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The rebuilt, rotated keys enter the logit MFMA as two bfloat16 terms,
// hi = bf16(x) and lo = bf16(x - hi) (x - hi is exact in binary32), so
// q . x = q . hi + q . lo carries ~16 significant bits of every key instead
// of bfloat16's 8: one rounding of the keys would cost up to ~1e-2 of output
// at sharp attention, the same order as the bfloat16 error bar.
// Adjacent values are converted in pairs (one v_cvt_pk_bf16_f32 each), and
// hi goes back to binary32 by shifting its bits into place.
__device__ __forceinline__ uint32_t cvt2_bf16(float x, float y) {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2));
}
__device__ __forceinline__ void split_bf16x8(f32x4 a, f32x4 b, bf16x8 &hi, bf16x8 &lo) {
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4 h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        h[k] = cvt2_bf16(v[2 * k], v[2 * k + 1]);
        const float h0 = __uint_as_float(h[k] << 16), h1 = __uint_as_float(h[k] & 0xffff0000u);
        l[k] = cvt2_bf16(v[2 * k] - h0, v[2 * k + 1] - h1);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// logits of one 16-key block: lg += q . (hi + lo) over the NP 32-dim pairs
template <int NP>
__device__ __forceinline__ f32x4 logits_hilo(const bf16x8 *qa, const f32x4 *acc, f32x4 lg) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        bf16x8 hi, lo;
        split_bf16x8(acc[2 * p], acc[2 * p + 1], hi, lo);
        lg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[p], hi, lg, 0, 0, 0);
        lg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[p], lo, lg, 0, 0, 0);
    }
    return lg;
}

// One launch takes both key sets.  With rebuilt keys (ts > 0 workgroups per
// row, 256 keys each) every workgroup then also takes its share of the static
// keys' 16-key blocks (one block per wave at the usual sizes), so the static
// logits cost no launch of their own; without them, the tt workgroups of the
// row only compute static logits.
template <int D, int GP, int NKB>
__global__ __launch_bounds__(256) void qk_mfma_kernel(const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ A,
                                                      const uint16_t *__restrict__ Bt,
                                                      const int32_t *__restrict__ sel,
                                                      const double *__restrict__ theta_rev,
                                                      const uint16_t *__restrict__ k_out,
                                                      const uint16_t *__restrict__ k_loc,
                                                      float *__restrict__ logits, int hkv, int G, int s,
                                                      int c, int r, int r_pad, int k, int OC, int KC, int w,
                                                      int wcap, int NK, int ts, int tt, float scale) {
    if (ts == 0) {  // no rebuilt keys: static logits only, no barrier
        qk_static_tile<D>(q, k_out, k_loc, logits, hkv, G, OC, KC, w, wcap, NK, scale, blockIdx.x, tt);
        return;
    }
    static_assert(GP <= 16, "query heads are the rows of one 16-row MFMA block");
    constexpr int NB = D / 16;      // 16-dim blocks
    constexpr int HB = NB / 2;      // blocks holding the first half of the dims
    constexpr int NP = NB / 2;      // 32-dim pairs of blocks (logit MFMA steps)
    constexpr int MB = 4;           // 16-key blocks per wave
    constexpr int STG = D / 8;      // B staging vectors per thread (r_pad <= 256)
    extern __shared__ __align__(16) uint16_t dyn[];
    uint16_t *Bs = dyn;             // D x (r_pad + 8)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, quad = lane >> 4;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    const int ldb = r_pad + 8;
    const int key_base = blockIdx.x * kQkMfmaTile + wave * 64;
    const bool active = key_base < KC;  // wave-uniform

    // The A side does not depend on the staged B: the chunk of every
    // selection position this wave's 64 keys touch (at most 64, one load per lane, then
    // shuffles) and the rotation rates are requested first, and the gathered
    // A rows of all four key blocks and the queries right after B is written
    // to LDS (the staging registers are free by then), before the barrier.
    const int pos0 = key_base / c;
    const int my_chunk = sel[static_cast<size_t>(bh) * k + min(pos0 + lane, k - 1)];
    // rotation rates (turns per position) of this lane's dims 16*hb + 4*quad + e
    double thr[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int e = 0; e < 4; ++e) thr[hb][e] = theta_rev[hb * 16 + quad * 4 + e];

    {
        // stage B[h] (transposed, d x r) with every load in flight
        const uint16_t *Btb = Bt + static_cast<size_t>(bh) * D * r;
        const int vpr = r_pad / 8, total = D * vpr;
        u32x4 tmp[STG];
#pragma unroll
        for (int i = 0; i < STG; ++i) {
            const int idx = tid + 256 * i;
            const int nr = idx / vpr, kc = (idx % vpr) * 8;
            tmp[i] = (idx < total && kc < r) ? *reinterpret_cast<const u32x4 *>(Btb + static_cast<size_t>(nr) * r + kc)
                                            : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < STG; ++i) {
            const int idx = tid + 256 * i;
            if (idx < total) *reinterpret_cast<u32x4 *>(Bs + (idx / vpr) * ldb + (idx % vpr) * 8) = tmp[i];
        }
    }
    // Gathered A row of this lane's key in a 16-key block, 8 rank values per
    // 32-wide rank block, through a buffer resource over this sequence's A:
    // keys past KC and rank columns past r read zeros without a memory
    // access, so no branch surrounds a load.
    const Rsrc ar = make_rsrc(A + static_cast<size_t>(b) * s * r, static_cast<uint32_t>(s) * r * 2);
    const Rsrc lr = make_rsrc(logits + static_cast<size_t>(bh) * G * NK, static_cast<uint32_t>(G) * NK * 4);
    u32x4 aop[MB][NKB];
    int pos[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int key = key_base + mb * 16 + row;
        const bool kv = active && key < KC;
        const int kk = key < KC ? key : key_base;
        const int chunk = __shfl(my_chunk, kk / c - pos0, 64);
        pos[mb] = chunk * c + kk % c;
        const int base = (pos[mb] * r + quad * 8) * 2;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            aop[mb][kb] = buf_ld128(ar, kv && kb * 32 + quad * 8 < r ? base + kb * 64 : kOob);
    }
    // the group's queries (raw bfloat16) as the logit MFMA's A operand: lane
    // (quad, row) holds head `row` (rows past G repeat the last head; their
    // outputs are dropped) in the permuted dim order
    bf16x8 qa[NP];
    {
        const uint16_t *qrow = q + (static_cast<size_t>(b) * hq + h * G + min(row, G - 1)) * D + quad * 4;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(qrow + 32 * p);
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(qrow + 32 * p + 16);
            qa[p] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
    }

    __syncthreads();  // the only barrier

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int kb0 = key_base + mb * 16;
        if (!active || kb0 >= KC) break;  // wave-uniform
        f32x4 acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const bf16x8 bop = __builtin_bit_cast(bf16x8, aop[mb][kb]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const bf16x8 aw = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(Bs + (nb * 16 + row) * ldb + kb * 32 + quad * 8));
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bop, acc[nb], 0, 0, 0);
            }
        }

        // RoPE of this lane's key at its original position: the angle in
        // turns, pos * theta_i / (2 pi), is reduced to [-1/2, 1/2] in double
        // precision and fed to the hardware sin/cos (which take turns)
        const double posd = static_cast<double>(pos[mb]);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double turns = posd * thr[hb][e];
                const float frac = static_cast<float>(turns - rint(turns));
                const float sn = __builtin_amdgcn_sinf(frac), cs = __builtin_amdgcn_cosf(frac);
                const float x1 = acc[hb][e], x2 = acc[hb + HB][e];
                acc[hb][e] = x1 * cs - x2 * sn;
                acc[hb + HB][e] = x2 * cs + x1 * sn;
            }
        }

        // logits[head, key] = sum over dims of q . K_rot: lane (quad, row)
        // ends with heads 4*quad + e of key kb0 + row
        const f32x4 lg = logits_hilo<NP>(qa, acc, f32x4{0.f, 0.f, 0.f, 0.f});
        const int key = kb0 + row;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int g = quad * 4 + e;
            buf_st32(lg[e] * scale, lr, key < KC && g < G ? (g * NK + OC + key) * 4 : kOob);
        }
    }
    qk_static_tile<D>(q, k_out, k_loc, logits, hkv, G, OC, KC, w, wcap, NK, scale, blockIdx.x, ts);
}

// 8 stored values of one 16-byte (bfloat16) or two 16-byte (binary32) loads.
template <typename T>
__device__ __forceinline__ void unpack8(const u32x4 *raw, float *v) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(raw[0][i] << 16);
            v[2 * i + 1] = __uint_as_float(raw[0][i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = __uint_as_float(raw[0][i]); v[4 + i] = __uint_as_float(raw[1][i]); }
    }
}

// ---------------------------------------------------------------------------
// Row-of-16 reduction (DPP inside each 16-lane row): every lane of the row
// ends with the row's result.
template <typename Op> __device__ __forceinline__ float row16_reduce(float v, Op op) {
    v = op(v, dpp_mov<0xB1>(v));
    v = op(v, dpp_mov<0x4E>(v));
    v = op(v, dpp_mov<0x141>(v));
    v = op(v, dpp_mov<0x140>(v));
    return v;
}

// Two floats that hold bfloat16 values, as two bfloat16 in one dword (exact).
// (v_perm_b32: the upper two bytes of a, then those of b)
__device__ __forceinline__ uint32_t pack2_exact(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// ---------------------------------------------------------------------------
// Fused attention (bfloat16, MFMA): rebuild + RoPE + logits + softmax-weighted
// values in one launch, the logits never leaving the workgroup.  Workgroup
// `tile` of a row (the XCD-aware order below maps the launch index to (row,
// tile)) takes rebuilt keys 256*tile .. +256 when tile < ts, 64 per wave
// exactly as the QK kernel, and each wave one 16-key block of the static keys
// (outlier chunks, then the local window: block 4*tile + wave).  Per wave:
//  1. the queries, the static block's keys and its value rows are requested,
//     then the gathered A rows of the four 16-key rebuilt blocks;
//  2. per pair of rebuilt blocks: Gather(A, I) . B on MFMA (each staged B
//     operand feeds both blocks), then per block RoPE in registers and logits
//     on MFMA (keys split into bfloat16 hi + lo); as soon as a block's A rows
//     are consumed its value rows are requested;
//  3. the static block's logits on MFMA.  Every block's logits come out with
//     lane (quad, row) holding heads 4*quad + e of key `row`, so each head's
//     softmax over the wave's 80 keys is a reduction inside a 16-lane row;
//  4. sum over keys of weight x V on MFMA.  The contraction runs over keys,
//     so each block's value rows (lane = key) are first turned column-major
//     by an MFMA against a 0/1 selector -- exact, one product per output --
//     whose output layout is the B operand of the weighted sum; the weights,
//     through LDS in the same key order, are its A operand (bfloat16 hi + lo);
//  5. the four waves' partials merged into the workgroup's (m, l, acc),
//     written for the merge kernel.
// With 16 heads per KV head the heads fill every row of the logit and
// weighted-sum MFMAs, so the kernel costs about the same at GQA 4 and 16.
// Workgroups past ts (more static blocks than rebuilt-key waves) skip the
// rebuild and its barrier (a workgroup-uniform branch); every workgroup
// reaches the final barrier.
template <int D, int GP, int NKB, bool IND, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ A, const uint16_t *__restrict__ Bt,
    const int32_t *__restrict__ chunks, const int32_t *__restrict__ sel_slot, const double *__restrict__ theta_rev,
    const uint16_t *__restrict__ k_out, const uint16_t *__restrict__ v_out, const uint16_t *__restrict__ k_loc,
    const uint16_t *__restrict__ v_loc, const uint16_t *__restrict__ vc, float2 *__restrict__ part_ml,
    float *__restrict__ part_acc, int hkv, int G, int s, int c, int r, int r_pad, int k, int cap, int OC, int KC,
    int w, int wcap, int ts, int T, int rows, float scale, int cshift, int kpw) {
    static_assert(GP <= 16, "query heads are the rows of one 16-row MFMA block");
    constexpr int NB = D / 16, HB = NB / 2, NP = NB / 2, MB = 4, STG = D / 8;
    constexpr int KB = D / 32;                      // 32-column slabs of a value row
    constexpr int PW = 84;                          // LDS row of one head's 80 weights
    constexpr int RP = D + 2;                       // merge record of one head: D sums, max, sum
    constexpr int RGN = GP * (PW > RP ? PW : RP);   // LDS floats of one wave
    extern __shared__ __align__(16) uint16_t dyn[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, quad = lane >> 4;
    // logits in base-2 units (log2(e) folded into the scale), so the softmax
    // takes v_exp_f32 directly; the split's max goes out in natural units
    constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
    const float scale2 = scale * kLog2e;
    // XCD-aware order: workgroups are dispatched to the 8 XCDs round-robin by
    // linear index, so tile t of row bh is given index (8*(bh/8)*T + 8*t) +
    // bh%8: all of a row's workgroups share one XCD, and the row's B, which
    // each of them stages, comes from HBM into that XCD's L2 once.  Indices
    // past the last row (rows rounded up to 8) exit at once.
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int bh = (idx / T) * 8 + xcd, tile = idx % T;
    if (bh >= rows) return;  // workgroup-uniform, before any barrier
    const int b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    const int ldb = NKB * 32 + 8;   // r_pad = 32 * NKB
    const bool rebuild = tile < ts;  // workgroup-uniform
    uint16_t *Bs = dyn;              // D x (r_pad + 8), rebuilding workgroups only
    // per wave: first its weights (GP x PW floats), then, once it has read
    // them, its merge record (GP x RP floats)
    float *rec = reinterpret_cast<float *>(dyn + (ts > 0 ? static_cast<size_t>(D) * ldb : 0));
    float *ps = rec + wave * RGN;
    const int key_base = tile * NW * kpw + wave * kpw;
    const bool active = rebuild && key_base < KC;  // wave-uniform
    const int kend = min(KC, key_base + kpw);       // end of this wave's rebuilt keys
    const int nstat = OC + w;
    const int sb0 = (tile * NW + wave) * 16;  // first key of this wave's static block

    // ---- 1. queries and the static block -------------------------------------------
    // the group's queries as the logit MFMA's A operand: lane (quad, row)
    // holds head `row` (rows past G repeat the last head; their outputs are
    // dropped) in the permuted dim order 32p + 4*quad + e, 32p + 16 + 4*quad + e
    bf16x8 qa[NP];
    {
        const uint16_t *qrow = q + (static_cast<size_t>(b) * hq + h * G + min(row, G - 1)) * D + quad * 4;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(qrow + 32 * p);
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(qrow + 32 * p + 16);
            qa[p] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
    }
    // the static block: keys in the same permuted dims (B operand), value
    // rows with lane (quad, row) holding key `row`, columns 32*kb + 8*quad .. +8
    const bool has_stat = sb0 < nstat;  // wave-uniform
    const int sk = min(sb0 + row, max(nstat - 1, 0));
    const uint16_t *skrow = sk < OC ? k_out + (static_cast<size_t>(bh) * OC + sk) * D
                                    : k_loc + (static_cast<size_t>(bh) * wcap + (sk - OC)) * D;
    const uint16_t *svrow = sk < OC ? v_out + (static_cast<size_t>(bh) * OC + sk) * D
                                    : v_loc + (static_cast<size_t>(bh) * wcap + (sk - OC)) * D;
    bf16x8 sko[NP];
    u32x4 svr[KB];
    if (has_stat) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(skrow + 32 * p + quad * 4);
            const u32x2 hi = *reinterpret_cast<const u32x2 *>(skrow + 32 * p + 16 + quad * 4);
            sko[p] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) svr[kb] = *reinterpret_cast<const u32x4 *>(svrow + kb * 32 + quad * 8);
    }

    // ---- 2. rebuilt blocks ---------------------------------------------------------
    f32x4 lg[MB + 1];  // logits, block MB is the static one
    u32x4 vr[MB][KB];  // value rows of the rebuilt blocks, laid out as svr
#pragma unroll
    for (int mb = 0; mb <= MB; ++mb) lg[mb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) vr[mb][kb] = u32x4{0u, 0u, 0u, 0u};
    if (rebuild) {
        const int pos0 = cshift >= 0 ? key_base >> cshift : key_base / c;
        const int my_chunk = chunks[static_cast<size_t>(bh) * k + min(pos0 + lane, k - 1)];
        // rotation rates (turns per position) of this lane's dims
        // 16*hb + 4*quad + e: theta_rev[4*quad + e] times the ratio of the
        // rates 16*hb dims apart, theta_rev[16*hb] / theta_rev[0]
        double thr0[4], rat[HB];
        const double inv_thr0 = 1.0 / theta_rev[0];
#pragma unroll
        for (int e = 0; e < 4; ++e) thr0[e] = theta_rev[quad * 4 + e];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) rat[hb] = theta_rev[hb * 16] * inv_thr0;
        {
            // stage B[h] (transposed, d x r) with every load in flight: row
            // nr of Bt, 8 rank values from kc; ranks past r read zeros
            // through the buffer resource's range check
            constexpr int VPR = NKB * 4, TOT = D * VPR, NT = 64 * NW, NIT = (TOT + NT - 1) / NT;
            const Rsrc brs = make_rsrc(Bt + static_cast<size_t>(bh) * D * r, static_cast<uint32_t>(D) * r * 2);
            u32x4 tmp[NIT];
#pragma unroll
            for (int i = 0; i < NIT; ++i) {
                const int ix = tid + NT * i;
                const int nr = ix / VPR, kc = (ix % VPR) * 8;
                tmp[i] = buf_ld128(brs, (ix < TOT && kc < r) ? (nr * r + kc) * 2 : kOob);
            }
#pragma unroll
            for (int i = 0; i < NIT; ++i) {
                const int ix = tid + NT * i;
                if (ix < TOT) *reinterpret_cast<u32x4 *>(Bs + (ix / VPR) * ldb + (ix % VPR) * 8) = tmp[i];
            }
        }
        // Gathered A row of this lane's key in each 16-key block, 8 rank
        // values per 32-wide rank block, through a buffer resource over this
        // sequence's A: keys past KC and rank columns past r read zeros
        // without a memory access, so no branch surrounds a load.
        const Rsrc ar = make_rsrc(A + static_cast<size_t>(b) * s * r, static_cast<uint32_t>(s) * r * 2);
        u32x4 aop[MB][NKB];
        int pos[MB], vkey[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int key = key_base + mb * 16 + row;
            const bool kv = active && key < kend;
            const int kk = key < kend ? key : key_base;
            const int kq = cshift >= 0 ? kk >> cshift : kk / c;  // c = 2^cshift: shifts
            const int chunk = __shfl(my_chunk, kq - pos0, 64);
            pos[mb] = chunk * c + (kk - kq * c);
            vkey[mb] = key < kend ? key : (KC > 0 ? KC - 1 : 0);  // a valid value row; its weight is 0
            const int base = (pos[mb] * r + quad * 8) * 2;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                aop[mb][kb] = buf_ld128(ar, kv && kb * 32 + quad * 8 < r ? base + kb * 64 : kOob);
        }
        __syncthreads();  // Bs staged (every wave of a rebuilding workgroup reaches it)

        // The blocks go in pairs (BP = 2, ranks 97..192): each staged Bt
        // operand read from LDS feeds both blocks' MFMAs, which halves the LDS
        // traffic of the rebuild.  With fewer or more rank blocks the second
        // block's registers do not fit beside the rest, so blocks go singly.
        constexpr int BP = (NKB >= 4 && NKB <= 6) ? 2 : 1;
#pragma unroll
        for (int mp = 0; mp < MB; mp += BP) {
            if (active && key_base + mp * 16 < kend) {  // wave-uniform
                // K^T[dim, key] = sum_r Bt[dim, r] A[key, r]: lane (quad, row)
                // ends with key `row`, dims 16*nb + 4*quad + e, of each block
                f32x4 acc[BP][NB];
#pragma unroll
                for (int x = 0; x < BP; ++x)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[x][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    bf16x8 bop[BP];
#pragma unroll
                    for (int x = 0; x < BP; ++x) bop[x] = __builtin_bit_cast(bf16x8, aop[mp + x][kb]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const bf16x8 aw = __builtin_bit_cast(
                            bf16x8, *reinterpret_cast<const u32x4 *>(Bs + (nb * 16 + row) * ldb + kb * 32 + quad * 8));
#pragma unroll
                        for (int x = 0; x < BP; ++x)
                            acc[x][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bop[x], acc[x][nb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int x = 0; x < BP; ++x) {
                    const int mb = mp + x, kb0 = key_base + mb * 16;
                    // the block's value rows, requested now that its A rows are consumed
                    {
                        const int key = vkey[mb];
                        const uint16_t *vrow;
                        if constexpr (IND) {
                            const int slot = min(max(sel_slot[static_cast<size_t>(bh) * k + key / c], 0), cap - 1);
                            vrow = vc + ((static_cast<size_t>(bh) * cap + slot) * c + key % c) * D;
                        } else {
                            vrow = vc + (static_cast<size_t>(bh) * KC + key) * D;
                        }
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb)
                            vr[mb][kb] = *reinterpret_cast<const u32x4 *>(vrow + kb * 32 + quad * 8);
                    }
                    // RoPE of this lane's key at its original position: the
                    // angle in turns, pos * theta_i / (2 pi), is reduced to
                    // [-1/2, 1/2] in double precision and fed to the hardware
                    // sin/cos (which take turns)
                    f32x4 *ac = acc[x];
                    const double posd = static_cast<double>(pos[mb]);
#pragma unroll
                    for (int hb = 0; hb < HB; ++hb) {
                        const double ph = posd * rat[hb];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const double turns = ph * thr0[e];
                            const float frac = static_cast<float>(turns - rint(turns));
                            const float sn = __builtin_amdgcn_sinf(frac), cs = __builtin_amdgcn_cosf(frac);
                            const float x1 = ac[hb][e], x2 = ac[hb + HB][e];
                            ac[hb][e] = x1 * cs - x2 * sn;
                            ac[hb + HB][e] = x2 * cs + x1 * sn;
                        }
                    }
                    const f32x4 l4 = logits_hilo<NP>(qa, ac, f32x4{0.f, 0.f, 0.f, 0.f});
                    const bool kv = kb0 + row < kend;
#pragma unroll
                    for (int e = 0; e < 4; ++e) lg[mb][e] = kv ? l4[e] * scale2 : -INFINITY;
                }
            }
        }
    }
    // ---- 3. the static block's logits ------------------------------------------------
    if (has_stat) {
        f32x4 l4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NP; ++p) l4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[p], sko[p], l4, 0, 0, 0);
        const bool kv = sb0 + row < nstat;
#pragma unroll
        for (int e = 0; e < 4; ++e) lg[MB][e] = kv ? l4[e] * scale2 : -INFINITY;
    } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) svr[kb] = u32x4{0u, 0u, 0u, 0u};
    }

    // ---- softmax per head 4*quad + e over the wave's 80 keys; weights to LDS -------
    float mrow[4], lrow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float m = lg[0][e];
#pragma unroll
        for (int mb = 1; mb <= MB; ++mb) m = fmaxf(m, lg[mb][e]);
        m = row16_reduce(m, [](float x, float y) { return fmaxf(x, y); });
        float l = 0.f;
#pragma unroll
        for (int mb = 0; mb <= MB; ++mb) {
            const float p = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lg[mb][e] - m);
            lg[mb][e] = p;
            l += p;
        }
        l = row16_reduce(l, [](float x, float y) { return x + y; });
        mrow[e] = m;
        lrow[e] = l;
        const int g = quad * 4 + e;
        if (g < GP) {
#pragma unroll
            for (int mb = 0; mb <= MB; ++mb) ps[g * PW + mb * 16 + row] = lg[mb][e];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- 4. sum of weight x V on MFMA ------------------------------------------------
    // 0/1 selectors: lane (row = n, quad = kq) of the B operand holds rows
    // 8*kq .. +8 of the 32 x 16 matrix with ones at (n + 16*half, n), so
    // V-slab x selector = the slab's columns 16*half .. +16, with lane
    // (quad, n) holding keys 4*quad + e of column n: a value row turned
    // column-major, each output one exact product
    bf16x8 sel01[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 8; ++j) sel01[hf][j] = static_cast<__bf16>(quad * 8 + j == row + 16 * hf ? 1.0f : 0.0f);
    // step st contracts the block pair (2*st, 2*st + 1) over the keys
    // {16*mb0 + 4*kq + e} then {16*mb1 + 4*kq + e}: the weights (A operand,
    // lane (head row, kq)) in that key order from LDS, the values (B operand)
    // from the two blocks' column-major outputs
    const int prow = min(row, GP - 1);
    f32x4 pacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 3; ++st) {
        const int mb0 = 2 * st, mb1 = 2 * st + 1;  // block MB = 4 is the static one, block 5 is empty
        const float4 p0 = *reinterpret_cast<const float4 *>(ps + prow * PW + mb0 * 16 + quad * 4);
        const float4 p1 = mb1 <= MB ? *reinterpret_cast<const float4 *>(ps + prow * PW + mb1 * 16 + quad * 4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
        bf16x8 phi, plo;
        split_bf16x8(f32x4{p0.x, p0.y, p0.z, p0.w}, f32x4{p1.x, p1.y, p1.z, p1.w}, phi, plo);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const u32x4 v0 = mb0 < MB ? vr[mb0][kb] : svr[kb];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const f32x4 t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v0), sel01[hf],
                                                                          f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                f32x4 t1 = {0.f, 0.f, 0.f, 0.f};
                if (mb1 < MB)
                    t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vr[mb1][kb]), sel01[hf],
                                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                else if (mb1 == MB)
                    t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, svr[kb]), sel01[hf],
                                                                 f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                const bf16x8 vop = __builtin_bit_cast(
                    bf16x8, u32x4{pack2_exact(t0[0], t0[1]), pack2_exact(t0[2], t0[3]), pack2_exact(t1[0], t1[1]),
                                  pack2_exact(t1[2], t1[3])});
                const int nb = kb * 2 + hf;  // output columns 16*nb .. +16
                pacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vop, pacc[nb], 0, 0, 0);
                pacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vop, pacc[nb], 0, 0, 0);
            }
        }
    }

    // ---- 5. this wave's partial per head into LDS (over its own weights, all
    //         read above), then the workgroup's four partials merged ---------------
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int g = quad * 4 + e;  // lane (quad, row): head g, column 16*nb + row
        if (g < G) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) ps[g * RP + nb * 16 + row] = pacc[nb][e];
            if (row == 0) {
                ps[g * RP + D] = mrow[e];
                ps[g * RP + D + 1] = lrow[e];
            }
        }
    }
    __syncthreads();  // every wave of the workgroup reaches it (no early exit above)
    for (int ix = tid; ix < G * D; ix += 64 * NW) {
        const int g = ix / D, i = ix % D;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, rec[wv * RGN + g * RP + D]);
        float Ls = 0.f, a = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) {
                const float *rr = rec + wv * RGN + g * RP;
                const float wgt = __builtin_amdgcn_exp2f(rr[D] - M);
                Ls += wgt * rr[D + 1];
                a += wgt * rr[i];
            }
        }
        const size_t rc = (static_cast<size_t>(bh) * G + g) * T + tile;
        part_acc[rc * D + i] = a;
        if (i == 0) part_ml[rc] = make_float2(M * kLn2, Ls);  // natural-log units for the merge kernel
    }
}

// ---------------------------------------------------------------------------
// PV over one split of 256 keys: partial (max, sum) and sum_key p * V[key].
// Thread (row group rg, column group cg) holds 8 columns of 256/(d/8) rows;
// every V load of the split is issued before the softmax weights are
// computed.  Partials are reduced across row groups with lane exchanges
// inside a wave and through LDS across the four waves.
// ---------------------------------------------------------------------------

// IND: the rebuilt block's V is looked up by slot (sel_slot); otherwise
// selection position i is cache slot i (a cache of exactly k slots, with the
// rebuilt keys in slot order).
template <typename T, int D, int GP, bool IND>
__global__ __launch_bounds__(256) void pv_kernel(const float *__restrict__ logits, const T *__restrict__ v_out,
                                                 const T *__restrict__ vc, const int32_t *__restrict__ sel_slot,
                                                 const T *__restrict__ v_loc, float2 *__restrict__ part_ml,
                                                 float *__restrict__ part_acc, int G, int OC, int KC, int c, int k,
                                                 int cap, int w, int wcap, int NK, int tiles) {
    constexpr int CG = D / 8;              // column groups of 8
    constexpr int RG = 256 / CG;           // row groups
    constexpr int RPT = kPvTile / RG;      // rows per thread
    constexpr int VPR = sizeof(T) == 2 ? 1 : 2;  // 16-byte vectors per 8 values
    constexpr int WRG = 64 / CG;           // row groups inside one wave
    __shared__ float ps[GP][kPvTile];
    __shared__ float red[4][GP][D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.y, tile = blockIdx.x;
    const int key0 = tile * kPvTile;
    const int cnt = min(kPvTile, NK - key0);
    const int cg = tid % CG, rg = tid / CG;

    // 1. the logits of this wave's heads first: the softmax then waits only
    //    for them, not for the V rows issued after them.  Every load below is
    //    unconditional (past the tile, the last key's row is read and weighted
    //    by zero), so the compiler's wait counts stay exact.
    constexpr int HPW = (GP + 3) / 4;  // heads per wave
    float lv[HPW][kPvTile / 64];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const int g = min(wave + 4 * hh, G - 1);
        const float *lg = logits + (static_cast<size_t>(bh) * G + g) * NK + key0;
#pragma unroll
        for (int i = 0; i < kPvTile / 64; ++i) lv[hh][i] = lg[min(lane + 64 * i, cnt - 1)];
    }
    // 2. the V rows of this thread's 8 columns; a rebuilt key i*c + t reads
    //    token t of cache slot sel_slot[i] (slots are looked up first, for
    //    every row, clamped into the block so the loads stay unconditional)
    int slot[RPT];
    if constexpr (IND) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int key = key0 + min(rg + RG * i, cnt - 1);
            const int p = KC > 0 ? min(max(key - OC, 0), KC - 1) : 0;
            slot[i] = min(max(sel_slot[static_cast<size_t>(bh) * k + p / c], 0), cap - 1);  // kept in the row
        }
    }
    u32x4 raw[RPT][VPR];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int key = key0 + min(rg + RG * i, cnt - 1);
        const T *sparse = IND ? vc + ((static_cast<size_t>(bh) * cap + slot[i]) * c + (key - OC) % c) * D
                              : vc + (static_cast<size_t>(bh) * KC + (key - OC)) * D;
        const T *vrow = key < OC ? v_out + (static_cast<size_t>(bh) * OC + key) * D
                      : key < OC + KC ? sparse
                                      : v_loc + (static_cast<size_t>(bh) * wcap + (key - OC - KC)) * D;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(vrow + cg * 8);
#pragma unroll
        for (int u = 0; u < VPR; ++u) raw[i][u] = src[u];
    }

    // 3. each head's softmax partial over the tile: (max, sum) to part_ml,
    //    the weights to LDS
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
        const int g = wave + 4 * hh;
        if (g >= GP) break;
        if (g >= G) {
            for (int i = lane; i < kPvTile; i += 64) ps[g][i] = 0.f;
            continue;
        }
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kPvTile / 64; ++i)
            if (lane + 64 * i < cnt) m = fmaxf(m, lv[hh][i]);
        m = wave_max(m);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < kPvTile / 64; ++i) {
            const int kk = lane + 64 * i;
            const float p = kk < cnt ? expf(lv[hh][i] - m) : 0.f;
            ps[g][kk] = p;
            sum += p;
        }
        sum = wave_sum(sum);
        if (lane == 0) part_ml[(static_cast<size_t>(bh) * G + g) * tiles + tile] = make_float2(m, sum);
    }
    __syncthreads();

    float acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[g][x] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int rr = rg + RG * i;
        float v[8];
        unpack8<T>(raw[i], v);
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float p = ps[g][rr];
#pragma unroll
            for (int x = 0; x < 8; ++x) acc[g][x] += p * v[x];
        }
    }
    if constexpr (CG == 16) {
        // sum over the wave's four row groups (lanes l, l+16, l+32, l+48) with
        // two halving permlane exchanges: lane group r ends with the values
        // r*(2*GP) .. r*(2*GP) + 2*GP - 1 of the flattened (head, column) list
        constexpr int NV = GP * 8;
        float a[NV];
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
            for (int x = 0; x < 8; ++x) a[g * 8 + x] = acc[g][x];
#pragma unroll
        for (int v = 0; v < NV / 2; ++v) a[v] = swap_sum32(a[v], a[v + NV / 2]);
#pragma unroll
        for (int v = 0; v < NV / 4; ++v) a[v] = swap_sum16(a[v], a[v + NV / 4]);
        const int r = lane >> 4;
#pragma unroll
        for (int v = 0; v < NV / 4; ++v) {
            const int f = r * (NV / 4) + v;
            red[wave][f >> 3][cg * 8 + (f & 7)] = a[v];
        }
    } else {
        // reduce the row groups of this wave (lane bits above the column group)
#pragma unroll
        for (int off = CG; off < 64; off <<= 1)
#pragma unroll
            for (int g = 0; g < GP; ++g)
#pragma unroll
                for (int x = 0; x < 8; ++x) acc[g][x] += __shfl_xor(acc[g][x], off, 64);
        if (lane < CG) {
#pragma unroll
            for (int g = 0; g < GP; ++g)
#pragma unroll
                for (int x = 0; x < 8; ++x) red[wave][g][cg * 8 + x] = acc[g][x];
        }
    }
    (void)WRG;
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, i = idx % D;
        part_acc[((static_cast<size_t>(bh) * G + g) * tiles + tile) * D + i] =
            red[0][g][i] + red[1][g][i] + red[2][g][i] + red[3][g][i];
    }
}

// out[b, g, :] = sum_t e^(m_t - M) acc_t / sum_t e^(m_t - M) l_t over the key
// splits t.  The record index (b*h_kv + h)*G + gi equals b*h_q + g of q/out.
template <typename T, int D>
__global__ __launch_bounds__(D) void combine_kernel(const float2 *__restrict__ part_ml,
                                                    const float *__restrict__ part_acc, T *__restrict__ out,
                                                    int tiles, int G, int rows) {
    // XCD-aware order, as the fused attention kernel's: query head g of row bh
    // (sequence, KV head) runs on XCD bh % 8, where that row's splits were
    // written.  Indices past the last row (rows rounded up to 8) exit at once.
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int bh = (j / G) * 8 + xcd;
    if (bh >= rows) return;
    const int bg = bh * G + j % G, i = threadIdx.x;
    const float2 *ml = part_ml + static_cast<size_t>(bg) * tiles;
    const float *pa = part_acc + static_cast<size_t>(bg) * tiles * D + i;
    constexpr int TMAX = 16;  // splits held in registers (all loads in flight); more are streamed
    if (tiles <= TMAX) {
        const Rsrc mr = make_rsrc(ml, static_cast<uint32_t>(tiles) * 8);
        const Rsrc ar = make_rsrc(pa - i, static_cast<uint32_t>(tiles) * D * 4);
        float m[TMAX], l[TMAX], a[TMAX];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            m[t] = __uint_as_float(buf_ld32(mr, t < tiles ? t * 8 : kOob));
            l[t] = __uint_as_float(buf_ld32(mr, t < tiles ? t * 8 + 4 : kOob));
            a[t] = __uint_as_float(buf_ld32(ar, t < tiles ? (t * D + i) * 4 : kOob));
        }
        float M = -INFINITY;
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if (t < tiles) M = fmaxf(M, m[t]);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < tiles) {
                const float wgt = expf(m[t] - M);
                L += wgt * l[t];
                acc += wgt * a[t];
            }
        }
        Elem<T>::st(out, static_cast<size_t>(bg) * D + i, acc / L);
        return;
    }
    float M = -INFINITY;
    for (int t = 0; t < tiles; ++t) M = fmaxf(M, ml[t].x);
    float L = 0.f, acc = 0.f;
    for (int t = 0; t < tiles; ++t) {
        const float wgt = expf(ml[t].x - M);
        L += wgt * ml[t].y;
        acc += wgt * pa[static_cast<size_t>(t) * D];
    }
    Elem<T>::st(out, static_cast<size_t>(bg) * D + i, acc / L);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_fetch(const Dims &dm, const void *v_host, void *vc, const int2 *misses, const int32_t *miss_count,
                        const uint32_t *vcode, unsigned long long *counters, int waves, hipStream_t st) {
    if (dm.k <= 0) return hipSuccess;
    const int rows = dm.b * dm.hkv;
    const int chunk_vec = dm.c * dm.d * dm.esize / 16;
    const size_t lds = static_cast<size_t>(rows + 1) * sizeof(int);
    auto go = [&](auto kern) {
        if (lds > 48 * 1024) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(kern, dim3(std::max(1, (waves + 3) / 4)), dim3(256), lds, st,
                           static_cast<const u32x4 *>(v_host), static_cast<u32x4 *>(vc), misses, miss_count, vcode,
                           counters, rows, dm.k, dm.cap, dm.n, chunk_vec);
        return hipGetLastError();
    };
    switch (chunk_vec) {
        case 64: return go(fetch_kernel<1>);
        case 128: return go(fetch_kernel<2>);
        case 256: return go(fetch_kernel<4>);
        default: return go(fetch_kernel<0>);
    }
}
template <typename T, int D>
static hipError_t qk_generic_t(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                               const void *Bt, const int32_t *sel, const double *theta, float *logits,
                               hipStream_t st) {
    const int t_out = (dm.OC + kQkTile - 1) / kQkTile;
    const int t_sp = (dm.KC + kQkTile - 1) / kQkTile;
    const int t_loc = (dm.w + kQkTile - 1) / kQkTile;
    const int tiles = t_out + t_sp + t_loc;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((qk_generic_kernel<T, D>), dim3(tiles, dm.b * dm.hkv), dim3(256), 0, st,
                       static_cast<const T *>(q), static_cast<const T *>(k_out), static_cast<const T *>(k_loc),
                       static_cast<const T *>(A), static_cast<const T *>(Bt), sel, theta, logits, dm.hkv,
                       dm.G, dm.s, dm.c, dm.r, dm.k, dm.OC, dm.KC, dm.w, dm.wcap, dm.NK, t_out, t_sp, dm.scale);
    return hipGetLastError();
}

template <int D, int GP, int NKB>
static hipError_t qk_mfma_t(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                            const void *Bt, const int32_t *sel, const double *theta_rev, float *logits,
                            hipStream_t st) {
    const int nstat = dm.OC + dm.w;
    const int ts = (dm.KC + kQkMfmaTile - 1) / kQkMfmaTile;  // rebuilt-key workgroups per row
    const int tt = (nstat + 63) / 64;                         // static-only workgroups per row (ts = 0)
    if (ts + tt == 0) return hipSuccess;
    const int r_pad = NKB * 32;
    const size_t lds = ts > 0 ? static_cast<size_t>(D) * (r_pad + 8) * sizeof(uint16_t) : 0;
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qk_mfma_kernel<D, GP, NKB>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    dim3 grid(ts > 0 ? ts : tt, dm.b * dm.hkv);
    hipLaunchKernelGGL((qk_mfma_kernel<D, GP, NKB>), grid, dim3(256), lds, st, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(Bt), sel, theta_rev,
                       static_cast<const uint16_t *>(k_out), static_cast<const uint16_t *>(k_loc), logits, dm.hkv,
                       dm.G, dm.s, dm.c, dm.r, r_pad, dm.k, dm.OC, dm.KC, dm.w, dm.wcap, dm.NK, ts, tt, dm.scale);
    return hipGetLastError();
}

// rank blocks of 32: the smallest supported count that covers the rank
template <int D, int GP>
static hipError_t qk_mfma_r(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                            const void *Bt, const int32_t *sel, const double *theta_rev, float *logits,
                            hipStream_t st) {
    const int need = (dm.r + 31) / 32;
    if (need <= 2) return qk_mfma_t<D, GP, 2>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
    if (need <= 4) return qk_mfma_t<D, GP, 4>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
    if (need <= 5) return qk_mfma_t<D, GP, 5>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
    if (need <= 6) return qk_mfma_t<D, GP, 6>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
    return qk_mfma_t<D, GP, 8>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
}

template <int D>
static hipError_t qk_bf16_d(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                            const void *Bt, const int32_t *sel, const double *theta_rev,
                            float *logits, hipStream_t st) {
    switch (dm.GP) {
        case 4: return qk_mfma_r<D, 4>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
        case 8: return qk_mfma_r<D, 8>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
        default: return qk_mfma_r<D, 16>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
    }
}

hipError_t launch_qk(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                     const void *Bt, const int32_t *sel, const double *theta, const double *theta_rev,
                     float *logits, hipStream_t st) {
    if (dm.bf16 && dm.r % 8 == 0)
        return dm.d == 128 ? qk_bf16_d<128>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st)
                           : qk_bf16_d<64>(dm, q, k_out, k_loc, A, Bt, sel, theta_rev, logits, st);
    if (dm.bf16)
        return dm.d == 128 ? qk_generic_t<uint16_t, 128>(dm, q, k_out, k_loc, A, Bt, sel, theta, logits, st)
                           : qk_generic_t<uint16_t, 64>(dm, q, k_out, k_loc, A, Bt, sel, theta, logits, st);
    return dm.d == 128 ? qk_generic_t<float, 128>(dm, q, k_out, k_loc, A, Bt, sel, theta, logits, st)
                       : qk_generic_t<float, 64>(dm, q, k_out, k_loc, A, Bt, sel, theta, logits, st);
}

template <typename T, int D, int GP>
static hipError_t pv_t(const Dims &dm, const float *logits, const void *v_out, const void *vc,
                       const int32_t *sel_slot, const void *v_loc, float2 *part_ml, float *part_acc,
                       hipStream_t st) {
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(dm.pv_tiles, dm.b * dm.hkv), dim3(256), 0, st, logits,
                           static_cast<const T *>(v_out), static_cast<const T *>(vc), sel_slot,
                           static_cast<const T *>(v_loc), part_ml, part_acc, dm.G, dm.OC, dm.KC, dm.c, dm.k, dm.cap,
                           dm.w, dm.wcap, dm.NK, dm.pv_tiles);
    };
    if (sel_slot) go(pv_kernel<T, D, GP, true>);
    else go(pv_kernel<T, D, GP, false>);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t pv_d(const Dims &dm, const float *logits, const void *v_out, const void *vc,
                       const int32_t *sel_slot, const void *v_loc, float2 *part_ml, float *part_acc,
                       hipStream_t st) {
    switch (dm.GP) {
        case 4: return pv_t<T, D, 4>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st);
        case 8: return pv_t<T, D, 8>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st);
        default: return pv_t<T, D, 16>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st);
    }
}

hipError_t launch_pv(const Dims &dm, const float *logits, const void *v_out, const void *vc, const int32_t *sel_slot,
                     const void *v_loc, float2 *part_ml, float *part_acc, hipStream_t st) {
    if (dm.bf16)
        return dm.d == 128 ? pv_d<uint16_t, 128>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st)
                           : pv_d<uint16_t, 64>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st);
    return dm.d == 128 ? pv_d<float, 128>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st)
                       : pv_d<float, 64>(dm, logits, v_out, vc, sel_slot, v_loc, part_ml, part_acc, st);
}


template <int D, int GP, int NKB, bool IND, int NW>
static hipError_t attn_t(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *chunks,
                         const int32_t *sel_slot, const double *theta_rev, const void *k_out, const void *v_out,
                         const void *k_loc, const void *v_loc, const void *vc, float2 *part_ml, float *part_acc,
                         hipStream_t st) {
    const int ts = (dm.KC + NW * dm.kpw - 1) / (NW * dm.kpw);
    const int T = attn_workgroups(dm);
    const int r_pad = NKB * 32;
    constexpr int RGN = GP * (84 > D + 2 ? 84 : D + 2);  // LDS floats per wave: weights, then merge record
    const size_t lds = (ts > 0 ? static_cast<size_t>(D) * (r_pad + 8) * sizeof(uint16_t) : 0) + static_cast<size_t>(NW) * RGN * sizeof(float);
    auto kern = attn_mfma_kernel<D, GP, NKB, IND, NW>;
    if (lds > 48 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    const int rows = dm.b * dm.hkv, rows8 = (rows + 7) / 8 * 8;
    hipLaunchKernelGGL(kern, dim3(T * rows8), dim3(64 * NW), lds, st, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(Bt), chunks, sel_slot,
                       theta_rev, static_cast<const uint16_t *>(k_out), static_cast<const uint16_t *>(v_out),
                       static_cast<const uint16_t *>(k_loc), static_cast<const uint16_t *>(v_loc),
                       static_cast<const uint16_t *>(vc), part_ml, part_acc, dm.hkv, dm.G, dm.s, dm.c, dm.r, r_pad,
                       dm.k, dm.cap, dm.OC, dm.KC, dm.w, dm.wcap, ts, T, rows, dm.scale,
                       (dm.c & (dm.c - 1)) == 0 ? __builtin_ctz(dm.c) : -1, dm.kpw);
    return hipGetLastError();
}

template <int D, int GP, bool IND>
static hipError_t attn_r(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *chunks,
                         const int32_t *sel_slot, const double *theta_rev, const void *k_out, const void *v_out,
                         const void *k_loc, const void *v_loc, const void *vc, float2 *part_ml, float *part_acc,
                         hipStream_t st) {
    const int need = (dm.r + 31) / 32;
#define SKV_ATTN(NKB) \
    attn_t<D, GP, NKB, IND, 4>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc, vc, part_ml, \
                               part_acc, st)
    if (need <= 2) return SKV_ATTN(2);
    if (need <= 4) return SKV_ATTN(4);
    if constexpr (D == 128) {
        // 8-wave workgroups (one per CU, sharing one staged B) at rank 129..160
        if (need <= 5 && dm.attn_nw == 8)
            return attn_t<D, GP, 5, IND, 8>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc,
                                            vc, part_ml, part_acc, st);
    }
    if (need <= 5) return SKV_ATTN(5);
    if (need <= 6) return SKV_ATTN(6);
    return SKV_ATTN(8);
#undef SKV_ATTN
}

template <int D, bool IND>
static hipError_t attn_g(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *chunks,
                         const int32_t *sel_slot, const double *theta_rev, const void *k_out, const void *v_out,
                         const void *k_loc, const void *v_loc, const void *vc, float2 *part_ml, float *part_acc,
                         hipStream_t st) {
    switch (dm.GP) {
        case 4:
            return attn_r<D, 4, IND>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc, vc,
                                     part_ml, part_acc, st);
        case 8:
            return attn_r<D, 8, IND>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc, vc,
                                     part_ml, part_acc, st);
        default:
            return attn_r<D, 16, IND>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc, vc,
                                      part_ml, part_acc, st);
    }
}

int attn_waves(const Dims &dm) { return dm.bf16 && dm.attn_nw == 8 && dm.d == 128 && (dm.r + 31) / 32 == 5 ? 8 : 4; }

int attn_workgroups(const Dims &dm) {
    const int nw = attn_waves(dm);
    const int ts = (dm.KC + nw * dm.kpw - 1) / (nw * dm.kpw);
    return std::max(ts, (dm.OC + dm.w + 16 * nw - 1) / (16 * nw));
}

hipError_t launch_attn(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *chunks,
                       const int32_t *sel_slot, const double *theta_rev, const void *k_out, const void *v_out,
                       const void *k_loc, const void *v_loc, const void *vc, float2 *part_ml, float *part_acc,
                       hipStream_t st) {
    if (!dm.bf16) return hipErrorInvalidValue;
    if (attn_workgroups(dm) <= 0) return hipSuccess;
    if (sel_slot) {
        return dm.d == 128 ? attn_g<128, true>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc,
                                               vc, part_ml, part_acc, st)
                           : attn_g<64, true>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc,
                                              vc, part_ml, part_acc, st);
    }
    return dm.d == 128 ? attn_g<128, false>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc, vc,
                                            part_ml, part_acc, st)
                       : attn_g<64, false>(dm, q, A, Bt, chunks, sel_slot, theta_rev, k_out, v_out, k_loc, v_loc, vc,
                                           part_ml, part_acc, st);
}

hipError_t launch_combine(const Dims &dm, const float2 *part_ml, const float *part_acc, void *out, int splits,
                          hipStream_t st) {
    const int rows = dm.b * dm.hkv, blocks = (rows + 7) / 8 * 8 * dm.G;
    if (dm.bf16) {
        if (dm.d == 128)
            hipLaunchKernelGGL((combine_kernel<uint16_t, 128>), dim3(blocks), dim3(128), 0, st, part_ml, part_acc,
                               static_cast<uint16_t *>(out), splits, dm.G, rows);
        else
            hipLaunchKernelGGL((combine_kernel<uint16_t, 64>), dim3(blocks), dim3(64), 0, st, part_ml, part_acc,
                               static_cast<uint16_t *>(out), splits, dm.G, rows);
    } else {
        if (dm.d == 128)
            hipLaunchKernelGGL((combine_kernel<float, 128>), dim3(blocks), dim3(128), 0, st, part_ml, part_acc,
                               static_cast<float *>(out), splits, dm.G, rows);
        else
            hipLaunchKernelGGL((combine_kernel<float, 64>), dim3(blocks), dim3(64), 0, st, part_ml, part_acc,
                               static_cast<float *>(out), splits, dm.G, rows);
    }
    return hipGetLastError();
}

}  // namespace skv
