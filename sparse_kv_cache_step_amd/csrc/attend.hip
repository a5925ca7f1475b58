// Attention half of the decode step (review page, section 三, Algorithm 2
// steps 3-4):
//   fetch    V of the chunks that missed the resident cache, read by the GPU
//            straight from pinned host memory (second stream);
//   qk       logits over [outlier keys; rebuilt keys; local keys], where the
//            rebuilt keys are Gather(A, I) . B on MFMA followed by RoPE at the
//            chunks' original positions, never written to memory;
//   pv       softmax-weighted values per key split, with split partials;
//   combine  merge of the split partials into the output.
#include "skv_device.h"

namespace skv {

// ---------------------------------------------------------------------------
// Host-V fetch: one wave copies one missing chunk (c * d elements, contiguous
// on both sides) from pinned host memory into its cache slot.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fetch_kernel(const u32x4 *__restrict__ v_host, u32x4 *__restrict__ vc,
                                                    const int2 *__restrict__ misses,
                                                    const int32_t *__restrict__ miss_count, int k, int n,
                                                    int chunk_vec) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y;
    const int cnt = miss_count[bh];
    const int2 *ml = misses + static_cast<size_t>(bh) * k;
    for (int m = blockIdx.x * 4 + wave; m < cnt; m += gridDim.x * 4) {
        const int2 e = ml[m];
        const u32x4 *src = v_host + (static_cast<size_t>(bh) * n + e.x) * chunk_vec;
        u32x4 *dst = vc + (static_cast<size_t>(bh) * k + e.y) * chunk_vec;
        int i = lane;
        for (; i + 64 < chunk_vec; i += 128) {
            const u32x4 a = __builtin_nontemporal_load(src + i);
            const u32x4 b = __builtin_nontemporal_load(src + i + 64);
            dst[i] = a;
            dst[i + 64] = b;
        }
        if (i < chunk_vec) dst[i] = __builtin_nontemporal_load(src + i);
    }
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
                                                         const int32_t *__restrict__ slot_chunk,
                                                         const double *__restrict__ theta,
                                                         float *__restrict__ logits, int hkv, int G, int s, int c,
                                                         int r, int k, int OC, int KC, int w, int NK, int t_out,
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
                                : k_loc + (static_cast<size_t>(bh) * w + key0) * D;
        for (int idx = threadIdx.x; idx < cnt * D; idx += 256) Ks[idx / D][idx % D] = Elem<T>::ld(src, idx);
    } else {
        const T *Bh = Bt + static_cast<size_t>(bh) * D * r;
        for (int idx = threadIdx.x; idx < cnt * D; idx += 256) {
            const int rr = idx / D, i = idx % D, key = key0 + rr;
            const int pos = slot_chunk[static_cast<size_t>(bh) * k + key / c] * c + key % c;
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
            const int pos = slot_chunk[static_cast<size_t>(bh) * k + key / c] * c + key % c;
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
// Rebuilt keys on MFMA (bfloat16).  Per (sequence, KV head) the rebuild is
// K[key, :] = A[pos(key), :] . B[h] with pos(key) = chunk(slot) * c + t, a
// genuine rank-r x d contraction.  A workgroup takes 256 keys (4 waves x 64);
// B[h] (stored transposed, d x r) is staged once in LDS and shared by the four
// waves, the gathered A rows feed the MFMA A operand straight from memory.
// v_mfma_f32_16x16x32_bf16 leaves lane l with keys 4*(l>>4)+e (e < 4) of a
// 16-key block and column (l & 15) of a 16-column block, so the RoPE pair
// (i, i + d/2) sits in one lane and is rotated in registers.  The logits for
// the GP (padded) query heads are reduced across the 16 column lanes with a
// halving exchange, leaving each lane with GP/4 finished logits.
// ---------------------------------------------------------------------------
template <int D, int GP>
__global__ __launch_bounds__(256) void qk_sparse_mfma_kernel(const uint16_t *__restrict__ q,
                                                             const uint16_t *__restrict__ A,
                                                             const uint16_t *__restrict__ Bt,
                                                             const int32_t *__restrict__ slot_chunk,
                                                             const double *__restrict__ theta,
                                                             const float2 *__restrict__ rope_off,
                                                             float *__restrict__ logits, int hkv, int G, int s,
                                                             int c, int r, int r_pad, int k, int OC, int KC, int NK,
                                                             float scale) {
    constexpr int NB = D / 16;  // 16-column blocks
    constexpr int HB = NB / 2;  // blocks holding the first half of the dims
    constexpr int MB = 4;       // 16-key blocks per wave
    constexpr int X = 4 * GP;   // logit partials per lane and key block
    extern __shared__ uint16_t Bs[];  // D rows of (r_pad + 8) rank entries
    __shared__ float qs[GP][D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, quad = lane >> 4;
    const int bh = blockIdx.y, b = bh / hkv, h = bh % hkv;
    const int hq = hkv * G;
    const int ldb = r_pad + 8;

    {
        const uint16_t *Btb = Bt + static_cast<size_t>(bh) * D * r;
        const int vpr = r_pad / 8;
        for (int idx = tid; idx < D * vpr; idx += 256) {
            const int nr = idx / vpr, kc = (idx % vpr) * 8;
            const u32x4 v = kc < r ? *reinterpret_cast<const u32x4 *>(Btb + static_cast<size_t>(nr) * r + kc)
                                   : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(Bs + nr * ldb + kc) = v;
        }
        for (int idx = tid; idx < GP * D; idx += 256) {
            const int g = idx / D, i = idx % D;
            qs[g][i] = g < G ? bf16_bits_to_f32(q[(static_cast<size_t>(b) * hq + h * G + g) * D + i]) * scale : 0.f;
        }
    }
    __syncthreads();

    const int key_base = blockIdx.x * kQkMfmaTile + wave * 64;
    if (key_base >= KC) return;  // no barrier follows
    const int32_t *sc = slot_chunk + static_cast<size_t>(bh) * k;

    const uint16_t *arow[MB];
    bool avalid[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int key = key_base + mb * 16 + row;
        avalid[mb] = key < KC;
        const int chunk = avalid[mb] ? sc[key / c] : 0;
        const int pos = chunk * c + (avalid[mb] ? key % c : 0);
        arow[mb] = A + (static_cast<size_t>(b) * s + pos) * r + quad * 8;
    }

    f32x4 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kb = 0; kb < r_pad / 32; ++kb) {
        const int kk = kb * 32 + quad * 8;
        bf16x8 aop[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const u32x4 v = (avalid[mb] && kk < r) ? *reinterpret_cast<const u32x4 *>(arow[mb] + kb * 32)
                                                   : u32x4{0u, 0u, 0u, 0u};
            aop[mb] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const bf16x8 bop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(Bs + (nb * 16 + row) * ldb + kk));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[mb], bop, acc[mb][nb], 0, 0, 0);
        }
    }

    // RoPE at pos = chunk * c + t: the chunk's angle chunk*c*theta_i is reduced
    // in double precision; the in-chunk offset t*theta_i comes from a table.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        float cb[HB], sb[HB];
        int prev = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = key_base + mb * 16 + quad * 4 + e;
            const bool kv = key < KC;
            const int chunk = kv ? sc[key / c] : 0;
            const int t = kv ? key % c : 0;
            if (chunk != prev) {
#pragma unroll
                for (int hb = 0; hb < HB; ++hb)
                    angle_sincos(static_cast<double>(chunk * c) * theta[hb * 16 + row], &sb[hb], &cb[hb]);
                prev = chunk;
            }
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                const float2 off = rope_off[t * (D / 2) + hb * 16 + row];
                const float cs = cb[hb] * off.x - sb[hb] * off.y;
                const float sn = sb[hb] * off.x + cb[hb] * off.y;
                const float x1 = acc[mb][hb][e], x2 = acc[mb][hb + HB][e];
                acc[mb][hb][e] = x1 * cs - x2 * sn;
                acc[mb][hb + HB][e] = x2 * cs + x1 * sn;
            }
        }
    }

    // logits: partial dots over this lane's columns, then a halving exchange
    // across the 16 lanes of a lane group.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        float part[X];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                float a = 0.f;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) a += qs[g][nb * 16 + row] * acc[mb][nb][e];
                part[e * GP + g] = a;
            }
#pragma unroll
        for (int bit = 8, cntv = X; bit >= 1; bit >>= 1, cntv >>= 1) {
            const bool upper = (row & bit) != 0;
            const int half = cntv / 2;
#pragma unroll
            for (int x = 0; x < X / 2; ++x) {
                if (x < half) {
                    const float send = upper ? part[x] : part[x + half];
                    const float keep = upper ? part[x + half] : part[x];
                    part[x] = keep + __shfl_xor(send, bit, 64);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < GP / 4; ++j) {
            const int xo = (GP / 4) * row + j;
            const int e = xo / GP, g = xo % GP;
            const int key = key_base + mb * 16 + quad * 4 + e;
            if (key < KC && g < G) logits[(static_cast<size_t>(bh) * G + g) * NK + OC + key] = part[j];
        }
    }
}

// ---------------------------------------------------------------------------
// PV over one split of 256 keys: p = exp(logit - m_split), partial (m, l) and
// sum_key p * V[key, :] for each query head of the group.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pv_kernel(const float *__restrict__ logits, const T *__restrict__ v_out,
                                                 const T *__restrict__ vc, const T *__restrict__ v_loc,
                                                 float2 *__restrict__ part_ml, float *__restrict__ part_acc,
                                                 int G, int OC, int KC, int w, int NK, int tiles) {
    constexpr int CP = D / 2;       // column pairs
    constexpr int NRG = 256 / CP;   // row groups
    __shared__ float ps[kMaxGroup][kPvTile];
    __shared__ float red[NRG][kMaxGroup][D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.y, tile = blockIdx.x;
    const int key0 = tile * kPvTile;
    const int cnt = min(kPvTile, NK - key0);
    for (int g = wave; g < G; g += 4) {
        const float *lg = logits + (static_cast<size_t>(bh) * G + g) * NK + key0;
        float v[kPvTile / 64];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kPvTile / 64; ++i) {
            const int kk = lane + 64 * i;
            v[i] = kk < cnt ? lg[kk] : -INFINITY;
            m = fmaxf(m, v[i]);
        }
        m = wave_max(m);
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < kPvTile / 64; ++i) {
            const int kk = lane + 64 * i;
            const float p = kk < cnt ? expf(v[i] - m) : 0.f;
            ps[g][kk] = p;
            sum += p;
        }
        sum = wave_sum(sum);
        if (lane == 0) part_ml[(static_cast<size_t>(bh) * G + g) * tiles + tile] = make_float2(m, sum);
    }
    __syncthreads();
    const int cp = tid % CP, rg = tid / CP;
    float a0[kMaxGroup], a1[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) { a0[g] = 0.f; a1[g] = 0.f; }
    for (int rr = rg; rr < cnt; rr += NRG) {
        const int key = key0 + rr;
        const T *vrow = key < OC ? v_out + (static_cast<size_t>(bh) * OC + key) * D
                      : key < OC + KC ? vc + (static_cast<size_t>(bh) * KC + (key - OC)) * D
                                      : v_loc + (static_cast<size_t>(bh) * w + (key - OC - KC)) * D;
        const float v0 = Elem<T>::ld(vrow, 2 * cp), v1 = Elem<T>::ld(vrow, 2 * cp + 1);
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) {
            if (g < G) {
                const float p = ps[g][rr];
                a0[g] += p * v0;
                a1[g] += p * v1;
            }
        }
    }
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
        if (g < G) { red[rg][g][2 * cp] = a0[g]; red[rg][g][2 * cp + 1] = a1[g]; }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, i = idx % D;
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < NRG; ++x) acc += red[x][g][i];
        part_acc[((static_cast<size_t>(bh) * G + g) * tiles + tile) * D + i] = acc;
    }
}

// out[b, g, :] = sum_t e^(m_t - M) acc_t / sum_t e^(m_t - M) l_t.  The linear
// index (b*h_kv + h)*G + gi of a split record equals b*h_q + g of q and out.
template <typename T, int D>
__global__ __launch_bounds__(D) void combine_kernel(const float2 *__restrict__ part_ml,
                                                    const float *__restrict__ part_acc, T *__restrict__ out,
                                                    int tiles) {
    const int bg = blockIdx.x, i = threadIdx.x;
    const float2 *ml = part_ml + static_cast<size_t>(bg) * tiles;
    float M = -INFINITY;
    for (int t = 0; t < tiles; ++t) M = fmaxf(M, ml[t].x);
    float L = 0.f, acc = 0.f;
    for (int t = 0; t < tiles; ++t) {
        const float wgt = expf(ml[t].x - M);
        L += wgt * ml[t].y;
        acc += wgt * part_acc[(static_cast<size_t>(bg) * tiles + t) * D + i];
    }
    Elem<T>::st(out, static_cast<size_t>(bg) * D + i, acc / L);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_fetch(const Dims &dm, const void *v_host, void *vc, const int2 *misses, const int32_t *miss_count,
                        int blocks_per_bh, hipStream_t st) {
    if (dm.k <= 0) return hipSuccess;
    const int chunk_vec = dm.c * dm.d * dm.esize / 16;
    dim3 grid(blocks_per_bh, dm.b * dm.hkv);
    hipLaunchKernelGGL(fetch_kernel, grid, dim3(256), 0, st, static_cast<const u32x4 *>(v_host),
                       static_cast<u32x4 *>(vc), misses, miss_count, dm.k, dm.n, chunk_vec);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t qk_generic_t(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                               const void *Bt, const int32_t *slot_chunk, const double *theta, float *logits,
                               bool include_sparse, hipStream_t st) {
    const int t_out = (dm.OC + kQkTile - 1) / kQkTile;
    const int t_sp = include_sparse ? (dm.KC + kQkTile - 1) / kQkTile : 0;
    const int t_loc = (dm.w + kQkTile - 1) / kQkTile;
    const int tiles = t_out + t_sp + t_loc;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((qk_generic_kernel<T, D>), dim3(tiles, dm.b * dm.hkv), dim3(256), 0, st,
                       static_cast<const T *>(q), static_cast<const T *>(k_out), static_cast<const T *>(k_loc),
                       static_cast<const T *>(A), static_cast<const T *>(Bt), slot_chunk, theta, logits, dm.hkv,
                       dm.G, dm.s, dm.c, dm.r, dm.k, dm.OC, dm.KC, dm.w, dm.NK, t_out, t_sp, dm.scale);
    return hipGetLastError();
}

template <int D, int GP>
static hipError_t qk_mfma_t(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *slot_chunk,
                            const double *theta, const float2 *rope_off, float *logits, hipStream_t st) {
    if (dm.KC <= 0) return hipSuccess;
    const size_t lds = static_cast<size_t>(D) * (dm.r_pad + 8) * sizeof(uint16_t);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(qk_sparse_mfma_kernel<D, GP>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid((dm.KC + kQkMfmaTile - 1) / kQkMfmaTile, dm.b * dm.hkv);
    hipLaunchKernelGGL((qk_sparse_mfma_kernel<D, GP>), grid, dim3(256), lds, st, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(A), static_cast<const uint16_t *>(Bt), slot_chunk, theta,
                       rope_off, logits, dm.hkv, dm.G, dm.s, dm.c, dm.r, dm.r_pad, dm.k, dm.OC, dm.KC, dm.NK,
                       dm.scale);
    return hipGetLastError();
}

template <int D>
static hipError_t qk_mfma_d(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *slot_chunk,
                            const double *theta, const float2 *rope_off, float *logits, hipStream_t st) {
    switch (dm.GP) {
        case 4: return qk_mfma_t<D, 4>(dm, q, A, Bt, slot_chunk, theta, rope_off, logits, st);
        case 8: return qk_mfma_t<D, 8>(dm, q, A, Bt, slot_chunk, theta, rope_off, logits, st);
        default: return qk_mfma_t<D, 16>(dm, q, A, Bt, slot_chunk, theta, rope_off, logits, st);
    }
}

hipError_t launch_qk(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                     const void *Bt, const int32_t *slot_chunk, const double *theta, const float2 *rope_off,
                     float *logits, hipStream_t st) {
    hipError_t e;
    if (dm.bf16 && dm.r % 8 == 0) {
        e = dm.d == 128 ? qk_generic_t<uint16_t, 128>(dm, q, k_out, k_loc, A, Bt, slot_chunk, theta, logits, false, st)
                        : qk_generic_t<uint16_t, 64>(dm, q, k_out, k_loc, A, Bt, slot_chunk, theta, logits, false, st);
        if (e != hipSuccess) return e;
        return dm.d == 128 ? qk_mfma_d<128>(dm, q, A, Bt, slot_chunk, theta, rope_off, logits, st)
                           : qk_mfma_d<64>(dm, q, A, Bt, slot_chunk, theta, rope_off, logits, st);
    }
    if (dm.bf16)
        return dm.d == 128 ? qk_generic_t<uint16_t, 128>(dm, q, k_out, k_loc, A, Bt, slot_chunk, theta, logits, true, st)
                           : qk_generic_t<uint16_t, 64>(dm, q, k_out, k_loc, A, Bt, slot_chunk, theta, logits, true, st);
    return dm.d == 128 ? qk_generic_t<float, 128>(dm, q, k_out, k_loc, A, Bt, slot_chunk, theta, logits, true, st)
                       : qk_generic_t<float, 64>(dm, q, k_out, k_loc, A, Bt, slot_chunk, theta, logits, true, st);
}

template <typename T, int D>
static hipError_t pv_t(const Dims &dm, const float *logits, const void *v_out, const void *vc, const void *v_loc,
                       float2 *part_ml, float *part_acc, hipStream_t st) {
    hipLaunchKernelGGL((pv_kernel<T, D>), dim3(dm.pv_tiles, dm.b * dm.hkv), dim3(256), 0, st, logits,
                       static_cast<const T *>(v_out), static_cast<const T *>(vc), static_cast<const T *>(v_loc),
                       part_ml, part_acc, dm.G, dm.OC, dm.KC, dm.w, dm.NK, dm.pv_tiles);
    return hipGetLastError();
}

hipError_t launch_pv(const Dims &dm, const float *logits, const void *v_out, const void *vc, const void *v_loc,
                     float2 *part_ml, float *part_acc, hipStream_t st) {
    if (dm.bf16)
        return dm.d == 128 ? pv_t<uint16_t, 128>(dm, logits, v_out, vc, v_loc, part_ml, part_acc, st)
                           : pv_t<uint16_t, 64>(dm, logits, v_out, vc, v_loc, part_ml, part_acc, st);
    return dm.d == 128 ? pv_t<float, 128>(dm, logits, v_out, vc, v_loc, part_ml, part_acc, st)
                       : pv_t<float, 64>(dm, logits, v_out, vc, v_loc, part_ml, part_acc, st);
}

hipError_t launch_combine(const Dims &dm, const float2 *part_ml, const float *part_acc, void *out, hipStream_t st) {
    const int blocks = dm.b * dm.hq;
    if (dm.bf16) {
        if (dm.d == 128)
            hipLaunchKernelGGL((combine_kernel<uint16_t, 128>), dim3(blocks), dim3(128), 0, st, part_ml, part_acc,
                               static_cast<uint16_t *>(out), dm.pv_tiles);
        else
            hipLaunchKernelGGL((combine_kernel<uint16_t, 64>), dim3(blocks), dim3(64), 0, st, part_ml, part_acc,
                               static_cast<uint16_t *>(out), dm.pv_tiles);
    } else {
        if (dm.d == 128)
            hipLaunchKernelGGL((combine_kernel<float, 128>), dim3(blocks), dim3(128), 0, st, part_ml, part_acc,
                               static_cast<float *>(out), dm.pv_tiles);
        else
            hipLaunchKernelGGL((combine_kernel<float, 64>), dim3(blocks), dim3(64), 0, st, part_ml, part_acc,
                               static_cast<float *>(out), dm.pv_tiles);
    }
    return hipGetLastError();
}

}  // namespace skv
