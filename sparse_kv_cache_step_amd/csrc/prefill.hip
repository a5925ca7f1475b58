// Prefill-side kernels of the ShadowKV step (review page, section 三,
// Algorithm 1 steps 2-5): RoPE of the pre-RoPE keys, chunk means
// (landmarks), each chunk's minimum token-to-landmark cosine, the static
// outlier / local-window buffers and the selectable-chunk bitmask; and the
// coded forms in which host V crosses PCIe.
#include <algorithm>

#include "skv_device.h"

namespace skv {

// Post-RoPE key pair (i, i + d/2) of one token, computed in double precision
// (angle, sin/cos, rotation) and rounded once to the storage type.  Prefill is
// off the decode path, so it affords the exact arithmetic: the stored keys and
// landmarks equal the correctly rounded values.
template <typename T>
__device__ __forceinline__ void rope_store_pair(const T *k_pre, const T *k_rope, size_t off, int i, int half,
                                                int pos, double theta, float &y1, float &y2) {
    if (k_rope) {
        y1 = Elem<T>::ld(k_rope, off + i);
        y2 = Elem<T>::ld(k_rope, off + i + half);
        return;
    }
    double sn, cs;
    sincos(static_cast<double>(pos) * theta, &sn, &cs);
    const double x1 = Elem<T>::ld(k_pre, off + i), x2 = Elem<T>::ld(k_pre, off + i + half);
    y1 = Elem<T>::rnd_d(x1 * cs - x2 * sn);
    y2 = Elem<T>::rnd_d(x2 * cs + x1 * sn);
}

// One wave per chunk.  Lane i < d/2 owns the RoPE pair (i, i + d/2).  The
// chunk mean is accumulated in double and rounded once; the cosines use the
// stored (rounded) keys and landmark and are accumulated in double.
template <typename T, int D>
__global__ __launch_bounds__(256) void landmarks_kernel(const T *__restrict__ k_pre,
                                                        const T *__restrict__ k_rope,
                                                        const double *__restrict__ theta,
                                                        T *__restrict__ landmarks,
                                                        float *__restrict__ min_cos, int n, int c, int s) {
    extern __shared__ float ys[];  // [4 waves][c][D] stored post-RoPE keys
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y;
    const int j = blockIdx.x * 4 + wave;
    if (j >= n) return;  // whole wave leaves together; no block barrier below
    constexpr int H = D / 2;
    const bool act = lane < H;
    float *y = ys + static_cast<size_t>(wave) * c * D;
    const size_t base = (static_cast<size_t>(bh) * s + static_cast<size_t>(j) * c) * D;
    double sum1 = 0.0, sum2 = 0.0;
    for (int t = 0; t < c; ++t) {
        float y1 = 0.f, y2 = 0.f;
        if (act) {
            rope_store_pair<T>(k_pre, k_rope, base + static_cast<size_t>(t) * D, lane, H, j * c + t, theta[lane], y1, y2);
            y[t * D + lane] = y1;
            y[t * D + lane + H] = y2;
        }
        sum1 += y1;
        sum2 += y2;
    }
    double l1 = act ? Elem<T>::rnd_d(sum1 / c) : 0.0;
    double l2 = act ? Elem<T>::rnd_d(sum2 / c) : 0.0;
    if (act) {
        const size_t lo = (static_cast<size_t>(bh) * n + j) * D;
        Elem<T>::st(landmarks, lo + lane, static_cast<float>(l1));
        Elem<T>::st(landmarks, lo + lane + H, static_cast<float>(l2));
    }
    const double lnorm = sqrt(wave_sum_d(l1 * l1 + l2 * l2));
    double mn = INFINITY;
    for (int t = 0; t < c; ++t) {
        const double y1 = act ? y[t * D + lane] : 0.0;
        const double y2 = act ? y[t * D + lane + H] : 0.0;
        const double dot = wave_sum_d(y1 * l1 + y2 * l2);
        const double den = sqrt(wave_sum_d(y1 * y1 + y2 * y2)) * lnorm;
        mn = fmin(mn, dot / (den > 1e-12 ? den : 1e-12));
    }
    if (lane == 0) min_cos[static_cast<size_t>(bh) * n + j] = static_cast<float>(mn);
}

// Gather the full-rank post-RoPE K and the V of every outlier chunk and of
// the last w tokens.  One wave per token row; RoPE is recomputed with the
// same arithmetic as landmarks_kernel, so the stored keys are identical to
// the ones the landmarks were built from.
template <typename T, int D>
__global__ __launch_bounds__(256) void gather_static_kernel(const T *__restrict__ k_pre,
                                                            const T *__restrict__ k_rope,
                                                            const T *__restrict__ v,
                                                            const int32_t *__restrict__ outliers,
                                                            const double *__restrict__ theta,
                                                            T *__restrict__ k_out, T *__restrict__ v_out,
                                                            T *__restrict__ k_loc, T *__restrict__ v_loc,
                                                            int s, int c, int o, int w, int wcap) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int bh = blockIdx.y;
    const int rr = blockIdx.x * 4 + wave;
    const int OC = o * c;
    if (rr >= OC + w) return;
    int pos;
    T *kd, *vd;
    size_t drow;
    if (rr < OC) {
        pos = outliers[static_cast<size_t>(bh) * o + rr / c] * c + rr % c;
        kd = k_out; vd = v_out; drow = static_cast<size_t>(bh) * OC + rr;
    } else {
        pos = s - w + (rr - OC);
        kd = k_loc; vd = v_loc; drow = static_cast<size_t>(bh) * wcap + (rr - OC);
    }
    constexpr int H = D / 2;
    const size_t src = (static_cast<size_t>(bh) * s + pos) * D;
    const size_t dst = drow * D;
    if (lane < H) {
        float y1, y2;
        rope_store_pair<T>(k_pre, k_rope, src, lane, H, pos, theta[lane], y1, y2);
        Elem<T>::st(kd, dst + lane, y1);
        Elem<T>::st(kd, dst + lane + H, y2);
        vd[dst + lane] = v[src + lane];
        vd[dst + lane + H] = v[src + lane + H];
    }
}

// Selectable chunks: outside the local window and not outliers.
__global__ void cand_mask_kernel(const int32_t *__restrict__ outliers, uint32_t *__restrict__ cand, int n,
                                 int n_loc, int o, int mask_words) {
    const int bh = blockIdx.y;
    const int wi = blockIdx.x * blockDim.x + threadIdx.x;
    if (wi >= mask_words) return;
    const int32_t *ol = outliers + static_cast<size_t>(bh) * o;
    uint32_t bits = 0;
    for (int bit = 0; bit < 32; ++bit) {
        const int j = wi * 32 + bit;
        if (j >= n - n_loc) break;
        int lo = 0, hi = o;  // binary search in the ascending outlier list
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (ol[mid] < j) lo = mid + 1; else hi = mid;
        }
        if (!(lo < o && ol[lo] == j)) bits |= 1u << bit;
    }
    cand[static_cast<size_t>(bh) * mask_words + wi] = bits;
}

// Outlier rows supplied by a caller must be strictly ascending and lie in
// [0, n - n_loc); counts offending rows.
__global__ void validate_outliers_kernel(const int32_t *__restrict__ outliers, int rows, int o, int limit,
                                         int32_t *__restrict__ bad) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const int32_t *ol = outliers + static_cast<size_t>(row) * o;
    bool ok = true;
    for (int a = 0; a < o; ++a) {
        ok = ok && ol[a] >= 0 && ol[a] < limit && (a == 0 || ol[a] > ol[a - 1]);
    }
    if (!ok) atomicAdd(bad, 1);
}

// Bt[b,h][i][e] = B[b,h][e][i]: the right factor stored column-major per head
// so a rank slice of one output column is contiguous.
template <typename T>
__global__ void transpose_b_kernel(const T *__restrict__ B, T *__restrict__ Bt, int r, int d) {
    const int bh = blockIdx.y;
    const size_t off = static_cast<size_t>(bh) * r * d;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < r * d; idx += gridDim.x * blockDim.x) {
        const int e = idx / d, i = idx % d;
        Bt[off + static_cast<size_t>(i) * r + e] = B[off + idx];
    }
}

__global__ void fill_i32_kernel(int32_t *p, int32_t value, size_t count) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < count;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = value;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static hipError_t allow_lds(const void *fn, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

template <typename T, int D>
static hipError_t landmarks_t(const Dims &dm, const void *k_pre, const void *k_rope, const double *theta,
                              void *landmarks, float *min_cos, hipStream_t st) {
    dim3 grid((dm.n + 3) / 4, dm.b * dm.hkv);
    size_t lds = 4ull * dm.c * D * sizeof(float);
    hipError_t e = allow_lds(reinterpret_cast<const void *>(landmarks_kernel<T, D>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((landmarks_kernel<T, D>), grid, dim3(256), lds, st, static_cast<const T *>(k_pre),
                       static_cast<const T *>(k_rope), theta, static_cast<T *>(landmarks), min_cos, dm.n, dm.c,
                       dm.s);
    return hipGetLastError();
}

hipError_t launch_landmarks(const Dims &dm, const void *k_pre, const void *k_rope, const double *theta,
                            void *landmarks, float *min_cos, hipStream_t st) {
    if (dm.bf16) {
        return dm.d == 128 ? landmarks_t<uint16_t, 128>(dm, k_pre, k_rope, theta, landmarks, min_cos, st)
                           : landmarks_t<uint16_t, 64>(dm, k_pre, k_rope, theta, landmarks, min_cos, st);
    }
    return dm.d == 128 ? landmarks_t<float, 128>(dm, k_pre, k_rope, theta, landmarks, min_cos, st)
                       : landmarks_t<float, 64>(dm, k_pre, k_rope, theta, landmarks, min_cos, st);
}

template <typename T, int D>
static hipError_t gather_t(const Dims &dm, const void *k_pre, const void *k_rope, const void *v,
                           const int32_t *outliers, const double *theta, void *k_out, void *v_out, void *k_loc,
                           void *v_loc, hipStream_t st) {
    const int rows = dm.OC + dm.w;
    if (rows == 0) return hipSuccess;
    dim3 grid((rows + 3) / 4, dm.b * dm.hkv);
    hipLaunchKernelGGL((gather_static_kernel<T, D>), grid, dim3(256), 0, st, static_cast<const T *>(k_pre),
                       static_cast<const T *>(k_rope), static_cast<const T *>(v), outliers, theta,
                       static_cast<T *>(k_out), static_cast<T *>(v_out), static_cast<T *>(k_loc),
                       static_cast<T *>(v_loc), dm.s, dm.c, dm.o, dm.w, dm.wcap);
    return hipGetLastError();
}

hipError_t launch_gather_static(const Dims &dm, const void *k_pre, const void *k_rope, const void *v,
                                const int32_t *outliers, const double *theta, void *k_out, void *v_out,
                                void *k_loc, void *v_loc, hipStream_t st) {
    if (dm.bf16) {
        return dm.d == 128
                   ? gather_t<uint16_t, 128>(dm, k_pre, k_rope, v, outliers, theta, k_out, v_out, k_loc, v_loc, st)
                   : gather_t<uint16_t, 64>(dm, k_pre, k_rope, v, outliers, theta, k_out, v_out, k_loc, v_loc, st);
    }
    return dm.d == 128 ? gather_t<float, 128>(dm, k_pre, k_rope, v, outliers, theta, k_out, v_out, k_loc, v_loc, st)
                       : gather_t<float, 64>(dm, k_pre, k_rope, v, outliers, theta, k_out, v_out, k_loc, v_loc, st);
}

hipError_t launch_cand_mask(const Dims &dm, const int32_t *outliers, uint32_t *cand, hipStream_t st) {
    dim3 grid((dm.mask_words + 255) / 256, dm.b * dm.hkv);
    hipLaunchKernelGGL(cand_mask_kernel, grid, dim3(256), 0, st, outliers, cand, dm.n, dm.n_loc, dm.o,
                       dm.mask_words);
    return hipGetLastError();
}

hipError_t launch_validate_outliers(const Dims &dm, const int32_t *outliers, int32_t *bad, hipStream_t st) {
    const int rows = dm.b * dm.hkv;
    hipLaunchKernelGGL(validate_outliers_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, outliers, rows,
                       dm.o, dm.n - dm.n_loc, bad);
    return hipGetLastError();
}

hipError_t launch_transpose_b(const Dims &dm, const void *B, void *Bt, hipStream_t st) {
    dim3 grid((dm.r * dm.d + 255) / 256, dm.b * dm.hkv);
    if (dm.bf16)
        hipLaunchKernelGGL(transpose_b_kernel<uint16_t>, grid, dim3(256), 0, st,
                           static_cast<const uint16_t *>(B), static_cast<uint16_t *>(Bt), dm.r, dm.d);
    else
        hipLaunchKernelGGL(transpose_b_kernel<float>, grid, dim3(256), 0, st, static_cast<const float *>(B),
                           static_cast<float *>(Bt), dm.r, dm.d);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int32_t value, size_t count, hipStream_t st) {
    if (count == 0) return hipSuccess;
    size_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, p, value, count);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode-token append: the key of the token generated at position `pos` is
// rotated exactly like the prefill keys (angle in double precision, result
// rounded once to the storage type) and written, with its value, to row
// `row` of its (sequence, KV head)'s local block.  Thread i owns the RoPE
// pair (i, i + d/2).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(D / 2) void append_kernel(const T *__restrict__ k_new, const T *__restrict__ v_new,
                                                       const double *__restrict__ theta, T *__restrict__ k_loc,
                                                       T *__restrict__ v_loc, int wcap, int row, int pos) {
    constexpr int H = D / 2;
    const int bh = blockIdx.x, i = threadIdx.x;
    const size_t src = static_cast<size_t>(bh) * D;
    const size_t dst = (static_cast<size_t>(bh) * wcap + row) * D;
    float y1, y2;
    rope_store_pair<T>(k_new, nullptr, src, i, H, pos, theta[i], y1, y2);
    Elem<T>::st(k_loc, dst + i, y1);
    Elem<T>::st(k_loc, dst + i + H, y2);
    v_loc[dst + i] = v_new[src + i];
    v_loc[dst + i + H] = v_new[src + i + H];
}

template <typename T, int D>
static hipError_t append_t(const Dims &dm, const void *k_new, const void *v_new, const double *theta, void *k_loc,
                           void *v_loc, int row, int pos, hipStream_t st) {
    hipLaunchKernelGGL((append_kernel<T, D>), dim3(dm.b * dm.hkv), dim3(D / 2), 0, st, static_cast<const T *>(k_new),
                       static_cast<const T *>(v_new), theta, static_cast<T *>(k_loc), static_cast<T *>(v_loc), dm.wcap,
                       row, pos);
    return hipGetLastError();
}

hipError_t launch_append(const Dims &dm, const void *k_new, const void *v_new, const double *theta, void *k_loc,
                         void *v_loc, int row, int pos, hipStream_t st) {
    if (dm.bf16)
        return dm.d == 128 ? append_t<uint16_t, 128>(dm, k_new, v_new, theta, k_loc, v_loc, row, pos, st)
                           : append_t<uint16_t, 64>(dm, k_new, v_new, theta, k_loc, v_loc, row, pos, st);
    return dm.d == 128 ? append_t<float, 128>(dm, k_new, v_new, theta, k_loc, v_loc, row, pos, st)
                       : append_t<float, 64>(dm, k_new, v_new, theta, k_loc, v_loc, row, pos, st);
}


// ---------------------------------------------------------------------------
// Host V in a lossless coded form (bfloat16 chunks of N = 512, 1024 or 2048
// values).  The V fetch is bound by PCIe, so each chunk crosses it in the
// smaller of two forms, in the chunk's own slot of the host buffer (2N bytes).
// Lane l of a chunk's wave owns values l*Q .. l*Q+Q-1 (Q = N / 64).  Both
// forms start with
//   N bytes      sign and mantissa of every value (bits 15 and 6..0), lane l's
//                Q bytes at l*Q,
// and keep the exponents (bits 14..7) as follows.
// The 12-bit form:
//   N / 2 bytes  4-bit offsets from the chunk's base, base = max(0, largest
//                exponent - 14), offset 15 marking an escape; lane l's at
//                N + l*Q/2, value q in bits 4*(q % 8) of word q / 8;
//   4 B each     the escapes: (value index << 8) | exponent, for values whose
//                exponent lies below the base (zeros, tiny values), in index
//                order, from N + N/2.
// The class form (about 10.6 bits a value on normally distributed values,
// whose exponents cluster a little below the chunk's largest): with
// top = max(largest exponent - 1, 0),
//   N / 4 bytes  2-bit classes: 0, 1, 2 = exponent top, top - 1, top - 2;
//                3 = in the side stream; lane l's at N + l*Q/4, value q in
//                bits 2*(q % 16) of word q / 16;
//   S bytes      the side stream, from N + N/4: a 3-bit code for each value of
//                class 3, in value order, code i in bits 3i .. 3i+2 (bit 0 of
//                byte 0 first): 0 = exponent top + 1, x in 1..6 = top - 2 - x,
//                7 = an escape; S = ceil(3 * count / 8) rounded up to 4;
//   4 B each     the escapes, as above, from N + N/4 + S.
// A chunk that takes neither form within 64 escapes (NaN and Inf, whose
// exponent 255 moves the window, or a spread of magnitudes) stays raw.  The
// chunk's code word (device memory) says which: 0 = raw; bit 31 alone = the
// 12-bit form, escape count in bits 16..23, base in bits 0..7; bits 31 and 30
// = the class form, S / 4 in bits 20..27, escape count in bits 8..15, top in
// bits 0..7.
// ---------------------------------------------------------------------------
template <int Q>
__global__ __launch_bounds__(256) void vcode_kernel(const uint16_t *__restrict__ v, uint8_t *__restrict__ out,
                                                    uint32_t *__restrict__ code, long long nchunks, int forms) {
    constexpr int N = 64 * Q;
    constexpr int SW = (3 * N / 8 + 3) / 4 + 4;  // side-stream words per wave (with slack)
    __shared__ uint32_t s_side[4][SW];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t *side = s_side[wave];
    const long long nw = static_cast<long long>(gridDim.x) * 4;
    for (long long ch = static_cast<long long>(blockIdx.x) * 4 + wave; ch < nchunks; ch += nw) {
        // this lane's Q values (2Q bytes: Q / 8 16-byte loads)
        const u32x4 *src = reinterpret_cast<const u32x4 *>(v + ch * N) + lane * (Q / 8);
        uint32_t w[Q / 2];
#pragma unroll
        for (int u = 0; u < Q / 8; ++u) {
            const u32x4 t = src[u];
            w[4 * u] = t[0]; w[4 * u + 1] = t[1]; w[4 * u + 2] = t[2]; w[4 * u + 3] = t[3];
        }
        auto expo = [&](int q) { return static_cast<int>((w[q >> 1] >> (16 * (q & 1) + 7)) & 0xffu); };
        int emax = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) emax = max(emax, expo(q));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) emax = max(emax, __shfl_xor(emax, off, 64));
        const int base = max(0, emax - 14), top = max(emax - 1, 0);
        // per value: 12-bit escape; class-form class and side code
        auto side_code = [&](int e) {  // 3-bit code of a class-3 exponent
            const int d = top - e;
            return e == top + 1 ? 0 : (d >= 3 && d <= 8 ? d - 2 : 7);
        };
        int esc12 = 0, n3 = 0, esc2 = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = expo(q), d = top - e;
            esc12 += e < base ? 1 : 0;
            if (d < 0 || d > 2) {
                ++n3;
                esc2 += side_code(e) == 7 ? 1 : 0;
            }
        }
        const int i12 = wave_incl_scan(esc12), i3 = wave_incl_scan(n3), i2 = wave_incl_scan(esc2);
        const int nesc12 = __builtin_amdgcn_readlane(i12, 63), n3t = __builtin_amdgcn_readlane(i3, 63),
                  nesc2 = __builtin_amdgcn_readlane(i2, 63);
        const int S = (3 * n3t + 31) / 32 * 4;
        const int size12 = (forms & 1) && nesc12 <= 64 ? 3 * N / 2 + 4 * nesc12 : 1 << 30;
        const int size2 =
            (forms & 2) && nesc2 <= 64 && N + N / 4 + S + 4 * nesc2 <= 2 * N ? N + N / 4 + S + 4 * nesc2 : 1 << 30;
        uint8_t *dst = out + ch * 2 * N;
        if (size12 >= (1 << 30) && size2 >= (1 << 30)) {  // stays raw
            u32x4 *d4 = reinterpret_cast<u32x4 *>(dst) + lane * (Q / 8);
#pragma unroll
            for (int u = 0; u < Q / 8; ++u) d4[u] = u32x4{w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]};
            if (lane == 0) code[ch] = 0u;
            continue;
        }
        // sign and mantissa bytes (both forms)
        uint32_t bw[Q / 4];
#pragma unroll
        for (int i = 0; i < Q / 4; ++i) bw[i] = 0u;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint32_t x = (w[q >> 1] >> (16 * (q & 1))) & 0xffffu;
            bw[q >> 2] |= (((x >> 8) & 0x80u) | (x & 0x7fu)) << (8 * (q & 3));
        }
        uint32_t *bp = reinterpret_cast<uint32_t *>(dst) + lane * (Q / 4);
#pragma unroll
        for (int i = 0; i < Q / 4; ++i) bp[i] = bw[i];
        if (size2 < size12) {
            // the class form: classes, side stream (built in LDS), escapes
            uint32_t cw[(Q + 15) / 16];
#pragma unroll
            for (int i = 0; i < (Q + 15) / 16; ++i) cw[i] = 0u;
            for (int i = lane; i < SW; i += 64) side[i] = 0u;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            int pos = 3 * (i3 - n3);   // this lane's first side-stream bit
            int slot = i2 - esc2;      // this lane's first escape entry
            uint32_t *ep = reinterpret_cast<uint32_t *>(dst + N + N / 4 + S);
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int e = expo(q), d = top - e;
                const int c = d >= 0 && d <= 2 ? d : 3;
                cw[q >> 4] |= static_cast<uint32_t>(c) << (2 * (q & 15));
                if (c == 3) {
                    const int x = side_code(e);
                    // a code may straddle two words
                    atomicOr(&side[pos >> 5], static_cast<uint32_t>(x) << (pos & 31));
                    if ((pos & 31) > 29) atomicOr(&side[(pos >> 5) + 1], static_cast<uint32_t>(x) >> (32 - (pos & 31)));
                    pos += 3;
                    if (x == 7) {
                        ep[slot] = (static_cast<uint32_t>(lane * Q + q) << 8) | static_cast<uint32_t>(e);
                        ++slot;
                    }
                }
            }
            if constexpr (Q == 8) {
                reinterpret_cast<uint16_t *>(dst + N)[lane] = static_cast<uint16_t>(cw[0]);
            } else {
                uint32_t *cp = reinterpret_cast<uint32_t *>(dst + N) + lane * (Q / 16);
#pragma unroll
                for (int i = 0; i < Q / 16; ++i) cp[i] = cw[i];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint32_t *sp = reinterpret_cast<uint32_t *>(dst + N + N / 4);
            for (int i = lane; i < S / 4; i += 64) sp[i] = side[i];
            if (lane == 0)
                code[ch] = 0xC0000000u | (static_cast<uint32_t>(S / 4) << 20) | (static_cast<uint32_t>(nesc2) << 8) |
                           static_cast<uint32_t>(top);
        } else {
            // the 12-bit form: offsets and escapes
            uint32_t nw4[Q / 8];
#pragma unroll
            for (int i = 0; i < Q / 8; ++i) nw4[i] = 0u;
            int slot = i12 - esc12;  // this lane's first escape entry
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int e = expo(q);
                const bool esc = e < base;
                nw4[q >> 3] |= static_cast<uint32_t>(esc ? 15 : e - base) << (4 * (q & 7));
                if (esc) {
                    reinterpret_cast<uint32_t *>(dst + 3 * N / 2)[slot] =
                        (static_cast<uint32_t>(lane * Q + q) << 8) | static_cast<uint32_t>(e);
                    ++slot;
                }
            }
            uint32_t *np = reinterpret_cast<uint32_t *>(dst + N) + lane * (Q / 8);
#pragma unroll
            for (int i = 0; i < Q / 8; ++i) np[i] = nw4[i];
            if (lane == 0) code[ch] = 0x80000000u | (static_cast<uint32_t>(nesc12) << 16) | static_cast<uint32_t>(base);
        }
    }
}

int vcode_values(const Dims &dm) {
    const int N = dm.c * dm.d;
    return dm.bf16 && (N == 512 || N == 1024 || N == 2048) ? N : 0;
}

hipError_t launch_vcode(const Dims &dm, int forms, const void *v, void *out, uint32_t *code, long long nchunks,
                        hipStream_t st) {
    if (nchunks <= 0) return hipSuccess;
    const int blocks = static_cast<int>(std::min<long long>((nchunks + 3) / 4, 8192));
    switch (vcode_values(dm)) {
        case 512:
            hipLaunchKernelGGL(vcode_kernel<8>, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(v),
                               static_cast<uint8_t *>(out), code, nchunks, forms);
            break;
        case 1024:
            hipLaunchKernelGGL(vcode_kernel<16>, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(v),
                               static_cast<uint8_t *>(out), code, nchunks, forms);
            break;
        case 2048:
            hipLaunchKernelGGL(vcode_kernel<32>, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(v),
                               static_cast<uint8_t *>(out), code, nchunks, forms);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace skv
