// Low-rank factors of the pre-RoPE keys on the device (review page, section
// 三, Algorithm 1 step 1: A, B <- SVD(K_pre)), in double precision.
//
// Per sequence the keys form the s x n matrix M (n = h_kv * d; column h*d + i
// is head h's dimension i).  The right singular vectors of M are the
// eigenvectors of the Gram matrix G = M^T M, and the rank-r factors are
// A = M V_r (= U_r S_r) and B = V_r^T split by head, so A . B is M's best
// rank-r approximation.  Kernels:
//   gram_kernel          G in 128 x 128 tiles of its upper triangle, the rows
//                        of M split into slices that each write a partial
//   gram_sum_kernel      G = the slices' partials summed in slice order,
//                        mirrored; the eigenvector accumulator set to I
//   jacobi_rot_kernel    one round of the parallel two-sided Jacobi method:
//                        for each of the round's n/2 disjoint index pairs the
//                        plane rotation that zeroes the pair's off-diagonal
//                        entry
//   jacobi_apply_kernel  G <- R^T G R (one 2 x 2 block per thread)
//   jacobi_vec_kernel    V <- V R
//   offdiag_kernel       off-diagonal and total squared sums (convergence)
//   gather_b_kernel      W = the r leading eigenvectors, and B
//   factor_a_kernel      A = M W, rounded once to the storage type
//
// Round order.  The matrix is kept in the order of the current round: round
// position i holds the index pair (2i, 2i+1), so a thread's 2 x 2 block is two
// 16-byte reads.  Between rounds every index except 0 moves one place along
// the cycle 2 -> 4 -> ... -> n-2 -> n-1 -> n-3 -> ... -> 3 -> 1 -> 2 (the
// circle method of round-robin tournaments): two indices at cycle places a
// and b are paired when a + b + 2t is a fixed value mod n - 1, which happens
// once in n - 1 rounds, so n - 1 rounds are one sweep over all pairs.  The
// rotated blocks and eigenvector columns are written straight to their next
// places (a second buffer); the eigenvalues end on the diagonal and their
// eigenvectors in the same columns of V.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <utility>
#include <vector>

#include "skv_device.h"
#include "skv_dims.h"

namespace skv {

namespace {

constexpr int kGT = 128;  // Gram tile (rows and columns)
constexpr int kGK = 16;   // rows of M per staged slab

// 8 consecutive stored values (16 B of bfloat16, 32 B of binary32) as doubles
template <typename T>
__device__ __forceinline__ void load8_f64(const T *p, bool ok, double *o) {
    if constexpr (sizeof(T) == 2) {
        const u32x4 r = ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[2 * e] = static_cast<double>(__uint_as_float(r[e] << 16));
            o[2 * e + 1] = static_cast<double>(__uint_as_float(r[e] & 0xffff0000u));
        }
    } else {
        u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u};
        if (ok) {
            r0 = reinterpret_cast<const u32x4 *>(p)[0];
            r1 = reinterpret_cast<const u32x4 *>(p)[1];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[e] = static_cast<double>(__uint_as_float(r0[e]));
            o[4 + e] = static_cast<double>(__uint_as_float(r1[e]));
        }
    }
}

// Place of index position x in the next round (see the header).
__device__ __forceinline__ int next_place(int x, int n) {
    if (x == 0) return 0;
    if (x == 1) return 2;
    if (x & 1) return x - 2;
    return x == n - 2 ? n - 1 : x + 2;
}

}  // namespace

// ---------------------------------------------------------------------------
// Partial Gram tiles.  Workgroup (pair, slice, seq): output tile (tp, tq),
// tp <= tq, over rows [slice * rps, min(s, (slice + 1) * rps)) of M.  Thread
// (ty, tx) accumulates rows tp*128 + ty + 16i and columns tq*128 + tx + 16j
// (i, j < 8) in double; slabs of 16 rows of both column ranges are staged in
// LDS as doubles, the next slab loaded into registers while this one is used.
// Columns past n read zeros.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void gram_kernel(const T *__restrict__ kp, double *__restrict__ part, int hkv,
                                                   int s, int d, int n, int nt, int rps, int nseq) {
    __shared__ double Ps[kGK][kGT];
    __shared__ double Qs[kGK][kGT];
    int x = blockIdx.x, tp = 0;
    while (x >= nt - tp) { x -= nt - tp; ++tp; }
    const int tq = tp + x;
    const int slice = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int t_begin = slice * rps, t_end = min(s, t_begin + rps);
    // staging: row tid / 16 of the slab, columns 8 * (tid % 16) .. + 8 of each tile
    const int srow = tid >> 4, scol = (tid & 15) * 8;
    const int pc = tp * kGT + scol, qc = tq * kGT + scol;
    const T *kseq = kp + static_cast<size_t>(seq) * hkv * s * d;
    auto src = [&](int col, int t) {  // M[t, col] of a column below n
        return kseq + (static_cast<size_t>(col / d) * s + t) * d + col % d;
    };
    double acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
    double pv[8], qv[8];
    {
        const int t = t_begin + srow;
        load8_f64(src(min(pc, n - 8), min(t, s - 1)), t < t_end && pc < n, pv);
        load8_f64(src(min(qc, n - 8), min(t, s - 1)), t < t_end && qc < n, qv);
    }
    for (int t0 = t_begin; t0 < t_end; t0 += kGK) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Ps[srow][scol + e] = pv[e];
            Qs[srow][scol + e] = qv[e];
        }
        __syncthreads();
        if (t0 + kGK < t_end) {
            const int t = t0 + kGK + srow;
            load8_f64(src(min(pc, n - 8), min(t, s - 1)), t < t_end && pc < n, pv);
            load8_f64(src(min(qc, n - 8), min(t, s - 1)), t < t_end && qc < n, qv);
        }
#pragma unroll 4
        for (int k = 0; k < kGK; ++k) {
            double a[8], b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = Ps[k][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = Qs[k][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    double *out = part + (static_cast<size_t>(slice) * nseq + seq) * n * n;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = tp * kGT + ty + 16 * i;
        if (p >= n) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = tq * kGT + tx + 16 * j;
            if (q < n) out[static_cast<size_t>(p) * n + q] = acc[i][j];
        }
    }
}

// G[p][q] = sum over slices (in slice order) of the tile holding (p, q) or
// its mirror; V = I.
__global__ __launch_bounds__(256) void gram_sum_kernel(const double *__restrict__ part, double *__restrict__ G,
                                                       double *__restrict__ V, int n, int ns, int nseq) {
    const size_t nn = static_cast<size_t>(n) * n;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    const int seq = blockIdx.y;
    if (idx >= nn) return;
    const int p = static_cast<int>(idx / n), q = static_cast<int>(idx % n);
    const size_t src = (p / kGT <= q / kGT) ? static_cast<size_t>(p) * n + q : static_cast<size_t>(q) * n + p;
    double sum = 0.0;
    for (int sl = 0; sl < ns; ++sl) sum += part[(static_cast<size_t>(sl) * nseq + seq) * nn + src];
    G[seq * nn + idx] = sum;
    V[seq * nn + idx] = p == q ? 1.0 : 0.0;
}

// The rotation (c, s) of round position i: with a = G[2i][2i], b =
// G[2i+1][2i+1], e = G[2i][2i+1], R = [[c, s], [-s, c]] makes the block of
// R^T G R at the pair diagonal: t = s/c is the root of smaller magnitude of
// t^2 + 2 theta t - 1 = 0, theta = (b - a) / (2e).  Entries negligible
// against the diagonal (or zero) are left alone.
__global__ __launch_bounds__(256) void jacobi_rot_kernel(const double *__restrict__ G, double2 *__restrict__ rot,
                                                         int n) {
    const int h = n / 2, i = blockIdx.x * 256 + threadIdx.x, seq = blockIdx.y;
    if (i >= h) return;
    const double *g = G + static_cast<size_t>(seq) * n * n;
    const double a = g[static_cast<size_t>(2 * i) * n + 2 * i], b = g[static_cast<size_t>(2 * i + 1) * n + 2 * i + 1];
    const double e = g[static_cast<size_t>(2 * i) * n + 2 * i + 1];
    double c = 1.0, sn = 0.0;
    if (e != 0.0 && fabs(e) > 1e-18 * sqrt(fabs(a) * fabs(b))) {
        const double theta = (b - a) / (2.0 * e);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        c = 1.0 / sqrt(t * t + 1.0);
        sn = t * c;
    }
    rot[static_cast<size_t>(seq) * h + i] = make_double2(c, sn);
}

// Block (i, j) of the round: X' = R_i^T X R_j, written at the next round's
// places of rows 2i, 2i+1 and columns 2j, 2j+1.  Every block of both
// triangles is a thread of its own (the matrix is stored whole), so each
// thread reads and writes only its own block.  Diagonal blocks are set
// diagonal.
__global__ __launch_bounds__(256) void jacobi_apply_kernel(const double *__restrict__ G, double *__restrict__ Gn,
                                                           const double2 *__restrict__ rot, int n) {
    const int h = n / 2, tiles = h / 16;
    const int bi = blockIdx.x / tiles, bj = blockIdx.x % tiles, seq = blockIdx.y;
    const int i = bi * 16 + (threadIdx.x >> 4), j = bj * 16 + (threadIdx.x & 15);
    const size_t base = static_cast<size_t>(seq) * n * n;
    const double *g = G + base;
    double *gn = Gn + base;
    const double2 x0 = *reinterpret_cast<const double2 *>(g + static_cast<size_t>(2 * i) * n + 2 * j);
    const double2 x1 = *reinterpret_cast<const double2 *>(g + static_cast<size_t>(2 * i + 1) * n + 2 * j);
    const double2 ri = rot[static_cast<size_t>(seq) * h + i], rj = rot[static_cast<size_t>(seq) * h + j];
    // Y = X R_j
    const double y00 = rj.x * x0.x - rj.y * x0.y, y01 = rj.y * x0.x + rj.x * x0.y;
    const double y10 = rj.x * x1.x - rj.y * x1.y, y11 = rj.y * x1.x + rj.x * x1.y;
    // X' = R_i^T Y
    double z00 = ri.x * y00 - ri.y * y10, z01 = ri.x * y01 - ri.y * y11;
    double z10 = ri.y * y00 + ri.x * y10, z11 = ri.y * y01 + ri.x * y11;
    if (i == j) z01 = z10 = 0.0;
    const size_t r0 = static_cast<size_t>(next_place(2 * i, n)) * n, r1 = static_cast<size_t>(next_place(2 * i + 1, n)) * n;
    const int c0 = next_place(2 * j, n), c1 = next_place(2 * j + 1, n);
    gn[r0 + c0] = z00;
    gn[r0 + c1] = z01;
    gn[r1 + c0] = z10;
    gn[r1 + c1] = z11;
}

// V <- V R_j on columns 2j, 2j+1 of every row, written at the next places.
__global__ __launch_bounds__(256) void jacobi_vec_kernel(const double *__restrict__ V, double *__restrict__ Vn,
                                                         const double2 *__restrict__ rot, int n) {
    const int h = n / 2;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    const int seq = blockIdx.y;
    if (idx >= static_cast<size_t>(n) * h) return;
    const int row = static_cast<int>(idx / h), j = static_cast<int>(idx % h);
    const size_t base = static_cast<size_t>(seq) * n * n + static_cast<size_t>(row) * n;
    const double2 v = *reinterpret_cast<const double2 *>(V + base + 2 * j);
    const double2 rj = rot[static_cast<size_t>(seq) * h + j];
    Vn[base + next_place(2 * j, n)] = rj.x * v.x - rj.y * v.y;
    Vn[base + next_place(2 * j + 1, n)] = rj.y * v.x + rj.x * v.y;
}

// Squared sums of the off-diagonal entries and of all entries: workgroup
// `blk` of 64 per matrix writes its share (a fixed order, so the sums are
// reproducible).
__global__ __launch_bounds__(256) void offdiag_kernel(const double *__restrict__ G, double2 *__restrict__ out, int n) {
    __shared__ double so[256], st[256];
    const size_t nn = static_cast<size_t>(n) * n;
    const int seq = blockIdx.y;
    const double *g = G + seq * nn;
    double off = 0.0, tot = 0.0;
    for (size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; idx < nn; idx += 64 * 256) {
        const double v = g[idx] * g[idx];
        tot += v;
        if (idx / n != idx % n) off += v;
    }
    so[threadIdx.x] = off;
    st[threadIdx.x] = tot;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            so[threadIdx.x] += so[threadIdx.x + w];
            st[threadIdx.x] += st[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) out[seq * 64 + blockIdx.x] = make_double2(so[0], st[0]);
}

// W[x][j] = V[x][sel[j]] (j < rr, double), and B[h][j][i] = V[h*d + i][sel[j]]
// rounded to the storage type (zero for rr <= j < r).
template <typename T>
__global__ __launch_bounds__(256) void gather_b_kernel(const double *__restrict__ V, const int32_t *__restrict__ sel,
                                                       double *__restrict__ W, T *__restrict__ B, int n, int d,
                                                       int r, int rr) {
    const int seq = blockIdx.y;
    const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<size_t>(n) * r) return;
    const int x = static_cast<int>(idx / r), j = static_cast<int>(idx % r);
    const double v = j < rr ? V[static_cast<size_t>(seq) * n * n + static_cast<size_t>(x) * n + sel[seq * rr + j]] : 0.0;
    if (j < rr) W[(static_cast<size_t>(seq) * n + x) * rr + j] = v;
    const int hh = x / d, i = x % d;
    Elem<T>::st(B, ((static_cast<size_t>(seq) * (n / d) + hh) * r + j) * d + i, Elem<T>::rnd_d(v));
}

// A[t][j] = M[t] . W[:, j] for j < rr (zero for rr <= j < r), accumulated in
// double and rounded once.  Workgroup: 64 rows t x 64 columns j; slabs of 32
// columns of M (transposed into LDS) and 32 rows of W.
template <typename T>
__global__ __launch_bounds__(256) void factor_a_kernel(const T *__restrict__ kp, const double *__restrict__ W,
                                                       T *__restrict__ A, int hkv, int s, int d, int r, int rr) {
    __shared__ double Ms[32][64 + 1];
    __shared__ double Ws[32][64];
    const int n = hkv * d;
    const int seq = blockIdx.z, t0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const T *kseq = kp + static_cast<size_t>(seq) * hkv * s * d;
    const double *wseq = W + static_cast<size_t>(seq) * n * rr;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    // staging: M rows t0 + tid / 4, columns x0 + 8 * (tid % 4) .. + 8;
    // W rows x0 + tid / 8, columns j0 + 8 * (tid % 8) .. + 8
    const int mt = tid >> 2, mx = (tid & 3) * 8, wx = tid >> 3, wj = (tid & 7) * 8;
    for (int x0 = 0; x0 < n; x0 += 32) {
        {
            const int t = t0 + mt, x = x0 + mx;
            double v[8];
            load8_f64(kseq + (static_cast<size_t>(x / d) * s + min(t, s - 1)) * d + x % d, t < s, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) Ms[mx + e][mt] = v[e];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = j0 + wj + e;
                Ws[wx][wj + e] = j < rr ? wseq[static_cast<size_t>(x0 + wx) * rr + j] : 0.0;
            }
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < 32; ++k) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = Ms[k][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Ws[k][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty + 16 * i;
        if (t >= s) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int jj = j0 + tx + 16 * j;
            if (jj < r) Elem<T>::st(A, (static_cast<size_t>(seq) * s + t) * r + jj, Elem<T>::rnd_d(jj < rr ? acc[i][j] : 0.0));
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: batches of up to 8 sequences; the eigensolver's sweeps run until
// the off-diagonal mass (sum of squares) is below 1e-28 of the total, or below
// 1e-20 and no longer falling tenfold per sweep (the rounding floor), or 30
// sweeps have run.  SKV_FACTOR_LOG=1 prints the measure after every sweep.
// ---------------------------------------------------------------------------
#define FZ_HIP(expr)                                                                         \
    do {                                                                                     \
        hipError_t e_ = (expr);                                                              \
        if (e_ != hipSuccess) {                                                              \
            *why = std::string(#expr) + ": " + hipGetErrorString(e_);                        \
            rc = -5;                                                                         \
            goto done;                                                                       \
        }                                                                                    \
    } while (0)

int factorize_device(int bf16, int batch, int hkv, int s, int d, int r, const void *k_pre, void *A, void *B,
                     hipStream_t st, std::string *why, int *sweeps_out) {
    const int n = hkv * d, h = n / 2, rr = r < n ? r : n;
    const int group = batch < 8 ? batch : 8;
    const int nt = (n + kGT - 1) / kGT, npair = nt * (nt + 1) / 2;
    int ns = (1024 + npair * group - 1) / (npair * group);
    const int max_ns = (s + 255) / 256;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    const int rps = ((s + ns - 1) / ns + kGK - 1) / kGK * kGK;
    const size_t nn = static_cast<size_t>(n) * n;
    const size_t esz = bf16 ? 2 : 4;
    double *part = nullptr, *G0 = nullptr, *G1 = nullptr, *V0 = nullptr, *V1 = nullptr, *W = nullptr;
    double2 *rot = nullptr, *offs = nullptr;
    int32_t *sel = nullptr;
    int rc = 0, max_sweeps = 0;
    std::vector<double2> offs_h(static_cast<size_t>(group) * 64);
    std::vector<double> diag(n);
    std::vector<int32_t> sel_h(static_cast<size_t>(group) * rr);
    std::vector<int32_t> order(n);
    const bool log_sweeps = std::getenv("SKV_FACTOR_LOG") != nullptr;
    FZ_HIP(hipMalloc(&part, static_cast<size_t>(ns) * group * nn * 8));
    FZ_HIP(hipMalloc(&G0, group * nn * 8));
    FZ_HIP(hipMalloc(&G1, group * nn * 8));
    FZ_HIP(hipMalloc(&V0, group * nn * 8));
    FZ_HIP(hipMalloc(&V1, group * nn * 8));
    FZ_HIP(hipMalloc(&W, static_cast<size_t>(group) * n * rr * 8));
    FZ_HIP(hipMalloc(&rot, static_cast<size_t>(group) * h * sizeof(double2)));
    FZ_HIP(hipMalloc(&offs, static_cast<size_t>(group) * 64 * sizeof(double2)));
    FZ_HIP(hipMalloc(&sel, static_cast<size_t>(group) * rr * 4));
    for (int g0 = 0; g0 < batch; g0 += group) {
        const int gc = batch - g0 < group ? batch - g0 : group;
        const char *kp = static_cast<const char *>(k_pre) + static_cast<size_t>(g0) * hkv * s * d * esz;
        char *Ag = static_cast<char *>(A) + static_cast<size_t>(g0) * s * r * esz;
        char *Bg = static_cast<char *>(B) + static_cast<size_t>(g0) * hkv * r * d * esz;
        if (bf16)
            hipLaunchKernelGGL(gram_kernel<uint16_t>, dim3(npair, ns, gc), dim3(256), 0, st,
                               reinterpret_cast<const uint16_t *>(kp), part, hkv, s, d, n, nt, rps, gc);
        else
            hipLaunchKernelGGL(gram_kernel<float>, dim3(npair, ns, gc), dim3(256), 0, st,
                               reinterpret_cast<const float *>(kp), part, hkv, s, d, n, nt, rps, gc);
        FZ_HIP(hipGetLastError());
        hipLaunchKernelGGL(gram_sum_kernel, dim3(static_cast<unsigned>((nn + 255) / 256), gc), dim3(256), 0, st, part,
                           G0, V0, n, ns, gc);
        FZ_HIP(hipGetLastError());
        double *Gc = G0, *Gn = G1, *Vc = V0, *Vn = V1;
        int sweep = 0;
        std::vector<double> prev_rel(gc, 1.0);
        for (; sweep < 30; ++sweep) {
            for (int round = 0; round < n - 1; ++round) {
                hipLaunchKernelGGL(jacobi_rot_kernel, dim3((h + 255) / 256, gc), dim3(256), 0, st, Gc, rot, n);
                hipLaunchKernelGGL(jacobi_apply_kernel, dim3((h / 16) * (h / 16), gc), dim3(256), 0, st, Gc, Gn, rot,
                                   n);
                hipLaunchKernelGGL(jacobi_vec_kernel, dim3(static_cast<unsigned>((static_cast<size_t>(n) * h + 255) / 256), gc),
                                   dim3(256), 0, st, Vc, Vn, rot, n);
                std::swap(Gc, Gn);
                std::swap(Vc, Vn);
            }
            FZ_HIP(hipGetLastError());
            hipLaunchKernelGGL(offdiag_kernel, dim3(64, gc), dim3(256), 0, st, Gc, offs, n);
            FZ_HIP(hipMemcpyAsync(offs_h.data(), offs, static_cast<size_t>(gc) * 64 * sizeof(double2),
                                  hipMemcpyDeviceToHost, st));
            FZ_HIP(hipStreamSynchronize(st));
            // converged: the off-diagonal mass is at 1e-28 of the total, or
            // it has reached the rounding floor (below 1e-20 and no longer
            // falling tenfold per sweep)
            bool done_all = true;
            for (int q = 0; q < gc; ++q) {
                double off = 0.0, tot = 0.0;
                for (int k = 0; k < 64; ++k) {
                    off += offs_h[q * 64 + k].x;
                    tot += offs_h[q * 64 + k].y;
                }
                const double rel = tot > 0.0 ? off / tot : 0.0;
                if (log_sweeps) fprintf(stderr, "factorize: sequence %d sweep %d off/total %.3e\n", g0 + q, sweep, rel);
                if (!(rel <= 1e-28 || (rel <= 1e-20 && rel > 0.1 * prev_rel[q]))) done_all = false;
                prev_rel[q] = rel;
            }
            if (done_all) {
                ++sweep;
                break;
            }
        }
        if (sweep > max_sweeps) max_sweeps = sweep;
        // the rr largest eigenvalues (ties: lower place first)
        for (int q = 0; q < gc; ++q) {
            FZ_HIP(hipMemcpy2DAsync(diag.data(), 8, Gc + q * nn, static_cast<size_t>(n + 1) * 8, 8, n,
                                    hipMemcpyDeviceToHost, st));
            FZ_HIP(hipStreamSynchronize(st));
            for (int x = 0; x < n; ++x) order[x] = x;
            std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return diag[a] > diag[b]; });
            for (int j = 0; j < rr; ++j) sel_h[static_cast<size_t>(q) * rr + j] = order[j];
        }
        FZ_HIP(hipMemcpyAsync(sel, sel_h.data(), static_cast<size_t>(gc) * rr * 4, hipMemcpyHostToDevice, st));
        {
            const dim3 gb(static_cast<unsigned>((static_cast<size_t>(n) * r + 255) / 256), gc);
            const dim3 ga((s + 63) / 64, (r + 63) / 64, gc);
            if (bf16) {
                hipLaunchKernelGGL(gather_b_kernel<uint16_t>, gb, dim3(256), 0, st, Vc, sel, W,
                                   reinterpret_cast<uint16_t *>(Bg), n, d, r, rr);
                hipLaunchKernelGGL(factor_a_kernel<uint16_t>, ga, dim3(256), 0, st,
                                   reinterpret_cast<const uint16_t *>(kp), W, reinterpret_cast<uint16_t *>(Ag), hkv,
                                   s, d, r, rr);
            } else {
                hipLaunchKernelGGL(gather_b_kernel<float>, gb, dim3(256), 0, st, Vc, sel, W,
                                   reinterpret_cast<float *>(Bg), n, d, r, rr);
                hipLaunchKernelGGL(factor_a_kernel<float>, ga, dim3(256), 0, st, reinterpret_cast<const float *>(kp),
                                   W, reinterpret_cast<float *>(Ag), hkv, s, d, r, rr);
            }
            FZ_HIP(hipGetLastError());
        }
        FZ_HIP(hipStreamSynchronize(st));
    }
done:
    (void)hipStreamSynchronize(st);
    if (part) (void)hipFree(part);
    if (G0) (void)hipFree(G0);
    if (G1) (void)hipFree(G1);
    if (V0) (void)hipFree(V0);
    if (V1) (void)hipFree(V1);
    if (W) (void)hipFree(W);
    if (rot) (void)hipFree(rot);
    if (offs) (void)hipFree(offs);
    if (sel) (void)hipFree(sel);
    if (sweeps_out) *sweeps_out = max_sweeps;
    return rc;
}
#undef FZ_HIP

}  // namespace skv
