// Low-rank factors of the pre-RoPE keys on the device (review page, section
// 三, Algorithm 1 step 1: A, B <- SVD(K_pre)), in double precision.
//
// Per sequence the keys form the s x n matrix M (n = h_kv * d; column h*d + i
// is head h's dimension i).  The right singular vectors of M are the
// eigenvectors of the Gram matrix G = M^T M, and the rank-r factors are
// A = M V_r (= U_r S_r) and B = V_r^T split by head, so A . B is M's best
// rank-r approximation.  Kernels:
//   gram_kernel          G in 128 x 128 tiles of its upper triangle on the
//                        fp64 matrix cores, the rows of M split into slices
//                        that each write a partial
//   gram_sum_kernel      G = the slices' partials summed in slice order,
//                        mirrored; the eigenvector accumulator set to I
//   the eigensolver, the parallel two-sided (cyclic) Jacobi method in one of
//   two round forms:
//     super-blocks of 2 JB indices, JB = 16 (the default) or 32:
//       jacobi_block_solve_kernel, jacobi_block_apply_kernel,
//       jacobi_block_vec_kernel (described at their definitions)
//     single index pairs:
//       jacobi_rot_kernel    for each of the round's n/2 disjoint index pairs
//                            the plane rotation that zeroes the pair's
//                            off-diagonal entry
//       jacobi_apply_kernel  G <- R^T G R (one 2 x 2 block per thread)
//       jacobi_vec_kernel    V <- V R
//   offdiag_kernel       off-diagonal and total squared sums (convergence)
//   diag_kernel          the eigenvalues (G's diagonal), read by the host to
//                        pick the r largest
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
// tp <= tq, over rows [slice * rps, min(s, (slice + 1) * rps)) of M.  Slabs of
// 16 rows of both column ranges are staged in LDS as doubles (the next slab
// loaded into registers while this one is used; columns past n read zeros),
// and wave w accumulates the 64 x 64 quadrant (rows 64 (w / 2), columns
// 64 (w % 2)) of the tile on the double-precision matrix cores: per 4 rows of
// the slab, 4 x 4 products of 16 x 16 blocks, the A operand the slab's P
// columns (M^T) and the B operand its Q columns.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) double f64x4;

// D += A B on the double-precision matrix cores, 16 x 16 x 4: lane l gives
// A[l % 16][l / 16] and B[l / 16][l % 16], and holds D[4 j + l / 16][l % 16]
// in element j (rows interleaved across the four elements).
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 d) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, d, 0, 0, 0);
}

constexpr int kGPad = kGT + 8;  // LDS row of a staged slab (doubles), off the 64-bank period

template <typename T>
__global__ __launch_bounds__(256) void gram_kernel(const T *__restrict__ kp, double *__restrict__ part, int hkv,
                                                   int s, int d, int n, int nt, int rps, int nseq) {
    __shared__ double Ps[kGK][kGPad];
    __shared__ double Qs[kGK][kGPad];
    int x = blockIdx.x, tp = 0;
    while (x >= nt - tp) { x -= nt - tp; ++tp; }
    const int tq = tp + x;
    const int slice = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
    const int wy = wave >> 1, wx = wave & 1;
    const int t_begin = slice * rps, t_end = min(s, t_begin + rps);
    // staging: row tid / 16 of the slab, columns 8 * (tid % 16) .. + 8 of each tile
    const int srow = tid >> 4, scol = (tid & 15) * 8;
    const int pc = tp * kGT + scol, qc = tq * kGT + scol;
    const T *kseq = kp + static_cast<size_t>(seq) * hkv * s * d;
    auto src = [&](int col, int t) {  // M[t, col] of a column below n
        return kseq + (static_cast<size_t>(col / d) * s + t) * d + col % d;
    };
    f64x4 acc[4][4] = {};
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
#pragma unroll
        for (int k0 = 0; k0 < kGK; k0 += 4) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = Ps[k0 + lk][64 * wy + 16 * i + lr];  // (M^T)[p][t] = M[t][p]
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Qs[k0 + lk][64 * wx + 16 * j + lr];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f64(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    double *out = part + (static_cast<size_t>(slice) * nseq + seq) * n * n;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int p = tp * kGT + 64 * wy + 16 * i + 4 * e + lk;
            if (p >= n) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = tq * kGT + 64 * wx + 16 * j + lr;
                if (q < n) out[static_cast<size_t>(p) * n + q] = acc[i][j][e];
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

// The rotation (c, s) of a pair with diagonal entries a, b and off-diagonal
// entry e: R = [[c, s], [-s, c]] makes the pair's block of R^T G R diagonal.
// t = s / c is the root of smaller magnitude of t^2 + 2 theta t - 1 = 0,
// theta = (b - a) / (2e), here written t = 2e sgn(h) / (|h| + sqrt(h^2 + 4e^2))
// with h = b - a (the Gram entries are far from overflowing the squares).
// c = 1 / sqrt(1 + t^2) comes from the hardware reciprocal square root refined
// by two Newton steps y <- y (3 - w y^2) / 2: w = 1 + t^2 lies in [1, 2], the
// estimate's relative error is about 2^-23 and each step squares it, so c is
// correct to a few ulps and c^2 + s^2 = 1 to the same.  Entries below 1e-18
// of sqrt(|a b|), or zero, are left alone.
__device__ __forceinline__ double2 jacobi_rotation(double a, double b, double e) {
    double c = 1.0, sn = 0.0;
    if (e != 0.0 && e * e > 1e-36 * fabs(a * b)) {
        const double h = b - a, e2 = 2.0 * e;
        const double t = (h >= 0.0 ? e2 : -e2) / (fabs(h) + sqrt(h * h + e2 * e2));
        const double w = fma(t, t, 1.0);
        double y = __builtin_amdgcn_rsq(w);
        y = y * fma(-0.5 * w, y * y, 1.5);
        y = y * fma(-0.5 * w, y * y, 1.5);
        c = y;
        sn = t * y;
    }
    return make_double2(c, sn);
}

// One round's rotations: position i pairs indices 2i and 2i + 1.
__global__ __launch_bounds__(256) void jacobi_rot_kernel(const double *__restrict__ G, double2 *__restrict__ rot,
                                                         int n) {
    const int h = n / 2, i = blockIdx.x * 256 + threadIdx.x, seq = blockIdx.y;
    if (i >= h) return;
    const double *g = G + static_cast<size_t>(seq) * n * n;
    rot[static_cast<size_t>(seq) * h + i] =
        jacobi_rotation(g[static_cast<size_t>(2 * i) * n + 2 * i], g[static_cast<size_t>(2 * i + 1) * n + 2 * i + 1],
                        g[static_cast<size_t>(2 * i) * n + 2 * i + 1]);
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

// ---------------------------------------------------------------------------
// Block Jacobi.  The n indices form nb = n / JB blocks of JB (16 or 32), kept
// (like the single indices above) in the order of the current round: round
// position I holds the block pair (2I, 2I+1), a JS = 2 JB index super-block,
// and between rounds the blocks move round the same cycle as single indices
// do (next_place over nb places), so nb - 1 rounds pair every two blocks
// once: a sweep.  A round:
//   jacobi_block_solve_kernel  each super-block's JS x JS diagonal tile,
//                              diagonalised in LDS by cyclic two-sided Jacobi
//                              sweeps (the plane rotations above, JS/2
//                              disjoint pairs at a time), giving the tile's
//                              orthogonal Q_I; the rotated tile goes to its
//                              next places
//   jacobi_block_apply_kernel  the other tiles: Q_I^T G_IJ Q_J at the next
//                              places, so that G <- J^T G J with
//                              J = diag(Q_0, Q_1, ...)
//   jacobi_block_vec_kernel    V <- V J
// As in the single-index method every pair of indices is rotated in every
// sweep (inside the super-block that holds both), in JB times fewer rounds,
// each a few small products instead of a pass per rotation.  The apply and
// eigenvector launches move all of G and V whatever JB is, so larger blocks
// (fewer rounds) move fewer bytes a sweep.
// ---------------------------------------------------------------------------
template <int JB>
struct JBlk {
    static constexpr int JS = 2 * JB;            // indices per super-block (a round position)
    static constexpr int Pad = JS + 1;           // LDS row stride of a JS x JS tile (doubles)
    static constexpr int NT = (JS / 2) * (JS / 2);  // solve threads: one 2 x 2 block each per step
    static constexpr int NBK = JS / 16;          // 16 x 16 MFMA blocks per tile side
};

// Index at position k (of JS) in step t (of JS - 1) of an inner sweep: index
// 0 stays, the others advance one place round a circle of JS - 1 each step,
// and the step pairs positions k and JS - 1 - k, so JS - 1 steps pair every
// two indices once.
template <int JS>
__device__ __forceinline__ int inner_pos(int k, int t) { return k == 0 ? 0 : 1 + (k - 1 + t) % (JS - 1); }

// Place in the next round of row or column u (< 2 JB) of super-block I.
template <int JB>
__device__ __forceinline__ int block_next(int I, int u, int nb) {
    return next_place(2 * I + u / JB, nb) * JB + u % JB;
}

// Workgroup (I, seq).  Inner sweeps run while the tile's off-diagonal mass is
// above 1e-30 of its total and still falling a hundredfold per sweep once
// below 1e-22 (the rounding floor), at most max_sweeps.  The tile is double
// buffered: a step reads its pairs' 2 x 2 diagonal blocks and its own block
// from one buffer and writes the other, so a step takes one barrier.  Each
// lane works out one rotation, its column pair's, and takes its row pair's
// from the lane of the same wave that holds it.
template <int JB>
__global__ __launch_bounds__(JBlk<JB>::NT) void jacobi_block_solve_kernel(const double *__restrict__ G,
                                                                        double *__restrict__ Gn,
                                                                        double *__restrict__ Qb, int n,
                                                                        int max_sweeps) {
    constexpr int JS = JBlk<JB>::JS, Pad = JBlk<JB>::Pad, NT = JBlk<JB>::NT, NW = NT / 64, H = JS / 2;
    __shared__ double S[2][JS][Pad];
    __shared__ double Qm[JS][Pad];
    __shared__ double red[2][NW];
    const int I = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x, nb = n / JB;
    const size_t base = static_cast<size_t>(seq) * n * n;
    const double *g = G + base + static_cast<size_t>(I) * JS * n + I * JS;
    for (int x = tid; x < JS * JS; x += NT) {
        const int u = x / JS, v = x % JS;
        S[0][u][v] = g[static_cast<size_t>(u) * n + v];
        Qm[u][v] = u == v ? 1.0 : 0.0;
    }
    __syncthreads();
    const int br = tid / H, bc = tid % H;  // this thread's 2 x 2 block: row pair br, column pair bc
    int cur = 0;
    double prev = 0.0;
    for (int sw = 0; sw < max_sweeps; ++sw) {
        double off = 0.0, tot = 0.0;
        for (int x = tid; x < JS * JS; x += NT) {
            const double v = S[cur][x / JS][x % JS];
            tot += v * v;
            if (x / JS != x % JS) off += v * v;
        }
        off = wave_sum_d(off);
        tot = wave_sum_d(tot);
        if ((tid & 63) == 0) {
            red[0][tid >> 6] = off;
            red[1][tid >> 6] = tot;
        }
        __syncthreads();
        double o = 0.0, a = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            o += red[0][w];
            a += red[1][w];
        }
        const bool stop = !(o > 1e-30 * a) || (sw > 0 && o <= 1e-22 * a && o > 0.01 * prev);
        prev = o;
        if (stop) break;  // the same in every thread (red is rewritten only after the steps' barriers)
        for (int t = 0; t < JS - 1; ++t) {
            const double(*X)[Pad] = S[cur];
            double(*Y)[Pad] = S[cur ^ 1];
            const int p0 = inner_pos<JS>(br, t), q0 = inner_pos<JS>(JS - 1 - br, t);
            const int p1 = inner_pos<JS>(bc, t), q1 = inner_pos<JS>(JS - 1 - bc, t);
            // this lane's rotation is pair bc's (bc = lane mod H, H dividing
            // 64); pair br's (br < H) is lane br's, read across the wave
            const double2 rj = jacobi_rotation(X[p1][p1], X[q1][q1], X[p1][q1]);
            const double2 ri = make_double2(__shfl(rj.x, br, 64), __shfl(rj.y, br, 64));
            const double x00 = X[p0][p1], x01 = X[p0][q1], x10 = X[q0][p1], x11 = X[q0][q1];
            const double y00 = rj.x * x00 - rj.y * x01, y01 = rj.y * x00 + rj.x * x01;
            const double y10 = rj.x * x10 - rj.y * x11, y11 = rj.y * x10 + rj.x * x11;
            double z00 = ri.x * y00 - ri.y * y10, z01 = ri.x * y01 - ri.y * y11;
            double z10 = ri.y * y00 + ri.x * y10, z11 = ri.y * y01 + ri.x * y11;
            if (br == bc) z01 = z10 = 0.0;
            Y[p0][p1] = z00;
            Y[p0][q1] = z01;
            Y[q0][p1] = z10;
            Y[q0][q1] = z11;
            // Q <- Q R on columns p1, q1 of rows 2 br and 2 br + 1 (this thread's alone)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const int row = 2 * br + w;
                const double qa = Qm[row][p1], qb = Qm[row][q1];
                Qm[row][p1] = rj.x * qa - rj.y * qb;
                Qm[row][q1] = rj.y * qa + rj.x * qb;
            }
            cur ^= 1;
            __syncthreads();
        }
    }
    double *q = Qb + (static_cast<size_t>(seq) * (n / JS) + I) * JS * JS;
    for (int x = tid; x < JS * JS; x += NT) {
        const int u = x / JS, v = x % JS;
        q[x] = Qm[u][v];
        Gn[base + static_cast<size_t>(block_next<JB>(I, u, nb)) * n + block_next<JB>(I, v, nb)] = S[cur][u][v];
    }
}

// One wave per tile pair (I, J), I < J: Y = Q_I^T G_IJ Q_J on the matrix
// cores (T = G_IJ Q_J, staged in LDS as the second product's B operand), Y
// written at tile (I, J)'s next places and its transpose at tile (J, I)'s,
// which keeps G exactly symmetric.
template <int JB>
__global__ __launch_bounds__(64) void jacobi_block_apply_kernel(const double *__restrict__ G, double *__restrict__ Gn,
                                                                const double *__restrict__ Qb, int n) {
    constexpr int JS = JBlk<JB>::JS, Pad = JBlk<JB>::Pad, NBK = JBlk<JB>::NBK;
    __shared__ double T[JS][Pad];
    const int ns = n / JS, seq = blockIdx.y, l = threadIdx.x, lr = l & 15, lk = l >> 4, nb = n / JB;
    int p = blockIdx.x, I = 0;
    while (p >= ns - 1 - I) {
        p -= ns - 1 - I;
        ++I;
    }
    const int J = I + 1 + p;
    const size_t base = static_cast<size_t>(seq) * n * n;
    const double *g = G + base + static_cast<size_t>(I) * JS * n + J * JS;
    const double *qi = Qb + (static_cast<size_t>(seq) * ns + I) * JS * JS;
    const double *qj = Qb + (static_cast<size_t>(seq) * ns + J) * JS * JS;
    // The contraction index k runs as 16 c + 4 (l / 16) + e: a lane reads four
    // consecutive k of its row (32 bytes, a whole 128-byte row segment per 16
    // lanes) and feeds them to four products, element e to the e-th.
    f64x4 acc[NBK][NBK] = {};
#pragma unroll
    for (int c = 0; c < JS / 16; ++c) {
        const int k0 = 16 * c + 4 * lk;
        f64x4 a[NBK];
#pragma unroll
        for (int rb = 0; rb < NBK; ++rb)
            a[rb] = *reinterpret_cast<const f64x4 *>(g + static_cast<size_t>(16 * rb + lr) * n + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double b[NBK];
#pragma unroll
            for (int cb = 0; cb < NBK; ++cb) b[cb] = qj[(k0 + e) * JS + 16 * cb + lr];
#pragma unroll
            for (int rb = 0; rb < NBK; ++rb)
#pragma unroll
                for (int cb = 0; cb < NBK; ++cb) acc[rb][cb] = mfma_f64(a[rb][e], b[cb], acc[rb][cb]);
        }
    }
#pragma unroll
    for (int rb = 0; rb < NBK; ++rb)
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                T[16 * rb + 4 * j + lk][16 * cb + lr] = acc[rb][cb][j];
                acc[rb][cb][j] = 0.0;
            }
    __syncthreads();
    // Y = Q_I^T T, accumulated in acc again
#pragma unroll 4
    for (int st = 0; st < JS / 4; ++st) {
        const int k = 4 * st + lk;
        double a[NBK], b[NBK];
#pragma unroll
        for (int rb = 0; rb < NBK; ++rb) a[rb] = qi[k * JS + 16 * rb + lr];  // (Q_I^T)[row][k] = Q_I[k][row]
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb) b[cb] = T[k][16 * cb + lr];
#pragma unroll
        for (int rb = 0; rb < NBK; ++rb)
#pragma unroll
            for (int cb = 0; cb < NBK; ++cb) acc[rb][cb] = mfma_f64(a[rb], b[cb], acc[rb][cb]);
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < NBK; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int u = 16 * rb + 4 * j + lk;
            const size_t row = base + static_cast<size_t>(block_next<JB>(I, u, nb)) * n;
#pragma unroll
            for (int cb = 0; cb < NBK; ++cb) {
                Gn[row + block_next<JB>(J, 16 * cb + lr, nb)] = acc[rb][cb][j];
                T[u][16 * cb + lr] = acc[rb][cb][j];
            }
        }
    __syncthreads();
    // tile (J, I): row v of it is column v of Y; a pass writes 64 / JS rows
    const int u = l % JS, cu = block_next<JB>(I, u, nb);
#pragma unroll 4
    for (int it = 0; it < JS * JS / 64; ++it) {
        const int v = it * (64 / JS) + l / JS;
        Gn[base + static_cast<size_t>(block_next<JB>(J, v, nb)) * n + cu] = T[u][v];
    }
}

// V <- V J: one wave per 64 rows of super-block J's JS columns, times Q_J on
// the matrix cores, written at the next round's column places (rows stay).
template <int JB>
__global__ __launch_bounds__(64) void jacobi_block_vec_kernel(const double *__restrict__ V, double *__restrict__ Vn,
                                                              const double *__restrict__ Qb, int n) {
    constexpr int JS = JBlk<JB>::JS, NBK = JBlk<JB>::NBK;
    const int ns = n / JS, J = blockIdx.y, seq = blockIdx.z, l = threadIdx.x, lr = l & 15, lk = l >> 4, nb = n / JB;
    const int r0 = blockIdx.x * 64;
    const size_t base = static_cast<size_t>(seq) * n * n;
    const double *qj = Qb + (static_cast<size_t>(seq) * ns + J) * JS * JS;
    // k runs as 16 c + 4 (l / 16) + e, as in the apply kernel
    f64x4 acc[4][NBK] = {};
#pragma unroll
    for (int c = 0; c < JS / 16; ++c) {
        const int k0 = 16 * c + 4 * lk;
        f64x4 a[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int row = r0 + rb * 16 + lr;
            a[rb] = row < n ? *reinterpret_cast<const f64x4 *>(V + base + static_cast<size_t>(row) * n + J * JS + k0)
                            : f64x4{0.0, 0.0, 0.0, 0.0};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            double b[NBK];
#pragma unroll
            for (int cb = 0; cb < NBK; ++cb) b[cb] = qj[(k0 + e) * JS + 16 * cb + lr];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int cb = 0; cb < NBK; ++cb) acc[rb][cb] = mfma_f64(a[rb][e], b[cb], acc[rb][cb]);
        }
    }
    int col[NBK];
#pragma unroll
    for (int cb = 0; cb < NBK; ++cb) col[cb] = block_next<JB>(J, 16 * cb + lr, nb);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = r0 + rb * 16 + 4 * j + lk;
            if (row < n) {
#pragma unroll
                for (int cb = 0; cb < NBK; ++cb) Vn[base + static_cast<size_t>(row) * n + col[cb]] = acc[rb][cb][j];
            }
        }
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

// out[seq][x] = G[seq][x][x]
__global__ __launch_bounds__(256) void diag_kernel(const double *__restrict__ G, double *__restrict__ out, int n) {
    const int x = blockIdx.x * 256 + threadIdx.x, seq = blockIdx.y;
    if (x < n) out[static_cast<size_t>(seq) * n + x] = G[static_cast<size_t>(seq) * n * n + static_cast<size_t>(x) * (n + 1)];
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

// 4 consecutive stored values as doubles (8 B of bfloat16, 16 B of binary32)
template <typename T>
__device__ __forceinline__ void load4_f64(const T *p, bool ok, double *o) {
    if constexpr (sizeof(T) == 2) {
        const u32x2 r = ok ? *reinterpret_cast<const u32x2 *>(p) : u32x2{0u, 0u};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            o[2 * e] = static_cast<double>(__uint_as_float(r[e] << 16));
            o[2 * e + 1] = static_cast<double>(__uint_as_float(r[e] & 0xffff0000u));
        }
    } else {
        const u32x4 r = ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = static_cast<double>(__uint_as_float(r[e]));
    }
}

constexpr int kFX = 16;  // columns of M (rows of W) per staged slab

// A[t][j] = M[t] . W[:, j] for j < rr (zero for rr <= j < r), accumulated in
// double and rounded once.  Workgroup: 64 rows t, every column j; wave w the
// 16 rows 16 w .. + 15, as NCB >= r / 16 products of 16 x 16 blocks on the
// double-precision matrix cores.  Slabs of 16 columns of M (transposed into
// LDS) and the same 16 rows of W (zero past rr) are staged, the next slab
// loaded into registers while this one is used.
template <typename T, int NCB>
__global__ __launch_bounds__(256) void factor_a_kernel(const T *__restrict__ kp, const double *__restrict__ W,
                                                       T *__restrict__ A, int hkv, int s, int d, int r, int rr) {
    constexpr int wcols = 16 * NCB, ncb = NCB;
    __shared__ double Ms[kFX][64 + 1];
    __shared__ double Ws[kFX][wcols + 8];
    const int n = hkv * d;
    const int seq = blockIdx.z, t0 = blockIdx.x * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
    const T *kseq = kp + static_cast<size_t>(seq) * hkv * s * d;
    const double *wseq = W + static_cast<size_t>(seq) * n * rr;
    // staging: M row t0 + tid / 4, columns x0 + 4 (tid % 4) .. + 4; W entries
    // tid + 256 u of the slab's 16 x wcols (u < ncb)
    const int mt = tid >> 2, mx = (tid & 3) * 4;
    auto load_slab = [&](int x0, double *mv, double *wv) {
        const int t = t0 + mt, x = x0 + mx;
        load4_f64(kseq + (static_cast<size_t>(x / d) * s + min(t, s - 1)) * d + x % d, t < s, mv);
#pragma unroll
        for (int u = 0; u < ncb; ++u) {
            const int e = tid + 256 * u, row = e / wcols, col = e % wcols;
            wv[u] = col < rr ? wseq[static_cast<size_t>(x0 + row) * rr + col] : 0.0;
        }
    };
    f64x4 acc[NCB] = {};
    double mv[4], wv[NCB];
    load_slab(0, mv, wv);
    for (int x0 = 0; x0 < n; x0 += kFX) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Ms[mx + e][mt] = mv[e];
#pragma unroll
        for (int u = 0; u < ncb; ++u) {
            const int e = tid + 256 * u;
            Ws[e / wcols][e % wcols] = wv[u];
        }
        __syncthreads();
        if (x0 + kFX < n) load_slab(x0 + kFX, mv, wv);
#pragma unroll
        for (int k0 = 0; k0 < kFX; k0 += 4) {
            const double a = Ms[k0 + lk][16 * wave + lr];  // A[row][k] = M[t0 + 16 w + row][x0 + k]
#pragma unroll
            for (int cb = 0; cb < ncb; ++cb) acc[cb] = mfma_f64(a, Ws[k0 + lk][16 * cb + lr], acc[cb]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int cb = 0; cb < ncb; ++cb) {
        const int jj = 16 * cb + lr;
        if (jj >= r) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 16 * wave + 4 * e + lk;
            if (t < s) Elem<T>::st(A, (static_cast<size_t>(seq) * s + t) * r + jj, Elem<T>::rnd_d(jj < rr ? acc[cb][e] : 0.0));
        }
    }
}

// factor_a_kernel with the fewest column blocks (of 4, 8, 10, 12, 16) that
// cover r <= 256
template <typename T>
void launch_factor_a(const T *kp, const double *W, T *A, int hkv, int s, int d, int r, int rr, dim3 grid,
                     hipStream_t st) {
    const int ncb = (r + 15) / 16;
    if (ncb <= 4) hipLaunchKernelGGL((factor_a_kernel<T, 4>), grid, dim3(256), 0, st, kp, W, A, hkv, s, d, r, rr);
    else if (ncb <= 8) hipLaunchKernelGGL((factor_a_kernel<T, 8>), grid, dim3(256), 0, st, kp, W, A, hkv, s, d, r, rr);
    else if (ncb <= 10) hipLaunchKernelGGL((factor_a_kernel<T, 10>), grid, dim3(256), 0, st, kp, W, A, hkv, s, d, r, rr);
    else if (ncb <= 12) hipLaunchKernelGGL((factor_a_kernel<T, 12>), grid, dim3(256), 0, st, kp, W, A, hkv, s, d, r, rr);
    else hipLaunchKernelGGL((factor_a_kernel<T, 16>), grid, dim3(256), 0, st, kp, W, A, hkv, s, d, r, rr);
}

// ---------------------------------------------------------------------------
// Host side: batches of up to 8 sequences; the eigensolver's sweeps run until
// the off-diagonal mass (sum of squares) is below 1e-22 of the total, or below
// 1e-20 and no longer falling tenfold per sweep (the rounding floor), or 30
// sweeps have run.  Each sweep's measure is read while the next sweep runs, so
// one sweep past the deciding one is done; the method converges quadratically
// there, so that sweep takes a mass below 1e-22 down to the rounding floor
// (about 1e-30 on these matrices).  SKV_FACTOR_LOG=1 prints the measure after
// every sweep.
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
    // row slices of the Gram launch: at least about 1024 workgroups, and of up
    // to four times that many the count whose workgroups fill the last round
    // of resident ones best (two per CU), slices of at least 256 rows
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                   hipSuccess || cus < 1)
        cus = 256;
    const int max_ns = (s + 255) / 256;
    const int ns0 = std::max(1, std::min(max_ns, (1024 + npair * group - 1) / (npair * group)));
    int ns = ns0;
    {
        const long long slots = 2LL * cus;
        double best = 0.0;
        for (int c = ns0; c <= std::min(max_ns, 4 * ns0); ++c) {
            const long long wgs = static_cast<long long>(npair) * group * c;
            const double fill = static_cast<double>(wgs) / static_cast<double>((wgs + slots - 1) / slots * slots);
            if (fill > best + 1e-9) {
                best = fill;
                ns = c;
            }
        }
    }
    const int rps = ((s + ns - 1) / ns + kGK - 1) / kGK * kGK;
    const size_t nn = static_cast<size_t>(n) * n;
    const size_t esz = bf16 ? 2 : 4;
    double *part = nullptr, *G0 = nullptr, *G1 = nullptr, *V0 = nullptr, *V1 = nullptr, *W = nullptr, *dg = nullptr;
    double2 *rot = nullptr, *offs = nullptr, *offs_pin = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    int32_t *sel = nullptr;
    int rc = 0, max_sweeps = 0;
    std::vector<double> diag(static_cast<size_t>(group) * n);
    std::vector<int32_t> sel_h(static_cast<size_t>(group) * rr);
    std::vector<int32_t> order(n);
    const bool log_sweeps = std::getenv("SKV_FACTOR_LOG") != nullptr;
    // block rounds: blocks of 16 where n is a multiple of 32 with at least 4
    // of them (the round cycle needs 4 places).  Blocks of 32 halve the
    // rounds and the apply and eigenvector passes a sweep, but their tile
    // solve (63 steps over 16 waves) costs more than that saves (128K b8:
    // 78.7 against 70.4 ms of rounds a layer); SKV_FACTOR_BLOCK=32 asks for
    // them where n is a multiple of 64 with at least 4, 0 keeps the
    // single-index rounds
    const char *fb = std::getenv("SKV_FACTOR_BLOCK");
    const int fbv = fb ? std::atoi(fb) : 1;
    const bool fit32 = n % 64 == 0 && n / 32 >= 4, fit16 = n % 32 == 0 && n / 16 >= 4;
    const int jb = fbv == 0 ? 0 : (fbv == 32 && fit32 ? 32 : (fit16 ? 16 : 0));
    const bool blockwise = jb > 0;
    const int js = 2 * jb, nsb = blockwise ? n / js : 0;
    // inner sweeps per super-block and round at most: one sweep a round costs
    // the fewest rounds' time (the outer sweeps finish what it leaves)
    const char *fi = std::getenv("SKV_FACTOR_INNER");
    const int inner = fi && std::atoi(fi) > 0 ? std::atoi(fi) : 1;
    double *Qb = nullptr;
    FZ_HIP(hipMalloc(&part, static_cast<size_t>(ns) * group * nn * 8));
    FZ_HIP(hipMalloc(&G0, group * nn * 8));
    FZ_HIP(hipMalloc(&G1, group * nn * 8));
    FZ_HIP(hipMalloc(&V0, group * nn * 8));
    FZ_HIP(hipMalloc(&V1, group * nn * 8));
    FZ_HIP(hipMalloc(&W, static_cast<size_t>(group) * n * rr * 8));
    FZ_HIP(hipMalloc(&dg, static_cast<size_t>(group) * n * 8));
    FZ_HIP(hipMalloc(&rot, static_cast<size_t>(group) * h * sizeof(double2)));
    FZ_HIP(hipMalloc(&offs, static_cast<size_t>(group) * 2 * 64 * sizeof(double2)));
    FZ_HIP(hipHostMalloc(reinterpret_cast<void **>(&offs_pin), static_cast<size_t>(group) * 2 * 64 * sizeof(double2),
                         hipHostMallocDefault));
    FZ_HIP(hipEventCreateWithFlags(&ev[0], hipEventDisableTiming));
    FZ_HIP(hipEventCreateWithFlags(&ev[1], hipEventDisableTiming));
    FZ_HIP(hipMalloc(&sel, static_cast<size_t>(group) * rr * 4));
    if (blockwise) FZ_HIP(hipMalloc(&Qb, static_cast<size_t>(group) * nsb * js * js * 8));
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
        // one sweep's rounds and its measure, read back through slot k % 2
        auto enqueue_sweep = [&](int k) -> hipError_t {
            if (blockwise) {
                for (int round = 0; round < n / jb - 1; ++round) {
                    if (jb == 32) {
                        hipLaunchKernelGGL(jacobi_block_solve_kernel<32>, dim3(nsb, gc), dim3(JBlk<32>::NT), 0, st,
                                           Gc, Gn, Qb, n, inner);
                        hipLaunchKernelGGL(jacobi_block_apply_kernel<32>, dim3(nsb * (nsb - 1) / 2, gc), dim3(64), 0,
                                           st, Gc, Gn, Qb, n);
                        hipLaunchKernelGGL(jacobi_block_vec_kernel<32>, dim3((n + 63) / 64, nsb, gc), dim3(64), 0, st,
                                           Vc, Vn, Qb, n);
                    } else {
                        hipLaunchKernelGGL(jacobi_block_solve_kernel<16>, dim3(nsb, gc), dim3(JBlk<16>::NT), 0, st,
                                           Gc, Gn, Qb, n, inner);
                        hipLaunchKernelGGL(jacobi_block_apply_kernel<16>, dim3(nsb * (nsb - 1) / 2, gc), dim3(64), 0,
                                           st, Gc, Gn, Qb, n);
                        hipLaunchKernelGGL(jacobi_block_vec_kernel<16>, dim3((n + 63) / 64, nsb, gc), dim3(64), 0, st,
                                           Vc, Vn, Qb, n);
                    }
                    std::swap(Gc, Gn);
                    std::swap(Vc, Vn);
                }
            } else {
                for (int round = 0; round < n - 1; ++round) {
                    hipLaunchKernelGGL(jacobi_rot_kernel, dim3((h + 255) / 256, gc), dim3(256), 0, st, Gc, rot, n);
                    hipLaunchKernelGGL(jacobi_apply_kernel, dim3((h / 16) * (h / 16), gc), dim3(256), 0, st, Gc, Gn,
                                       rot, n);
                    hipLaunchKernelGGL(jacobi_vec_kernel,
                                       dim3(static_cast<unsigned>((static_cast<size_t>(n) * h + 255) / 256), gc),
                                       dim3(256), 0, st, Vc, Vn, rot, n);
                    std::swap(Gc, Gn);
                    std::swap(Vc, Vn);
                }
            }
            const size_t slot = static_cast<size_t>(k & 1) * group * 64;
            hipLaunchKernelGGL(offdiag_kernel, dim3(64, gc), dim3(256), 0, st, Gc, offs + slot, n);
            hipError_t e = hipGetLastError();
            if (e == hipSuccess)
                e = hipMemcpyAsync(offs_pin + slot, offs + slot, static_cast<size_t>(gc) * 64 * sizeof(double2),
                                   hipMemcpyDeviceToHost, st);
            if (e == hipSuccess) e = hipEventRecord(ev[k & 1], st);
            return e;
        };
        std::vector<double> prev_rel(gc, 1.0);
        int queued = 1;
        FZ_HIP(enqueue_sweep(0));
        for (int sweep = 0; sweep < 30; ++sweep) {
            // the next sweep is queued before this one's measure is read, so
            // the device stays busy while the host waits; a sweep past
            // convergence only refines the result
            if (queued < 30) FZ_HIP(enqueue_sweep(queued++));
            FZ_HIP(hipEventSynchronize(ev[sweep & 1]));
            const double2 *m = offs_pin + static_cast<size_t>(sweep & 1) * group * 64;
            // converged: the off-diagonal mass is at 1e-22 of the total, or
            // it has reached the rounding floor (below 1e-20 and no longer
            // falling tenfold per sweep)
            bool done_all = true;
            for (int q = 0; q < gc; ++q) {
                double off = 0.0, tot = 0.0;
                for (int k = 0; k < 64; ++k) {
                    off += m[q * 64 + k].x;
                    tot += m[q * 64 + k].y;
                }
                const double rel = tot > 0.0 ? off / tot : 0.0;
                if (log_sweeps) fprintf(stderr, "factorize: sequence %d sweep %d off/total %.3e\n", g0 + q, sweep, rel);
                if (!(rel <= 1e-22 || (rel <= 1e-20 && rel > 0.1 * prev_rel[q]))) done_all = false;
                prev_rel[q] = rel;
            }
            if (done_all) {
                // the queued sweep's measure, for the log
                if (log_sweeps && queued == sweep + 2) {
                    FZ_HIP(hipEventSynchronize(ev[(queued - 1) & 1]));
                    const double2 *mq = offs_pin + static_cast<size_t>((queued - 1) & 1) * group * 64;
                    for (int q = 0; q < gc; ++q) {
                        double off = 0.0, tot = 0.0;
                        for (int k = 0; k < 64; ++k) {
                            off += mq[q * 64 + k].x;
                            tot += mq[q * 64 + k].y;
                        }
                        fprintf(stderr, "factorize: sequence %d sweep %d (queued) off/total %.3e\n", g0 + q,
                                queued - 1, tot > 0.0 ? off / tot : 0.0);
                    }
                }
                break;
            }
        }
        const int sweep = queued;
        if (sweep > max_sweeps) max_sweeps = sweep;
        // the rr largest eigenvalues (ties: lower place first), the diagonals
        // gathered on the device and read in one copy
        hipLaunchKernelGGL(diag_kernel, dim3((n + 255) / 256, gc), dim3(256), 0, st, Gc, dg, n);
        FZ_HIP(hipGetLastError());
        FZ_HIP(hipMemcpyAsync(diag.data(), dg, static_cast<size_t>(gc) * n * 8, hipMemcpyDeviceToHost, st));
        FZ_HIP(hipStreamSynchronize(st));
        for (int q = 0; q < gc; ++q) {
            const double *dq = diag.data() + static_cast<size_t>(q) * n;
            for (int x = 0; x < n; ++x) order[x] = x;
            std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return dq[a] > dq[b]; });
            for (int j = 0; j < rr; ++j) sel_h[static_cast<size_t>(q) * rr + j] = order[j];
        }
        FZ_HIP(hipMemcpyAsync(sel, sel_h.data(), static_cast<size_t>(gc) * rr * 4, hipMemcpyHostToDevice, st));
        {
            const dim3 gb(static_cast<unsigned>((static_cast<size_t>(n) * r + 255) / 256), gc);
            const dim3 ga((s + 63) / 64, 1, gc);
            if (bf16) {
                hipLaunchKernelGGL(gather_b_kernel<uint16_t>, gb, dim3(256), 0, st, Vc, sel, W,
                                   reinterpret_cast<uint16_t *>(Bg), n, d, r, rr);
                launch_factor_a(reinterpret_cast<const uint16_t *>(kp), W, reinterpret_cast<uint16_t *>(Ag), hkv, s,
                                d, r, rr, ga, st);
            } else {
                hipLaunchKernelGGL(gather_b_kernel<float>, gb, dim3(256), 0, st, Vc, sel, W,
                                   reinterpret_cast<float *>(Bg), n, d, r, rr);
                launch_factor_a(reinterpret_cast<const float *>(kp), W, reinterpret_cast<float *>(Ag), hkv, s, d, r,
                                rr, ga, st);
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
    if (dg) (void)hipFree(dg);
    if (rot) (void)hipFree(rot);
    if (offs) (void)hipFree(offs);
    if (offs_pin) (void)hipHostFree(offs_pin);
    if (ev[0]) (void)hipEventDestroy(ev[0]);
    if (ev[1]) (void)hipEventDestroy(ev[1]);
    if (sel) (void)hipFree(sel);
    if (Qb) (void)hipFree(Qb);
    if (sweeps_out) *sweeps_out = max_sweeps;
    return rc;
}
#undef FZ_HIP

}  // namespace skv
