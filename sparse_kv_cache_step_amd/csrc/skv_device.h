// Device-side helpers shared by the gfx950 kernels of the ShadowKV decode
// step: storage conversions, wave64 reductions and scans, order-preserving
// float keys for radix selection, and RoPE with a double-precision angle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "skv_dims.h"

namespace skv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Raw buffer access.  A buffer resource covers `bytes` bytes from `base`
// (bytes < kOob, checked on the host by the layer's shape validation); a load at an offset at or past the end returns zeros and a
// store there is dropped, by the hardware and without a memory access.
// Kernels use this for predicated loads and stores: every lane issues the
// same instruction (kOob as the offset switches a lane off), so there are no
// branches around memory operations and the compiler's wait counts stay
// exact.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
constexpr int kOob = 0x7fff0000;  // an offset past every resource, far from 2^32

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld128(Rsrc r, int off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ uint32_t buf_ld32(Rsrc r, int off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
__device__ __forceinline__ void buf_st32(float v, Rsrc r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_st64(float2 v, Rsrc r, int off) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v.x), __float_as_uint(v.y)}, r, off, 0, 0);
}
__device__ __forceinline__ void buf_st128(float4 v, Rsrc r, int off) {
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)}, r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Storage types: binary32 (float) or bfloat16 carried as its 16 raw bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Nearest bfloat16 of a double, rounded once (ties to even): 8 significant
// bits, binary32's exponent range (subnormal spacing 2^-133).
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
    if (x == 0.0 || !isfinite(x)) return f32_to_bf16_bits(static_cast<float>(x));
    int e;
    frexp(x, &e);
    int q = e - 8;
    if (q < -133) q = -133;
    const double y = ldexp(rint(ldexp(x, -q)), q);  // a bfloat16 value (or 2^128)
    return static_cast<uint16_t>(__float_as_uint(static_cast<float>(y)) >> 16);
}

template <typename T> struct Elem;

template <> struct Elem<float> {
    static __device__ __forceinline__ float ld(const float *p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float *p, size_t i, float v) { p[i] = v; }
    // storage value of a double (one rounding)
    static __device__ __forceinline__ float rnd_d(double v) { return static_cast<float>(v); }
};

template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t *p, size_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void st(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }
    static __device__ __forceinline__ float rnd_d(double v) { return bf16_bits_to_f32(f64_to_bf16_bits(v)); }
};

// ---------------------------------------------------------------------------
// Wave64 reductions.
// ---------------------------------------------------------------------------
// The float reductions take the four in-row steps with DPP moves (quad
// exchanges, then the mirrors within 8 and within 16 lanes) and the two
// cross-row steps with the gfx950 permlane swaps, so no step goes through
// LDS.  Every step combines a lane with its partner symmetrically, so all 64
// lanes end with bitwise the same result.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <typename Op> __device__ __forceinline__ float wave_reduce(float v, Op op) {
    v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
    v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
    v = op(v, dpp_mov<0x141>(v));  // row_half_mirror: lane i <-> 7 - i within 8
    v = op(v, dpp_mov<0x140>(v));  // row_mirror: lane i <-> 15 - i within 16
    // rows 0/1 and 2/3: the swap leaves row 2j in one result and row 2j+1 in
    // the other, lane for lane
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    // lanes l and l + 32 likewise
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each row of
// 16 lanes with DPP row shifts (lanes shifted in from outside the row add 0),
// then each row adds the totals of the rows before it, read from lanes 15,
// 31 and 47.  No step goes through LDS.
template <int CTRL> __device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_i32<0x111>(x);  // row_shr:1
    x += dpp_i32<0x112>(x);  // row_shr:2
    x += dpp_i32<0x114>(x);  // row_shr:4
    x += dpp_i32<0x118>(x);  // row_shr:8
    const int row = (threadIdx.x & 63) >> 4;
    const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
              t2 = __builtin_amdgcn_readlane(x, 47);
    return x + (row > 0 ? t0 : 0) + (row > 1 ? t1 : 0) + (row > 2 ? t2 : 0);
}

__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// Merge two (running max, sum of exp(x - max)) pairs.
__device__ __forceinline__ void ms_merge(float &m, float &s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    if (mn == -INFINITY) { m = mn; s = 0.f; return; }
    s = s * expf(m - mn) + s2 * expf(m2 - mn);
    m = mn;
}

// (max, sum) merge across lanes whose index differs in the bits of `mask_bits`
// (xor distances 1, 2, 4, ... up to the highest bit set).
__device__ __forceinline__ void ms_reduce_lanes(float &m, float &s, int width) {
    for (int off = 1; off < width; off <<= 1) {
        float m2 = __shfl_xor(m, off, kWave);
        float s2 = __shfl_xor(s, off, kWave);
        ms_merge(m, s, m2, s2);
    }
}

// Exclusive count of `flag` over the threads of the block (thread order) and
// the block total.  Every thread of the block must call it.  `wcnt` holds at
// least blockDim.x / 64 ints of shared memory.
__device__ __forceinline__ int block_excl_count(bool flag, int *wcnt, int *total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    const uint64_t m = __ballot(flag);
    const uint64_t lt = lane ? (~0ull >> (kWave - lane)) : 0ull;
    const int pre = __popcll(m & lt);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < nwaves; ++w) {
        int c = wcnt[w];
        before += (w < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return before + pre;
}

// ---------------------------------------------------------------------------
// Order-preserving 32-bit key of a float (larger float -> larger key, -0 and
// +0 equal); 0 is below every finite or infinite value's key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float x) {
    x = x + 0.0f;  // -0 -> +0
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// RoPE.  The angle pos * theta is formed in double precision and reduced to
// [-pi, pi] with a two-part 2*pi before single-precision sin/cos, so large
// positions (2.5e5) keep ~1e-7 accuracy.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void angle_sincos(double a, float *sn, float *cs) {
    const double kInv2Pi = 0.15915494309189535;
    const double k2PiHi = 6.283185307179586;
    const double k2PiLo = 2.4492935982947064e-16;
    double turns = rint(a * kInv2Pi);
    double red = fma(-turns, k2PiHi, a);
    red = fma(-turns, k2PiLo, red);
    sincosf(static_cast<float>(red), sn, cs);
}

__device__ __forceinline__ void rope_rotate(float x1, float x2, float sn, float cs, float &y1, float &y2) {
    y1 = x1 * cs - x2 * sn;
    y2 = x2 * cs + x1 * sn;
}

__device__ __forceinline__ bool mask_bit(const uint32_t *words, int j) {
    return (words[j >> 5] >> (j & 31)) & 1u;
}

}  // namespace skv
