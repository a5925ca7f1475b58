// Derived sizes of one layer and the kernel launchers of the ShadowKV step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace skv {

// Tile sizes.
constexpr int kScoreTile = 256;   // chunks per scoring workgroup (4 waves x 64)
constexpr int kSelectThreads = 1024;  // one workgroup per (sequence, KV head) row
constexpr int kGroupSlice = 1024;     // chunks per group-score workgroup
constexpr int kQkTile = 64;       // keys per generic QK workgroup
constexpr int kQkMfmaTile = 256;  // keys per MFMA QK workgroup (4 waves x 64)
constexpr int kPvTile = 256;      // keys per PV workgroup
constexpr int kMaxGroup = 16;     // query heads per KV head

struct Dims {
    int b, hq, hkv, d, s, c, r, o, k;
    int cap;         // V cache slots (chunks) per (sequence, KV head), >= k
    int w;           // local keys attended: the window, plus the tokens appended so far
    int wcap;        // rows of the local K/V buffers: window + append capacity
    int n;           // chunks per sequence
    int n_loc;       // chunks of the local window
    int G;           // query heads per KV head
    int GP;          // G rounded up to 4, 8 or 16 (MFMA QK variant)
    int mask_words;  // ceil(n / 32)
    int score_tiles; // ceil(n / kScoreTile): scoring workgroups per row
    int wtiles;      // ceil(n / 64): 64-chunk softmax tiles per row
    int OC, KC, NK;  // outlier keys, rebuilt keys, all keys per (b, h_kv) (NK with w)
    int pv_tiles;    // ceil(NK / kPvTile)
    int esize;       // bytes per stored element
    int bf16;        // storage type
    int r_pad;       // rank rounded up to 32
    float scale;     // 1 / sqrt(d)
    int tslice;      // chunks per slice of the two-pass Top-K (0: by k)
    int kpw;         // rebuilt keys per wave of the fused attention kernel (64, 48, 32 or 16)
    int attn_nw;     // waves per fused attention workgroup (4, or 8 where built)
};

// Low-rank key factors of `batch` sequences (A, B <- SVD(K_pre) through the
// Gram matrix's eigenvectors, in double precision; see factor.hip).  Returns
// 0, or -5 with the failing HIP call in *why.
int factorize_device(int bf16, int batch, int hkv, int s, int d, int r, const void *k_pre, void *A, void *B,
                     hipStream_t st, std::string *why, int *sweeps_out);

// ---- launchers (return the launch status) ----------------------------------
// Prefill.
hipError_t launch_landmarks(const Dims &dm, const void *k_pre, const void *k_rope, const double *theta,
                            void *landmarks, float *min_cos, hipStream_t st);
hipError_t launch_topo(const Dims &dm, const float *min_cos, int32_t *outliers, uint32_t *gscratch, int keys_in_lds,
                       hipStream_t st);
hipError_t launch_gather_static(const Dims &dm, const void *k_pre, const void *k_rope, const void *v,
                                const int32_t *outliers, const double *theta, void *k_out, void *v_out,
                                void *k_loc, void *v_loc, hipStream_t st);
hipError_t launch_cand_mask(const Dims &dm, const int32_t *outliers, uint32_t *cand, hipStream_t st);
hipError_t launch_transpose_b(const Dims &dm, const void *B, void *Bt, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, int32_t value, size_t count, hipStream_t st);
// Host V's coded forms (prefill.hip): chunk values N when the layer's chunks
// can take it (bfloat16, N in {512, 1024, 2048}), else 0; the encoder writes
// nchunks chunks of v (raw, contiguous) into out (2N bytes each, coded or
// raw) and each chunk's code word.
int vcode_values(const Dims &dm);
// forms: bit 0 allows the 12-bit form, bit 1 the class form.
hipError_t launch_vcode(const Dims &dm, int forms, const void *v, void *out, uint32_t *code, long long nchunks,
                        hipStream_t st);
hipError_t launch_validate_outliers(const Dims &dm, const int32_t *outliers, int32_t *bad, hipStream_t st);
// Decode-token append: rotate the new key (pre-RoPE, (b, h_kv, d)) at `pos`
// and write it and its value to row `row` of the local buffers.
hipError_t launch_append(const Dims &dm, const void *k_new, const void *v_new, const double *theta, void *k_loc,
                         void *v_loc, int row, int pos, hipStream_t st);

// Decode.
// Query rows of a scoring launch.  q is laid out (b, h_q, w_obs, d); scored
// row g' (0 <= g' < G * wp) of KV head h is query head h*G + g'/wp at window
// position o_base + g'%wp.  The decode step scores one query per head
// (w_obs = wp = 1, o_base = 0); the SnapKV-style selection scores up to
// kMaxGroup (head, window position) rows per pass.
struct QRows {
    int w_obs, o_base, wp;
};
// score_wgs: workgroups of the persistent bfloat16 scoring kernel (0: two
// 64-chunk tiles per wave).  U and stats hold G * wp scored rows per KV head.
hipError_t launch_score(const Dims &dm, const void *q, const void *landmarks, const uint32_t *cand,
                        float *P, float2 *stats, int score_wgs, QRows qr, hipStream_t st);
// Group score: kbounds holds one (min, max) key pair per row and slice of
// kGroupSlice chunks.
int group_slices(const Dims &dm);
hipError_t launch_group(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                        uint32_t *keys, uint2 *kbounds, hipStream_t st);
// LDS of the select kernel: dynamic part (slot arrays, and the keys when they
// fit) and static part.
size_t select_dynamic_lds(const Dims &dm, bool keys_in_lds);
size_t select_static_lds();
// Selection and cache update: sel (b, h_kv, k) ascending chunks, sel_slot
// (b, h_kv, k) the cache slot of each; slot_chunk / slot_stamp (b, h_kv, cap)
// the chunk each slot holds (-1: empty) and the stamp of its last selection;
// `stamp` is this selection's (one more than the previous selection's).
hipError_t launch_select(const Dims &dm, const uint32_t *keys, const uint2 *kbounds, int32_t *sel,
                         int32_t *sel_slot, int32_t *slot_chunk, uint32_t *slot_stamp, uint32_t stamp,
                         int2 *misses, int32_t *miss_count, unsigned long long *counters, int keys_in_lds,
                         hipStream_t st);
// The decode path's selection in two kernels: the group score with a
// slice-local Top-K (topk_slices(dm) slices of topk_slice(dm) chunks per row,
// up to k candidates each: cand_key / cand_idx (b, h_kv, slices, k),
// cand_count (b, h_kv, slices)), then the selection over the candidates with
// the cache update of launch_select.
int topk_slice(const Dims &dm);
int topk_slices(const Dims &dm);
size_t group_topk_lds(const Dims &dm);
size_t select_cand_lds(const Dims &dm);
hipError_t launch_group_topk(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                             uint32_t *cand_key, int32_t *cand_idx, int32_t *cand_count, hipStream_t st);
hipError_t launch_select_cand(const Dims &dm, const uint32_t *cand_key, const int32_t *cand_idx,
                              const int32_t *cand_count, int32_t *sel, int32_t *sel_slot, int32_t *slot_chunk,
                              uint32_t *slot_stamp, uint32_t stamp, int2 *misses, int32_t *miss_count,
                              unsigned long long *counters, hipStream_t st);
// The group score and the selection in one kernel (one workgroup per row,
// the keys in LDS): launch_group's S2 and launch_select's outputs.
size_t select_fused_lds(const Dims &dm);
hipError_t launch_select_fused(const Dims &dm, const float *P, const float2 *stats, const uint32_t *cand, float *S2,
                               int32_t *sel, int32_t *sel_slot, int32_t *slot_chunk, uint32_t *slot_stamp,
                               uint32_t stamp, int2 *misses, int32_t *miss_count, unsigned long long *counters,
                               hipStream_t st);
// SnapKV-style selection: accumulate a pass's summed attention, then pool
// it into S2, selection keys and slice bounds.
hipError_t launch_snap_accum(const Dims &dm, const float *S2, float *acc, float weight, int first, hipStream_t st);
hipError_t launch_snap_pool(const Dims &dm, const float *acc, const uint32_t *cand, float *S2, uint32_t *keys,
                            uint2 *kbounds, int pool, hipStream_t st);
hipError_t launch_fetch(const Dims &dm, const void *v_host, void *vc, const int2 *misses,
                        const int32_t *miss_count, const uint32_t *vcode, unsigned long long *counters, int waves,
                        hipStream_t st);
// The rebuilt block's key i*c + t is token t of chunk chunks[i]; its value
// is in cache slot sel_slot[i], or slot i when sel_slot is null (a cache of
// exactly k slots, chunks = the slots' chunks).
hipError_t launch_qk(const Dims &dm, const void *q, const void *k_out, const void *k_loc, const void *A,
                     const void *Bt, const int32_t *chunks, const double *theta, const double *theta_rev,
                     float *logits, hipStream_t st);
hipError_t launch_pv(const Dims &dm, const float *logits, const void *v_out, const void *vc, const int32_t *sel_slot,
                     const void *v_loc, float2 *part_ml, float *part_acc, hipStream_t st);
// Fused attention (bfloat16 only): logits and PV partials in one launch,
// attn_workgroups(dm) workgroups per row, one split partial each; then
// launch_combine with splits = attn_workgroups(dm).
int attn_workgroups(const Dims &dm);
// Waves per fused attention workgroup for dm (8 only where that variant is built).
int attn_waves(const Dims &dm);
hipError_t launch_attn(const Dims &dm, const void *q, const void *A, const void *Bt, const int32_t *chunks,
                       const int32_t *sel_slot, const double *theta_rev, const void *k_out, const void *v_out,
                       const void *k_loc, const void *v_loc, const void *vc, float2 *part_ml, float *part_acc,
                       hipStream_t st);
// out = merge of `splits` partials per (sequence, query head).
hipError_t launch_combine(const Dims &dm, const float2 *part_ml, const float *part_acc, void *out, int splits,
                          hipStream_t st);
}  // namespace skv
