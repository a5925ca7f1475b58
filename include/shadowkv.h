/*
 * shadowkv.h -- C ABI of the MI355X (gfx950) ShadowKV sparse decode step.
 *
 * The method is the one described on the review page "ShadowKV: KV Cache in
 * Shadows for High-Throughput Long-Context LLM Inference" (xllm-io
 * paper-review blog), section 三 技术架构: Algorithm 1 (Pre-filling) builds
 * per-layer metadata once; Algorithm 2 (Decoding) runs per layer and per
 * generated token.  The per-layer cache that loads only the set difference
 * between consecutive steps follows the Telegram write-up "Ускорение
 * E2E-инференса через оптимизацию KV-кэша. Часть II".
 *
 * Conventions for every entry point
 *   - Tensors are dense and row-major with the shapes given below; their
 *     element type is the layer's `dtype` (binary32 or bfloat16) unless an
 *     integer type is named.  "device" pointers are HIP device memory of the
 *     GPU that was current when the layer was created; "pinned host" pointers
 *     come from shadowkv_host_alloc (or hipHostMalloc).
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     Calls enqueue work on it and return without waiting unless noted.
 *   - Return value: SKV_OK (0) or a negative SKV_E_* code; the message is in
 *     shadowkv_last_error() (per calling thread).  On a shape/argument error
 *     nothing is enqueued and the layer is unchanged.
 *   - A layer handle is not thread-safe; different layers may be used from
 *     different threads and streams.
 *
 * Ownership: the caller owns every pointer it passes.  Device inputs are
 * read only by the work enqueued by the call (keep them alive until that
 * work has run).  The pinned host V buffer is borrowed for the layer's
 * lifetime.  The library owns its copies of A and B, the landmarks, the
 * outlier and local buffers, the resident V cache with its slot map, all
 * scratch, the layer's events, and two HIP streams per device (shared by the
 * layers on it) for the optional fetch / rebuild overlap.
 */
#ifndef SHADOWKV_H
#define SHADOWKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
enum { SKV_F32 = 0, SKV_BF16 = 1 };

/* Status codes. */
enum {
    SKV_OK = 0,
    SKV_E_INVAL = -1,  /* null pointer, bad dtype, host buffer not pinned   */
    SKV_E_SHAPE = -2,  /* sizes violate the constraints listed below        */
    SKV_E_STATE = -3,  /* decode before prefill/load                        */
    SKV_E_NOMEM = -4,  /* device or pinned-host allocation failed           */
    SKV_E_HIP = -5     /* a HIP runtime call failed (text in last_error)    */
};

/*
 * Layer sizes (Algorithm 1's input list plus the key-parameter table of
 * section 三: chunk 8, rank 160, 48 outlier chunks, budget 1.56 %).
 * Constraints (SKV_E_SHAPE otherwise):
 *   batch >= 1; heads_kv >= 1; heads_q a multiple of heads_kv with
 *   group = heads_q / heads_kv <= 16; head_dim in {64, 128};
 *   1 <= chunk <= 64 and seq_len a positive multiple of chunk;
 *   local_window a multiple of chunk, 0 <= local_window <= seq_len;
 *   n = seq_len / chunk, n_loc = local_window / chunk;
 *   0 <= n_outlier <= n - n_loc; 0 <= top_k <= n - n_loc - n_outlier and
 *   top_k <= 4096; at least one attended key; 1 <= rank <= 256 (a multiple
 *   of 8 for bfloat16);
 *   rope_base > 0; 0 <= max_new <= 2^20;
 *   cache_chunks 0 (= top_k) or top_k <= cache_chunks <= n - n_loc - n_outlier,
 *   at most 16384.
 */
typedef struct {
    int32_t batch;         /* b: sequences decoded together                  */
    int32_t heads_q;       /* h_q: query heads                               */
    int32_t heads_kv;      /* h_kv: key/value heads (GQA: q head g -> g/group)*/
    int32_t head_dim;      /* d                                              */
    int32_t seq_len;       /* s: context tokens held by the layer            */
    int32_t chunk;         /* c: tokens per chunk (landmark granularity)     */
    int32_t rank;          /* r: rank of the pre-RoPE key factors            */
    int32_t n_outlier;     /* o: outlier chunks kept at full rank on the GPU */
    int32_t top_k;         /* k: chunks selected per (sequence, KV head)     */
    int32_t local_window;  /* w: last tokens always attended (dense)         */
    float rope_base;       /* RoPE base (theta_i = base^(-2i/d))             */
    int32_t dtype;         /* SKV_F32 or SKV_BF16                            */
    int32_t max_new;       /* decode tokens shadowkv_append may add to the
                              local block (0: none)                          */
    int32_t cache_chunks;  /* C: V chunks resident in HBM per (sequence, KV
                              head).  0 or top_k: the set-difference cache
                              (a step reuses what the previous step loaded);
                              larger: least recently used, keeping besides
                              the selection the C - k chunks selected most
                              recently (equal steps: lower chunk index)     */
} skv_config;

typedef struct skv_layer skv_layer;

/* Counters accumulated by the decode steps since creation or the last
 * shadowkv_reset_stats.  hits/misses count chunks per (sequence, KV head);
 * bytes_h2d is what the V fetch read from pinned host memory (raw chunks at
 * 2 bytes a value, coded ones in their coded size: see shadowkv_prefill_meta). */
typedef struct {
    int64_t steps;
    int64_t hits;
    int64_t misses;
    int64_t bytes_h2d;
} skv_stats;

/* Create a layer: validates `cfg` and allocates every device buffer the
 * layer will use (nothing is allocated later).  *out receives the handle. */
int shadowkv_layer_create(const skv_config *cfg, skv_layer **out);

/* Release the layer's memory, stream and events (synchronizes its streams). */
void shadowkv_layer_destroy(skv_layer *layer);

/*
 * Algorithm 1 (Pre-filling), steps 2-5, on the device.  Step 1's factors are
 * inputs (shadowkv_factorize computes them on the device; any factors of the
 * documented shapes will do).
 *   k_pre       device (b, h_kv, s, d)  pre-RoPE keys.
 *   k_rope      device (b, h_kv, s, d)  post-RoPE keys, or NULL: then they
 *               are computed here from k_pre (rotate-half RoPE, 0-based
 *               positions, angle reduced in double precision) and rounded
 *               to dtype.
 *   v           device (b, h_kv, s, d)  values.
 *   A           device (b, s, r)        left factor, shared by the KV heads.
 *   B           device (b, h_kv, r, d)  right factor per KV head;
 *               A[b] . B[b,h] approximates head h's pre-RoPE keys.
 *   v_host      pinned host (b, h_kv, s, d) bytes of dtype: receives V (the
 *               offload of step 5), each chunk in its own c*d-value slot; must
 *               stay allocated while the layer is used.  For bfloat16 layers
 *               with N = c*d in {512, 1024, 2048} a chunk is written in the
 *               smaller of two lossless coded forms, because the decode
 *               step's V fetch is bound by PCIe.  Lane l of 64 owns values
 *               l*Q .. l*Q+Q-1 (Q = N/64); both forms start with N bytes of
 *               sign and mantissa (lane l's at l*Q).
 *               The 12-bit form: N/2 bytes of 4-bit exponent offsets from
 *               the base, the chunk's largest exponent minus 14 (at least
 *               0), lane l's at N + l*Q/2, value q at bits 4*(q % 8) of
 *               32-bit word q/8, offset 15 marking an escape; then from
 *               N + N/2 4 bytes per escape, (value index << 8) | exponent,
 *               for the values whose exponent lies below the base.
 *               The class form: with top = the largest exponent minus 1 (at
 *               least 0), N/4 bytes of 2-bit classes, lane l's at
 *               N + l*Q/4, value q at bits 2*(q % 16) of 32-bit word q/16:
 *               0, 1, 2 = exponent top, top-1, top-2, 3 = in the side
 *               stream; from N + N/4 the side stream of S bytes (a multiple
 *               of 4), a 3-bit code per class-3 value in value order, code i
 *               at bits 3i..3i+2 (bit 0 of byte 0 first): 0 = top+1, x in
 *               1..6 = top-2-x, 7 = an escape; then from N + N/4 + S the
 *               escapes as above.
 *               A chunk with more than 64 escapes in both forms stays raw.
 *               SKV_T_V_CODES gives each chunk's form; the fetch restores V
 *               bit for bit.
 * Computes the chunk means of the post-RoPE keys (landmarks), each chunk's
 * minimum cosine to its landmark, the n_outlier chunks with the lowest
 * minimum (ties: lower index; chunks of the local window excluded), gathers
 * the full-rank post-RoPE K and V of outlier chunks and of the last
 * local_window tokens, marks the remaining chunks selectable, writes V to
 * v_host (raw or coded, above) and empties the resident V cache.
 */
int shadowkv_prefill_meta(skv_layer *layer, const void *k_pre, const void *k_rope,
                          const void *v, const void *A, const void *B,
                          void *v_host, void *stream);

/*
 * Install precomputed prefill metadata instead of computing it (resume from
 * saved metadata).  All device pointers except v_host (pinned host, already
 * holding V of shape (b, h_kv, s, d), raw: the fetch reads it as it is):
 *   landmarks (b, h_kv, n, d); outliers int32 (b, h_kv, o), each row
 *   strictly ascending, values in [0, n - n_loc); k_out, v_out
 *   (b, h_kv, o*c, d) post-RoPE; k_loc, v_loc (b, h_kv, w, d) post-RoPE;
 *   A (b, s, r); B (b, h_kv, r, d).
 * Also empties the resident V cache.
 */
int shadowkv_load_meta(skv_layer *layer, const void *landmarks, const int32_t *outliers,
                       const void *k_out, const void *v_out, const void *k_loc,
                       const void *v_loc, const void *A, const void *B,
                       void *v_host, void *stream);

/*
 * Decode-token append: the token generated at position seq_len + t (t =
 * tokens appended since the last prefill_meta / load_meta) joins the dense
 * local block, the third key block of Algorithm 2 step 4, and every later
 * decode step attends to it.  The pages do not describe generation beyond the
 * decoding step; this reading keeps generated tokens dense and uncompressed.
 *   k_new  device (b, h_kv, d)  the token's pre-RoPE key; rotated here at its
 *          position exactly like the prefill keys and rounded to dtype.
 *   v_new  device (b, h_kv, d)  its value.
 * Enqueued on `stream` (later decode steps must be ordered after it).
 * SKV_E_STATE before prefill_meta / load_meta; SKV_E_SHAPE once max_new
 * tokens have been appended.  prefill_meta and load_meta empty the appended
 * part of the block.
 */
int shadowkv_append(skv_layer *layer, const void *k_new, const void *v_new, void *stream);

/*
 * SnapKV-style fixed selection (the SnapKV review page, section on the core
 * formulas: importance S_i as attention summed over heads and queries, then
 * TopK, the compressed cache, and average pooling of the scores).  Taken at
 * the chunk granularity of this layer: each query of an observation window
 * scores the selectable chunks by softmax(q . L^T / sqrt(d)); S sums those
 * probabilities over the KV group's query heads and the window's queries; S
 * is average-pooled over `pool` neighbouring chunks (zero padding, divided
 * by `pool`); the k selectable chunks of largest pooled S (ties to the lower
 * index) become the layer's selection and stay fixed: later decode steps
 * skip scoring and selection, the first of them fetches the V of the chunks
 * not yet resident, and the rest fetch nothing.  prefill_meta, load_meta and
 * reset_cache return the layer to per-step selection.
 *   q_obs  device (b, h_q, w_obs, d)  post-RoPE queries of the window.
 *   w_obs  1 ..= 4096 window queries; pool odd, 1 ..= 63.
 * Enqueued on `stream`.  SKV_E_STATE before prefill_meta / load_meta;
 * SKV_E_SHAPE for top_k = 0, a bad w_obs or pool, or q_obs of 1 GiB or more.
 * The hit / miss counters count the selection as one step.
 */
int shadowkv_snapkv_select(skv_layer *layer, const void *q_obs, int w_obs, int pool, void *stream);
/* (A second selection before any decode step first fetches the V that the
 * previous selection still owes, on `stream`, so the cache stays lossless.) */

/*
 * Algorithm 2 (Decoding): one step of one layer for all b sequences.
 *   q    device (b, h_q, d)  post-RoPE queries.
 *   out  device (b, h_q, d)  attention output.
 * Steps: P = q . L^T / sqrt(d) over selectable chunks; the group score S2
 * (each head's softmax over selectable chunks, averaged over the heads of a
 * KV group -- the page leaves S2 undefined, this is the reading taken);
 * I = ArgTopK(S2, k) per (sequence, KV head) with ties to the lower index;
 * the set difference against the previous step's resident chunks; V of the
 * missing chunks read from v_host (after the selection; beside the key
 * rebuild on a second stream if shadowkv_set_overlap enabled it); the
 * selected keys rebuilt as Gather(A, I) . B and rotated at their original
 * positions; softmax attention over
 * [outlier keys; rebuilt keys; local-window keys] with the matching values.
 * Enqueued on `stream`; `out` is valid once `stream` has reached this point.
 * SKV_E_STATE before prefill_meta / load_meta.
 */
int shadowkv_decode_step(skv_layer *layer, const void *q, void *out, void *stream);

/*
 * shadowkv_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, same results; it calls no hipMalloc, hipFree
 * or other allocating routine.  The step's scratch (landmark scores, tile
 * statistics, group scores, selection keys or candidates, logits, split
 * partials) lives in one 128 MiB device array per GPU, held from the first
 * call on that GPU until the process ends, instead of in the layer's own
 * buffers.  Every layer and every call on one GPU shares that array: calls
 * that overlap on one GPU (different streams, not ordered) race and give
 * wrong results.  Per-kernel timing is not recorded, and the score reads of
 * shadowkv_read (SKV_T_SCORES, SKV_T_GROUP_SCORES) keep the last
 * shadowkv_decode_step's values.  SKV_E_SHAPE, before any work is enqueued,
 * when the layer's step needs more than 128 MiB of scratch (e.g. b = 48 at
 * 60K with GQA 4 needs ~84 MB, the GLM-shaped 244K b = 12 ~64 MB).
 */
int shadowkv_decode_step_noalloc(skv_layer *layer, const void *q, void *out, void *stream);

/* Empty the resident V cache (all later chunks load again).  The cache is
 * lossless, so outputs do not change; only the hit counts do. */
int shadowkv_reset_cache(skv_layer *layer, void *stream);

/* Read the counters.  Waits for the work this layer's calls enqueued last
 * (on whatever stream they were given), not for the rest of the device. */
int shadowkv_get_stats(skv_layer *layer, skv_stats *out);
int shadowkv_reset_stats(skv_layer *layer);

/* Debug / test access to the layer's device state.  shadowkv_read copies
 * tensor `which` into dst (device or host memory, `bytes` must equal
 * shadowkv_tensor_bytes) ordered on `stream`. */
enum {
    SKV_T_LANDMARKS = 0,    /* dtype (b, h_kv, n, d)                          */
    SKV_T_MIN_COS = 1,      /* f32 (b, h_kv, n): prefill cosine minimum       */
    SKV_T_OUTLIERS = 2,     /* int32 (b, h_kv, o), ascending                  */
    SKV_T_CAND_MASK = 3,    /* uint32 (b, h_kv, ceil(n/32)): selectable bits  */
    SKV_T_SCORES = 4,       /* f32 (b, h_kv, n, G): exp(P - max of P over the
                               64-chunk tile), 0 off-candidate (last step)    */
    SKV_T_GROUP_SCORES = 5, /* f32 (b, h_kv, n): last step's S2, 0 masked     */
    SKV_T_SELECTION = 6,    /* int32 (b, h_kv, k): last step's I, ascending   */
    SKV_T_SLOT_CHUNKS = 7,  /* int32 (b, h_kv, C): chunk held by each slot,
                               -1 if empty (C = cache_chunks)                 */
    SKV_T_CACHE_V = 8,      /* dtype (b, h_kv, C*c, d): resident V by slot    */
    SKV_T_K_OUT = 9,        /* dtype (b, h_kv, o*c, d)                        */
    SKV_T_V_OUT = 10,
    SKV_T_K_LOC = 11,       /* dtype (b, h_kv, w + max_new, d): the window's
                               keys, then the appended ones                   */
    SKV_T_V_LOC = 12,
    SKV_T_SELECTION_SLOTS = 13, /* int32 (b, h_kv, k): slot holding the i-th
                                   selected chunk                             */
    SKV_T_V_CODES = 14,     /* uint32 (b, h_kv, n): each host V chunk's code
                               word (forms: shadowkv_prefill_meta): 0 raw;
                               bit 31 alone: 12-bit form, escape count in bits
                               16..23, base in bits 0..7; bits 31 and 30: class
                               form, S/4 in bits 20..27, escape count in bits
                               8..15, top in bits 0..7                         */
    SKV_T_COUNT = 15
};
size_t shadowkv_tensor_bytes(const skv_layer *layer, int which);
int shadowkv_read(skv_layer *layer, int which, void *dst, size_t bytes, void *stream);

/* Schedule of the host-V fetch (Algorithm 2 step 3 runs the fetch and the
 * key rebuild "in parallel"; the review page credits multi-stream overlap
 * with a 2x latency cut).  enable != 0: the fetch runs on a second stream
 * beside the key rebuild.  0 (the default): both run in order on the
 * caller's stream.  On MI355X the device-initiated PCIe reads of the fetch
 * slow every other kernel's memory traffic, so running beside them gains
 * less than the cross-queue synchronisation costs.  Outputs are identical
 * either way. */
int shadowkv_set_overlap(skv_layer *layer, int enable);

/* Per-kernel timing with HIP events recorded on the stream each kernel runs
 * on.  While enabled, every decode step records a start/stop pair around
 * each kernel.  shadowkv_get_timing waits for those events, writes the summed
 * milliseconds of each kernel (SKV_K_COUNT entries) and the number of steps
 * they cover, and clears the record. */
enum {
    SKV_K_SCORE = 0,    /* landmark scores + per-tile softmax partials      */
    SKV_K_SELECT = 1,   /* group score S2, ArgTopK, set difference          */
    SKV_K_FETCH = 2,    /* V of missing chunks from pinned host memory      */
    SKV_K_QK = 3,       /* logits: static keys, rebuilt keys + RoPE         */
    SKV_K_PV = 4,       /* probabilities times values, split merge          */
    SKV_K_ATTN = 5,     /* fused rebuild + logits + PV, split merge: bfloat16
                           on one queue (QK and PV then read 0); otherwise 0 */
    SKV_K_COUNT = 6
};
int shadowkv_set_timing(skv_layer *layer, int enable);
int shadowkv_get_timing(skv_layer *layer, double *ms_out, int64_t *steps_out);

/*
 * Low-rank factors of the pre-RoPE keys (the ShadowKV review page, section
 * 三, Algorithm 1 step 1, A, B <- SVD(K_pre); computed once per sequence,
 * before decoding).  Per sequence the keys form the s x n matrix M,
 * n = heads_kv * head_dim, column h*head_dim + i = head h's dimension i; with
 * V_r the eigenvectors of M^T M for its `rank` largest eigenvalues (the
 * leading right singular vectors of M), A = M V_r and B = V_r^T split by
 * head, so A[b] . B[b, h] is the best rank-`rank` approximation of head h's
 * keys.  Everything runs on the device in double precision: the Gram matrix,
 * a parallel cyclic two-sided Jacobi eigensolver on 32-index super-blocks
 * (until the off-diagonal mass, a sum of squares, is below 1e-22 of the total
 * or has stopped falling at its rounding floor below 1e-20; at most 30
 * sweeps, and one sweep past the deciding one, which was queued while its
 * measure was read and, the convergence being quadratic there, ends near the
 * rounding floor), and A = M V_r; A and B are rounded once to `dtype`.
 *   k_pre  device (batch, heads_kv, seq_len, head_dim), `dtype`
 *   A      device (batch, seq_len, rank), written
 *   B      device (batch, heads_kv, rank, head_dim), written
 * With rank > n the columns past n are zero.  The call allocates its own
 * device scratch (about 1.3 GB at n = 1024: the Gram partials of up to 16 row
 * slices, two copies of the matrix and of the eigenvectors for 8 sequences at
 * a time), runs on
 * `stream`, reads back the convergence measure once per sweep (through a
 * small pinned buffer) and the eigenvalues at the end, and returns when the
 * factors are written.
 * SKV_E_INVAL for a null pointer or a bad dtype; SKV_E_SHAPE unless
 * batch, heads_kv, seq_len >= 1, head_dim in {64, 128}, rank in [1, 256],
 * heads_kv * head_dim <= 2048 (the eigensolver's cost grows as n^3: a sweep is
 * n/16 - 1 rounds over two n x n matrices); SKV_E_HIP if an allocation, launch or
 * copy fails.  `sweeps_out` (may be NULL) receives the sweeps the slowest batch
 * took.
 */
int shadowkv_factorize(int dtype, int batch, int heads_kv, int seq_len, int head_dim, int rank,
                       const void *k_pre, void *A, void *B, void *stream, int *sweeps_out);

/* Pinned host memory that the device can read directly. */
int shadowkv_host_alloc(size_t bytes, void **out);
int shadowkv_host_free(void *ptr);

/* Message of the last failing call on this thread ("" if none). */
const char *shadowkv_last_error(void);

/* Equivalent bandwidth of section 三's 核心公式:
 *   B~ = 2 S B_gpu / (S/C + 2 (K + O) C + (1 - alpha) K C B_gpu / B_pcie)
 * S tokens, C chunk size, K selected and O outlier chunks, alpha the cache
 * hit rate; the result has the unit of b_gpu. */
double shadowkv_equiv_bandwidth(double S, double C, double K, double O, double alpha,
                                double b_gpu, double b_pcie);

/* Measurement aid, not part of the method: the best rate (1e9 B/s) at which a
 * plain streaming kernel reads `bytes` (>= 1 MiB; make it larger than the
 * device's last-level cache) of device memory at `buf`, over `reps` passes at
 * each of a few launch shapes.  The caller owns `buf`; its contents are read,
 * never written.  Runs on `stream` and waits for it.  SKV_E_INVAL for a null
 * pointer, reps < 1 or too few bytes; SKV_E_HIP if a launch or event fails. */
int shadowkv_probe_hbm_read(const void *buf, size_t bytes, int reps, void *stream, double *gbps_out);

/* Measurement aid, not part of the method: the host-issued alternative to the
 * device-initiated V fetch (the review page, section 三, Algorithm 2 step 3;
 * the pages overlap host-driven copies with the key rebuild).  Copies
 * n_chunks chunks of chunk_bytes from the pinned host buffer `host`
 * (host_bytes long; chunk i starts at host_chunk[i] * chunk_bytes, a host
 * array) to consecutive chunks of the device buffer `dev`, first with one
 * hipMemcpyAsync per chunk, then with one hipMemcpyBatchAsync, `reps` times
 * each on `stream`, and returns the best rate (1e9 B/s) of each (the batch
 * rate is 0 when the HIP runtime in the process lacks the call).  The caller
 * owns all buffers; `dev` must hold n_chunks * chunk_bytes.  Waits for the
 * stream.  SKV_E_INVAL for a null pointer, a chunk outside the host buffer,
 * reps or n_chunks < 1; SKV_E_HIP if a copy or event fails. */
int shadowkv_probe_host_copies(const void *host, size_t host_bytes, void *dev, size_t chunk_bytes, int n_chunks,
                               const int64_t *host_chunk, int reps, void *stream, double *gbps_each,
                               double *gbps_batch);

#ifdef __cplusplus
}
#endif

#endif /* SHADOWKV_H */
