// Host runtime and C ABI of the ShadowKV decode step (declared in
// include/shadowkv.h): per-layer device state, argument validation, the
// two-stream schedule of one decode step, counters and per-kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "shadowkv.h"
#include "skv_dims.h"

using skv::Dims;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

#define SKV_HIP(expr)                                                                          \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess) return fail(SKV_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Validates a configuration and derives the sizes the kernels use.
int make_dims(const skv_config &c, Dims *dm, std::string *why) {
    auto bad = [&](const char *m) { *why = m; return SKV_E_SHAPE; };
    if (c.dtype != SKV_F32 && c.dtype != SKV_BF16) { *why = "dtype must be SKV_F32 or SKV_BF16"; return SKV_E_INVAL; }
    if (c.batch < 1 || c.heads_kv < 1) return bad("batch and heads_kv must be >= 1");
    if (c.heads_q < c.heads_kv || c.heads_q % c.heads_kv) return bad("heads_q must be a multiple of heads_kv");
    if (c.heads_q / c.heads_kv > skv::kMaxGroup) return bad("heads_q / heads_kv must be <= 16");
    if (c.head_dim != 64 && c.head_dim != 128) return bad("head_dim must be 64 or 128");
    if (c.chunk < 1 || c.chunk > 64) return bad("chunk must be in [1, 64]");
    if (c.seq_len < c.chunk || c.seq_len % c.chunk) return bad("seq_len must be a positive multiple of chunk");
    if (c.local_window < 0 || c.local_window % c.chunk || c.local_window > c.seq_len)
        return bad("local_window must be a multiple of chunk in [0, seq_len]");
    const int n = c.seq_len / c.chunk, n_loc = c.local_window / c.chunk;
    if (c.n_outlier < 0 || c.n_outlier > n - n_loc) return bad("n_outlier must be in [0, n - n_loc]");
    if (c.top_k < 0 || c.top_k > n - n_loc - c.n_outlier) return bad("top_k must be in [0, n - n_loc - n_outlier]");
    if (c.top_k > 4096) return bad("top_k must be <= 4096");
    if (c.rank < 1 || c.rank > 256) return bad("rank must be in [1, 256]");
    // the bfloat16 rebuild reads 8 rank values per 16-byte load of an A or B row
    if (c.dtype == SKV_BF16 && c.rank % 8) return bad("bfloat16 layers need rank a multiple of 8");
    if (!(c.rope_base > 0.f)) return bad("rope_base must be > 0");
    if (c.max_new < 0 || c.max_new > (1 << 20)) return bad("max_new must be in [0, 2^20]");
    if (c.cache_chunks != 0 && (c.cache_chunks < c.top_k || c.cache_chunks > n - n_loc - c.n_outlier))
        return bad("cache_chunks must be 0 or in [top_k, n - n_loc - n_outlier]");
    if (c.cache_chunks > 16384) return bad("cache_chunks must be <= 16384");
    const long long nk = 1LL * c.n_outlier * c.chunk + 1LL * c.top_k * c.chunk + c.local_window;
    if (nk < 1) return bad("at least one key must be attended");
    const long long seq_elems = 1LL * c.batch * c.heads_kv * c.seq_len * c.head_dim;
    if (seq_elems >= (1LL << 40)) return bad("tensor too large");
    // kernels address each (sequence, KV head) row of a tensor, and each
    // sequence of A, through buffer resources of less than 1 GiB
    const long long es = c.dtype == SKV_BF16 ? 2 : 4;
    if (1LL * n * c.head_dim * es >= (1LL << 30) || 1LL * n * (c.heads_q / c.heads_kv) * 4 >= (1LL << 30) ||
        1LL * c.seq_len * c.rank * es >= (1LL << 30))
        return bad("a per-row tensor would reach 1 GiB (sequence too long)");
    if ((1LL * c.n_outlier * c.chunk + 1LL * c.top_k * c.chunk + c.local_window + c.max_new) * (c.heads_q / c.heads_kv) * 4 >=
        (1LL << 30))
        return bad("a per-row logit block would reach 1 GiB");
    Dims &d = *dm;
    d.b = c.batch; d.hq = c.heads_q; d.hkv = c.heads_kv; d.d = c.head_dim; d.s = c.seq_len; d.c = c.chunk;
    d.r = c.rank; d.o = c.n_outlier; d.k = c.top_k; d.w = c.local_window;
    d.cap = c.cache_chunks > 0 ? c.cache_chunks : c.top_k;
    d.wcap = c.local_window + c.max_new;
    d.n = n; d.n_loc = n_loc; d.G = c.heads_q / c.heads_kv;
    d.GP = d.G <= 4 ? 4 : (d.G <= 8 ? 8 : 16);
    d.mask_words = (n + 31) / 32;
    d.score_tiles = (n + skv::kScoreTile - 1) / skv::kScoreTile;
    d.wtiles = (n + 63) / 64;
    d.OC = c.n_outlier * c.chunk; d.KC = c.top_k * c.chunk; d.NK = static_cast<int>(nk);
    d.pv_tiles = (d.NK + skv::kPvTile - 1) / skv::kPvTile;
    d.esize = c.dtype == SKV_BF16 ? 2 : 4;
    d.bf16 = c.dtype == SKV_BF16;
    d.r_pad = round_up(c.rank, 32);
    d.kpw = 64;  // rebuilt keys per wave of the fused attention kernel
    d.attn_nw = 4;
    d.scale = 1.0f / std::sqrt(static_cast<float>(c.head_dim));
    return SKV_OK;
}

// The sizes of a decode step whose local block holds `w_local` keys.
Dims dims_with_local(const Dims &dm, int w_local) {
    Dims d = dm;
    d.w = w_local;
    d.NK = d.OC + d.KC + w_local;
    d.pv_tiles = (d.NK + skv::kPvTile - 1) / skv::kPvTile;
    return d;
}

struct Mark {
    int kernel;
    hipEvent_t start, stop;
};

// Streams shared by every layer on one device.  The host-V fetch waits on
// PCIe for microseconds per read; a wave doing so slows the memory traffic of
// every other wave on its CU.  So the fetch stream is confined by a CU mask to
// a few CUs, and the key-rebuild stream that runs beside it to the rest.
// Masked streams own hardware queues, so they are created once per device
// (not per layer).  SKV_FETCH_CUS sets the fetch CU count (0: no masks).
struct DevStreams {
    bool ready = false;
    hipStream_t fetch = nullptr, comp = nullptr;
    int fetch_cus = 0;
    // staging of host V's coded form on its way to the host (the prefill's
    // offload on the fetch stream; allocated by the first prefill that codes,
    // kept until the process ends)
    void *stage = nullptr;
};
constexpr size_t kStageBytes = size_t(64) << 20;
std::mutex g_dev_mutex;
DevStreams g_dev[64];

int device_streams(int device, DevStreams **out) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (device < 0 || device >= 64) return fail(SKV_E_INVAL, "device index out of range");
    DevStreams &ds = g_dev[device];
    if (!ds.ready) {
        int ncu = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || ncu <= 0)
            return fail(SKV_E_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed");
        int fcu = 0;
        if (const char *e = std::getenv("SKV_FETCH_CUS")) fcu = std::atoi(e);
        fcu = std::max(0, std::min(fcu, ncu / 2));
        // "block": the fetch takes the first fcu CUs and the compute stream
        // skips the whole 32-CU block they sit in; "spread": the fetch CUs are
        // spaced evenly and the compute stream takes every other CU.
        bool block = false;
        if (const char *e = std::getenv("SKV_FETCH_CU_MODE")) block = std::strcmp(e, "block") == 0;
        if (fcu > 0) {
            const int words = (ncu + 31) / 32;
            std::vector<uint32_t> fm(words, 0u), cm(words, 0u);
            const int stride = ncu / fcu;
            for (int cu = 0; cu < ncu; ++cu) {
                const bool is_fetch = block ? cu < fcu : ((cu % stride == 0) && (cu / stride < fcu));
                const bool is_comp = block ? cu >= ((fcu + 31) / 32) * 32 : !is_fetch;
                if (is_fetch) fm[cu / 32] |= 1u << (cu % 32);
                if (is_comp) cm[cu / 32] |= 1u << (cu % 32);
            }
            if (hipExtStreamCreateWithCUMask(&ds.fetch, words, fm.data()) != hipSuccess ||
                hipExtStreamCreateWithCUMask(&ds.comp, words, cm.data()) != hipSuccess) {
                (void)hipGetLastError();
                if (ds.fetch) (void)hipStreamDestroy(ds.fetch);
                ds.fetch = ds.comp = nullptr;
                fcu = 0;
            }
        }
        if (fcu == 0 && (hipStreamCreateWithFlags(&ds.fetch, hipStreamNonBlocking) != hipSuccess ||
                         hipStreamCreateWithFlags(&ds.comp, hipStreamNonBlocking) != hipSuccess))
            return fail(SKV_E_HIP, "creating the fetch / compute streams failed");
        ds.fetch_cus = fcu;
        ds.ready = true;
    }
    *out = &ds;
    return SKV_OK;
}

// The device's staging buffer for host V's coded form (allocated once).
int device_stage(int device, void **out) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (device < 0 || device >= 64) return fail(SKV_E_INVAL, "device index out of range");
    DevStreams &ds = g_dev[device];
    if (!ds.stage && hipMalloc(&ds.stage, kStageBytes) != hipSuccess) {
        ds.stage = nullptr;
        return fail(SKV_E_NOMEM, "staging buffer for host V (64 MiB) could not be allocated");
    }
    *out = ds.stage;
    return SKV_OK;
}

}  // namespace

struct skv_layer {
    skv_config cfg{};
    Dims dm{};
    int device = 0;
    int lds_limit = 0;
    std::vector<void *> allocs;
    // parameters and metadata
    void *A = nullptr, *Bt = nullptr, *L = nullptr;
    void *k_out = nullptr, *v_out = nullptr, *k_loc = nullptr, *v_loc = nullptr;
    uint32_t *cand = nullptr;
    int32_t *outliers = nullptr;
    float *min_cos = nullptr;
    double *theta = nullptr;      // theta_i = base^(-2i/d)
    double *theta_rev = nullptr;  // theta_i / (2 pi): turns per position
    // resident V cache
    void *vc = nullptr;
    int32_t *slot_chunk = nullptr;   // (b, h_kv, cap): chunk held by each cache slot, -1 empty
    uint32_t *slot_stamp = nullptr;  // (b, h_kv, cap): stamp of the slot chunk's last selection
    int32_t *sel_slot = nullptr;     // (b, h_kv, k): cache slot of each selected chunk
    uint32_t stamp = 0;              // selections made (stamps of the cache's LRU order)
    // per-step scratch
    int32_t *sel = nullptr;
    float *P = nullptr, *S2 = nullptr, *logits = nullptr, *part_acc = nullptr;
    float2 *stats = nullptr, *part_ml = nullptr;
    int2 *misses = nullptr;
    int32_t *miss_count = nullptr;
    unsigned long long *counters = nullptr;  // hits, misses, steps, bytes read from host V
    uint32_t *keys = nullptr;    // selection keys (b, h_kv, n)
    uint2 *kbounds = nullptr;    // (min, max) selectable key per row and group slice
    int select_keys_in_lds = 1, topo_keys_in_lds = 1;
    // the decode selection through slice-local candidates (group_topk +
    // select over the candidates) when both fit in LDS; else group + select
    bool topk_cand = false;
    // the one-pass selection with the group score computed in the same
    // kernel (no group kernel)
    bool select_fused = false;
    int cus = 0;
    uint32_t *cand_key = nullptr;  // (b, h_kv, slices, k)
    int32_t *cand_idx = nullptr;   // (b, h_kv, slices, k)
    int32_t *cand_count = nullptr; // (b, h_kv, slices)
    int32_t *bad = nullptr;
    // host V
    void *v_host_dev = nullptr;
    // (b, h_kv, n): each host V chunk's code word (0: raw; else which coded
    // form the prefill wrote, see prefill.hip); vcoded: the prefill codes
    uint32_t *vcode = nullptr;
    bool vcoded = false;
    int vforms = 3;  // coded forms the prefill may pick: bit 0 the 12-bit form, bit 1 the class form
    bool ready = false;
    // shared per-device streams for the host-V fetch and the key rebuild
    hipStream_t copy = nullptr, comp = nullptr;
    hipEvent_t ev_sel = nullptr, ev_fetch = nullptr, ev_qk = nullptr;
    // recorded on the caller's stream at the end of every call that enqueues
    // work: the counters and timings are read after it, so reading them waits
    // for this layer's work only
    hipEvent_t ev_done = nullptr;
    int fetch_waves = 256;
    int score_wgs = 0;  // workgroups of the scoring kernel (0: two tiles per wave)
    int n_app = 0;      // decode tokens appended to the local block since the last prefill / load
    // bfloat16 on one queue: rebuild, logits and PV in one fused launch
    // instead of the separate QK and PV launches
    bool fused = false;
    // SnapKV-style fixed selection: decode steps keep the selection (no
    // scoring or selection); the missing V is fetched by the first of them
    bool fixed = false, fetch_pending = false;
    float *snap_acc = nullptr;  // (b, h_kv, n) summed attention of the observation window
    // timing
    bool overlap = false;  // fetch beside the key rebuild (true) or before it
    bool timing = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;
    std::vector<Mark> marks;
    int64_t timed_steps = 0;
};

// Per-step scratch of a decode step: written and read within one step.
struct StepScratch {
    float *P;            // U (b, h_kv, n, G): exp(P - tile max)
    float2 *stats;       // (b, h_kv, G, ceil(n/64)) tile (max, sum)
    float *S2;           // (b, h_kv, n) group scores
    uint32_t *keys;      // (b, h_kv, n) selection keys (one-pass selection)
    uint2 *kbounds;      // (b, h_kv, group slices) key bounds
    uint32_t *cand_key;  // (b, h_kv, slices, k) slice candidates (two-pass selection)
    int32_t *cand_idx;
    int32_t *cand_count; // (b, h_kv, slices)
    float *logits;       // (b, h_q, NK) (separate QK + PV kernels)
    float2 *part_ml;     // (b, h_q, splits) split (max, sum)
    float *part_acc;     // (b, h_q, splits, d) split sums
};

namespace {

int dalloc(skv_layer *ly, size_t bytes, void **p) {
    if (bytes == 0) bytes = 256;
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(SKV_E_NOMEM, std::string("hipMalloc(") + std::to_string(bytes) + "): " + hipGetErrorString(e));
    }
    ly->allocs.push_back(*p);
    return SKV_OK;
}

template <typename P>
int dalloc_t(skv_layer *ly, size_t bytes, P **p) {
    void *v = nullptr;
    int rc = dalloc(ly, bytes, &v);
    *p = static_cast<P *>(v);
    return rc;
}

void release(skv_layer *ly) {
    // the layer's work ends at ev_done on the caller's stream (every call that
    // enqueues work records it) and on the shared copy and rebuild streams
    if (ly->ev_done) (void)hipEventSynchronize(ly->ev_done);
    if (ly->copy) (void)hipStreamSynchronize(ly->copy);
    if (ly->comp) (void)hipStreamSynchronize(ly->comp);
    for (void *p : ly->allocs) (void)hipFree(p);
    ly->allocs.clear();
    for (hipEvent_t e : ly->ev_pool) (void)hipEventDestroy(e);
    ly->ev_pool.clear();
    if (ly->ev_sel) (void)hipEventDestroy(ly->ev_sel);
    if (ly->ev_fetch) (void)hipEventDestroy(ly->ev_fetch);
    if (ly->ev_qk) (void)hipEventDestroy(ly->ev_qk);
    if (ly->ev_done) (void)hipEventDestroy(ly->ev_done);
}

// The end of the layer's latest enqueued work on `st`.
int mark_done(skv_layer *ly, hipStream_t st) {
    SKV_HIP(hipEventRecord(ly->ev_done, st));
    return SKV_OK;
}

hipEvent_t pool_event(skv_layer *ly) {
    if (ly->ev_used == ly->ev_pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        ly->ev_pool.push_back(e);
    }
    return ly->ev_pool[ly->ev_used++];
}

// Brackets one kernel launch with timing events when timing is enabled.
struct Timed {
    skv_layer *ly;
    int kernel;
    hipStream_t st;
    hipEvent_t stop = nullptr;
    Timed(skv_layer *l, int k, hipStream_t s, bool on) : ly(l), kernel(k), st(s) {
        if (!on || !ly->timing) return;
        hipEvent_t start = pool_event(ly);
        stop = pool_event(ly);
        if (!start || !stop) { stop = nullptr; return; }
        (void)hipEventRecord(start, st);
        ly->marks.push_back({kernel, start, stop});
    }
    ~Timed() {
        if (stop) (void)hipEventRecord(stop, st);
    }
};

int check_pinned(const void *host, void **dev) {
    if (!host) return fail(SKV_E_INVAL, "v_host is null");
    hipError_t e = hipHostGetDevicePointer(dev, const_cast<void *>(host), 0);
    if (e != hipSuccess || !*dev) {
        (void)hipGetLastError();
        return fail(SKV_E_INVAL, "v_host is not pinned, device-mapped host memory (use shadowkv_host_alloc)");
    }
    return SKV_OK;
}

}  // namespace

extern "C" {

const char *shadowkv_last_error(void) { return g_last_error.c_str(); }

int shadowkv_factorize(int dtype, int batch, int heads_kv, int seq_len, int head_dim, int rank, const void *k_pre,
                       void *A, void *B, void *stream, int *sweeps_out) {
    if (!k_pre || !A || !B) return fail(SKV_E_INVAL, "null k_pre, A or B");
    if (dtype != SKV_F32 && dtype != SKV_BF16) return fail(SKV_E_INVAL, "dtype must be SKV_F32 or SKV_BF16");
    if (batch < 1 || heads_kv < 1 || seq_len < 1) return fail(SKV_E_SHAPE, "batch, heads_kv and seq_len must be >= 1");
    if (head_dim != 64 && head_dim != 128) return fail(SKV_E_SHAPE, "head_dim must be 64 or 128");
    if (rank < 1 || rank > 256) return fail(SKV_E_SHAPE, "rank must be in [1, 256]");
    if (heads_kv * head_dim > 2048) return fail(SKV_E_SHAPE, "heads_kv * head_dim must be <= 2048");
    std::string why;
    const int rc = skv::factorize_device(dtype == SKV_BF16, batch, heads_kv, seq_len, head_dim, rank, k_pre, A, B,
                                         static_cast<hipStream_t>(stream), &why, sweeps_out);
    return rc ? fail(SKV_E_HIP, why) : SKV_OK;
}

double shadowkv_equiv_bandwidth(double S, double C, double K, double O, double alpha, double b_gpu, double b_pcie) {
    return 2.0 * S * b_gpu / (S / C + 2.0 * (K + O) * C + (1.0 - alpha) * K * C * b_gpu / b_pcie);
}

int shadowkv_host_alloc(size_t bytes, void **out) {
    if (!out) return fail(SKV_E_INVAL, "out is null");
    *out = nullptr;
    // SKV_HOST_NONCOHERENT=1 asks for coarse-grained (non-coherent) pages,
    // which the GPU may cache; V on the host is written once (prefill) and
    // then only read, so either kind is correct.
    unsigned flags = hipHostMallocMapped;
    if (const char *e = std::getenv("SKV_HOST_NONCOHERENT"))
        if (std::atoi(e) != 0) flags |= hipHostMallocNonCoherent;
    hipError_t e = hipHostMalloc(out, bytes ? bytes : 1, flags);
    if (e != hipSuccess) return fail(SKV_E_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    return SKV_OK;
}

int shadowkv_host_free(void *ptr) {
    if (!ptr) return SKV_OK;
    SKV_HIP(hipHostFree(ptr));
    return SKV_OK;
}

int shadowkv_layer_create(const skv_config *cfg, skv_layer **out) {
    if (!cfg || !out) return fail(SKV_E_INVAL, "null argument");
    *out = nullptr;
    Dims dm{};
    std::string why;
    int rc = make_dims(*cfg, &dm, &why);
    if (rc) return fail(rc, why);
    // SKV_TOPK_SLICE (a multiple of 64): chunks per slice of the two-pass Top-K
    if (const char *e = std::getenv("SKV_TOPK_SLICE")) {
        const int v = std::atoi(e);
        if (v >= 64 && v % 64 == 0) dm.tslice = v;
    }

    skv_layer *ly = new skv_layer();
    ly->cfg = *cfg;
    ly->dm = dm;
    auto bail = [&](int code) {
        std::string msg = g_last_error;
        release(ly);
        delete ly;
        g_last_error = msg;
        return code;
    };
    if (hipGetDevice(&ly->device) != hipSuccess) return bail(fail(SKV_E_HIP, "hipGetDevice failed"));
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, ly->device) != hipSuccess)
        return bail(fail(SKV_E_HIP, "hipDeviceGetAttribute(MaxSharedMemoryPerBlock) failed"));
    ly->lds_limit = lds;
    // rebuilt keys per wave of the fused attention kernel: 64 (measured at
    // 128K b8 and the GLM shape, 48 and 32 keys per wave were slower: their
    // extra workgroups each stage B again); SKV_ATTN_KPW (48, 32 or 16) forces
    // another
    // waves per fused attention workgroup: 8 (one workgroup per CU, one
    // staged B for 512 keys) when the launch then still fits the CUs at once,
    // else 4 (measured: 128K b8 31.9 -> 30.7 us, GLM-shaped 244K b12 31.9 ->
    // 30.9 us with 8; 60K b48, three rounds of workgroups, 89 -> 128 us);
    // SKV_ATTN_WAVES (4 or 8) forces it
    {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, ly->device) != hipSuccess || cus < 1)
            return bail(fail(SKV_E_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed"));
        ly->cus = cus;
        Dims t = dims_with_local(dm, dm.wcap);
        t.attn_nw = 8;
        dm.attn_nw = skv::attn_waves(t) == 8 && static_cast<long long>(dm.b) * dm.hkv * skv::attn_workgroups(t) <= cus
                         ? 8 : 4;
        if (const char *e = std::getenv("SKV_ATTN_WAVES")) dm.attn_nw = std::atoi(e) == 8 ? 8 : 4;
        ly->dm.attn_nw = dm.attn_nw;
    }
    if (const char *e = std::getenv("SKV_ATTN_KPW")) {
        const int v = std::atoi(e);
        if (v == 64 || v == 48 || v == 32 || v == 16) dm.kpw = v;
        ly->dm.kpw = dm.kpw;
    }
    // Scoring grid: 0 picks two 64-chunk tiles per wave; SKV_SCORE_WGS
    // overrides the workgroup count for tuning.
    ly->score_wgs = 0;
    if (const char *e = std::getenv("SKV_SCORE_WGS")) ly->score_wgs = std::max(1, std::atoi(e));
    // bfloat16 takes the fused kernel at every group size (its weighted sum
    // runs on MFMA, whose 16 rows the heads fill at GQA 16); SKV_ATTN_FUSED=0
    // or 1 forces the separate QK + PV kernels or the fused one
    ly->fused = dm.bf16 != 0;
    if (const char *e = std::getenv("SKV_ATTN_FUSED")) ly->fused = dm.bf16 != 0 && std::atoi(e) != 0;
    // host V crosses PCIe in a coded form where the chunks allow it;
    // SKV_HOST_V_CODE=0 keeps it raw, 1 allows only the 12-bit form
    ly->vcoded = skv::vcode_values(dm) > 0;
    if (const char *e = std::getenv("SKV_HOST_V_CODE")) {
        const int f = std::atoi(e);
        ly->vcoded = ly->vcoded && f != 0;
        ly->vforms = f == 1 ? 1 : 3;  // 1: the 12-bit form only
    }

    const size_t B = dm.b, HKV = dm.hkv, HQ = dm.hq, D = dm.d, S = dm.s, E = dm.esize;
    const size_t bh = B * HKV;
#define ALLOC(ptr, bytes) \
    if ((rc = dalloc_t(ly, (bytes), &ly->ptr))) return bail(rc)
    ALLOC(A, B * S * dm.r * E);
    ALLOC(Bt, bh * D * dm.r * E);
    ALLOC(L, bh * dm.n * D * E);
    ALLOC(cand, bh * dm.mask_words * 4);
    ALLOC(outliers, bh * dm.o * 4);
    ALLOC(min_cos, bh * dm.n * 4);
    ALLOC(k_out, bh * dm.OC * D * E);
    ALLOC(v_out, bh * dm.OC * D * E);
    ALLOC(k_loc, bh * dm.wcap * D * E);
    ALLOC(v_loc, bh * dm.wcap * D * E);
    ALLOC(vc, bh * dm.cap * dm.c * D * E);
    ALLOC(slot_chunk, bh * dm.cap * 4);
    ALLOC(slot_stamp, bh * dm.cap * 4);
    ALLOC(sel, bh * dm.k * 4);
    ALLOC(sel_slot, bh * dm.k * 4);
    // U and the tile statistics hold up to kMaxGroup scored rows per KV head
    // (the SnapKV-style selection scores (head, window position) rows)
    ALLOC(P, bh * skv::kMaxGroup * dm.n * 4);
    ALLOC(stats, bh * skv::kMaxGroup * dm.wtiles * sizeof(float2));
    ALLOC(snap_acc, bh * dm.n * 4);
    ALLOC(S2, bh * dm.n * 4);
    ALLOC(misses, bh * dm.k * sizeof(int2));
    ALLOC(miss_count, bh * 4);
    // logits and split partials sized for a full local block (window plus
    // every appended token)
    const Dims dfull = dims_with_local(dm, dm.wcap);
    ALLOC(logits, B * HQ * dfull.NK * 4);
    // split partials: PV's key tiles, or the fused kernel's one split per workgroup
    const size_t splits = std::max<size_t>(dfull.pv_tiles, skv::attn_workgroups(dfull));
    ALLOC(part_ml, B * HQ * splits * sizeof(float2));
    ALLOC(part_acc, B * HQ * splits * D * 4);
    ALLOC(counters, 4 * sizeof(unsigned long long));
    ALLOC(vcode, bh * dm.n * 4);
    ALLOC(bad, 4);
    ALLOC(theta, D / 2 * sizeof(double));
    ALLOC(theta_rev, D / 2 * sizeof(double));
    const size_t lds_cap = static_cast<size_t>(ly->lds_limit);
    ly->select_keys_in_lds = skv::select_dynamic_lds(dm, true) + skv::select_static_lds() <= lds_cap;
    ly->topo_keys_in_lds = static_cast<size_t>(dm.n) * 4 + skv::select_static_lds() <= lds_cap;
    if (skv::select_dynamic_lds(dm, false) + skv::select_static_lds() > lds_cap)
        return bail(fail(SKV_E_SHAPE, "top_k too large for the select kernel's shared memory"));
    ALLOC(keys, bh * dm.n * 4);
    // measured on MI355X: with few rows the one-workgroup-per-row selection
    // leaves most CUs idle and the candidates win (GLM-shaped 244K b12, 24
    // rows: 47.4 against 53.4 us); at 64 rows they are even and at 384 rows
    // (60K b48) they lose (66.2 against 56.8 us).  SKV_SELECT_CAND=0/1 forces
    // either where both fit.
    ly->topk_cand = dm.k > 0 && skv::group_topk_lds(dm) + skv::select_static_lds() <= lds_cap &&
                    skv::select_cand_lds(dm) + skv::select_static_lds() <= lds_cap;
    const bool cand_fits = ly->topk_cand;
    ly->topk_cand = cand_fits && bh < 64;
    if (const char *e = std::getenv("SKV_SELECT_CAND")) ly->topk_cand = cand_fits && std::atoi(e) != 0;
    // The group score inside the selection kernel, where the rows alone fill
    // the CUs: one CU reads a row's U at a fraction of the device rate, so
    // with fewer rows the wide group kernel wins (measured on MI355X: 60K
    // b48, 384 rows: 44.4 against 47.5 us for group + select; 128K b8, 64
    // rows: 28.9 against 26.9 us, and splitting each row's score over four
    // workgroups, the last of which selects, 29.2 us).  SKV_SELECT_FUSED=0/1
    // forces either where it fits.
    {
        const bool fits = skv::select_fused_lds(dm) + skv::select_static_lds() <= lds_cap;
        bool want = fits && !ly->topk_cand && static_cast<long long>(bh) >= ly->cus;
        if (const char *e = std::getenv("SKV_SELECT_FUSED")) want = fits && std::atoi(e) != 0;
        if (const char *e = std::getenv("SKV_SELECT_CAND")) want = want && std::atoi(e) == 0;
        ly->select_fused = want;
        if (want) ly->topk_cand = false;
    }
    {
        const size_t cslots = ly->topk_cand ? bh * skv::topk_slices(dm) * dm.k : 0;
        ALLOC(cand_key, cslots * 4);
        ALLOC(cand_idx, cslots * 4);
        ALLOC(cand_count, (ly->topk_cand ? bh * skv::topk_slices(dm) : 0) * 4);
    }
    ALLOC(kbounds, bh * skv::group_slices(dm) * sizeof(uint2));
#undef ALLOC

    // RoPE rates: theta_i = base^(-2i/d) in double, and the same in turns
    // (theta_i / 2 pi) for the hardware sin/cos.
    std::vector<double> th(D / 2), thr(D / 2);
    for (size_t i = 0; i < D / 2; ++i) {
        th[i] = std::pow(static_cast<double>(cfg->rope_base), -2.0 * i / D);
        thr[i] = th[i] / (2.0 * 3.14159265358979323846);
    }
    if (hipMemcpy(ly->theta, th.data(), th.size() * sizeof(double), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(ly->theta_rev, thr.data(), thr.size() * sizeof(double), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemset(ly->counters, 0, 4 * sizeof(unsigned long long)) != hipSuccess ||
        (dm.wcap > 0 && (hipMemset(ly->k_loc, 0, bh * dm.wcap * D * E) != hipSuccess ||
                         hipMemset(ly->v_loc, 0, bh * dm.wcap * D * E) != hipSuccess)) ||
        (dm.cap > 0 && hipMemset(ly->vc, 0, bh * dm.cap * dm.c * D * E) != hipSuccess))
        return bail(fail(SKV_E_HIP, "initialising layer tables failed"));
    DevStreams *ds = nullptr;
    if ((rc = device_streams(ly->device, &ds))) return bail(rc);
    ly->copy = ds->fetch;
    ly->comp = ds->comp;
    if (hipEventCreateWithFlags(&ly->ev_sel, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ly->ev_fetch, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ly->ev_qk, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ly->ev_done, hipEventDisableTiming) != hipSuccess)
        return bail(fail(SKV_E_HIP, "creating events failed"));

    // Host-V fetch: enough waves to keep PCIe busy (a few hundred chunk reads
    // in flight while waves decode the coded forms), not so many that the
    // slow host reads crowd the memory path of the kernels running beside
    // them (measured, 128K b8 with the class form: 128 waves 43.4 GB/s of
    // coded bytes, 256 52.4, 512 50.7, 1024 52.2).  SKV_FETCH_WAVES overrides the
    // default for tuning.
    if (const char *e = std::getenv("SKV_FETCH_WAVES")) ly->fetch_waves = std::max(4, std::atoi(e));

    *out = ly;
    return SKV_OK;
}

void shadowkv_layer_destroy(skv_layer *layer) {
    if (!layer) return;
    release(layer);
    delete layer;
}

static int install_common(skv_layer *ly, const void *A, const void *B, void *v_host, hipStream_t st) {
    const Dims &dm = ly->dm;
    SKV_HIP(hipMemcpyAsync(ly->A, A, static_cast<size_t>(dm.b) * dm.s * dm.r * dm.esize, hipMemcpyDefault, st));
    SKV_HIP(skv::launch_transpose_b(dm, B, ly->Bt, st));
    SKV_HIP(skv::launch_cand_mask(dm, ly->outliers, ly->cand, st));
    SKV_HIP(skv::launch_fill_i32(ly->slot_chunk, -1, static_cast<size_t>(dm.b) * dm.hkv * dm.cap, st));
    ly->fixed = ly->fetch_pending = false;
    (void)v_host;
    return SKV_OK;
}

int shadowkv_prefill_meta(skv_layer *ly, const void *k_pre, const void *k_rope, const void *v, const void *A,
                          const void *B, void *v_host, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    if ((!k_pre && !k_rope) || !v || !A || !B) return fail(SKV_E_INVAL, "null input pointer");
    void *vdev = nullptr;
    int rc = check_pinned(v_host, &vdev);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const Dims &dm = ly->dm;
    ly->ready = false;
    // Step 5's V offload (a DMA copy over PCIe, tens of milliseconds at long
    // context) runs on the layer's copy stream beside steps 2-4's kernels,
    // which need only HBM; the caller's stream waits for it at the end.
    SKV_HIP(hipEventRecord(ly->ev_sel, st));
    SKV_HIP(hipStreamWaitEvent(ly->copy, ly->ev_sel, 0));
    const long long nchunks = static_cast<long long>(dm.b) * dm.hkv * dm.n;
    if (ly->vcoded) {
        // chunk by chunk into a coded form, through the device's staging
        // buffer, 64 MiB at a time (the chunks of V are contiguous)
        void *stage = nullptr;
        if ((rc = device_stage(ly->device, &stage))) return rc;
        const long long cb = 2LL * skv::vcode_values(dm), per = static_cast<long long>(kStageBytes) / cb;
        for (long long c0 = 0; c0 < nchunks; c0 += per) {
            const long long cnt = std::min(per, nchunks - c0);
            SKV_HIP(skv::launch_vcode(dm, ly->vforms, static_cast<const char *>(v) + c0 * cb, stage, ly->vcode + c0, cnt,
                                      ly->copy));
            SKV_HIP(hipMemcpyAsync(static_cast<char *>(v_host) + c0 * cb, stage, static_cast<size_t>(cnt * cb),
                                   hipMemcpyDeviceToHost, ly->copy));
        }
    } else {
        SKV_HIP(hipMemcpyAsync(v_host, v, static_cast<size_t>(dm.b) * dm.hkv * dm.s * dm.d * dm.esize,
                               hipMemcpyDeviceToHost, ly->copy));
        SKV_HIP(skv::launch_fill_i32(reinterpret_cast<int32_t *>(ly->vcode), 0, static_cast<size_t>(nchunks), ly->copy));
    }
    SKV_HIP(hipEventRecord(ly->ev_fetch, ly->copy));
    SKV_HIP(skv::launch_landmarks(dm, k_pre, k_rope, ly->theta, ly->L, ly->min_cos, st));
    SKV_HIP(skv::launch_topo(dm, ly->min_cos, ly->outliers, ly->keys, ly->topo_keys_in_lds, st));
    SKV_HIP(skv::launch_gather_static(dm, k_pre, k_rope, v, ly->outliers, ly->theta, ly->k_out, ly->v_out,
                                      ly->k_loc, ly->v_loc, st));
    if ((rc = install_common(ly, A, B, v_host, st))) return rc;
    SKV_HIP(hipStreamWaitEvent(st, ly->ev_fetch, 0));
    ly->v_host_dev = vdev;
    ly->n_app = 0;
    ly->ready = true;
    return mark_done(ly, st);
}

int shadowkv_load_meta(skv_layer *ly, const void *landmarks, const int32_t *outliers, const void *k_out,
                       const void *v_out, const void *k_loc, const void *v_loc, const void *A, const void *B,
                       void *v_host, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    const Dims &dm = ly->dm;
    if (!landmarks || !A || !B || (dm.o > 0 && (!outliers || !k_out || !v_out)) || (dm.w > 0 && (!k_loc || !v_loc)))
        return fail(SKV_E_INVAL, "null input pointer");
    void *vdev = nullptr;
    int rc = check_pinned(v_host, &vdev);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const size_t bh = static_cast<size_t>(dm.b) * dm.hkv, E = dm.esize, D = dm.d;
    ly->ready = false;
    if (dm.o > 0) {
        SKV_HIP(hipMemcpyAsync(ly->outliers, outliers, bh * dm.o * 4, hipMemcpyDefault, st));
        SKV_HIP(skv::launch_fill_i32(ly->bad, 0, 1, st));
        SKV_HIP(skv::launch_validate_outliers(dm, ly->outliers, ly->bad, st));
        int32_t nbad = 0;
        SKV_HIP(hipMemcpyAsync(&nbad, ly->bad, 4, hipMemcpyDeviceToHost, st));
        SKV_HIP(hipStreamSynchronize(st));
        if (nbad) return fail(SKV_E_SHAPE, "outlier rows must be strictly ascending and lie in [0, n - n_loc)");
        SKV_HIP(hipMemcpyAsync(ly->k_out, k_out, bh * dm.OC * D * E, hipMemcpyDefault, st));
        SKV_HIP(hipMemcpyAsync(ly->v_out, v_out, bh * dm.OC * D * E, hipMemcpyDefault, st));
    }
    SKV_HIP(hipMemcpyAsync(ly->L, landmarks, bh * dm.n * D * E, hipMemcpyDefault, st));
    if (dm.w > 0) {
        // (b, h_kv, w, d) into the local buffers' rows of w + max_new
        const size_t row = static_cast<size_t>(dm.w) * D * E, pitch = static_cast<size_t>(dm.wcap) * D * E;
        SKV_HIP(hipMemcpy2DAsync(ly->k_loc, pitch, k_loc, row, row, bh, hipMemcpyDefault, st));
        SKV_HIP(hipMemcpy2DAsync(ly->v_loc, pitch, v_loc, row, row, bh, hipMemcpyDefault, st));
    }
    // the caller's host V is raw
    SKV_HIP(skv::launch_fill_i32(reinterpret_cast<int32_t *>(ly->vcode), 0, bh * dm.n, st));
    if ((rc = install_common(ly, A, B, v_host, st))) return rc;
    ly->v_host_dev = vdev;
    ly->n_app = 0;
    ly->ready = true;
    return mark_done(ly, st);
}

int shadowkv_append(skv_layer *ly, const void *k_new, const void *v_new, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    if (!k_new || !v_new) return fail(SKV_E_INVAL, "null k_new or v_new");
    if (!ly->ready) return fail(SKV_E_STATE, "append before prefill_meta / load_meta");
    const Dims &dm = ly->dm;
    if (ly->n_app >= dm.wcap - dm.w) return fail(SKV_E_SHAPE, "the local block is full (max_new tokens appended)");
    hipStream_t st = static_cast<hipStream_t>(stream);
    SKV_HIP(skv::launch_append(dm, k_new, v_new, ly->theta, ly->k_loc, ly->v_loc, dm.w + ly->n_app,
                               dm.s + ly->n_app, st));
    ++ly->n_app;
    return mark_done(ly, st);
}

int shadowkv_snapkv_select(skv_layer *ly, const void *q_obs, int w_obs, int pool, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    if (!q_obs) return fail(SKV_E_INVAL, "null q_obs");
    if (!ly->ready) return fail(SKV_E_STATE, "snapkv_select before prefill_meta / load_meta");
    if (w_obs < 1 || w_obs > 4096) return fail(SKV_E_SHAPE, "w_obs must be in [1, 4096]");
    if (pool < 1 || pool > 63 || pool % 2 == 0) return fail(SKV_E_SHAPE, "pool must be odd, in [1, 63]");
    const Dims &dm = ly->dm;
    if (dm.k <= 0) return fail(SKV_E_SHAPE, "top_k is 0: there is nothing to select");
    if (static_cast<double>(dm.b) * dm.hkv * dm.G * w_obs * dm.d * dm.esize >= static_cast<double>(1u << 30))
        return fail(SKV_E_SHAPE, "q_obs must be smaller than 1 GiB");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // A selection made by an earlier call whose missing V no decode step has
    // fetched yet: its chunks already own their cache slots, so they would
    // count as hits of this selection.  Fetch them first, which keeps the
    // cache lossless.
    if (ly->fetch_pending) {
        SKV_HIP(skv::launch_fetch(dm, ly->v_host_dev, ly->vc, ly->misses, ly->miss_count, ly->vcode, ly->counters, ly->fetch_waves, st));
        ly->fetch_pending = false;
    }
    // passes of up to kMaxGroup (head, window position) rows per KV head
    const int wp_max = std::max(1, skv::kMaxGroup / dm.G);
    for (int o0 = 0; o0 < w_obs; o0 += wp_max) {
        const int wp = std::min(wp_max, w_obs - o0);
        Dims dv = dm;  // the pass's scored rows as the group's heads
        dv.G = dm.G * wp;
        dv.GP = dv.G <= 4 ? 4 : (dv.G <= 8 ? 8 : 16);
        SKV_HIP(skv::launch_score(dm, q_obs, ly->L, ly->cand, ly->P, ly->stats, ly->score_wgs,
                                  skv::QRows{w_obs, o0, wp}, st));
        SKV_HIP(skv::launch_group(dv, ly->P, ly->stats, ly->cand, ly->S2, ly->keys, ly->kbounds, st));
        SKV_HIP(skv::launch_snap_accum(dm, ly->S2, ly->snap_acc, static_cast<float>(dv.G), o0 == 0, st));
    }
    SKV_HIP(skv::launch_snap_pool(dm, ly->snap_acc, ly->cand, ly->S2, ly->keys, ly->kbounds, pool, st));
    SKV_HIP(skv::launch_select(dm, ly->keys, ly->kbounds, ly->sel, ly->sel_slot, ly->slot_chunk,
                               ly->slot_stamp, ++ly->stamp, ly->misses, ly->miss_count, ly->counters,
                               ly->select_keys_in_lds, st));
    ly->fixed = true;
    ly->fetch_pending = true;
    return mark_done(ly, st);
}

// One decode step (Algorithm 2) with its per-step scratch in `sc`.  `timed`:
// bracket the kernels with the layer's timing events when timing is on.
static int decode_impl(skv_layer *ly, const void *q, void *out, hipStream_t st, const Dims &dm,
                       const StepScratch &sc, bool timed) {
    // with exactly k cache slots the slots hold the selection: the rebuilt
    // keys go in slot order and PV reads the cache contiguously; a larger
    // cache holds other chunks too, so the keys go in selection order and PV
    // looks up each chunk's slot
    const bool by_slot = dm.cap == dm.k;
    const int32_t *qk_chunks = by_slot ? ly->slot_chunk : ly->sel;
    const int32_t *pv_slots = by_slot ? nullptr : ly->sel_slot;
    // a fixed (SnapKV-style) selection skips scoring and selection, and
    // fetches only once, on the first step after it was made
    const bool select = !ly->fixed, fetch = select || ly->fetch_pending;
    if (select) {
        {
            Timed t(ly, SKV_K_SCORE, st, timed);
            SKV_HIP(skv::launch_score(dm, q, ly->L, ly->cand, sc.P, sc.stats, ly->score_wgs, skv::QRows{1, 0, 1},
                                      st));
        }
        {
            Timed t(ly, SKV_K_SELECT, st, timed);
            if (ly->select_fused) {
                SKV_HIP(skv::launch_select_fused(dm, sc.P, sc.stats, ly->cand, sc.S2, ly->sel, ly->sel_slot,
                                                 ly->slot_chunk, ly->slot_stamp, ++ly->stamp, ly->misses,
                                                 ly->miss_count, ly->counters, st));
            } else if (ly->topk_cand) {
                SKV_HIP(skv::launch_group_topk(dm, sc.P, sc.stats, ly->cand, sc.S2, sc.cand_key, sc.cand_idx,
                                               sc.cand_count, st));
                SKV_HIP(skv::launch_select_cand(dm, sc.cand_key, sc.cand_idx, sc.cand_count, ly->sel,
                                                ly->sel_slot, ly->slot_chunk, ly->slot_stamp, ++ly->stamp,
                                                ly->misses, ly->miss_count, ly->counters, st));
            } else {
                SKV_HIP(skv::launch_group(dm, sc.P, sc.stats, ly->cand, sc.S2, sc.keys, sc.kbounds, st));
                SKV_HIP(skv::launch_select(dm, sc.keys, sc.kbounds, ly->sel, ly->sel_slot, ly->slot_chunk,
                                           ly->slot_stamp, ++ly->stamp, ly->misses, ly->miss_count, ly->counters,
                                           ly->select_keys_in_lds, st));
            }
        }
    }
    if (ly->overlap) {
        // fork: the fetch of missing V on the fetch stream, the key rebuild
        // and logits on the compute stream; join before PV
        SKV_HIP(hipEventRecord(ly->ev_sel, st));
        SKV_HIP(hipStreamWaitEvent(ly->copy, ly->ev_sel, 0));
        SKV_HIP(hipStreamWaitEvent(ly->comp, ly->ev_sel, 0));
        if (fetch) {
            Timed t(ly, SKV_K_FETCH, ly->copy, timed);
            SKV_HIP(skv::launch_fetch(dm, ly->v_host_dev, ly->vc, ly->misses, ly->miss_count, ly->vcode, ly->counters, ly->fetch_waves,
                                      ly->copy));
        }
        SKV_HIP(hipEventRecord(ly->ev_fetch, ly->copy));
        {
            Timed t(ly, SKV_K_QK, ly->comp, timed);
            SKV_HIP(skv::launch_qk(dm, q, ly->k_out, ly->k_loc, ly->A, ly->Bt, qk_chunks, ly->theta,
                                   ly->theta_rev, sc.logits, ly->comp));
        }
        SKV_HIP(hipEventRecord(ly->ev_qk, ly->comp));
        SKV_HIP(hipStreamWaitEvent(st, ly->ev_qk, 0));
        SKV_HIP(hipStreamWaitEvent(st, ly->ev_fetch, 0));
    } else {
        // one queue: the fetch runs alone on PCIe, then attention
        if (fetch) {
            Timed t(ly, SKV_K_FETCH, st, timed);
            SKV_HIP(skv::launch_fetch(dm, ly->v_host_dev, ly->vc, ly->misses, ly->miss_count, ly->vcode, ly->counters, ly->fetch_waves,
                                      st));
        }
        if (ly->fused) {
            Timed t(ly, SKV_K_ATTN, st, timed);
            SKV_HIP(skv::launch_attn(dm, q, ly->A, ly->Bt, qk_chunks, pv_slots, ly->theta_rev, ly->k_out, ly->v_out,
                                     ly->k_loc, ly->v_loc, ly->vc, sc.part_ml, sc.part_acc, st));
            SKV_HIP(skv::launch_combine(dm, sc.part_ml, sc.part_acc, out, skv::attn_workgroups(dm), st));
        } else {
            Timed t(ly, SKV_K_QK, st, timed);
            SKV_HIP(skv::launch_qk(dm, q, ly->k_out, ly->k_loc, ly->A, ly->Bt, qk_chunks, ly->theta,
                                   ly->theta_rev, sc.logits, st));
        }
    }
    ly->fetch_pending = false;
    if (ly->overlap || !ly->fused) {
        Timed t(ly, SKV_K_PV, st, timed);
        SKV_HIP(skv::launch_pv(dm, sc.logits, ly->v_out, ly->vc, pv_slots, ly->v_loc, sc.part_ml,
                               sc.part_acc, st));
        SKV_HIP(skv::launch_combine(dm, sc.part_ml, sc.part_acc, out, dm.pv_tiles, st));
    }
    if (timed && ly->timing) ++ly->timed_steps;
    return mark_done(ly, st);
}

int shadowkv_decode_step(skv_layer *ly, const void *q, void *out, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    if (!q || !out) return fail(SKV_E_INVAL, "null q or out");
    if (!ly->ready) return fail(SKV_E_STATE, "decode_step before prefill_meta / load_meta");
    const Dims dm = dims_with_local(ly->dm, ly->dm.w + ly->n_app);
    const StepScratch sc{ly->P, ly->stats, ly->S2, ly->keys, ly->kbounds, ly->cand_key, ly->cand_idx,
                         ly->cand_count, ly->logits, ly->part_ml, ly->part_acc};
    return decode_impl(ly, q, out, static_cast<hipStream_t>(stream), dm, sc, true);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decoding without allocation.  shadowkv_decode_step_noalloc takes the step's
// scratch (the buffers of StepScratch) from `scratch`, a file-scope device
// array of kStaticScratchBytes, instead of the layer's own.  In host code
// `scratch` names a host-side stand-in, never a device address: its device
// address is looked up once per device (with that device current) and only
// that address reaches kernels.  Every call on one GPU shares its array.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kStaticScratchBytes = size_t(128) << 20;  // 128 MiB per GPU
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_dev[64] = {};  // device address of `scratch` on each device

int static_scratch(int device, void **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (device < 0 || device >= 64) return fail(SKV_E_INVAL, "device index out of range");
    if (!g_scratch_dev[device]) {
        int cur = -1;
        SKV_HIP(hipGetDevice(&cur));
        if (cur != device) SKV_HIP(hipSetDevice(device));
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) SKV_HIP(hipSetDevice(cur));
        if (e != hipSuccess || !p)
            return fail(SKV_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_dev[device] = p;
    }
    *out = g_scratch_dev[device];
    return SKV_OK;
}

// The step's scratch carved from `base` in 256-byte aligned pieces, only the
// buffers this layer's schedule uses; returns the bytes taken (base null:
// the size only, every pointer null).
size_t carve_step_scratch(const skv_layer *ly, const Dims &dm, char *base, StepScratch *sc) {
    size_t used = 0;
    auto take = [&](size_t bytes) -> char * {
        const size_t off = (used + 255) / 256 * 256;
        used = off + std::max<size_t>(bytes, 4);
        return base ? base + off : nullptr;
    };
    const size_t bh = static_cast<size_t>(dm.b) * dm.hkv, hq = static_cast<size_t>(dm.b) * dm.hq;
    *sc = StepScratch{};
    if (!ly->fixed) {  // scoring and selection run
        sc->P = reinterpret_cast<float *>(take(bh * dm.G * dm.n * 4));
        sc->stats = reinterpret_cast<float2 *>(take(bh * dm.G * dm.wtiles * sizeof(float2)));
        sc->S2 = reinterpret_cast<float *>(take(bh * dm.n * 4));
        if (ly->topk_cand) {
            const size_t cs = bh * skv::topk_slices(dm);
            sc->cand_key = reinterpret_cast<uint32_t *>(take(cs * dm.k * 4));
            sc->cand_idx = reinterpret_cast<int32_t *>(take(cs * dm.k * 4));
            sc->cand_count = reinterpret_cast<int32_t *>(take(cs * 4));
        } else {
            sc->keys = reinterpret_cast<uint32_t *>(take(bh * dm.n * 4));
            sc->kbounds = reinterpret_cast<uint2 *>(take(bh * skv::group_slices(dm) * sizeof(uint2)));
        }
    }
    const bool separate = ly->overlap || !ly->fused;
    if (separate) sc->logits = reinterpret_cast<float *>(take(hq * dm.NK * 4));
    const size_t splits = separate ? static_cast<size_t>(dm.pv_tiles) : skv::attn_workgroups(dm);
    sc->part_ml = reinterpret_cast<float2 *>(take(hq * splits * sizeof(float2)));
    sc->part_acc = reinterpret_cast<float *>(take(hq * splits * dm.d * 4));
    return used;
}

}  // namespace

extern "C" {

int shadowkv_decode_step_noalloc(skv_layer *ly, const void *q, void *out, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    if (!q || !out) return fail(SKV_E_INVAL, "null q or out");
    const Dims dm = dims_with_local(ly->dm, ly->dm.w + ly->n_app);
    StepScratch sc{};
    const size_t need = carve_step_scratch(ly, dm, nullptr, &sc);
    if (need > kStaticScratchBytes)
        return fail(SKV_E_SHAPE, "this layer's decode step needs " + std::to_string(need) +
                                     " bytes of scratch; the static scratch holds " +
                                     std::to_string(kStaticScratchBytes) + " (use shadowkv_decode_step)");
    if (!ly->ready) return fail(SKV_E_STATE, "decode_step before prefill_meta / load_meta");
    void *base = nullptr;
    int rc = static_scratch(ly->device, &base);
    if (rc) return rc;
    carve_step_scratch(ly, dm, static_cast<char *>(base), &sc);
    return decode_impl(ly, q, out, static_cast<hipStream_t>(stream), dm, sc, false);
}

int shadowkv_reset_cache(skv_layer *ly, void *stream) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    hipStream_t st = static_cast<hipStream_t>(stream);
    SKV_HIP(hipStreamWaitEvent(st, ly->ev_fetch, 0));
    SKV_HIP(skv::launch_fill_i32(ly->slot_chunk, -1, static_cast<size_t>(ly->dm.b) * ly->dm.hkv * ly->dm.cap, st));
    ly->fixed = ly->fetch_pending = false;
    return mark_done(ly, st);
}

// The counters are read and cleared on the layer's copy stream after the
// layer's latest work: neither waits for anything else on the device.
int shadowkv_get_stats(skv_layer *ly, skv_stats *out) {
    if (!ly || !out) return fail(SKV_E_INVAL, "null argument");
    unsigned long long c[4] = {0, 0, 0, 0};
    SKV_HIP(hipStreamWaitEvent(ly->copy, ly->ev_done, 0));
    SKV_HIP(hipMemcpyAsync(c, ly->counters, sizeof(c), hipMemcpyDeviceToHost, ly->copy));
    SKV_HIP(hipStreamSynchronize(ly->copy));
    out->hits = static_cast<int64_t>(c[0]);
    out->misses = static_cast<int64_t>(c[1]);
    out->steps = static_cast<int64_t>(c[2]);
    out->bytes_h2d = static_cast<int64_t>(c[3]);  // counted by the fetch: what crossed PCIe
    return SKV_OK;
}

int shadowkv_reset_stats(skv_layer *ly) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    SKV_HIP(hipStreamWaitEvent(ly->copy, ly->ev_done, 0));
    SKV_HIP(skv::launch_fill_i32(reinterpret_cast<int32_t *>(ly->counters), 0, 8, ly->copy));
    SKV_HIP(hipStreamSynchronize(ly->copy));
    return SKV_OK;
}

static const void *tensor_ptr(const skv_layer *ly, int which, size_t *bytes) {
    const Dims &dm = ly->dm;
    const size_t bh = static_cast<size_t>(dm.b) * dm.hkv, E = dm.esize, D = dm.d;
    switch (which) {
        case SKV_T_LANDMARKS: *bytes = bh * dm.n * D * E; return ly->L;
        case SKV_T_MIN_COS: *bytes = bh * dm.n * 4; return ly->min_cos;
        case SKV_T_OUTLIERS: *bytes = bh * dm.o * 4; return ly->outliers;
        case SKV_T_CAND_MASK: *bytes = bh * dm.mask_words * 4; return ly->cand;
        case SKV_T_SCORES: *bytes = bh * dm.n * dm.G * 4; return ly->P;
        case SKV_T_GROUP_SCORES: *bytes = bh * dm.n * 4; return ly->S2;
        case SKV_T_SELECTION: *bytes = bh * dm.k * 4; return ly->sel;
        case SKV_T_SLOT_CHUNKS: *bytes = bh * dm.cap * 4; return ly->slot_chunk;
        case SKV_T_CACHE_V: *bytes = bh * dm.cap * dm.c * D * E; return ly->vc;
        case SKV_T_SELECTION_SLOTS: *bytes = bh * dm.k * 4; return ly->sel_slot;
        case SKV_T_V_CODES: *bytes = bh * dm.n * 4; return ly->vcode;
        case SKV_T_K_OUT: *bytes = bh * dm.OC * D * E; return ly->k_out;
        case SKV_T_V_OUT: *bytes = bh * dm.OC * D * E; return ly->v_out;
        case SKV_T_K_LOC: *bytes = bh * dm.wcap * D * E; return ly->k_loc;
        case SKV_T_V_LOC: *bytes = bh * dm.wcap * D * E; return ly->v_loc;
        default: *bytes = 0; return nullptr;
    }
}

size_t shadowkv_tensor_bytes(const skv_layer *ly, int which) {
    if (!ly) return 0;
    size_t bytes = 0;
    tensor_ptr(ly, which, &bytes);
    return bytes;
}

int shadowkv_read(skv_layer *ly, int which, void *dst, size_t bytes, void *stream) {
    if (!ly || !dst) return fail(SKV_E_INVAL, "null argument");
    size_t need = 0;
    const void *src = tensor_ptr(ly, which, &need);
    if (!src) return fail(SKV_E_INVAL, "unknown tensor id");
    if (bytes != need) return fail(SKV_E_SHAPE, "byte count does not match the tensor size");
    if (need == 0) return SKV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    SKV_HIP(hipStreamWaitEvent(st, ly->ev_fetch, 0));
    SKV_HIP(hipMemcpyAsync(dst, src, need, hipMemcpyDefault, st));
    return SKV_OK;
}

int shadowkv_set_overlap(skv_layer *ly, int enable) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    ly->overlap = enable != 0;
    return SKV_OK;
}

int shadowkv_set_timing(skv_layer *ly, int enable) {
    if (!ly) return fail(SKV_E_INVAL, "layer is null");
    ly->timing = enable != 0;
    return SKV_OK;
}

int shadowkv_get_timing(skv_layer *ly, double *ms_out, int64_t *steps_out) {
    if (!ly || !ms_out) return fail(SKV_E_INVAL, "null argument");
    for (int i = 0; i < SKV_K_COUNT; ++i) ms_out[i] = 0.0;
    for (const Mark &m : ly->marks) {
        float ms = 0.f;
        SKV_HIP(hipEventSynchronize(m.stop));  // this kernel's own stream, up to its stop
        SKV_HIP(hipEventElapsedTime(&ms, m.start, m.stop));
        ms_out[m.kernel] += ms;
    }
    if (steps_out) *steps_out = ly->timed_steps;
    ly->marks.clear();
    ly->ev_used = 0;
    ly->timed_steps = 0;
    return SKV_OK;
}

}  // extern "C"
