/*
 * ShadowKV sparse decode step -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference
 * that the HIP library is checked against.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark load it.  It shares no code,
 * header or table with the HIP library, and includes nothing from it.
 *
 * What it follows (the review page "ShadowKV: KV Cache in Shadows for
 * High-Throughput Long-Context LLM Inference", xllm-io paper-review blog):
 *   - section 三 技术架构, "Algorithm 1: Pre-filling"  -> orc_prefill
 *   - section 三 技术架构, "Algorithm 2: Decoding"     -> orc_decode, orc_attend
 *   - section 三 技术架构, 核心公式, equivalent-bandwidth formula
 *                                                      -> orc_equiv_bandwidth
 *   - section 三 关键参数 table (chunk 8, rank 160, 48 outlier chunks, 1.56%)
 * and the Telegram write-up "Ускорение E2E-инференса через оптимизацию
 * KV-кэша. Часть II" (per-layer cache that loads only the set difference
 * between consecutive steps; lossless) -- the cache itself is simulated in
 * the Python wrapper, because the attended set never depends on it.
 *
 * Every floating-point step is carried out in double precision.  Where the
 * storage type is bfloat16 the oracle rounds (round-to-nearest-even) exactly
 * where the stored tensors are rounded: the post-RoPE keys and the chunk
 * means (landmarks).  Where a floating-point value decides an index (which
 * chunks are outliers, which chunks are selected) the value is first rounded
 * to binary32, the precision the GPU takes that decision in, and exact ties
 * go to the lower index.
 *
 * Readings taken where the page is silent or garbled (each is also recorded
 * in the repository's design notes):
 *   S2 (undefined in Algorithm 2 step 2): softmax over candidate chunks of
 *     each query head's scores P = q.L^T / sqrt(d), averaged over the query
 *     heads of one KV group.
 *   The third key block of Algorithm 2 step 4 (its subscript is lost): the
 *     last w context tokens, dense and post-RoPE.
 *   Outlier, selected and local chunks partition the context: the local
 *     window's chunks are never outliers, and neither outliers nor local
 *     chunks are selectable.
 *   RoPE: rotate-half pairs (i, i + d/2), theta_i = base^(-2i/d), 0-based
 *     positions.  The query is supplied already rotated.
 *   GQA: query head g reads KV head g / (h_q / h_kv).
 *   Cosine: denominator max(|a||b|, 1e-12).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t b;       /* sequences                              */
    int32_t h_q;     /* query heads                            */
    int32_t h_kv;    /* key/value heads                        */
    int32_t d;       /* head dimension (even)                  */
    int32_t s;       /* context length, a multiple of c        */
    int32_t c;       /* chunk size                             */
    int32_t r;       /* SVD rank                               */
    int32_t o;       /* outlier chunks per (sequence, KV head) */
    int32_t k;       /* selected chunks per (sequence, KV head)*/
    int32_t w;       /* local window in tokens, a multiple of c*/
    double rope_base;
    int32_t bf16;    /* 1: stored tensors are bfloat16         */
    int32_t n_app;   /* decode tokens appended after the window:
                        the local block holds w + n_app tokens  */
    int32_t plant;   /* 0 always, except in the tests that show a
                        parity case would catch a broken rebuild:
                        ORC_PLANT_* below                       */
} orc_cfg;

/* Deliberate mistakes in the rebuilt-key block of orc_attend, planted only by
 * the tests that check a parity case discriminates (a correct kernel must be
 * far closer to the unplanted oracle than any of these). */
enum {
    ORC_PLANT_NONE = 0,
    ORC_PLANT_ZERO_REBUILT = 1,     /* rebuilt keys replaced by zeros          */
    ORC_PLANT_NO_ROPE_REBUILT = 2,  /* rebuilt keys left unrotated             */
    ORC_PLANT_POS_PLUS_ONE = 3,     /* rebuilt keys rotated one position late  */
    ORC_PLANT_NO_OUTLIERS = 4,      /* outlier block left out of the softmax   */
    /* Not a mistake: rebuilt, rotated keys rounded to bfloat16 before the
     * logits, the quantisation point of the bfloat16 kernels.  Its distance
     * from the unplanted result is the share of the error bar it uses. */
    ORC_PLANT_BF16_REBUILT = 5
};

enum { ORC_OK = 0, ORC_E_SHAPE = -2, ORC_E_NOMEM = -4 };

/* ------------------------------------------------------------------------ */
/* bfloat16 rounding from its definition: 8 significant bits, the exponent  */
/* range of binary32 (normal numbers down to 2^-126, subnormal spacing      */
/* 2^-133), round to nearest with ties to even, overflow to infinity.       */
/* ------------------------------------------------------------------------ */
double orc_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                  /* x = m * 2^e, 0.5 <= |m| < 1        */
    int q = e - 8;                 /* spacing of 8-bit significands      */
    if (q < -133) q = -133;        /* subnormal range                    */
    double scaled = ldexp(x, -q);  /* exact: only the exponent changes   */
    double rounded = nearbyint(scaled);   /* default mode: ties to even  */
    double y = ldexp(rounded, q);
    /* largest finite bfloat16 is (2 - 2^-7) * 2^127 */
    if (fabs(y) > ldexp(2.0 - ldexp(1.0, -7), 127)) return copysign(INFINITY, x);
    return y;
}

/* In-place rounding of an array (used for the factors A and B). */
void orc_round_bf16_n(double *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) x[i] = orc_round_bf16(x[i]);
}

static double store(const orc_cfg *cfg, double x)
{
    return cfg->bf16 ? orc_round_bf16(x) : (double)(float)x;
}

/* ------------------------------------------------------------------------ */
/* RoPE, rotate-half form, at one position.                                 */
/* ------------------------------------------------------------------------ */
void orc_rope_row(const double *x, double *y, int32_t d, double pos, double base)
{
    int32_t half = d / 2;
    for (int32_t i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)d);
        double a = pos * theta;
        double cs = cos(a), sn = sin(a);
        double x1 = x[i], x2 = x[i + half];
        y[i] = x1 * cs - x2 * sn;
        y[i + half] = x2 * cs + x1 * sn;
    }
}

/* ------------------------------------------------------------------------ */
/* ArgTopK: the k largest keys among valid entries, exact ties to the lower */
/* index, returned in ascending index order.                                */
/* ------------------------------------------------------------------------ */
typedef struct { double key; int32_t idx; } keyed;

static int by_key_desc(const void *pa, const void *pb)
{
    const keyed *a = (const keyed *)pa, *b = (const keyed *)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

static int by_int_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int orc_topk(const double *key, const uint8_t *valid, int32_t n, int32_t k, int32_t *out)
{
    keyed *items = (keyed *)malloc(sizeof(keyed) * (size_t)(n > 0 ? n : 1));
    if (!items) return ORC_E_NOMEM;
    int32_t m = 0;
    for (int32_t j = 0; j < n; ++j)
        if (!valid || valid[j]) { items[m].key = key[j]; items[m].idx = j; ++m; }
    if (k > m) { free(items); return ORC_E_SHAPE; }
    qsort(items, (size_t)m, sizeof(keyed), by_key_desc);
    for (int32_t i = 0; i < k; ++i) out[i] = items[i].idx;
    qsort(out, (size_t)k, sizeof(int32_t), by_int_asc);
    free(items);
    return ORC_OK;
}

static int check_cfg(const orc_cfg *g)
{
    if (g->b < 1 || g->h_kv < 1 || g->h_q < g->h_kv || g->h_q % g->h_kv) return ORC_E_SHAPE;
    if (g->d < 2 || g->d % 2 || g->c < 1 || g->s < g->c || g->s % g->c) return ORC_E_SHAPE;
    if (g->w < 0 || g->w % g->c || g->w > g->s) return ORC_E_SHAPE;
    int32_t n = g->s / g->c, n_loc = g->w / g->c;
    if (g->o < 0 || g->o > n - n_loc) return ORC_E_SHAPE;
    if (g->k < 0 || g->k > n - n_loc - g->o) return ORC_E_SHAPE;
    if ((int64_t)g->o * g->c + (int64_t)g->k * g->c + g->w < 1) return ORC_E_SHAPE;
    if (g->r < 1) return ORC_E_SHAPE;
    if (g->n_app < 0) return ORC_E_SHAPE;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Algorithm 1 (Pre-filling), steps 2-5, per (sequence, KV head).           */
/*   k_pre, v      : (b, h_kv, s, d)  pre-RoPE keys, values                 */
/*   landmarks     : (b, h_kv, n, d)  chunk means of the post-RoPE keys     */
/*   min_cos       : (b, h_kv, n)     min over the chunk's tokens of the    */
/*                                    cosine to the chunk's landmark        */
/*   outliers      : (b, h_kv, o)     ascending chunk indices               */
/*   k_out, v_out  : (b, h_kv, o*c, d) post-RoPE K / V of outlier chunks    */
/*   k_loc, v_loc  : (b, h_kv, w, d)  post-RoPE K / V of the last w tokens  */
/*   cand          : (b, h_kv, n)     1 for selectable chunks               */
/* Step 1 (the SVD) is a library routine called from the Python wrapper.    */
/* ------------------------------------------------------------------------ */
int orc_prefill(const orc_cfg *cfg, const double *k_pre, const double *v,
                double *landmarks, double *min_cos, int32_t *outliers,
                double *k_out, double *v_out, double *k_loc, double *v_loc,
                uint8_t *cand)
{
    int rc = check_cfg(cfg);
    if (rc) return rc;
    const int32_t B = cfg->b, H = cfg->h_kv, d = cfg->d, s = cfg->s, c = cfg->c;
    const int32_t n = s / c, n_loc = cfg->w / c, o = cfg->o, w = cfg->w;
    int failed = 0;

#pragma omp parallel for schedule(dynamic) reduction(| : failed)
    for (int32_t bh = 0; bh < B * H; ++bh) {
        const double *K = k_pre + (size_t)bh * s * d;
        const double *Vh = v + (size_t)bh * s * d;
        double *Kr = (double *)malloc(sizeof(double) * (size_t)s * d);
        double *key = (double *)malloc(sizeof(double) * (size_t)n);
        uint8_t *valid = (uint8_t *)malloc((size_t)n);
        if (!Kr || !key || !valid) { free(Kr); free(key); free(valid); failed = 1; continue; }

        /* K_RoPE: every token rotated at its own position, then stored. */
        for (int32_t t = 0; t < s; ++t) {
            orc_rope_row(K + (size_t)t * d, Kr + (size_t)t * d, d, (double)t, cfg->rope_base);
            for (int32_t i = 0; i < d; ++i) Kr[(size_t)t * d + i] = store(cfg, Kr[(size_t)t * d + i]);
        }

        double *Lh = landmarks + (size_t)bh * n * d;
        double *mh = min_cos + (size_t)bh * n;
        for (int32_t j = 0; j < n; ++j) {
            /* Step 2: Reduce(K_RoPE) -- the chunk mean, stored. */
            for (int32_t i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int32_t t = 0; t < c; ++t) acc += Kr[((size_t)j * c + t) * d + i];
                Lh[(size_t)j * d + i] = store(cfg, acc / c);
            }
            /* Step 3: CosineSimilarity(C, K_RoPE); step 4's Min over tokens. */
            double lnorm = 0.0;
            for (int32_t i = 0; i < d; ++i) lnorm += Lh[(size_t)j * d + i] * Lh[(size_t)j * d + i];
            lnorm = sqrt(lnorm);
            double mn = INFINITY;
            for (int32_t t = 0; t < c; ++t) {
                const double *x = Kr + ((size_t)j * c + t) * d;
                double dot = 0.0, xn = 0.0;
                for (int32_t i = 0; i < d; ++i) { dot += x[i] * Lh[(size_t)j * d + i]; xn += x[i] * x[i]; }
                double den = sqrt(xn) * lnorm;
                double cs = dot / (den > 1e-12 ? den : 1e-12);
                if (cs < mn) mn = cs;
            }
            mh[j] = mn;
        }

        /* Step 4: ArgTopK(-Min(S), o) over chunks outside the local window;  */
        /* the decision is taken on binary32-rounded values.                  */
        for (int32_t j = 0; j < n; ++j) { key[j] = -(double)(float)mh[j]; valid[j] = (uint8_t)(j < n - n_loc); }
        int32_t *oh = outliers + (size_t)bh * o;
        if (orc_topk(key, valid, n, o, oh)) failed = 1;

        /* Static GPU-resident buffers: outlier chunks and the local window. */
        for (int32_t a = 0; a < o; ++a)
            for (int32_t t = 0; t < c; ++t) {
                size_t src = ((size_t)oh[a] * c + t) * d, dst = ((size_t)bh * o * c + (size_t)a * c + t) * d;
                memcpy(k_out + dst, Kr + src, sizeof(double) * d);
                memcpy(v_out + dst, Vh + src, sizeof(double) * d);
            }
        for (int32_t t = 0; t < w; ++t) {
            size_t src = (size_t)(s - w + t) * d, dst = ((size_t)bh * w + t) * d;
            memcpy(k_loc + dst, Kr + src, sizeof(double) * d);
            memcpy(v_loc + dst, Vh + src, sizeof(double) * d);
        }

        /* Selectable chunks: outside the local window and not outliers. */
        uint8_t *ch = cand + (size_t)bh * n;
        for (int32_t j = 0; j < n; ++j) ch[j] = (uint8_t)(j < n - n_loc);
        for (int32_t a = 0; a < o; ++a) ch[oh[a]] = 0;

        free(Kr); free(key); free(valid);
    }
    return failed ? ORC_E_NOMEM : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Algorithm 2 steps 3-4 for a given selection: rebuild the selected keys   */
/* as Gather(A, I) times B, rotate them at their original positions, gather */
/* V, and attend over [outlier keys; rotated rebuilt keys; local keys].     */
/*   q     : (b, h_q, d)      post-RoPE queries                             */
/*   sel   : (b, h_kv, k)     selected chunk indices                        */
/*   A     : (b, s, r)        low-rank left factor (shared by the KV heads) */
/*   Bf    : (b, h_kv, r, d)  low-rank right factor, per KV head            */
/*   v_host: (b, h_kv, s, d)  offloaded values                              */
/*   out   : (b, h_q, d)      softmax(q K^T / sqrt(d)) V, unrounded         */
/* ------------------------------------------------------------------------ */
int orc_attend(const orc_cfg *cfg, const double *q, const int32_t *sel,
               const double *A, const double *Bf, const double *v_host,
               const double *k_out, const double *v_out,
               const double *k_loc, const double *v_loc, double *out)
{
    int rc = check_cfg(cfg);
    if (rc) return rc;
    const int32_t Bn = cfg->b, H = cfg->h_kv, Hq = cfg->h_q, G = Hq / H, d = cfg->d;
    const int32_t s = cfg->s, c = cfg->c, r = cfg->r, o = cfg->o, k = cfg->k;
    const int32_t w = cfg->w + cfg->n_app;  /* local block: the window, then the appended tokens */
    const int32_t nk = o * c + k * c + w;
    const double scale = 1.0 / sqrt((double)d);
    int failed = 0;

#pragma omp parallel for schedule(dynamic) reduction(| : failed)
    for (int32_t bh = 0; bh < Bn * H; ++bh) {
        const int32_t b = bh / H;
        double *Ks = (double *)malloc(sizeof(double) * (size_t)nk * d);
        double *Vs = (double *)malloc(sizeof(double) * (size_t)nk * d);
        double *row = (double *)malloc(sizeof(double) * (size_t)d);
        double *logit = (double *)malloc(sizeof(double) * (size_t)nk);
        if (!Ks || !Vs || !row || !logit) { free(Ks); free(Vs); free(row); free(logit); failed = 1; continue; }

        /* [K_outlier; ...] */
        memcpy(Ks, k_out + (size_t)bh * o * c * d, sizeof(double) * (size_t)o * c * d);
        memcpy(Vs, v_out + (size_t)bh * o * c * d, sizeof(double) * (size_t)o * c * d);
        /* [...; RoPE(K_sparse); ...] with K_sparse = Gather(A, I) B */
        const double *Bh = Bf + (size_t)bh * r * d;
        for (int32_t a = 0; a < k; ++a) {
            int32_t chunk = sel[(size_t)bh * k + a];
            for (int32_t t = 0; t < c; ++t) {
                int64_t pos = (int64_t)chunk * c + t;
                const double *Ar = A + ((size_t)b * s + (size_t)pos) * r;
                for (int32_t i = 0; i < d; ++i) {
                    double acc = 0.0;
                    for (int32_t e = 0; e < r; ++e) acc += Ar[e] * Bh[(size_t)e * d + i];
                    row[i] = acc;
                }
                size_t dst = ((size_t)o * c + (size_t)a * c + t) * d;
                if (cfg->plant == ORC_PLANT_ZERO_REBUILT)
                    for (int32_t i = 0; i < d; ++i) row[i] = 0.0;
                if (cfg->plant == ORC_PLANT_NO_ROPE_REBUILT)
                    memcpy(Ks + dst, row, sizeof(double) * d);
                else
                    orc_rope_row(row, Ks + dst, d, (double)pos + (cfg->plant == ORC_PLANT_POS_PLUS_ONE),
                                 cfg->rope_base);
                if (cfg->plant == ORC_PLANT_BF16_REBUILT)
                    for (int32_t i = 0; i < d; ++i) Ks[dst + i] = orc_round_bf16(Ks[dst + i]);
                memcpy(Vs + dst, v_host + ((size_t)bh * s + (size_t)pos) * d, sizeof(double) * d);
            }
        }
        /* [...; K_local] */
        size_t base = ((size_t)o * c + (size_t)k * c) * d;
        memcpy(Ks + base, k_loc + (size_t)bh * w * d, sizeof(double) * (size_t)w * d);
        memcpy(Vs + base, v_loc + (size_t)bh * w * d, sizeof(double) * (size_t)w * d);

        /* softmax(q K^T / sqrt(d)) V for each query head of the group. */
        const int32_t j0 = cfg->plant == ORC_PLANT_NO_OUTLIERS ? o * c : 0;
        for (int32_t gi = 0; gi < G; ++gi) {
            int32_t g = (bh % H) * G + gi;
            const double *qg = q + ((size_t)b * Hq + g) * d;
            double mx = -INFINITY;
            for (int32_t j = 0; j < nk; ++j) {
                double acc = 0.0;
                for (int32_t i = 0; i < d; ++i) acc += qg[i] * Ks[(size_t)j * d + i];
                logit[j] = j < j0 ? -INFINITY : acc * scale;
                if (logit[j] > mx) mx = logit[j];
            }
            double z = 0.0;
            for (int32_t j = 0; j < nk; ++j) { logit[j] = exp(logit[j] - mx); z += logit[j]; }
            double *og = out + ((size_t)b * Hq + g) * d;
            for (int32_t i = 0; i < d; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < nk; ++j) acc += logit[j] * Vs[(size_t)j * d + i];
                og[i] = acc / z;
            }
        }
        free(Ks); free(Vs); free(row); free(logit);
    }
    return failed ? ORC_E_NOMEM : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Algorithm 2 (Decoding), one step for all sequences and heads.            */
/*   P   : (b, h_q, n)   chunk scores q.L^T / sqrt(d); -inf off-candidate   */
/*   S2  : (b, h_kv, n)  group score: per-head softmax over candidates,     */
/*                       averaged over the group; 0 off-candidate           */
/*   sel : (b, h_kv, k)  ArgTopK(S2, k), ascending                          */
/*   out : (b, h_q, d)   attention output (see orc_attend)                  */
/* ------------------------------------------------------------------------ */
int orc_decode(const orc_cfg *cfg, const double *q, const double *landmarks,
               const uint8_t *cand, const double *A, const double *Bf,
               const double *v_host, const double *k_out, const double *v_out,
               const double *k_loc, const double *v_loc,
               double *P, double *S2, int32_t *sel, double *out)
{
    int rc = check_cfg(cfg);
    if (rc) return rc;
    const int32_t Bn = cfg->b, H = cfg->h_kv, Hq = cfg->h_q, G = Hq / H, d = cfg->d;
    const int32_t n = cfg->s / cfg->c, k = cfg->k;
    const double scale = 1.0 / sqrt((double)d);
    int failed = 0;

#pragma omp parallel for schedule(dynamic) reduction(| : failed)
    for (int32_t bh = 0; bh < Bn * H; ++bh) {
        const int32_t b = bh / H, h = bh % H;
        const uint8_t *ch = cand + (size_t)bh * n;
        const double *Lh = landmarks + (size_t)bh * n * d;
        double *s2 = S2 + (size_t)bh * n;
        double *key = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!key) { failed = 1; continue; }
        for (int32_t j = 0; j < n; ++j) s2[j] = 0.0;

        for (int32_t gi = 0; gi < G; ++gi) {
            int32_t g = h * G + gi;
            const double *qg = q + ((size_t)b * Hq + g) * d;
            double *Pg = P + ((size_t)b * Hq + g) * n;
            /* Step 1: P = MatMul(Q, L^T), scaled as attention logits. */
            double mx = -INFINITY;
            for (int32_t j = 0; j < n; ++j) {
                if (!ch[j]) { Pg[j] = -INFINITY; continue; }
                double acc = 0.0;
                for (int32_t i = 0; i < d; ++i) acc += qg[i] * Lh[(size_t)j * d + i];
                Pg[j] = acc * scale;
                if (Pg[j] > mx) mx = Pg[j];
            }
            /* S2: this head's softmax over candidates, averaged over G heads. */
            double z = 0.0;
            for (int32_t j = 0; j < n; ++j) if (ch[j]) z += exp(Pg[j] - mx);
            for (int32_t j = 0; j < n; ++j) if (ch[j]) s2[j] += exp(Pg[j] - mx) / z / G;
        }
        /* Step 2: I = ArgTopK(S2, k), decided on binary32-rounded scores. */
        for (int32_t j = 0; j < n; ++j) key[j] = (double)(float)s2[j];
        if (orc_topk(key, ch, n, k, sel + (size_t)bh * k)) failed = 1;
        free(key);
    }
    if (failed) return ORC_E_NOMEM;
    /* Steps 3-4: gather V, rebuild and rotate K, attend. */
    return orc_attend(cfg, q, sel, A, Bf, v_host, k_out, v_out, k_loc, v_loc, out);
}

/* ------------------------------------------------------------------------ */
/* Equivalent bandwidth (section 三, 核心公式):                               */
/*   B~ = 2 S B_GPU / ( S/C + 2 (K + O) C + (1 - alpha) K C B_GPU / B_PCIe ) */
/* ------------------------------------------------------------------------ */
double orc_equiv_bandwidth(double S, double C, double K, double O, double alpha,
                           double b_gpu, double b_pcie)
{
    return 2.0 * S * b_gpu / (S / C + 2.0 * (K + O) * C + (1.0 - alpha) * K * C * b_gpu / b_pcie);
}
