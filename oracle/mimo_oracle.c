/*
 * mimo_oracle.c -- plain, slow, fp64 CPU oracle for the MiMo-V2.6-Flash attention layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file; only the
 * test-suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no code, header,
 * table or constant generator with the HIP library; it is written from the pages' description of the
 * layer, not from the GPU kernels.
 *
 * What it computes (all arithmetic in IEEE double; tensors are passed either as bf16 bit patterns or as
 * doubles, chosen by the f64 argument of each entry point, and decoded exactly):
 *
 *   Source pages (cited by title and section):
 *   [P1] "feat(models): add MiMo-V2.6-Flash-RL support" (miles pull request 3648), PR body and the commit
 *        messages in its conversation: per-layer KV heads (8 on sliding-window layers, 4 on global),
 *        192-dim Q/K with 128-dim V, learnable sink on the sliding-window layers only, V scaled by 0.707
 *        before attention; the SWA window covers the query plus sliding_window_size (128) previous keys.
 *   [P2] miles docs "MiMo-V2.6-Flash", section 1 "Model Introduction" (hybrid attention, RoPE bases 1e4 /
 *        1e7, partial RoPE on 64 of 192 dims, V scale 0.707), section 5.1 "Parallelism" (THD packing) and
 *        section 5.4 "Notable quirks" (129-key window, window_size = (128, 0)).
 *   [P5] Megatron-Bridge API docs "mimo_v2_flash_bridge", module summary: partial rotary on about a
 *        third of the head dims, separate RoPE bases for full and sliding-window layers.
 *
 *   Readings taken where the pages are silent (each is listed with its reason in the design notes):
 *   - softmax scale 1/sqrt(192) (the Q/K head width); the sink logit is not scaled;
 *   - sink: one fp32 logit per query head; it joins the softmax denominator only (a virtual key
 *     with a zero value); NULL or -inf means no sink;
 *   - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads) (contiguous groups);
 *   - RoPE: dims 0..63 rotated in rotate-half pairs (d, d+32), angle pos * base^(-d/32) for
 *     d = 0..31; dims 64..191 untouched; the position restarts at 0 at every cu_seqlens boundary;
 *   - window w >= 0: query at position p sees keys at positions max(0, p - w) .. p (w = 128 gives
 *     129 keys); w = -1: plain causal;
 *   - V scale is the literal 0.707; LSE is the natural log of the full denominator incl. the sink;
 *   - no dropout.
 *
 *   Forward, for a query row (token i, head h) of sequence b at position p:
 *     q' = RoPE(q[i,h], p),  k'_j = RoPE(k[j,kv], p_j)
 *     s_j = q'.k'_j / sqrt(192)  for j in W(i)
 *     Z = exp(sink_h) + sum_j exp(s_j)         (max-shifted in the code)
 *     LSE = ln Z,  O = sum_j exp(s_j - LSE) * (0.707 * v[j,kv])
 *   Backward (exact gradient of the forward above; D from a given O, or from the exact O):
 *     P_j = exp(s_j - LSE), D = dO.O, dP_j = 0.707 * dO.v_j, dS_j = P_j (dP_j - D)
 *     dq' += dS_j k'_j / sqrt(192);  dk'_j += dS_j q' / sqrt(192);  dv_j += 0.707 P_j dO
 *     dsink_h += -exp(sink_h - LSE) * D
 *     dq = RoPE^T(dq') = RoPE(dq', -p), dk likewise.
 *   Decode: the forward for one query at an explicit position against cache rows that already hold
 *   rotated K and unscaled V, plus the current token (rotated here).
 *   Cached prefill: the forward for a chunk of new tokens at explicit positions against cache rows (the
 *   keys just before the chunk, rotated K, unscaled V) plus the chunk's own keys, causally.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define DQK 192
#define DV 128
#define NROT 64
#define NHALF 32
#define VSCALE 0.707

static double bf(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element idx of a tensor that holds either bf16 bit patterns (f64 == 0) or doubles (f64 == 1). */
static double X(const void *p, size_t idx, int f64)
{
    return f64 ? ((const double *)p)[idx] : bf(((const uint16_t *)p)[idx]);
}

/* Rotate dims 0..63 of x (192 doubles) in place by angle sign * pos * base^(-d/32), pairs (d, d+32). */
static void rope(double *x, double pos, double base, double sign)
{
    for (int d = 0; d < NHALF; ++d) {
        double theta = sign * pos * pow(base, -(double)d / (double)NHALF);
        double c = cos(theta), s = sin(theta);
        double a = x[d], b = x[d + NHALF];
        x[d] = a * c - b * s;
        x[d + NHALF] = b * c + a * s;
    }
}

/* Index of the sequence that holds token t: the b with cu[b] <= t < cu[b+1]. */
static int seq_of(const int32_t *cu, int batch, int64_t t)
{
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

/* ---------------------------------------------------------------------------------------------
 * A prefill layer: pointers and sizes, plus the rotated K of every token (built once per call).
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    const void *q, *k, *v;       /* [T,hq,192], [T,hkv,192], [T,hkv,128] (bf16 bits or doubles) */
    const double *sink;          /* [hq] or NULL */
    const int32_t *cu;           /* [batch+1] */
    int batch, hq, hkv, window;
    int64_t T;
    double base;
    double *kr;                  /* rotated K, fp64 [T,hkv,192] */
    const void *out_given;       /* O [T,hq,128] used for D, or NULL for the exact O */
    const void *dout;            /* dO [T,hq,128] (backward only) */
    int f64;                     /* element type of q, k, v, out_given, dout: 0 bf16 bits, 1 double */
} layer_t;

static int layer_init(layer_t *L)
{
    L->kr = (double *)malloc(sizeof(double) * (size_t)(L->T > 0 ? L->T : 1) * L->hkv * DQK);
    if (!L->kr) return -1;
    for (int b = 0; b < L->batch; ++b)
        for (int64_t j = L->cu[b]; j < L->cu[b + 1]; ++j)
            for (int g = 0; g < L->hkv; ++g) {
                double *dst = L->kr + ((size_t)j * L->hkv + g) * DQK;
                size_t base = ((size_t)j * L->hkv + g) * DQK;
                for (int d = 0; d < DQK; ++d) dst[d] = X(L->k, base + d, L->f64);
                rope(dst, (double)(j - L->cu[b]), L->base, 1.0);
            }
    return 0;
}

/* One query row of the forward: fills qr (rotated q), the key range [j0, j1], the scores s[] (length
 * j1-j0+1), LSE and the exact O (128).  s must hold at least j1-j0+1 doubles. */
static void row_forward(const layer_t *L, int64_t i, int h, double *qr, int64_t *j0o, int64_t *j1o,
                        double *s, double *lse, double *o)
{
    int b = seq_of(L->cu, L->batch, i);
    int64_t start = L->cu[b];
    int64_t p = i - start;
    int kv = h / (L->hq / L->hkv);
    size_t qbase = ((size_t)i * L->hq + h) * DQK;
    for (int d = 0; d < DQK; ++d) qr[d] = X(L->q, qbase + d, L->f64);
    rope(qr, (double)p, L->base, 1.0);

    int64_t j0 = start, j1 = i;
    if (L->window >= 0 && i - L->window > j0) j0 = i - L->window;
    double scale = 1.0 / sqrt((double)DQK);
    double m = -INFINITY;
    for (int64_t j = j0; j <= j1; ++j) {
        const double *kj = L->kr + ((size_t)j * L->hkv + kv) * DQK;
        double acc = 0.0;
        for (int d = 0; d < DQK; ++d) acc += qr[d] * kj[d];
        s[j - j0] = acc * scale;
        if (s[j - j0] > m) m = s[j - j0];
    }
    double sk = L->sink ? L->sink[h] : -INFINITY;
    if (sk > m) m = sk;
    double z = (sk == -INFINITY) ? 0.0 : exp(sk - m);
    for (int64_t j = j0; j <= j1; ++j) z += exp(s[j - j0] - m);
    double l = m + log(z);
    for (int e = 0; e < DV; ++e) o[e] = 0.0;
    for (int64_t j = j0; j <= j1; ++j) {
        double pj = exp(s[j - j0] - l);
        size_t vbase = ((size_t)j * L->hkv + kv) * DV;
        for (int e = 0; e < DV; ++e) o[e] += pj * (VSCALE * X(L->v, vbase + e, L->f64));
    }
    *j0o = j0;
    *j1o = j1;
    *lse = l;
}

/* D for row (i,h): dO . O with O the given bf16 output or the exact one. */
static double row_D(const layer_t *L, int64_t i, int h, const double *o_exact)
{
    size_t base = ((size_t)i * L->hq + h) * DV;
    double D = 0.0;
    if (L->out_given) {
        for (int e = 0; e < DV; ++e) D += X(L->dout, base + e, L->f64) * X(L->out_given, base + e, L->f64);
    } else {
        for (int e = 0; e < DV; ++e) D += X(L->dout, base + e, L->f64) * o_exact[e];
    }
    return D;
}

/* ---------------------------------------------------------------------------------------------
 * A tiny thread pool: run fn(ctx, unit) for unit = 0..n-1 over nthreads threads.  The units are
 * independent outputs, so the split does not change any arithmetic.
 * ------------------------------------------------------------------------------------------- */
typedef void (*unit_fn)(void *ctx, int64_t unit, double *scratch);
typedef struct {
    unit_fn fn;
    void *ctx;
    int64_t n;
    int64_t next;
    pthread_mutex_t mu;
    size_t scratch_len;
    int failed;
} pool_t;

static void *pool_worker(void *arg)
{
    pool_t *P = (pool_t *)arg;
    double *scratch = (double *)malloc(sizeof(double) * P->scratch_len);
    if (!scratch) {
        pthread_mutex_lock(&P->mu);
        P->failed = 1;
        pthread_mutex_unlock(&P->mu);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&P->mu);
        int64_t u = P->next++;
        pthread_mutex_unlock(&P->mu);
        if (u >= P->n) break;
        P->fn(P->ctx, u, scratch);
    }
    free(scratch);
    return NULL;
}

static int run_pool(unit_fn fn, void *ctx, int64_t n, int nthreads, size_t scratch_len)
{
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < nthreads) nthreads = n > 0 ? (int)n : 1;
    pool_t P = {fn, ctx, n, 0, PTHREAD_MUTEX_INITIALIZER, scratch_len, 0};
    pthread_t th[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, pool_worker, &P) != 0) break;
        ++started;
    }
    if (started == 0) pool_worker(&P);
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
    return P.failed ? -1 : 0;
}

static size_t max_keys(const layer_t *L)
{
    int64_t m = 1;
    for (int b = 0; b < L->batch; ++b) {
        int64_t len = L->cu[b + 1] - L->cu[b];
        if (len > m) m = len;
    }
    if (L->window >= 0 && (int64_t)L->window + 1 < m) m = (int64_t)L->window + 1;
    return (size_t)m;
}

/* ---------------------------------------------------------------------------------------------
 * Forward over a list of (token, head) rows: row r = token * hq + head.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    const layer_t *L;
    const int64_t *rows;
    double *out, *lse;
} fwd_ctx;

static void fwd_unit(void *c, int64_t r, double *scratch)
{
    fwd_ctx *C = (fwd_ctx *)c;
    const layer_t *L = C->L;
    int64_t row = C->rows ? C->rows[r] : r;
    int64_t i = row / L->hq;
    int h = (int)(row % L->hq);
    double qr[DQK], o[DV], l;
    int64_t j0, j1;
    row_forward(L, i, h, qr, &j0, &j1, scratch, &l, o);
    memcpy(C->out + (size_t)r * DV, o, sizeof o);
    if (C->lse) C->lse[r] = l;
}

static int check_args(const int32_t *cu, int batch, int64_t T, int hq, int hkv, int window)
{
    if (batch < 0 || T < 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0 || window < -1) return -1;
    if (batch == 0) return T == 0 ? 0 : -1;
    if (cu[0] != 0 || cu[batch] != T) return -1;
    for (int b = 0; b < batch; ++b)
        if (cu[b + 1] < cu[b]) return -1;
    return 0;
}

/* rows == NULL means every row 0..T*hq-1 (out [T*hq,128], lse [T*hq] in row order). */
int oracle_prefill_rows(const void *q, const void *k, const void *v, const double *sink,
                        const int32_t *cu_seqlens, int batch, int64_t total_tokens, int window,
                        double rope_base, int n_q_heads, int n_kv_heads, const int64_t *rows,
                        int64_t n_rows, double *out, double *lse, int f64, int nthreads)
{
    if (check_args(cu_seqlens, batch, total_tokens, n_q_heads, n_kv_heads, window)) return -1;
    layer_t L = {q, k, v, sink, cu_seqlens, batch, n_q_heads, n_kv_heads, window, total_tokens,
                 rope_base, NULL, NULL, NULL, f64};
    if (rows == NULL) n_rows = total_tokens * n_q_heads;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total_tokens * n_q_heads) return -1;
    if (n_rows == 0) return 0;
    if (layer_init(&L)) return -2;
    fwd_ctx C = {&L, rows, out, lse};
    int rc = run_pool(fwd_unit, &C, n_rows, nthreads, max_keys(&L));
    free(L.kr);
    return rc;
}

/* ---------------------------------------------------------------------------------------------
 * Backward.
 * ------------------------------------------------------------------------------------------- */

/* Full backward: one unit per (sequence, KV head); every query row of that sequence for every Q head of
 * the group contributes to that unit's dk/dv, so units never write the same dk/dv element.  dq rows are
 * owned by exactly one unit too.  dsink contributions are kept per unit and summed afterwards in unit
 * order, so the result does not depend on the thread count. */
typedef struct {
    const layer_t *L;
    double *dq, *dk, *dv;        /* unrotated gradients are produced at the end */
    double *dsink_part;          /* [batch*hkv, hq] */
} bwd_ctx;

static void bwd_unit(void *c, int64_t unit, double *scratch)
{
    bwd_ctx *C = (bwd_ctx *)c;
    const layer_t *L = C->L;
    int b = (int)(unit / L->hkv), kv = (int)(unit % L->hkv);
    int G = L->hq / L->hkv;
    double scale = 1.0 / sqrt((double)DQK);
    for (int h = kv * G; h < (kv + 1) * G; ++h) {
        for (int64_t i = L->cu[b]; i < L->cu[b + 1]; ++i) {
            double qr[DQK], o[DV], l;
            int64_t j0, j1;
            row_forward(L, i, h, qr, &j0, &j1, scratch, &l, o);
            double D = row_D(L, i, h, o);
            double dOd[DV];
            for (int e = 0; e < DV; ++e) dOd[e] = X(L->dout, ((size_t)i * L->hq + h) * DV + e, L->f64);
            double *dqi = C->dq + ((size_t)i * L->hq + h) * DQK;
            for (int64_t j = j0; j <= j1; ++j) {
                double P = exp(scratch[j - j0] - l);
                size_t vbase = ((size_t)j * L->hkv + kv) * DV;
                double dP = 0.0;
                for (int e = 0; e < DV; ++e) dP += dOd[e] * X(L->v, vbase + e, L->f64);
                dP *= VSCALE;
                double dS = P * (dP - D);
                const double *kj = L->kr + ((size_t)j * L->hkv + kv) * DQK;
                double *dkj = C->dk + ((size_t)j * L->hkv + kv) * DQK;
                double *dvj = C->dv + ((size_t)j * L->hkv + kv) * DV;
                for (int d = 0; d < DQK; ++d) {
                    dqi[d] += dS * kj[d] * scale;
                    dkj[d] += dS * qr[d] * scale;
                }
                for (int e = 0; e < DV; ++e) dvj[e] += VSCALE * P * dOd[e];
            }
            if (L->sink && L->sink[h] != -INFINITY)
                C->dsink_part[(size_t)unit * L->hq + h] += -exp(L->sink[h] - l) * D;
        }
    }
    /* undo the rotation on this unit's rows: dq rows of the group's heads, dk rows of this KV head */
    for (int64_t i = L->cu[b]; i < L->cu[b + 1]; ++i) {
        double p = (double)(i - L->cu[b]);
        for (int h = kv * G; h < (kv + 1) * G; ++h)
            rope(C->dq + ((size_t)i * L->hq + h) * DQK, p, L->base, -1.0);
        rope(C->dk + ((size_t)i * L->hkv + kv) * DQK, p, L->base, -1.0);
    }
}

/* out_given: bf16 O used for D = dO.O (the backward's "given the forward outputs" contract), or NULL to
 * take D from the exact fp64 O.  dq/dk/dv are fully written (zero where nothing attends). dsink may be
 * NULL; it must be non-NULL only when sink is. */
int oracle_prefill_bwd(const void *q, const void *k, const void *v, const double *sink,
                       const void *out_given, const void *dout, const int32_t *cu_seqlens,
                       int batch, int64_t total_tokens, int window, double rope_base, int n_q_heads,
                       int n_kv_heads, double *dq, double *dk, double *dv, double *dsink, int f64, int nthreads)
{
    if (check_args(cu_seqlens, batch, total_tokens, n_q_heads, n_kv_heads, window)) return -1;
    layer_t L = {q, k, v, sink, cu_seqlens, batch, n_q_heads, n_kv_heads, window, total_tokens,
                 rope_base, NULL, out_given, dout, f64};
    memset(dq, 0, sizeof(double) * (size_t)total_tokens * n_q_heads * DQK);
    memset(dk, 0, sizeof(double) * (size_t)total_tokens * n_kv_heads * DQK);
    memset(dv, 0, sizeof(double) * (size_t)total_tokens * n_kv_heads * DV);
    if (dsink) memset(dsink, 0, sizeof(double) * n_q_heads);
    if (batch == 0) return 0;
    if (layer_init(&L)) return -2;
    int64_t units = (int64_t)batch * n_kv_heads;
    double *part = (double *)calloc((size_t)units * n_q_heads, sizeof(double));
    if (!part) { free(L.kr); return -2; }
    bwd_ctx C = {&L, dq, dk, dv, part};
    int rc = run_pool(bwd_unit, &C, units, nthreads, max_keys(&L));
    if (dsink)
        for (int64_t u = 0; u < units; ++u)
            for (int h = 0; h < n_q_heads; ++h) dsink[h] += part[(size_t)u * n_q_heads + h];
    free(part);
    free(L.kr);
    return rc;
}

/* dq for a list of rows (row = token*hq + head): out dq_rows [n_rows,192]. */
typedef struct {
    const layer_t *L;
    const int64_t *rows;
    double *dq;
} dq_ctx;

static void dq_unit(void *c, int64_t r, double *scratch)
{
    dq_ctx *C = (dq_ctx *)c;
    const layer_t *L = C->L;
    int64_t i = C->rows[r] / L->hq;
    int h = (int)(C->rows[r] % L->hq);
    int kv = h / (L->hq / L->hkv);
    double scale = 1.0 / sqrt((double)DQK);
    double qr[DQK], o[DV], l, dq[DQK] = {0};
    int64_t j0, j1;
    row_forward(L, i, h, qr, &j0, &j1, scratch, &l, o);
    double D = row_D(L, i, h, o);
    size_t obase = ((size_t)i * L->hq + h) * DV;
    for (int64_t j = j0; j <= j1; ++j) {
        double P = exp(scratch[j - j0] - l);
        size_t vbase = ((size_t)j * L->hkv + kv) * DV;
        double dP = 0.0;
        for (int e = 0; e < DV; ++e) dP += X(L->dout, obase + e, L->f64) * X(L->v, vbase + e, L->f64);
        double dS = P * (VSCALE * dP - D);
        const double *kj = L->kr + ((size_t)j * L->hkv + kv) * DQK;
        for (int d = 0; d < DQK; ++d) dq[d] += dS * kj[d] * scale;
    }
    int b = seq_of(L->cu, L->batch, i);
    rope(dq, (double)(i - L->cu[b]), L->base, -1.0);
    memcpy(C->dq + (size_t)r * DQK, dq, sizeof dq);
}

int oracle_bwd_dq_rows(const void *q, const void *k, const void *v, const double *sink,
                       const void *out_given, const void *dout, const int32_t *cu_seqlens,
                       int batch, int64_t total_tokens, int window, double rope_base, int n_q_heads,
                       int n_kv_heads, const int64_t *rows, int64_t n_rows, double *dq_rows,
                       int f64, int nthreads)
{
    if (check_args(cu_seqlens, batch, total_tokens, n_q_heads, n_kv_heads, window)) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total_tokens * n_q_heads) return -1;
    if (n_rows == 0) return 0;
    layer_t L = {q, k, v, sink, cu_seqlens, batch, n_q_heads, n_kv_heads, window, total_tokens,
                 rope_base, NULL, out_given, dout, f64};
    if (layer_init(&L)) return -2;
    dq_ctx C = {&L, rows, dq_rows};
    int rc = run_pool(dq_unit, &C, n_rows, nthreads, max_keys(&L));
    free(L.kr);
    return rc;
}

/* dk, dv for a list of key rows (keyrow = token*hkv + kv head): out dk_rows [n,192], dv_rows [n,128].
 * Every query row (i, h) with h in the KV head's group and the key inside W(i) contributes. */
typedef struct {
    const layer_t *L;
    const int64_t *rows;
    double *dk, *dv;
} dkv_ctx;

static void dkv_unit(void *c, int64_t r, double *scratch)
{
    dkv_ctx *C = (dkv_ctx *)c;
    const layer_t *L = C->L;
    int64_t j = C->rows[r] / L->hkv;
    int kv = (int)(C->rows[r] % L->hkv);
    int G = L->hq / L->hkv;
    int b = seq_of(L->cu, L->batch, j);
    double scale = 1.0 / sqrt((double)DQK);
    double dk[DQK] = {0}, dv[DV] = {0};
    size_t vbase = ((size_t)j * L->hkv + kv) * DV;
    for (int h = kv * G; h < (kv + 1) * G; ++h) {
        for (int64_t i = j; i < L->cu[b + 1]; ++i) {
            if (L->window >= 0 && i - j > L->window) break;
            double qr[DQK], o[DV], l;
            int64_t j0, j1;
            row_forward(L, i, h, qr, &j0, &j1, scratch, &l, o);
            double D = row_D(L, i, h, o);
            size_t obase = ((size_t)i * L->hq + h) * DV;
            double P = exp(scratch[j - j0] - l);
            double dP = 0.0;
            for (int e = 0; e < DV; ++e) dP += X(L->dout, obase + e, L->f64) * X(L->v, vbase + e, L->f64);
            double dS = P * (VSCALE * dP - D);
            for (int d = 0; d < DQK; ++d) dk[d] += dS * qr[d] * scale;
            for (int e = 0; e < DV; ++e) dv[e] += VSCALE * P * X(L->dout, obase + e, L->f64);
        }
    }
    rope(dk, (double)(j - L->cu[b]), L->base, -1.0);
    memcpy(C->dk + (size_t)r * DQK, dk, sizeof dk);
    memcpy(C->dv + (size_t)r * DV, dv, sizeof dv);
}

int oracle_bwd_dkv_rows(const void *q, const void *k, const void *v, const double *sink,
                        const void *out_given, const void *dout, const int32_t *cu_seqlens,
                        int batch, int64_t total_tokens, int window, double rope_base, int n_q_heads,
                        int n_kv_heads, const int64_t *key_rows, int64_t n_rows, double *dk_rows,
                        double *dv_rows, int f64, int nthreads)
{
    if (check_args(cu_seqlens, batch, total_tokens, n_q_heads, n_kv_heads, window)) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (key_rows[r] < 0 || key_rows[r] >= total_tokens * n_kv_heads) return -1;
    if (n_rows == 0) return 0;
    layer_t L = {q, k, v, sink, cu_seqlens, batch, n_q_heads, n_kv_heads, window, total_tokens,
                 rope_base, NULL, out_given, dout, f64};
    if (layer_init(&L)) return -2;
    dkv_ctx C = {&L, key_rows, dk_rows, dv_rows};
    int rc = run_pool(dkv_unit, &C, n_rows, nthreads, max_keys(&L));
    free(L.kr);
    return rc;
}

/* dsink for a list of heads: one unit per head, summing over every token in token order. */
typedef struct {
    const layer_t *L;
    const int32_t *heads;
    double *dsink;
} ds_ctx;

static void ds_unit(void *c, int64_t r, double *scratch)
{
    ds_ctx *C = (ds_ctx *)c;
    const layer_t *L = C->L;
    int h = C->heads[r];
    double acc = 0.0;
    if (L->sink && L->sink[h] != -INFINITY) {
        for (int64_t i = 0; i < L->T; ++i) {
            double qr[DQK], o[DV], l;
            int64_t j0, j1;
            row_forward(L, i, h, qr, &j0, &j1, scratch, &l, o);
            double D = row_D(L, i, h, o);
            acc += -exp(L->sink[h] - l) * D;
        }
    }
    C->dsink[r] = acc;
}

int oracle_bwd_dsink_heads(const void *q, const void *k, const void *v, const double *sink,
                           const void *out_given, const void *dout, const int32_t *cu_seqlens,
                           int batch, int64_t total_tokens, int window, double rope_base,
                           int n_q_heads, int n_kv_heads, const int32_t *heads, int n_heads,
                           double *dsink_out, int f64, int nthreads)
{
    if (check_args(cu_seqlens, batch, total_tokens, n_q_heads, n_kv_heads, window)) return -1;
    for (int r = 0; r < n_heads; ++r)
        if (heads[r] < 0 || heads[r] >= n_q_heads) return -1;
    if (n_heads == 0) return 0;
    layer_t L = {q, k, v, sink, cu_seqlens, batch, n_q_heads, n_kv_heads, window, total_tokens,
                 rope_base, NULL, out_given, dout, f64};
    if (layer_init(&L)) return -2;
    ds_ctx C = {&L, heads, dsink_out};
    int rc = run_pool(ds_unit, &C, n_heads, nthreads, max_keys(&L));
    free(L.kr);
    return rc;
}

/* ---------------------------------------------------------------------------------------------
 * Decode: one new token per sequence against a KV cache.
 *   q [batch,hq,192] and k_new [batch,hkv,192] are unrotated and sit at positions[b];
 *   v_new [batch,hkv,128]; the cache rows cu_cache[b] .. cu_cache[b+1]-1 hold rotated K [.,hkv,192]
 *   and unscaled V [.,hkv,128], oldest first.  With window w >= 0 the query sees the last min(n_b, w)
 *   cache rows plus itself; with w = -1 every cache row plus itself.
 *   rows: list of b*hq + h (NULL = all), out [n_rows,128].
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    const void *q, *kn, *vn, *kc, *vc;
    const int32_t *cuc, *pos;
    const double *sink;
    int batch, hq, hkv, window;
    double base;
    const int64_t *rows;
    double *out, *lse;
    int f64;
} dec_ctx;

static void dec_unit(void *c, int64_t r, double *s)
{
    dec_ctx *C = (dec_ctx *)c;
    int64_t row = C->rows ? C->rows[r] : r;
    int b = (int)(row / C->hq), h = (int)(row % C->hq);
    int kv = h / (C->hq / C->hkv);
    double scale = 1.0 / sqrt((double)DQK);
    double qr[DQK], kn[DQK];
    for (int d = 0; d < DQK; ++d) qr[d] = X(C->q, ((size_t)b * C->hq + h) * DQK + d, C->f64);
    for (int d = 0; d < DQK; ++d) kn[d] = X(C->kn, ((size_t)b * C->hkv + kv) * DQK + d, C->f64);
    rope(qr, (double)C->pos[b], C->base, 1.0);
    rope(kn, (double)C->pos[b], C->base, 1.0);
    int64_t c0 = C->cuc[b], c1 = C->cuc[b + 1];
    if (C->window >= 0 && c1 - c0 > C->window) c0 = c1 - C->window;
    int64_t n = c1 - c0;   /* cache keys, then the current token as key n */
    double m = -INFINITY;
    for (int64_t j = 0; j <= n; ++j) {
        double acc = 0.0;
        if (j < n) {
            size_t kbase = ((size_t)(c0 + j) * C->hkv + kv) * DQK;
            for (int d = 0; d < DQK; ++d) acc += qr[d] * X(C->kc, kbase + d, C->f64);
        } else {
            for (int d = 0; d < DQK; ++d) acc += qr[d] * kn[d];
        }
        s[j] = acc * scale;
        if (s[j] > m) m = s[j];
    }
    double sk = C->sink ? C->sink[h] : -INFINITY;
    if (sk > m) m = sk;
    double z = (sk == -INFINITY) ? 0.0 : exp(sk - m);
    for (int64_t j = 0; j <= n; ++j) z += exp(s[j] - m);
    double l = m + log(z);
    double o[DV] = {0};
    for (int64_t j = 0; j <= n; ++j) {
        double p = exp(s[j] - l);
        const void *vt = (j < n) ? C->vc : C->vn;
        size_t vbase = (j < n) ? ((size_t)(c0 + j) * C->hkv + kv) * DV : ((size_t)b * C->hkv + kv) * DV;
        for (int e = 0; e < DV; ++e) o[e] += p * (VSCALE * X(vt, vbase + e, C->f64));
    }
    memcpy(C->out + (size_t)r * DV, o, sizeof o);
    if (C->lse) C->lse[r] = l;
}

int oracle_decode_rows(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                       const void *v_cache, const int32_t *cu_cache, const int32_t *positions,
                       const double *sink, int batch, int window, double rope_base, int n_q_heads,
                       int n_kv_heads, const int64_t *rows, int64_t n_rows, double *out, double *lse,
                       int f64, int nthreads)
{
    if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || window < -1)
        return -1;
    if (batch == 0) return 0;
    int64_t maxn = 1;
    for (int b = 0; b < batch; ++b) {
        if (cu_cache[b + 1] < cu_cache[b] || positions[b] < 0) return -1;
        int64_t n = cu_cache[b + 1] - cu_cache[b];
        if (n + 1 > maxn) maxn = n + 1;
    }
    if (rows == NULL) n_rows = (int64_t)batch * n_q_heads;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= (int64_t)batch * n_q_heads) return -1;
    if (n_rows == 0) return 0;
    dec_ctx C = {q, k_new, v_new, k_cache, v_cache, cu_cache, positions, sink, batch, n_q_heads,
                 n_kv_heads, window, rope_base, rows, out, lse, f64};
    return run_pool(dec_unit, &C, n_rows, nthreads, (size_t)maxn);
}

/* ---------------------------------------------------------------------------------------------
 * Prefill of a chunk of new tokens over a cached prefix (the serving engine prefills long prompts in
 * chunks of up to 49152 tokens against its KV cache: SGLang cookbook page "MiMo-V2.6", section 2
 * "Configuration tips", "Context length and memory"; the cache holds rotated K and unscaled V as in
 * decode).  Sequence b has n_b cache rows cu_cache[b] ..
 * cu_cache[b+1]-1, the keys at positions positions[b]-n_b .. positions[b]-1 in that order, and new tokens
 * cu_q[b] .. cu_q[b+1]-1 at positions positions[b], positions[b]+1, ...  New token i attends the cache
 * rows and the new tokens 0..i, limited to key positions >= its own position - window when window >= 0,
 * with the sink in the denominator.  With no cache rows and positions 0 this is the plain prefill; a
 * chunk of one token is decode.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
    const void *q, *k, *v, *kc, *vc;
    const int32_t *cuq, *cuc, *pos;
    const double *sink;
    int batch, hq, hkv, window;
    double base;
    const int64_t *rows;
    double *out, *lse;
    int f64;
} pc_ctx;

static void pc_unit(void *c, int64_t r, double *s)
{
    pc_ctx *C = (pc_ctx *)c;
    int64_t row = C->rows ? C->rows[r] : r;
    int64_t t = row / C->hq;
    int h = (int)(row % C->hq);
    int kv = h / (C->hq / C->hkv);
    int b = seq_of(C->cuq, C->batch, t);
    int64_t i = t - C->cuq[b];                       /* index of the token inside its chunk */
    int64_t n = C->cuc[b + 1] - C->cuc[b];           /* cache rows of the sequence */
    double p = (double)C->pos[b] + (double)i;        /* position of this query */
    double scale = 1.0 / sqrt((double)DQK);
    double qr[DQK], kr[DQK];
    for (int d = 0; d < DQK; ++d) qr[d] = X(C->q, ((size_t)t * C->hq + h) * DQK + d, C->f64);
    rope(qr, p, C->base, 1.0);
    /* keys in position order: cache rows j = 0 .. n-1, then new tokens j = n .. n+i; key j sits at
     * position pos[b] - n + j, and the window keeps positions >= p - window */
    int64_t nk = n + i + 1;
    int64_t j0 = 0;
    if (C->window >= 0 && nk - 1 - C->window > 0) j0 = nk - 1 - C->window;
    double m = -INFINITY;
    for (int64_t j = j0; j < nk; ++j) {
        double acc = 0.0;
        if (j < n) {
            size_t kb = ((size_t)(C->cuc[b] + j) * C->hkv + kv) * DQK;
            for (int d = 0; d < DQK; ++d) acc += qr[d] * X(C->kc, kb + d, C->f64);
        } else {
            size_t kb = ((size_t)(C->cuq[b] + j - n) * C->hkv + kv) * DQK;
            for (int d = 0; d < DQK; ++d) kr[d] = X(C->k, kb + d, C->f64);
            rope(kr, (double)C->pos[b] + (double)(j - n), C->base, 1.0);
            for (int d = 0; d < DQK; ++d) acc += qr[d] * kr[d];
        }
        s[j - j0] = acc * scale;
        if (s[j - j0] > m) m = s[j - j0];
    }
    double sk = C->sink ? C->sink[h] : -INFINITY;
    if (sk > m) m = sk;
    double z = (sk == -INFINITY) ? 0.0 : exp(sk - m);
    for (int64_t j = j0; j < nk; ++j) z += exp(s[j - j0] - m);
    double l = m + log(z);
    double o[DV] = {0};
    for (int64_t j = j0; j < nk; ++j) {
        double pj = exp(s[j - j0] - l);
        const void *vt = (j < n) ? C->vc : C->v;
        size_t vb = (j < n) ? ((size_t)(C->cuc[b] + j) * C->hkv + kv) * DV
                            : ((size_t)(C->cuq[b] + j - n) * C->hkv + kv) * DV;
        for (int e = 0; e < DV; ++e) o[e] += pj * (VSCALE * X(vt, vb + e, C->f64));
    }
    memcpy(C->out + (size_t)r * DV, o, sizeof o);
    if (C->lse) C->lse[r] = l;
}

int oracle_prefill_cached_rows(const void *q, const void *k, const void *v, const void *k_cache,
                               const void *v_cache, const int32_t *cu_q, const int32_t *cu_cache,
                               const int32_t *positions, const double *sink, int batch, int window,
                               double rope_base, int n_q_heads, int n_kv_heads, const int64_t *rows,
                               int64_t n_rows, double *out, double *lse, int f64, int nthreads)
{
    if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || window < -1)
        return -1;
    if (batch == 0) return 0;
    if (cu_q[0] != 0 || cu_cache[0] != 0) return -1;
    int64_t maxk = 1;
    for (int b = 0; b < batch; ++b) {
        if (cu_q[b + 1] < cu_q[b] || cu_cache[b + 1] < cu_cache[b]) return -1;
        int64_t n = cu_cache[b + 1] - cu_cache[b];
        if (positions[b] < n) return -1;             /* the cache rows precede the chunk */
        int64_t nk = n + (cu_q[b + 1] - cu_q[b]);
        if (nk > maxk) maxk = nk;
    }
    int64_t all = (int64_t)cu_q[batch] * n_q_heads;
    if (rows == NULL) n_rows = all;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= all) return -1;
    if (n_rows == 0) return 0;
    pc_ctx C = {q, k, v, k_cache, v_cache, cu_q, cu_cache, positions, sink, batch, n_q_heads, n_kv_heads,
                window, rope_base, rows, out, lse, f64};
    return run_pool(pc_unit, &C, n_rows, nthreads, (size_t)maxk);
}

/* The rotation alone, for tests: rows of 192 bf16 values at the given positions -> rotated fp64. */
int oracle_rope(const void *x, const int32_t *positions, int64_t n_rows, double rope_base, int f64,
                double *out)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int d = 0; d < DQK; ++d) out[r * DQK + d] = X(x, (size_t)r * DQK + d, f64);
        rope(out + r * DQK, (double)positions[r], rope_base, 1.0);
    }
    return 0;
}
