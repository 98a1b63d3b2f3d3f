/*
 * Reference CPU implementation of the variable-length packed attention
 * forward, in double precision.  TEST INFRASTRUCTURE ONLY: the library under
 * test never links, loads or calls this file; only the test-suite, the smoke
 * check and the benchmark's CPU-baseline leg do.
 *
 * What it computes (the plain definition, no blocking, no online rescaling):
 * for sequence b, query row i, query head h
 *   kv head         c = h / (H / H_kv)                  (boostr varlen_attention.rs,
 *                                                        varlen_attention_fwd: GQA mapping)
 *   score           s_j = scale * <q_i, k_j>           (same function, dot product times scale;
 *                                                        SparseAttnSharedkv README, formula)
 *   allowed keys    A(i) = { j < Lk : causal -> j <= i+delta, window -> i+delta-wl <= j <= i+delta+wr }
 *                   with delta = Lk - Lq (queries aligned to the end of the keys)
 *   m = max over A(i) of s_j, and over the sink logit sigma_h when sinks are given
 *   Z = sum over A(i) of exp(s_j - m)  [+ exp(sigma_h - m)]
 *   O = sum over A(i) of exp(s_j - m) / Z * v_j,     LSE = m + ln Z
 * The three passes (max, sum of exponentials, normalised weights times V)
 * follow the order of the boostr CPU forward.  A row with no allowed key and
 * no sink gets O = 0, LSE = -inf.
 *
 * Readings taken where the pages are silent or disagree:
 *   - causal alignment is bottom-right (query i sits at key position
 *     i + Lk - Lq); it equals the boostr top-left mask whenever Lq == Lk;
 *   - window bounds are inclusive, -1 meaning unbounded on that side
 *     (SparseAttnSharedkv README, ori_win_left / ori_win_right rows);
 *   - a sink is one unscaled logit per query head that adds exp(sigma - m) to
 *     the denominator, has no value row, and is part of the returned LSE;
 *   - paged K/V row j of sequence b lives in block block_table[b][j / bs],
 *     slot j % bs, and the key length is seqused_k[b] (README, PageAttention
 *     constraints and seqused_kv row).
 *
 * Inputs are float32 or raw bfloat16 bit patterns, widened exactly on the fly.
 *
 * The backward (oracle_varlen_bwd, contiguous K/V) follows the steps of the
 * boostr CPU backward varlen_attention_bwd, given the forward's out and lse:
 * for sequence b, query row i, head h (kv head c):
 *   Dv   = sum_d dout[i,d] * out[i,d]
 *   for every allowed key j:  s = scale <q_i, k_j>,  p = exp(s - lse_i),
 *                             dp = <dout_i, v_j>,  ds = p (dp - Dv)
 *                             dq_i += scale ds k_j,  dk_j += scale ds q_i,  dv_j += p dout_i
 * dk and dv of kv head c sum over the H/H_kv query heads that share it.  The
 * allowed-key set is the forward's (bottom-right causal, inclusive window);
 * a sink only enters through lse (its own logit gets no gradient here).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t dtype;              /* 0: float32, 1: bfloat16 bits, 2: binary16 bits */
    int32_t B, H, Hkv, D;
    int32_t causal, wl, wr;     /* window: -1 = unbounded                  */
    double scale;
    const void *q, *k, *v;      /* q [T_q,H,D]; k,v [T_k,Hkv,D] or caches  */
    const int32_t *cu_q;        /* [B+1]                                   */
    const int32_t *cu_k;        /* [B+1], contiguous mode                  */
    const int32_t *seqused_k;   /* [B], paged mode                         */
    const int32_t *block_table; /* [B, bt_stride], NULL = contiguous mode  */
    int32_t bt_stride, block_size;
    const float *sinks;         /* [H] or NULL                             */
    const float *alibi;         /* [H] slopes or NULL: score of (i, j) gets
                                 * - slope_h * |i + Lk - Lq - j|         */
} oracle_args;

/* IEEE 754 binary16 -> double, exact: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 is subnormal (fraction * 2^-24), 31 is inf/NaN. */
double oracle_half_to_double(uint16_t h)
{
    const int e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m | 0x400), e - 25);
    return (h & 0x8000) ? -v : v;
}

static double widen(int dtype, const void *base, size_t idx)
{
    if (dtype == 0)
        return (double)((const float *)base)[idx];
    if (dtype == 2)
        return oracle_half_to_double(((const uint16_t *)base)[idx]);
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int key_len(const oracle_args *a, int b)
{
    return a->block_table ? a->seqused_k[b] : a->cu_k[b + 1] - a->cu_k[b];
}

/* element offset of K/V row j (logical position in sequence b), kv head c */
static size_t kv_offset(const oracle_args *a, int b, int j, int c)
{
    size_t row;
    if (a->block_table) {
        int32_t blk = a->block_table[(size_t)b * a->bt_stride + j / a->block_size];
        row = (size_t)blk * a->block_size + (size_t)(j % a->block_size);
    } else {
        row = (size_t)a->cu_k[b] + (size_t)j;
    }
    return (row * a->Hkv + c) * (size_t)a->D;
}

/* ALiBi term of query i, key j (0 without slopes) */
static double alibi_bias(const oracle_args *a, int h, long i, long j, long delta)
{
    if (!a->alibi) return 0.0;
    const long dist = i + delta - j;
    return -(double)a->alibi[h] * (double)(dist < 0 ? -dist : dist);
}

static int is_allowed(const oracle_args *a, long i, long j, long delta)
{
    long p = i + delta;
    if (a->causal && j > p) return 0;
    if (a->wl >= 0 && j < p - a->wl) return 0;
    if (a->wr >= 0 && j > p + a->wr) return 0;
    return 1;
}

/* one (sequence, query row, head): writes D outputs and one LSE */
static void one_row(const oracle_args *a, int b, int i, int h, double *scores,
                    double *o, double *lse_out)
{
    const int D = a->D;
    const int Lq = a->cu_q[b + 1] - a->cu_q[b];
    const int Lk = key_len(a, b);
    const long delta = (long)Lk - (long)Lq;
    const int c = h / (a->H / a->Hkv);
    const size_t qoff = (((size_t)a->cu_q[b] + i) * a->H + h) * (size_t)D;

    /* pass 1: allowed scores and their maximum (the sink takes part) */
    double m = -INFINITY;
    for (int j = 0; j < Lk; ++j) {
        if (!is_allowed(a, i, j, delta)) continue;
        size_t koff = kv_offset(a, b, j, c);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += widen(a->dtype, a->q, qoff + d) * widen(a->dtype, a->k, koff + d);
        scores[j] = dot * a->scale + alibi_bias(a, h, i, j, delta);
        if (scores[j] > m) m = scores[j];
    }
    if (a->sinks && (double)a->sinks[h] > m) m = (double)a->sinks[h];

    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (m == -INFINITY) { /* nothing to attend to: O = 0, LSE = -inf */
        *lse_out = -INFINITY;
        return;
    }

    /* pass 2: denominator */
    double Z = 0.0;
    for (int j = 0; j < Lk; ++j)
        if (is_allowed(a, i, j, delta)) Z += exp(scores[j] - m);
    if (a->sinks) Z += exp((double)a->sinks[h] - m);

    /* pass 3: normalised weights times value rows */
    for (int j = 0; j < Lk; ++j) {
        if (!is_allowed(a, i, j, delta)) continue;
        double w = exp(scores[j] - m) / Z;
        size_t voff = kv_offset(a, b, j, c);
        for (int d = 0; d < D; ++d) o[d] += w * widen(a->dtype, a->v, voff + d);
    }
    *lse_out = m + log(Z);
}

/* ---------------------------------------------------------------- threads */

typedef struct {
    const oracle_args *a;
    /* full mode */
    const int32_t *unit_b, *unit_i0;  /* (sequence, first row) per unit      */
    int64_t n_units;
    /* row-list mode */
    const int64_t *pairs;             /* token * H + head                    */
    int64_t n_pairs;
    double *out, *lse;
    int max_lk;
    int64_t next;                     /* shared work counter                 */
} pool_t;

enum { ROWS_PER_UNIT = 64 };

static int seq_of_token(const oracle_args *a, int64_t t)
{
    int lo = 0, hi = a->B - 1; /* last b with cu_q[b] <= t */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (a->cu_q[mid] <= t) lo = mid; else hi = mid - 1;
    }
    /* skip empty sequences that share the same start */
    while (lo + 1 <= a->B - 1 && a->cu_q[lo + 1] <= t) ++lo;
    return lo;
}

static void *worker(void *arg)
{
    pool_t *p = (pool_t *)arg;
    const oracle_args *a = p->a;
    double *scores = (double *)malloc(sizeof(double) * (size_t)(p->max_lk > 0 ? p->max_lk : 1));
    if (!scores) return NULL;
    for (;;) {
        int64_t u = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
        if (p->pairs) {
            if (u >= p->n_pairs) break;
            int64_t t = p->pairs[u] / a->H;
            int h = (int)(p->pairs[u] % a->H);
            int b = seq_of_token(a, t);
            one_row(a, b, (int)(t - a->cu_q[b]), h, scores,
                    p->out + (size_t)u * a->D, p->lse + u);
        } else {
            if (u >= p->n_units) break;
            int b = p->unit_b[u / a->H], i0 = p->unit_i0[u / a->H];
            int h = (int)(u % a->H);
            int Lq = a->cu_q[b + 1] - a->cu_q[b];
            int i1 = i0 + ROWS_PER_UNIT < Lq ? i0 + ROWS_PER_UNIT : Lq;
            for (int i = i0; i < i1; ++i) {
                size_t t = (size_t)a->cu_q[b] + i;
                one_row(a, b, i, h, scores, p->out + (t * a->H + h) * (size_t)a->D,
                        p->lse + t * a->H + h);
            }
        }
    }
    free(scores);
    return NULL;
}

static int check_args(const oracle_args *a)
{
    if (!a || a->B < 0 || a->H <= 0 || a->Hkv <= 0 || a->D <= 0) return -1;
    if (a->H % a->Hkv != 0) return -1;
    if (!a->q || !a->k || !a->v || !a->cu_q) return -1;
    if (a->block_table ? (!a->seqused_k || a->block_size <= 0) : !a->cu_k) return -1;
    if (a->dtype < 0 || a->dtype > 2) return -1;
    return 0;
}

static int run_pool(pool_t *p, int nthreads)
{
    const oracle_args *a = p->a;
    int max_lk = 0;
    for (int b = 0; b < a->B; ++b)
        if (key_len(a, b) > max_lk) max_lk = key_len(a, b);
    p->max_lk = max_lk;
    p->next = 0;
    if (nthreads < 1) nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int started = 0;
    for (int k = 0; k < nthreads; ++k)
        if (pthread_create(&th[k], NULL, worker, p) == 0) ++started;
    if (started == 0) worker(p);
    for (int k = 0; k < started; ++k) pthread_join(th[k], NULL);
    free(th);
    return 0;
}

/* All rows: out [T_q, H, D], lse [T_q, H] (float64, caller-allocated). */
int oracle_varlen_fwd(const oracle_args *a, double *out, double *lse, int nthreads)
{
    if (check_args(a) || !out || !lse) return -1;
    int64_t n = 0;
    for (int b = 0; b < a->B; ++b) {
        int Lq = a->cu_q[b + 1] - a->cu_q[b];
        n += (Lq + ROWS_PER_UNIT - 1) / ROWS_PER_UNIT;
    }
    int32_t *ub = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    int32_t *ui = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
    if (!ub || !ui) { free(ub); free(ui); return -2; }
    int64_t u = 0;
    for (int b = 0; b < a->B; ++b) {
        int Lq = a->cu_q[b + 1] - a->cu_q[b];
        for (int i0 = 0; i0 < Lq; i0 += ROWS_PER_UNIT) { ub[u] = b; ui[u] = i0; ++u; }
    }
    pool_t p;
    memset(&p, 0, sizeof p);
    p.a = a; p.unit_b = ub; p.unit_i0 = ui; p.n_units = n * a->H;
    p.out = out; p.lse = lse;
    int rc = run_pool(&p, nthreads);
    free(ub); free(ui);
    return rc;
}

/* Selected (token, head) pairs only: pairs[n] = token * H + head;
 * out [n, D], lse [n]. */
int oracle_varlen_fwd_rows(const oracle_args *a, const int64_t *pairs, int64_t n_pairs,
                           double *out, double *lse, int nthreads)
{
    if (check_args(a) || !pairs || !out || !lse || a->B < 1) return -1;
    int64_t T = a->cu_q[a->B];
    for (int64_t u = 0; u < n_pairs; ++u)
        if (pairs[u] < 0 || pairs[u] >= T * a->H) return -1;
    pool_t p;
    memset(&p, 0, sizeof p);
    p.a = a; p.pairs = pairs; p.n_pairs = n_pairs; p.out = out; p.lse = lse;
    return run_pool(&p, nthreads);
}

/* ---------------------------------------------------------------- backward */

typedef struct {
    const oracle_args *a;
    const double *dout, *out, *lse;
    double *dq, *dk, *dv;
    int64_t n_units;   /* B * Hkv: one (sequence, kv head) per unit */
    int64_t next;
} bwd_pool_t;

/* all query rows of sequence b and the query heads of kv head c */
static void bwd_unit(const bwd_pool_t *p, int b, int c)
{
    const oracle_args *a = p->a;
    const int D = a->D, g = a->H / a->Hkv;
    const int Lq = a->cu_q[b + 1] - a->cu_q[b];
    const int Lk = a->cu_k[b + 1] - a->cu_k[b];
    const long delta = (long)Lk - (long)Lq;
    for (int h = c * g; h < (c + 1) * g; ++h) {
        for (int i = 0; i < Lq; ++i) {
            const size_t t = (size_t)a->cu_q[b] + i;
            const size_t qoff = (t * a->H + h) * (size_t)D;
            const double l = p->lse[t * a->H + h];
            double dv_row = 0.0;
            for (int d = 0; d < D; ++d) dv_row += p->dout[qoff + d] * p->out[qoff + d];
            for (int j = 0; j < Lk; ++j) {
                if (!is_allowed(a, i, j, delta)) continue;
                const size_t koff = kv_offset(a, b, j, c);
                double s = 0.0, dp = 0.0;
                for (int d = 0; d < D; ++d) {
                    s += widen(a->dtype, a->q, qoff + d) * widen(a->dtype, a->k, koff + d);
                    dp += p->dout[qoff + d] * widen(a->dtype, a->v, koff + d);
                }
                s = s * a->scale + alibi_bias(a, h, i, j, delta);
                const double pr = exp(s - l);
                const double ds = pr * (dp - dv_row);
                for (int d = 0; d < D; ++d) {
                    p->dq[qoff + d] += a->scale * ds * widen(a->dtype, a->k, koff + d);
                    p->dk[koff + d] += a->scale * ds * widen(a->dtype, a->q, qoff + d);
                    p->dv[koff + d] += pr * p->dout[qoff + d];
                }
            }
        }
    }
}

static void *bwd_worker(void *arg)
{
    bwd_pool_t *p = (bwd_pool_t *)arg;
    for (;;) {
        int64_t u = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
        if (u >= p->n_units) break;
        bwd_unit(p, (int)(u / p->a->Hkv), (int)(u % p->a->Hkv));
    }
    return NULL;
}

/* Contiguous K/V only.  dout, out [T_q,H,D] and lse [T_q,H] in float64;
 * dq [T_q,H,D], dk, dv [T_k,Hkv,D] float64, caller-allocated (zeroed here). */
int oracle_varlen_bwd(const oracle_args *a, const double *dout, const double *out, const double *lse,
                      double *dq, double *dk, double *dv, int nthreads)
{
    if (check_args(a) || a->block_table || !dout || !out || !lse || !dq || !dk || !dv) return -1;
    const size_t Tq = a->B > 0 ? (size_t)a->cu_q[a->B] : 0, Tk = a->B > 0 ? (size_t)a->cu_k[a->B] : 0;
    memset(dq, 0, sizeof(double) * Tq * a->H * a->D);
    memset(dk, 0, sizeof(double) * Tk * a->Hkv * a->D);
    memset(dv, 0, sizeof(double) * Tk * a->Hkv * a->D);
    bwd_pool_t p;
    memset(&p, 0, sizeof p);
    p.a = a; p.dout = dout; p.out = out; p.lse = lse; p.dq = dq; p.dk = dk; p.dv = dv;
    p.n_units = (int64_t)a->B * a->Hkv;
    if (nthreads < 1) nthreads = 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -2;
    int started = 0;
    for (int k = 0; k < nthreads; ++k)
        if (pthread_create(&th[k], NULL, bwd_worker, &p) == 0) ++started;
    if (started == 0) bwd_worker(&p);
    for (int k = 0; k < started; ++k) pthread_join(th[k], NULL);
    free(th);
    return 0;
}
