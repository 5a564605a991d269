/*
 * Attention oracle: a plain, slow, obviously correct CPU definition of the
 * graph protocol's `attention` op, in f64.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg call this code. It shares nothing with the
 * HIP library (no headers, helpers or tables) and the library never calls it.
 *
 * What it computes (graph protocol op catalogue, op `attention`: its summary,
 * inputs, and the params heads, headDim, kvHeads, vHeadDim, causal,
 * posOffset, scale, softcap, window and the alibi family; features
 * `attention.softcap` and `attention.bias`):
 *
 *   for every query head h and query row t, with pos = posOffset + t and
 *   g = floor(h * G / H) the key/value head h reads:
 *     visible(s)  causal:      pos - window < s <= pos   (window 0: s <= pos)
 *                 non-causal:  |pos - s| <= window        (window 0: every s)
 *                 with a window and sinks > 0, the keys s < sinks are also
 *                 visible (causal rows still need s <= pos): the attention
 *                 sinks the IR schema pairs with `window` (op_attention and
 *                 slot_kv, property `sinks`), read as StreamingLLM's kept
 *                 initial tokens
 *     x_s = scale * sum_d q[t, h*D + d] * k[s, g*D + d]
 *     x_s = softcap * tanh(x_s / softcap)         if softcap > 0
 *     x_s = x_s - slope[h] * |pos - s|            if ALiBi slopes are given
 *     x_s = x_s + pb_weight[b(pos, s), h]         with a bucketed position bias
 *     x_s = x_s + bias[(h,) t, s]                 if a bias is given
 *     out[t, h*Dv + e] = sum_s exp(x_s - M) v[s, g*Dv + e] / sum_s exp(x_s - M)
 *       over the visible s, with M the largest visible x_s (the catalogue's
 *       max-subtracted softmax); a row with no visible key is 0.
 *
 * Two further score terms the IR schema lists on its attention op, with no
 * rule on the pages (the readings are the published methods they are named
 * after):
 *   position_bias {weight, buckets}: T5's bucketed relative position bias.
 *     buckets holds ascending distance thresholds starting at 0; the bucket
 *     of a key is the last threshold <= |pos - s|, plus pb_n for a key after
 *     the query when the table is bidirectional (T5's encoder layout); the
 *     term is pb_weight[bucket, h], added where ALiBi is.
 *   relative_kv {key, value, max_distance}: Shaw et al.'s relative position
 *     representations. With r = clip(s - pos, -max, max) + max, the key
 *     embedding rel_k[r] is added to k before the product with q (so it is
 *     scaled with it) and rel_v[r] to v in the weighted sum.
 *
 * Parity unpinned (a reading, not a fact the pages fix, so nothing outside
 * this definition can confirm it): the zero output of a row with no visible
 * key. The ALiBi term -slope * |pos - s| is, on non-causal rows, MPT's
 * bidirectional bias (its "full" form: minus the absolute key - query
 * distance), and on causal rows it differs from BLOOM's slope * s and MPT's
 * slope * (s - (S - 1)) only by a per-row constant, which the softmax
 * removes; the tests pin both against those models' own constructions.
 *
 * The resolution of absent parameters (defaults, slope tables) happens in the
 * Python wrapper beside this file; this core takes resolved numbers.
 * Every input is an f32 array and is widened to f64 (exact); all arithmetic
 * is f64 in the order written above, with no blocking or reordering.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t T, S, H, G, D, Dv;
    int32_t causal;
    int64_t pos_offset;
    double scale;
    double softcap;        /* 0: off */
    int64_t window;        /* 0: off */
    const double* slopes;  /* NULL: no ALiBi; else H entries */
    int32_t bias_kind;     /* 0 none, 1 [T,S], 2 [H,T,S] */
    int64_t sinks;         /* 0: none; with a window, keys s < sinks stay visible */
    const float* pb_weight;      /* NULL: no position bias; else [pb_n or 2 pb_n, H] */
    const int64_t* pb_bounds;    /* pb_n ascending distance thresholds, the first 0 */
    int64_t pb_n;
    int32_t pb_bidirectional;    /* keys after the query use the second pb_n rows */
    const float* rel_k;          /* NULL: no relative keys; else [2 rel_max + 1, D] */
    const float* rel_v;          /* NULL: no relative values; else [2 rel_max + 1, Dv] */
    int64_t rel_max;
} oracle_attention_args;

typedef struct {
    const oracle_attention_args* a;
    const float *q, *k, *v, *bias;
    const int64_t* rows;
    int64_t nrows;
    double* out;
    int64_t first, step;   /* this worker's share of the (row, head) items */
} worker_job;

static int key_visible(const oracle_attention_args* a, int64_t pos, int64_t s)
{
    /* an attention sink: one of the first `sinks` keys, kept in view beside the window */
    const int sink = a->window > 0 && s < a->sinks;
    if (a->causal) {
        if (s > pos) return 0;
        if (sink) return 1;
        if (a->window > 0 && !(pos - a->window < s)) return 0;
        return 1;
    }
    if (a->window > 0 && !sink) {
        int64_t dist = pos > s ? pos - s : s - pos;
        if (dist > a->window) return 0;
    }
    return 1;
}

/* The position-bias row of key s for a query at pos: the last threshold not
 * above the distance, in the second half for later keys when bidirectional. */
static int64_t pb_row(const oracle_attention_args* a, int64_t pos, int64_t s)
{
    const int64_t dist = pos > s ? pos - s : s - pos;
    int64_t b = 0;
    for (int64_t i = 0; i < a->pb_n; ++i)
        if (a->pb_bounds[i] <= dist) b = i;
    if (a->pb_bidirectional && s > pos) b += a->pb_n;
    return b;
}

/* The relative-embedding row of key s for a query at pos. */
static int64_t rel_row(const oracle_attention_args* a, int64_t pos, int64_t s)
{
    int64_t r = s - pos;
    if (r < -a->rel_max) r = -a->rel_max;
    if (r > a->rel_max) r = a->rel_max;
    return r + a->rel_max;
}

/* One (query row, head): the definition above, written out. */
static void attend_row(const worker_job* j, int64_t ri, int64_t h, double* x, unsigned char* vis)
{
    const oracle_attention_args* a = j->a;
    const int64_t t = j->rows ? j->rows[ri] : ri;
    const int64_t pos = a->pos_offset + t;
    const int64_t g = (h * a->G) / a->H;
    const int64_t D = a->D, Dv = a->Dv;
    const float* qrow = j->q + t * (a->H * D) + h * D;
    double* orow = j->out + ri * (a->H * Dv) + h * Dv;

    int any = 0;
    double M = -INFINITY;
    for (int64_t s = 0; s < a->S; ++s) {
        vis[s] = (unsigned char)key_visible(a, pos, s);
        if (!vis[s]) continue;
        const float* krow = j->k + s * (a->G * D) + g * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (double)krow[d];
        if (a->rel_k) {
            const float* rk = a->rel_k + rel_row(a, pos, s) * D;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (double)rk[d];
        }
        double xs = a->scale * dot;
        if (a->softcap > 0.0) xs = a->softcap * tanh(xs / a->softcap);
        if (a->slopes) {
            double dist = (double)(pos > s ? pos - s : s - pos);
            xs -= a->slopes[h] * dist;
        }
        if (a->pb_weight) xs += (double)a->pb_weight[pb_row(a, pos, s) * a->H + h];
        if (a->bias_kind == 1) xs += (double)j->bias[t * a->S + s];
        if (a->bias_kind == 2) xs += (double)j->bias[(h * a->T + t) * a->S + s];
        x[s] = xs;
        if (!any || xs > M) M = xs;
        any = 1;
    }
    for (int64_t e = 0; e < Dv; ++e) orow[e] = 0.0;
    if (!any) return;

    double L = 0.0;
    for (int64_t s = 0; s < a->S; ++s) {
        if (!vis[s]) continue;
        double p = exp(x[s] - M);
        L += p;
        const float* vrow = j->v + s * (a->G * Dv) + g * Dv;
        for (int64_t e = 0; e < Dv; ++e) orow[e] += p * (double)vrow[e];
        if (a->rel_v) {
            const float* rv = a->rel_v + rel_row(a, pos, s) * Dv;
            for (int64_t e = 0; e < Dv; ++e) orow[e] += p * (double)rv[e];
        }
    }
    for (int64_t e = 0; e < Dv; ++e) orow[e] /= L;
}

static void* worker(void* arg)
{
    worker_job* j = (worker_job*)arg;
    const int64_t S = j->a->S > 0 ? j->a->S : 1;
    double* x = (double*)malloc(sizeof(double) * (size_t)S);
    unsigned char* vis = (unsigned char*)malloc((size_t)S);
    if (!x || !vis) {
        free(x);
        free(vis);
        return (void*)1;
    }
    const int64_t items = j->nrows * j->a->H;
    for (int64_t it = j->first; it < items; it += j->step)
        attend_row(j, it / j->a->H, it % j->a->H, x, vis);
    free(x);
    free(vis);
    return NULL;
}

/*
 * out: f64 [nrows, H*Dv], row i holding query row rows[i] (or row i when rows
 * is NULL, in which case nrows must be T). Returns 0 on success, -1 on bad
 * arguments, -2 when memory or threads run out.
 */
int oracle_attention(const oracle_attention_args* a, const float* q, const float* k,
                     const float* v, const float* bias, const int64_t* rows, int64_t nrows,
                     double* out, int nthreads)
{
    if (!a || !q || !out || a->H <= 0 || a->G <= 0 || a->H % a->G || a->D <= 0 || a->Dv <= 0)
        return -1;
    if (a->S > 0 && (!k || !v)) return -1;
    if (a->bias_kind && !bias) return -1;
    if (!rows && nrows != a->T) return -1;
    if (nthreads < 1) nthreads = 1;
    const int64_t items = nrows * a->H;
    if (nthreads > items) nthreads = (int)(items > 0 ? items : 1);

    worker_job* jobs = (worker_job*)calloc((size_t)nthreads, sizeof(worker_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(jobs);
        free(tids);
        return -2;
    }
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        worker_job w = {a, q, k, v, bias, rows, nrows, out, i, nthreads};
        jobs[i] = w;
        if (pthread_create(&tids[i], NULL, worker, &jobs[i]) != 0) {
            rc = -2;
            break;
        }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        void* res = NULL;
        pthread_join(tids[i], &res);
        if (res) rc = -2;
    }
    free(jobs);
    free(tids);
    return rc;
}
