/*
 * Plain CPU oracle of the FreeSolo-Linear (FS-L) attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code with the HIP library.
 *
 * Everything here is deliberately slow and literal: one head at a time, one
 * query at a time, floating point in fp64. Inputs arrive as float32 arrays
 * whose values are exact copies of the fp32 or bf16 tensors the GPU reads, so
 * the upcast to double is exact.
 *
 * Sources (the pages this follows):
 *  [D]  "FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
 *       Extrapolation" digest (paper.rainbus.top), sections "前置知识"
 *       (RoPE, NoPE), "核心方法" (core method), "方法步骤详情" (six steps),
 *       "局限与改进" (erf bound g_h >= erf(2)).
 *  [S]  ai.info summary of the same paper, "Methodology in Plain English" and
 *       "Why This Matters" (pool of P+W cells updated every B tokens, bounded
 *       state O(((P+W)s + w + B + s)d)).
 *
 * Readings taken where the pages leave a step open (each repeated at its
 * function): the long branch may use the cells that lie wholly before the
 * window of the block's first query; the window holds w keys including the
 * query itself; RoPE is the rotate-half pairing with base 10000 at absolute
 * positions; the erf bias is lambda_h * a_c * erf(sigma_h (i - c s) / (2 s));
 * the pool is the W most recent eligible cells plus the P best older ones under
 * (a desc, index asc); top-K under (score desc, index asc); the mix is
 * out = o_win + gamma_h * o_long / sqrt(mean(o_long^2) + eps).
 *
 * Cell statistics are stored as float32 (the rounding of the fp64 value), and
 * every selection decision is taken in fp64 from those stored values.
 *
 * Parity pins: every function below is pinned by a CPU test against closed
 * forms, library routines or brute force (the test module that exercises the
 * oracle lists which pin covers which function).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t N;       /* tokens */
    int32_t d;       /* head dim (even) */
    int32_t w;       /* window width, keys [i-w+1, i] */
    int32_t s;       /* cell size */
    int32_t P;       /* kept high-norm cells; -1 = no pruning (FS) */
    int32_t W;       /* kept recent cells */
    int32_t K;       /* cells read per query */
    int32_t B;       /* query block */
    int32_t pad_;
    double scale;    /* softmax scale of both branches */
    double rho;      /* weight of the content term in the cell score */
    double rope_base;
    double rms_eps;
    double sigma;    /* per-head erf width */
    double lambda;   /* per-head weight of the norm-weighted bias */
    double gamma;    /* per-head mixing coefficient */
} orc_head;

/* ------------------------------------------------------------------------ */
/* Cells and blocks ([D] core method: cells of s tokens, blocks of B queries) */

int64_t orc_num_cells(const orc_head *p) { return p->N / p->s; }

int64_t orc_num_blocks(const orc_head *p) { return (p->N + p->B - 1) / p->B; }

/* Cells eligible for query block b: those wholly before the window of the
 * block's first query t0 = b*B, i.e. floor((t0 - w + 1) / s), at least 0.
 * ([D] core method: a block shares one available set; reading of where the
 * long branch's cells end relative to the window.) */
int64_t orc_eligible(int64_t b, const orc_head *p)
{
    int64_t x = b * (int64_t)p->B - (int64_t)p->w + 1;
    if (x <= 0) return 0;
    int64_t nb = x / p->s;
    int64_t C = orc_num_cells(p);
    return nb < C ? nb : C;
}

/* Mean key and max key norm of every complete cell ([D] core method and step
 * 3; [S] methodology: mean key for routing, largest token-key norm as a
 * query-independent priority). Sums run in fp64 in token order (mean) and in
 * coordinate order with fused multiply-add (squared norm); the results are
 * rounded once to float32. */
void orc_cell_stats(const float *k, const orc_head *p, float *kbar, float *amax)
{
    const int64_t C = orc_num_cells(p);
    const int d = p->d, s = p->s;
    for (int64_t c = 0; c < C; ++c) {
        const float *cell = k + c * s * (int64_t)d;
        for (int x = 0; x < d; ++x) {
            double acc = 0.0;
            for (int j = 0; j < s; ++j) acc += (double)cell[(int64_t)j * d + x];
            kbar[c * d + x] = (float)(acc / (double)s);
        }
        double best = 0.0;
        for (int j = 0; j < s; ++j) {
            double ss = 0.0;
            for (int x = 0; x < d; ++x) {
                double e = (double)cell[(int64_t)j * d + x];
                ss = fma(e, e, ss);
            }
            if (ss > best) best = ss;
        }
        amax[c] = (float)sqrt(best);
    }
}

/* ------------------------------------------------------------------------ */
/* Norm prune ([D] step 4 and core method; [S] methodology: the W most recent
 * cells plus the P cells of highest max key norm, at most P+W, updated only at
 * block boundaries). Reading: the P best are taken among the eligible cells
 * that are not recent, ties by lower index. With P = -1 (FS) every eligible
 * cell is kept. Returns the pool size; pool[] is ascending. */

typedef struct { float a; int32_t idx; } orc_akey;

static int cmp_akey(const void *pa, const void *pb)
{
    const orc_akey *a = (const orc_akey *)pa, *b = (const orc_akey *)pb;
    if (a->a > b->a) return -1;
    if (a->a < b->a) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

static int cmp_i32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

int32_t orc_pool(const float *amax, int64_t b, const orc_head *p, int32_t *pool)
{
    const int64_t nb = orc_eligible(b, p);
    if (p->P < 0) {
        for (int64_t c = 0; c < nb; ++c) pool[c] = (int32_t)c;
        return (int32_t)nb;
    }
    const int64_t m = nb > p->W ? nb - p->W : 0; /* older cells: [0, m) */
    int32_t n = 0;
    if (m > 0 && p->P > 0) {
        orc_akey *keys = (orc_akey *)malloc(sizeof(orc_akey) * (size_t)m);
        for (int64_t c = 0; c < m; ++c) { keys[c].a = amax[c]; keys[c].idx = (int32_t)c; }
        qsort(keys, (size_t)m, sizeof(orc_akey), cmp_akey);
        int64_t take = m < p->P ? m : p->P;
        for (int64_t t = 0; t < take; ++t) pool[n++] = keys[t].idx;
        free(keys);
        qsort(pool, (size_t)n, sizeof(int32_t), cmp_i32);
    }
    for (int64_t c = m; c < nb; ++c) pool[n++] = (int32_t)c;
    return n;
}

/* ------------------------------------------------------------------------ */
/* Cell score and top-K ([D] core method and step 5: content match plus a
 * norm-weighted erf relative-position bias, top K cells; [D] limits section:
 * for available cells the erf factor is at least erf(2); [S] methodology: the
 * bias grows with distance and is scaled by the cell norm).
 * Reading: score = fma(rho, q.kbar_c, (lambda * a_c) * erf(sigma (i - c s) / (2 s))),
 * the dot product a left-to-right fused multiply-add chain in fp64. The K best
 * under (score desc, index asc) are kept (all of them if the pool is no larger
 * than K) and reported ascending, padded with -1. *margin receives the gap
 * between the K-th and (K+1)-th best score (+inf if no (K+1)-th). */

double orc_cell_score(const float *q_i, int64_t i, const float *kbar_c, float a_c,
                      int64_t c, const orc_head *p)
{
    double content = 0.0;
    for (int x = 0; x < p->d; ++x) content = fma((double)q_i[x], (double)kbar_c[x], content);
    double arg = (p->sigma * (double)(i - c * (int64_t)p->s)) / (2.0 * (double)p->s);
    double bias = (p->lambda * (double)a_c) * erf(arg);
    return fma(p->rho, content, bias);
}

typedef struct { double sc; int32_t idx; } orc_skey;

static int cmp_skey(const void *pa, const void *pb)
{
    const orc_skey *a = (const orc_skey *)pa, *b = (const orc_skey *)pb;
    if (a->sc > b->sc) return -1;
    if (a->sc < b->sc) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

int32_t orc_select(const float *q_i, int64_t i, const float *kbar, const float *amax,
                   const int32_t *pool, int32_t npool, const orc_head *p,
                   int32_t *sel, double *margin)
{
    const int d = p->d;
    int32_t nsel = 0;
    double gap = INFINITY;
    if (npool > 0) {
        orc_skey *sk = (orc_skey *)malloc(sizeof(orc_skey) * (size_t)npool);
        for (int32_t t = 0; t < npool; ++t) {
            int64_t c = pool[t];
            sk[t].sc = orc_cell_score(q_i, i, kbar + c * d, amax[c], c, p);
            sk[t].idx = (int32_t)c;
        }
        qsort(sk, (size_t)npool, sizeof(orc_skey), cmp_skey);
        nsel = npool < p->K ? npool : p->K;
        for (int32_t t = 0; t < nsel; ++t) sel[t] = sk[t].idx;
        if (npool > p->K) gap = sk[p->K - 1].sc - sk[p->K].sc;
        free(sk);
        qsort(sel, (size_t)nsel, sizeof(int32_t), cmp_i32);
    }
    for (int32_t t = nsel; t < p->K; ++t) sel[t] = -1;
    if (margin) *margin = gap;
    return nsel;
}

/* ------------------------------------------------------------------------ */
/* RoPE ([D] prerequisites: rotate q_i and k_j by R(i), R(j) so that their dot
 * product depends only on the offset; used only inside the local window).
 * Reading: rotate-half pairing (x[m], x[m + d/2]), angle t * base^(-2m/d). */
void orc_rope(const float *x, int64_t t, const orc_head *p, double *out)
{
    const int half = p->d / 2;
    for (int m = 0; m < half; ++m) {
        double theta = pow(p->rope_base, -2.0 * (double)m / (double)p->d);
        double ang = (double)t * theta;
        double cs = cos(ang), sn = sin(ang);
        double a = (double)x[m], b = (double)x[m + half];
        out[m] = a * cs - b * sn;
        out[m + half] = b * cs + a * sn;
    }
}

/* Local branch ([D] core method and step 2: standard RoPE attention in a
 * window of width w). Reading: keys j in [max(0, i-w+1), i]. qrot is R(i)q_i;
 * krot holds R(j)k_j for every j of the window (rows of a [N][d] array). */
void orc_window(const double *qrot, const double *krot, const float *v, int64_t i,
                const orc_head *p, double *o)
{
    const int d = p->d;
    int64_t j0 = i - p->w + 1;
    if (j0 < 0) j0 = 0;
    const int64_t n = i - j0 + 1;
    double *l = (double *)malloc(sizeof(double) * (size_t)n);
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        const double *kr = krot + (j0 + t) * d;
        double dot = 0.0;
        for (int x = 0; x < d; ++x) dot += qrot[x] * kr[x];
        l[t] = p->scale * dot;
        if (l[t] > mx) mx = l[t];
    }
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) { l[t] = exp(l[t] - mx); sum += l[t]; }
    for (int x = 0; x < d; ++x) o[x] = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        const float *vr = v + (j0 + t) * d;
        for (int x = 0; x < d; ++x) o[x] += l[t] * (double)vr[x];
    }
    for (int x = 0; x < d; ++x) o[x] /= sum;
    free(l);
}

/* Long branch readout ([D] core method and step 6; NoPE prerequisite: softmax
 * attention over the raw, unrotated tokens of the selected cells, at most K*s
 * tokens; the position bias takes no part in it). An empty selection gives 0. */
void orc_readout(const float *q_i, const float *k, const float *v, const int32_t *sel,
                 int32_t nsel, const orc_head *p, double *o)
{
    const int d = p->d, s = p->s;
    for (int x = 0; x < d; ++x) o[x] = 0.0;
    if (nsel <= 0) return;
    const int64_t n = (int64_t)nsel * s;
    double *l = (double *)malloc(sizeof(double) * (size_t)n);
    double mx = -INFINITY;
    for (int32_t u = 0; u < nsel; ++u)
        for (int j = 0; j < s; ++j) {
            const float *kr = k + ((int64_t)sel[u] * s + j) * d;
            double dot = 0.0;
            for (int x = 0; x < d; ++x) dot += (double)q_i[x] * (double)kr[x];
            double val = p->scale * dot;
            l[(int64_t)u * s + j] = val;
            if (val > mx) mx = val;
        }
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) { l[t] = exp(l[t] - mx); sum += l[t]; }
    for (int32_t u = 0; u < nsel; ++u)
        for (int j = 0; j < s; ++j) {
            const float *vr = v + ((int64_t)sel[u] * s + j) * d;
            double pw = l[(int64_t)u * s + j];
            for (int x = 0; x < d; ++x) o[x] += pw * (double)vr[x];
        }
    for (int x = 0; x < d; ++x) o[x] /= sum;
    free(l);
}

/* Branch mix ([D] core method and step 6: the long output goes through
 * RMSNorm and is added to the local branch with a per-head learned weight).
 * Reading: RMSNorm over d without a gain vector, eps added to the mean square. */
void orc_mix(const double *o_win, const double *o_long, const orc_head *p, double *out)
{
    const int d = p->d;
    double ms = 0.0;
    for (int x = 0; x < d; ++x) ms += o_long[x] * o_long[x];
    ms /= (double)d;
    double den = sqrt(ms + p->rms_eps);
    for (int x = 0; x < d; ++x) out[x] = o_win[x] + p->gamma * (o_long[x] / den);
}

/* ------------------------------------------------------------------------ */
/* Whole forward for one head at a list of query rows. q, k, v are [N][d].
 * Outputs per row r: out/o_win/o_long [nrows][d], sel [nrows][K], margin
 * [nrows]; pool_out (nullable) receives the pool of every block as
 * [nblk][pool_cap] padded with -1; kbar_out [C][d] and amax_out [C]
 * (nullable) receive the cell statistics. Because the method is causal, the
 * output at row i equals the output at the last row of the sequence cut
 * after token i, which is also the definition of a decode step. */
int orc_forward_head(const float *q, const float *k, const float *v, const orc_head *p,
                     const int64_t *rows, int64_t nrows, double *out, double *o_win,
                     double *o_long, int32_t *sel, double *margin, int32_t *pool_out,
                     int32_t pool_cap, float *kbar_out, float *amax_out, int nthreads)
{
    const int d = p->d;
    const int64_t N = p->N, C = orc_num_cells(p), nblk = orc_num_blocks(p);
    if (d <= 0 || (d & 1) || p->s <= 0 || p->B <= 0 || p->w <= 0 || p->K <= 0 || N <= 0)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    float *kbar = (float *)malloc(sizeof(float) * (size_t)(C > 0 ? C : 1) * d);
    float *amax = (float *)malloc(sizeof(float) * (size_t)(C > 0 ? C : 1));
    orc_cell_stats(k, p, kbar, amax);
    if (kbar_out) memcpy(kbar_out, kbar, sizeof(float) * (size_t)C * d);
    if (amax_out) memcpy(amax_out, amax, sizeof(float) * (size_t)C);

    const int64_t cap = p->P < 0 ? (C > 0 ? C : 1) : (int64_t)p->P + p->W;
    /* pools of the blocks the rows fall in */
    char *need_blk = (char *)calloc((size_t)nblk, 1);
    char *need_tok = (char *)calloc((size_t)N, 1);
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows[r];
        if (i < 0 || i >= N) { free(kbar); free(amax); free(need_blk); free(need_tok); return -2; }
        need_blk[i / p->B] = 1;
        int64_t j0 = i - p->w + 1;
        if (j0 < 0) j0 = 0;
        for (int64_t j = j0; j <= i; ++j) need_tok[j] = 1;
    }
    if (pool_out) for (int64_t b = 0; b < nblk; ++b) need_blk[b] = 1;
    int32_t *pools = (int32_t *)malloc(sizeof(int32_t) * (size_t)nblk * (size_t)(cap > 0 ? cap : 1));
    int32_t *npools = (int32_t *)calloc((size_t)nblk, sizeof(int32_t));
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nblk; ++b)
        if (need_blk[b]) npools[b] = orc_pool(amax, b, p, pools + b * cap);
    if (pool_out) {
        for (int64_t b = 0; b < nblk; ++b)
            for (int64_t t = 0; t < pool_cap; ++t)
                pool_out[b * pool_cap + t] = (t < npools[b] && t < cap) ? pools[b * cap + t] : -1;
    }
    /* rotated keys of every position some window needs */
    double *krot = (double *)malloc(sizeof(double) * (size_t)N * d);
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        if (need_tok[j]) orc_rope(k + j * d, j, p, krot + j * d);

    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        const int64_t b = i / p->B;
        double *qrot = (double *)malloc(sizeof(double) * d);
        double *ow = (double *)malloc(sizeof(double) * d);
        double *ol = (double *)malloc(sizeof(double) * d);
        int32_t *sl = (int32_t *)malloc(sizeof(int32_t) * (size_t)p->K);
        double mg;
        orc_rope(q + i * d, i, p, qrot);
        orc_window(qrot, krot, v, i, p, ow);
        int32_t nsel = orc_select(q + i * d, i, kbar, amax, pools + b * cap, npools[b], p, sl, &mg);
        orc_readout(q + i * d, k, v, sl, nsel, p, ol);
        orc_mix(ow, ol, p, out + r * d);
        if (o_win) memcpy(o_win + r * d, ow, sizeof(double) * d);
        if (o_long) memcpy(o_long + r * d, ol, sizeof(double) * d);
        if (sel) memcpy(sel + r * p->K, sl, sizeof(int32_t) * (size_t)p->K);
        if (margin) margin[r] = mg;
        free(qrot); free(ow); free(ol); free(sl);
    }
    free(krot); free(pools); free(npools); free(need_blk); free(need_tok);
    free(kbar); free(amax);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of one head, for training ([D] method steps, training paragraph:
 * the hard top-P / top-K indices receive no gradient; [S] "Methodology in
 * Plain English", training paragraph: the routing scalars sigma_h, lambda_h
 * stay fixed while the per-head mixing weight is learned).
 *
 * With the forward's selection sel [N][K] (ascending, -1 padded) held fixed,
 * out is a differentiable function of q, k, v and gamma. Given
 * dout = dL/dout [N][d] this accumulates dq, dk, dv [N][d] (zeroed here) and
 * returns dgamma in *dgamma. Per query i, for each branch with output o and
 * upstream gradient dO, and D = dO . o:
 *   P_j = softmax_j(l_j), dS_j = P_j (dO . v_j - D), dv_j += P_j dO,
 *   and the gradient of l_j = scale a . b_j goes to a (scale dS_j b_j) and to
 *   b_j (scale dS_j a).
 * Window: a = R(i) q_i, b_j = R(j) k_j, dO = dout_i; the rotated gradients are
 * turned back with R(t)^T = R(-t). Long branch: a = q_i, b_j = k_j over the
 * tokens of the selected cells; with r = sqrt(mean(o^2) + eps) and y = o / r,
 * dgamma += dout_i . y, dy = gamma dout_i and dO = (dy - y (dy . y) / d) / r
 * (RMSNorm's backward). An empty selection contributes nothing. fp64
 * throughout, queries in order. Returns 0, or -1 for bad parameters. */

/* R(t)^T x = R(-t) x for the rotate-half pairing, angle t * base^(-2m/d) */
static void orc_rope_back(const double *x, int64_t t, const orc_head *p, double *out)
{
    const int half = p->d / 2;
    for (int m = 0; m < half; ++m) {
        double theta = pow(p->rope_base, -2.0 * (double)m / (double)p->d);
        double ang = (double)t * theta;
        double cs = cos(ang), sn = sin(ang);
        double a = x[m], b = x[m + half];
        out[m] = a * cs + b * sn;
        out[m + half] = b * cs - a * sn;
    }
}

/* softmax backward over n keys for one query: a [d] the query-side operand,
 * brow(t) / vrow(t) the key-side operand and value of key t; accumulates
 * da [d], db_t and dv_t (through the callbacks' destinations) */
typedef struct {
    const double *b;  /* key-side operands, rows of d (or NULL: use bf) */
    const float *bf;
    const float *v;
    const int64_t *idx; /* key t -> row index */
    double *db;        /* gradient rows of the key-side operand */
    double *dv;        /* gradient rows of v */
} orc_keys;

static void orc_softmax_back(const double *a, const orc_keys *K, int64_t n, const double *dO,
                             const orc_head *p, double *da, double *o_out)
{
    const int d = p->d;
    double *l = (double *)malloc(sizeof(double) * (size_t)n);
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        const int64_t j = K->idx[t];
        double dot = 0.0;
        for (int x = 0; x < d; ++x) dot += a[x] * (K->b ? K->b[j * d + x] : (double)K->bf[j * d + x]);
        l[t] = p->scale * dot;
        if (l[t] > mx) mx = l[t];
    }
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) { l[t] = exp(l[t] - mx); sum += l[t]; }
    for (int64_t t = 0; t < n; ++t) l[t] /= sum; /* P_t */
    double *o = (double *)calloc((size_t)d, sizeof(double));
    for (int64_t t = 0; t < n; ++t) {
        const float *vr = K->v + K->idx[t] * d;
        for (int x = 0; x < d; ++x) o[x] += l[t] * (double)vr[x];
    }
    if (o_out) memcpy(o_out, o, sizeof(double) * d);
    double D = 0.0;
    for (int x = 0; x < d; ++x) D += dO[x] * o[x];
    for (int64_t t = 0; t < n; ++t) {
        const int64_t j = K->idx[t];
        const float *vr = K->v + j * d;
        double dP = 0.0;
        for (int x = 0; x < d; ++x) dP += dO[x] * (double)vr[x];
        const double dS = l[t] * (dP - D);
        for (int x = 0; x < d; ++x) {
            const double bx = K->b ? K->b[j * d + x] : (double)K->bf[j * d + x];
            da[x] += p->scale * dS * bx;
            K->db[j * d + x] += p->scale * dS * a[x];
            K->dv[j * d + x] += l[t] * dO[x];
        }
    }
    free(o);
    free(l);
}

int orc_backward_head(const float *q, const float *k, const float *v, const float *dout,
                      const int32_t *sel, const orc_head *p, double *dq, double *dk,
                      double *dv, double *dgamma)
{
    const int d = p->d, s = p->s;
    const int64_t N = p->N;
    if (d <= 0 || (d & 1) || s <= 0 || p->w <= 0 || p->K <= 0 || N <= 0) return -1;
    memset(dq, 0, sizeof(double) * (size_t)N * d);
    memset(dk, 0, sizeof(double) * (size_t)N * d);
    memset(dv, 0, sizeof(double) * (size_t)N * d);
    double *krot = (double *)malloc(sizeof(double) * (size_t)N * d);
    double *dkrot = (double *)calloc((size_t)N * d, sizeof(double));
    for (int64_t j = 0; j < N; ++j) orc_rope(k + j * d, j, p, krot + j * d);
    double *qrot = (double *)malloc(sizeof(double) * d);
    double *dqrot = (double *)malloc(sizeof(double) * d);
    double *back = (double *)malloc(sizeof(double) * d);
    double *dO = (double *)malloc(sizeof(double) * d);
    double *o = (double *)malloc(sizeof(double) * d);
    double *qd = (double *)malloc(sizeof(double) * d);
    int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)(p->w > (int64_t)p->K * s ? p->w : (int64_t)p->K * s));
    double dg = 0.0;
    for (int64_t i = 0; i < N; ++i) {
        /* local branch */
        int64_t j0 = i - p->w + 1;
        if (j0 < 0) j0 = 0;
        const int64_t nw = i - j0 + 1;
        for (int64_t t = 0; t < nw; ++t) idx[t] = j0 + t;
        orc_rope(q + i * d, i, p, qrot);
        for (int x = 0; x < d; ++x) { dqrot[x] = 0.0; dO[x] = (double)dout[i * d + x]; }
        orc_keys kw = {krot, NULL, v, idx, dkrot, dv};
        orc_softmax_back(qrot, &kw, nw, dO, p, dqrot, NULL);
        orc_rope_back(dqrot, i, p, back);
        for (int x = 0; x < d; ++x) dq[i * d + x] += back[x];
        /* long branch over the selected cells' tokens */
        int64_t nl = 0;
        for (int u = 0; u < p->K; ++u) {
            const int32_t c = sel[i * p->K + u];
            if (c < 0) continue;
            for (int j = 0; j < s; ++j) idx[nl++] = (int64_t)c * s + j;
        }
        if (nl == 0) continue;
        /* forward of the branch for y, then RMSNorm's backward for dO */
        {
            double *l = (double *)malloc(sizeof(double) * (size_t)nl);
            double mx = -INFINITY, sum = 0.0;
            for (int64_t t = 0; t < nl; ++t) {
                double dot = 0.0;
                for (int x = 0; x < d; ++x) dot += (double)q[i * d + x] * (double)k[idx[t] * d + x];
                l[t] = p->scale * dot;
                if (l[t] > mx) mx = l[t];
            }
            for (int64_t t = 0; t < nl; ++t) { l[t] = exp(l[t] - mx); sum += l[t]; }
            for (int x = 0; x < d; ++x) o[x] = 0.0;
            for (int64_t t = 0; t < nl; ++t)
                for (int x = 0; x < d; ++x) o[x] += (l[t] / sum) * (double)v[idx[t] * d + x];
            free(l);
        }
        double ms = 0.0;
        for (int x = 0; x < d; ++x) ms += o[x] * o[x];
        const double r = sqrt(ms / (double)d + p->rms_eps);
        double dyy = 0.0;
        for (int x = 0; x < d; ++x) {
            const double y = o[x] / r;
            dg += (double)dout[i * d + x] * y;
            dyy += p->gamma * (double)dout[i * d + x] * y;
        }
        for (int x = 0; x < d; ++x) {
            const double y = o[x] / r;
            dO[x] = (p->gamma * (double)dout[i * d + x] - y * dyy / (double)d) / r;
        }
        for (int x = 0; x < d; ++x) { qd[x] = (double)q[i * d + x]; dqrot[x] = 0.0; }
        orc_keys kl = {NULL, k, v, idx, dk, dv};
        orc_softmax_back(qd, &kl, nl, dO, p, dqrot, NULL);
        for (int x = 0; x < d; ++x) dq[i * d + x] += dqrot[x];
    }
    for (int64_t j = 0; j < N; ++j) {
        orc_rope_back(dkrot + j * d, j, p, back);
        for (int x = 0; x < d; ++x) dk[j * d + x] += back[x];
    }
    *dgamma = dg;
    free(krot); free(dkrot); free(qrot); free(dqrot); free(back); free(dO); free(o); free(qd); free(idx);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* FS-B: beam search over two causal forests of balanced trees ([S]
 * "Methodology in Plain English", FS-B paragraph: one tree over the full
 * prefix and one over cells whose norm exceeds a threshold; each node keeps a
 * mean key, a radius bounding its children, the largest cell norm and the
 * earliest position; a beam of 16 nodes per level descends each tree under a
 * provable upper bound of the cell score beneath a node; the union of both
 * beams is reranked with token-level log-sum-exp scores and the top 4 cells
 * are read. [D] method step 5 and novelty: two balanced forests, log depth,
 * O(N log^2 N) including radix-sort construction; [S] key contributions 3:
 * "causal forests").
 *
 * Readings where the pages leave the structure open:
 *  - Lists: list 0 holds every complete cell, list 1 the cells with a_c > tau
 *    (tau a per-head input; the pages set it once per checkpoint from data),
 *    both in position order.
 *  - Causal forest: every aligned segment [a 2^k, (a+1) 2^k) of a list holds a
 *    perfect binary tree whose leaves are the segment's cells ordered by
 *    (code asc, list index asc), code a 32-bit sign hash of kbar_c over 32
 *    given projection rows (bit 31-b set iff proj_b . kbar_c > 0). A block whose
 *    prefix holds m entries of a list searches the segments of m's binary
 *    decomposition (largest first): O(log N) trees of depth O(log N).
 *  - Node: mean key mu = float(sum of its leaves' kbar / count) (fp64 sum in
 *    leaf order); radius r = max over children of |mu_child - mu| + r_child
 *    (leaves 0), scaled by (1 + 2^-40) against rounding; amax and pmin the
 *    largest a_c and smallest c s beneath.
 *  - Bound (for rho, lambda, sigma >= 0): ub = fma(rho, fma(|q|, r, q . mu),
 *    (lambda amax) erf(sigma (i - pmin) / (2 s))); at a leaf it is the cell score.
 *  - Beam, per forest: start from the decomposition's roots; while the beam
 *    holds an internal node, replace every internal node by its two children
 *    and keep the `beam` best candidates under (ub desc, node key asc), the key
 *    ordering forest, level, segment and heap index.
 *  - Rerank: every distinct cell of the two final beams by
 *    lse_c = log sum_j exp(scale q . k_j) over its s raw tokens (fp64); the K best
 *    under (lse desc, cell asc), reported ascending and padded with -1.
 */

typedef struct {
    const float *proj;  /* [32][d] projection rows of the code */
    double tau;         /* list 1 holds the cells with a_c > tau */
    int32_t beam;       /* nodes kept per level */
    int32_t pad_;
} orc_fsb;

uint32_t orc_fsb_code(const float *x, const float *proj, int d)
{
    uint32_t code = 0;
    for (int b = 0; b < 32; ++b) {
        double dot = 0.0;
        for (int t = 0; t < d; ++t) dot = fma((double)proj[b * d + t], (double)x[t], dot);
        if (dot > 0.0) code |= 1u << (31 - b);
    }
    return code;
}

typedef struct {          /* one perfect tree: heap order, nodes 1 .. 2L-1, leaves L .. 2L-1 */
    int64_t L;
    int32_t *cell;        /* [L] leaf cells in leaf order */
    float *mu;            /* [2L][d] */
    double *rad;          /* [2L] */
    float *amax;          /* [2L] */
    int64_t *pmin;        /* [2L] */
} orc_fsb_tree;

typedef struct { uint32_t code; int64_t idx; int32_t cell; } orc_leafkey;

static int cmp_leafkey(const void *pa, const void *pb)
{
    const orc_leafkey *a = (const orc_leafkey *)pa, *b = (const orc_leafkey *)pb;
    if (a->code != b->code) return a->code < b->code ? -1 : 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

static double orc_dist(const float *a, const float *b, int d)
{
    double acc = 0.0;
    for (int x = 0; x < d; ++x) {
        double e = (double)a[x] - (double)b[x];
        acc = fma(e, e, acc);
    }
    return sqrt(acc);
}

/* the tree of segment [a 2^k, (a+1) 2^k) of a list (list[] of cells, codes[] per cell) */
void orc_fsb_build_tree(const int32_t *list, int64_t a, int k, const uint32_t *codes, const float *kbar,
                        const float *amax, const orc_head *p, orc_fsb_tree *t)
{
    const int d = p->d;
    const int64_t L = (int64_t)1 << k, base = a * L;
    orc_leafkey *lk = (orc_leafkey *)malloc(sizeof(orc_leafkey) * (size_t)L);
    for (int64_t u = 0; u < L; ++u) {
        lk[u].idx = base + u;
        lk[u].cell = list[base + u];
        lk[u].code = codes[lk[u].cell];
    }
    qsort(lk, (size_t)L, sizeof(orc_leafkey), cmp_leafkey);
    t->L = L;
    t->cell = (int32_t *)malloc(sizeof(int32_t) * (size_t)L);
    t->mu = (float *)malloc(sizeof(float) * (size_t)(2 * L) * d);
    t->rad = (double *)calloc((size_t)(2 * L), sizeof(double));
    t->amax = (float *)malloc(sizeof(float) * (size_t)(2 * L));
    t->pmin = (int64_t *)malloc(sizeof(int64_t) * (size_t)(2 * L));
    for (int64_t u = 0; u < L; ++u) t->cell[u] = lk[u].cell;
    free(lk);
    for (int64_t j = 1; j < 2 * L; ++j) {
        int depth = 0;
        while (((int64_t)1 << (depth + 1)) <= j) ++depth;
        const int64_t n = L >> depth, first = (j - ((int64_t)1 << depth)) * n;
        float am = -INFINITY;
        int64_t pm = INT64_MAX;
        for (int x = 0; x < d; ++x) {
            double sum = 0.0;
            for (int64_t u = first; u < first + n; ++u) sum = sum + (double)kbar[(int64_t)t->cell[u] * d + x];
            t->mu[j * d + x] = (float)(sum / (double)n);
        }
        for (int64_t u = first; u < first + n; ++u) {
            const int32_t c = t->cell[u];
            if (amax[c] > am) am = amax[c];
            if ((int64_t)c * p->s < pm) pm = (int64_t)c * p->s;
        }
        t->amax[j] = am;
        t->pmin[j] = pm;
    }
    for (int64_t j = L - 1; j >= 1; --j) {
        const double r0 = orc_dist(t->mu + 2 * j * d, t->mu + j * d, d) + t->rad[2 * j];
        const double r1 = orc_dist(t->mu + (2 * j + 1) * d, t->mu + j * d, d) + t->rad[2 * j + 1];
        t->rad[j] = (r0 > r1 ? r0 : r1) * (1.0 + 0x1p-40);
    }
}

static void orc_fsb_free_tree(orc_fsb_tree *t)
{
    free(t->cell); free(t->mu); free(t->rad); free(t->amax); free(t->pmin);
    t->L = 0;
}

/* the upper bound of node j of tree t for query q_i at position i (|q| given) */
double orc_fsb_bound(const orc_fsb_tree *t, int64_t j, const float *q_i, double qn, int64_t i, const orc_head *p)
{
    double content = 0.0;
    for (int x = 0; x < p->d; ++x) content = fma((double)q_i[x], (double)t->mu[j * p->d + x], content);
    const double tt = fma(qn, t->rad[j], content);
    const double arg = (p->sigma * (double)(i - t->pmin[j])) / (2.0 * (double)p->s);
    const double g = arg >= 6.0 ? 1.0 : erf(arg);
    return fma(p->rho, tt, (p->lambda * (double)t->amax[j]) * g);
}

typedef struct { double ub; int64_t key; const orc_fsb_tree *t; int64_t j; } orc_cand;

static int cmp_cand(const void *pa, const void *pb)
{
    const orc_cand *a = (const orc_cand *)pa, *b = (const orc_cand *)pb;
    if (a->ub > b->ub) return -1;
    if (a->ub < b->ub) return 1;
    return (a->key > b->key) - (a->key < b->key);
}

static int64_t orc_fsb_key(int T, int k, int64_t a, int64_t j)
{
    return ((int64_t)T << 40) | ((int64_t)k << 34) | (a << (k + 1)) | j;
}

/* FS-B selection for one head at the given query rows. q, k: [N][d]; sel: [nrows][K];
 * lse_out (nullable): [nrows][K] the rerank scores of the selected cells, aligned
 * with sel (NaN for padding). Returns 0, -1 for bad parameters. */
int orc_fsb_select(const float *q, const float *k, const orc_head *p, const orc_fsb *fb,
                   const int64_t *rows, int64_t nrows, int32_t *sel, double *lse_out)
{
    const int d = p->d, s = p->s, K = p->K;
    const int64_t C = orc_num_cells(p);
    if (d <= 0 || (d & 1) || s <= 0 || K <= 0 || fb->beam < 1 || p->rho < 0 || p->lambda < 0 || p->sigma < 0)
        return -1;
    float *kbar = (float *)malloc(sizeof(float) * (size_t)(C > 0 ? C : 1) * d);
    float *amax = (float *)malloc(sizeof(float) * (size_t)(C > 0 ? C : 1));
    orc_cell_stats(k, p, kbar, amax);
    uint32_t *codes = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(C > 0 ? C : 1));
    for (int64_t c = 0; c < C; ++c) codes[c] = orc_fsb_code(kbar + c * d, fb->proj, d);
    int32_t *list[2];
    int64_t len[2] = {0, 0};
    list[0] = (int32_t *)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    list[1] = (int32_t *)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    for (int64_t c = 0; c < C; ++c) {
        list[0][len[0]++] = (int32_t)c;
        if ((double)amax[c] > fb->tau) list[1][len[1]++] = (int32_t)c;
    }
    /* every complete segment's tree, built once: trees[T][k][a] */
    int kmax = 0;
    while (((int64_t)1 << (kmax + 1)) <= C) ++kmax;
    orc_fsb_tree **trees[2];
    for (int T = 0; T < 2; ++T) {
        trees[T] = (orc_fsb_tree **)calloc((size_t)kmax + 1, sizeof(orc_fsb_tree *));
        for (int kk = 0; kk <= kmax; ++kk) {
            const int64_t nseg = len[T] >> kk;
            trees[T][kk] = (orc_fsb_tree *)calloc((size_t)(nseg > 0 ? nseg : 1), sizeof(orc_fsb_tree));
            for (int64_t a = 0; a < nseg; ++a)
                orc_fsb_build_tree(list[T], a, kk, codes, kbar, amax, p, &trees[T][kk][a]);
        }
    }
    const int B = fb->beam;
    orc_cand *cand = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(2 * B + 64));
    orc_cand *beam = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)(2 * B + 64));
    int32_t *ucell = (int32_t *)malloc(sizeof(int32_t) * (size_t)(2 * B));
    orc_skey *rk = (orc_skey *)malloc(sizeof(orc_skey) * (size_t)(2 * B));
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        const float *qi = q + i * d;
        double qq = 0.0;
        for (int x = 0; x < d; ++x) qq = fma((double)qi[x], (double)qi[x], qq);
        const double qn = sqrt(qq);
        const int64_t nb = orc_eligible(i / p->B, p);
        int nu = 0;
        for (int T = 0; T < 2; ++T) {
            int64_t m = 0;
            if (T == 0) m = nb;
            else while (m < len[1] && list[1][m] < nb) ++m;
            int nc = 0;
            int64_t base = 0;
            for (int kk = kmax; kk >= 0; --kk)
                if ((m >> kk) & 1) {
                    const int64_t a = base >> kk;
                    const orc_fsb_tree *t = &trees[T][kk][a];
                    cand[nc].t = t; cand[nc].j = 1; cand[nc].key = orc_fsb_key(T, kk, a, 1);
                    cand[nc].ub = orc_fsb_bound(t, 1, qi, qn, i, p);
                    ++nc;
                    base += (int64_t)1 << kk;
                }
            qsort(cand, (size_t)nc, sizeof(orc_cand), cmp_cand);
            int nbm = nc < B ? nc : B;
            memcpy(beam, cand, sizeof(orc_cand) * (size_t)nbm);
            for (;;) {
                int internal = 0;
                for (int u = 0; u < nbm; ++u) internal |= beam[u].j < beam[u].t->L;
                if (!internal) break;
                nc = 0;
                for (int u = 0; u < nbm; ++u) {
                    if (beam[u].j >= beam[u].t->L) { cand[nc++] = beam[u]; continue; }
                    for (int ch = 0; ch < 2; ++ch) {
                        const int64_t j = 2 * beam[u].j + ch;
                        cand[nc] = beam[u];
                        cand[nc].j = j;
                        cand[nc].key = (beam[u].key & ~(((int64_t)1 << 34) - 1)) |
                                       ((beam[u].key & (((int64_t)1 << 34) - 1)) - beam[u].j + j);
                        cand[nc].ub = orc_fsb_bound(beam[u].t, j, qi, qn, i, p);
                        ++nc;
                    }
                }
                qsort(cand, (size_t)nc, sizeof(orc_cand), cmp_cand);
                nbm = nc < B ? nc : B;
                memcpy(beam, cand, sizeof(orc_cand) * (size_t)nbm);
            }
            for (int u = 0; u < nbm; ++u) {
                const int32_t c = beam[u].t->cell[beam[u].j - beam[u].t->L];
                int dup = 0;
                for (int v2 = 0; v2 < nu; ++v2) dup |= ucell[v2] == c;
                if (!dup) ucell[nu++] = c;
            }
        }
        /* rerank by token-level log-sum-exp */
        for (int u = 0; u < nu; ++u) {
            const int32_t c = ucell[u];
            double mx = -INFINITY;
            double *l = (double *)malloc(sizeof(double) * (size_t)s);
            for (int jt = 0; jt < s; ++jt) {
                const float *kr = k + ((int64_t)c * s + jt) * d;
                double dot = 0.0;
                for (int x = 0; x < d; ++x) dot = fma((double)qi[x], (double)kr[x], dot);
                l[jt] = p->scale * dot;
                if (l[jt] > mx) mx = l[jt];
            }
            double sum = 0.0;
            for (int jt = 0; jt < s; ++jt) sum = sum + exp(l[jt] - mx);
            rk[u].sc = mx + log(sum);
            rk[u].idx = c;
            free(l);
        }
        qsort(rk, (size_t)nu, sizeof(orc_skey), cmp_skey);
        const int nsel = nu < K ? nu : K;
        int32_t *sl = sel + r * K;
        for (int u = 0; u < nsel; ++u) sl[u] = rk[u].idx;
        qsort(sl, (size_t)nsel, sizeof(int32_t), cmp_i32);
        for (int u = nsel; u < K; ++u) sl[u] = -1;
        if (lse_out)
            for (int u = 0; u < K; ++u) {
                double val = NAN;
                for (int v2 = 0; v2 < nsel; ++v2)
                    if (rk[v2].idx == sl[u]) val = rk[v2].sc;
                lse_out[r * K + u] = u < nsel ? val : NAN;
            }
    }
    for (int T = 0; T < 2; ++T) {
        for (int kk = 0; kk <= kmax; ++kk) {
            const int64_t nseg = len[T] >> kk;
            for (int64_t a = 0; a < nseg; ++a) orc_fsb_free_tree(&trees[T][kk][a]);
            free(trees[T][kk]);
        }
        free(trees[T]);
        free(list[T]);
    }
    free(cand); free(beam); free(ucell); free(rk); free(codes); free(kbar); free(amax);
    return 0;
}

/* the forward at the given rows with a given selection sel [nrows][K] (ascending,
 * -1 padded): window, readout over the given cells, mix (for selections made by
 * another rule, such as FS-B) */
int orc_forward_rows_sel(const float *q, const float *k, const float *v, const orc_head *p,
                         const int64_t *rows, int64_t nrows, const int32_t *sel, double *out,
                         double *o_win, double *o_long)
{
    const int d = p->d;
    const int64_t N = p->N;
    if (d <= 0 || (d & 1) || p->s <= 0 || p->w <= 0 || p->K <= 0 || N <= 0) return -1;
    double *krot = (double *)malloc(sizeof(double) * (size_t)N * d);
    for (int64_t j = 0; j < N; ++j) orc_rope(k + j * d, j, p, krot + j * d);
    double *qrot = (double *)malloc(sizeof(double) * d);
    double *ow = (double *)malloc(sizeof(double) * d);
    double *ol = (double *)malloc(sizeof(double) * d);
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        if (i < 0 || i >= N) { free(krot); free(qrot); free(ow); free(ol); return -2; }
        orc_rope(q + i * d, i, p, qrot);
        orc_window(qrot, krot, v, i, p, ow);
        int32_t nsel = 0;
        while (nsel < p->K && sel[r * p->K + nsel] >= 0) ++nsel;
        orc_readout(q + i * d, k, v, sel + r * p->K, nsel, p, ol);
        orc_mix(ow, ol, p, out + r * d);
        if (o_win) memcpy(o_win + r * d, ow, sizeof(double) * d);
        if (o_long) memcpy(o_long + r * d, ol, sizeof(double) * d);
    }
    free(krot); free(qrot); free(ow); free(ol);
    return 0;
}

/* one segment tree, copied out (for the pins): cell [L], mu [2L][d], rad/amax/pmin [2L] */
void orc_fsb_tree_dump(const int32_t *list, int64_t a, int k, const uint32_t *codes, const float *kbar,
                       const float *amax, const orc_head *p, int32_t *cell, float *mu, double *rad, float *am,
                       int64_t *pmin)
{
    orc_fsb_tree t;
    orc_fsb_build_tree(list, a, k, codes, kbar, amax, p, &t);
    const int64_t L = t.L;
    memcpy(cell, t.cell, sizeof(int32_t) * (size_t)L);
    memcpy(mu, t.mu, sizeof(float) * (size_t)(2 * L) * p->d);
    memcpy(rad, t.rad, sizeof(double) * (size_t)(2 * L));
    memcpy(am, t.amax, sizeof(float) * (size_t)(2 * L));
    memcpy(pmin, t.pmin, sizeof(int64_t) * (size_t)(2 * L));
    orc_fsb_free_tree(&t);
}

/* the bound of every node of one segment tree for query q_i at position i (for the pins): ub [2L] */
void orc_fsb_tree_bounds(const int32_t *list, int64_t a, int k, const uint32_t *codes, const float *kbar,
                         const float *amax, const orc_head *p, const float *q_i, int64_t i, double *ub)
{
    orc_fsb_tree t;
    orc_fsb_build_tree(list, a, k, codes, kbar, amax, p, &t);
    double qq = 0.0;
    for (int x = 0; x < p->d; ++x) qq = fma((double)q_i[x], (double)q_i[x], qq);
    const double qn = sqrt(qq);
    for (int64_t j = 1; j < 2 * t.L; ++j) ub[j] = orc_fsb_bound(&t, j, q_i, qn, i, p);
    orc_fsb_free_tree(&t);
}
