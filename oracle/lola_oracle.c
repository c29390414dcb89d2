/*
 * LoLA layer oracle -- plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through the
 * seeded input generator.
 *
 * What it computes (sources: "LoLA: Low-Rank Linear Attention met Sparse
 * Caching", technical summary on gist.science, sections "Methodologie: LoLA",
 * "Het Self-Recall Error (SRE) Mechanisme" with its SRE equation, and
 * "Inferentiestrategie", steps 1-4; the paper abstract on shd-paper.top for
 * the three memory systems):
 *
 *   Every past key/value pair of a (sequence b, KV head g) chain lives in one
 *   of three memories: the sliding window (last w tokens, exact softmax), the
 *   sparse cache (at most C pairs, exact softmax) or the linear state
 *   H (F x D), s (F) of linear attention with the feature map
 *   phi(x) = [softmax(W x); softmax(-W x)].
 *
 *   The sequence is processed in update intervals of L tokens.  For each
 *   interval [a, e):
 *     read   -- each query t in [a, e) uses the memories as they stand at the
 *               interval start.  Softmax keys: the exact last-w window of t
 *               (t included) and the cache.  Linear keys: the state H, s plus
 *               the keys that left the window earlier in this interval and
 *               have not been managed yet ("pending": a-w <= j <= t-w).
 *               The output is one shared denominator over all of them:
 *                 o = (sum_soft e^(l_j - m) v_j + e^-m (H^T phi(q) + sum_pend kappa_j v_j))
 *                   / (sum_soft e^(l_j - m)     + e^-m (s^T phi(q) + sum_pend kappa_j))
 *               with l_j = tau q.k_j, kappa_j = phi(q).phi(k_j), m = max l (0 if none).
 *     manage -- at the interval end the pairs that left the window during
 *               the interval (positions max(0,a-w) .. e-1-w) and the cached
 *               pairs are scored with the self-recall error against the
 *               interval-start state:
 *                 SRE(k, v | H, s) = || H^T phi(k) / (s . phi(k)) - v ||^2
 *               (prediction taken as 0 when s . phi(k) = 0, i.e. an empty
 *               state).  The C highest (ties: older position first) stay in
 *               the cache; every other one is folded into the state by an
 *               outer product: H += phi(k) v^T, s += phi(k).
 *
 * Readings where the pages are silent (order of read and management, pending
 * keys, empty state, tie order, window membership, combination weights,
 * softmax scale) follow the list in the design notes; each is marked
 * "reading:" where it is used below.  The scoring and cache policies other
 * than the SRE (lo_cfg.policy) are described at their enum.
 *
 * Everything is fp64, loops are plain, nothing is blocked or fused.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_q_heads, n_kv_heads, head_dim, feat_half;
    int32_t window, cache_cap, chunk;
    int32_t policy; /* how candidates are scored, one of lo_policy */
    double scale;   /* tau on q.k; 0 -> 1/sqrt(head_dim) (reading: no scale inside phi) */
} lo_cfg;

/* Scoring and cache policies.  The method scores every candidate by its SRE at
 * every interval ("Inferentiestrategie", steps 1-2).  Step 2 also says the kept
 * pairs live in a min-heap or a FIFO depending on the implementation, and the
 * summary's contributions and ablations name two other scorers, the magnitude
 * of the attention weights and the softmax approximation error, without
 * formulas.  Readings implemented here (all keep the C highest scores, ties to
 * the older position, exactly as the SRE policy):
 *   LO_SRE        the method: SRE against the interval-start state, every
 *                 candidate rescored at every interval.
 *   LO_SRE_STALE  min-heap of stale scores: a pair is scored by SRE once, in
 *                 the interval in which it leaves the window; a cached pair
 *                 keeps that score and is never rescored.
 *   LO_FIFO       first in, first out: the score is the position, so the C
 *                 most recent candidates stay and the oldest are folded.
 *   LO_ATTN       attention-weight magnitude: with q_h (h in the KV head's
 *                 query heads) the last query of the interval, the score of u
 *                 is sum_h softmax over the candidates of tau q_h.k_u.
 *   LO_KERR       softmax approximation error: with p_hu that softmax weight
 *                 and l_hu = phi(q_h).phi(k_u) / sum over the candidates of
 *                 phi(q_h).phi(k) the weight linear attention gives the same
 *                 candidate, the score is sum_h |p_hu - l_hu|. */
enum { LO_SRE = 0, LO_SRE_STALE = 1, LO_FIFO = 2, LO_ATTN = 3, LO_KERR = 4 };

/* Optional per-interval log, indexed [b][g][interval] (and a candidate or
 * cache slot index last).  Any pointer may be NULL. */
typedef struct {
    int32_t max_intervals; /* NI: intervals per call that the arrays hold */
    int32_t max_cand;      /* maxU: candidate slots per interval (>= C + L) */
    int32_t* n_cand;       /* [B][Hkv][NI]            |U| */
    int64_t* cand_pos;     /* [B][Hkv][NI][maxU]       candidate positions, cache first then leaving keys */
    double* cand_sre;      /* [B][Hkv][NI][maxU]       their scores (self-recall errors for LO_SRE) */
    int64_t* own_kept;     /* [B][Hkv][NI][C]          the oracle's own kept set, by rank, -1 padded */
} lo_log;

typedef struct {
    double *H, *s;           /* [F][D], [F] */
    int wn;                  /* window entries held (<= w), ascending positions */
    int64_t* wpos;
    double *wk, *wv;         /* [w][D] */
    int cn;                  /* cache entries held (<= C), no order */
    int64_t* cpos;
    double *ck, *cv;         /* [C][D] */
    double* cscore;          /* [C] the score each cached pair was kept with */
    int64_t n_folded;
} lo_chain;

typedef struct {
    lo_cfg cfg;
    int B;
    double* W;        /* [Hkv][Fh][D] */
    int64_t* t0;      /* [B] tokens seen */
    lo_chain* ch;     /* [B*Hkv] */
} lo_state;

/* ------------------------------------------------------------------ */
/* feature map and self-recall error                                   */
/* ------------------------------------------------------------------ */

/* phi(x) = [softmax(W x); softmax(-W x)], each half normalised on its own
 * (feature map fixed by the layer configuration; the pages only say it is a
 * low-rank feature map approximating the exponential kernel). */
void lo_phi(const double* W, int Fh, int D, const double* x, double* out)
{
    double* z = (double*)malloc(sizeof(double) * (size_t)Fh);
    double zmax = -INFINITY, zmin = INFINITY;
    for (int i = 0; i < Fh; ++i) {
        double acc = 0.0;
        for (int j = 0; j < D; ++j) acc += W[(size_t)i * D + j] * x[j];
        z[i] = acc;
        if (acc > zmax) zmax = acc;
        if (acc < zmin) zmin = acc;
    }
    double sp = 0.0, sn = 0.0;
    for (int i = 0; i < Fh; ++i) {
        out[i] = exp(z[i] - zmax);
        out[Fh + i] = exp(-z[i] + zmin);
        sp += out[i];
        sn += out[Fh + i];
    }
    for (int i = 0; i < Fh; ++i) {
        out[i] /= sp;
        out[Fh + i] /= sn;
    }
    free(z);
}

/* SRE(k, v | H, s) = || H^T phi(k) / (s . phi(k)) - v ||^2  (SRE equation of
 * the "Self-Recall Error" section).  reading: an empty state (s . phi = 0)
 * predicts the zero vector. */
double lo_sre(int F, int D, const double* H, const double* s, const double* phik, const double* v)
{
    double d = 0.0;
    for (int i = 0; i < F; ++i) d += phik[i] * s[i];
    double e = 0.0;
    for (int j = 0; j < D; ++j) {
        double r = 0.0;
        if (d > 0.0) {
            double n = 0.0;
            for (int i = 0; i < F; ++i) n += phik[i] * H[(size_t)i * D + j];
            r = n / d;
        }
        double diff = r - v[j];
        e += diff * diff;
    }
    return e;
}

/* ------------------------------------------------------------------ */
/* state                                                               */
/* ------------------------------------------------------------------ */

static void chain_alloc(lo_chain* c, const lo_cfg* cfg)
{
    int F = 2 * cfg->feat_half, D = cfg->head_dim, w = cfg->window, C = cfg->cache_cap;
    c->H = (double*)calloc((size_t)F * D, sizeof(double));
    c->s = (double*)calloc((size_t)F, sizeof(double));
    c->wn = 0;
    c->wpos = (int64_t*)calloc((size_t)(w > 0 ? w : 1), sizeof(int64_t));
    c->wk = (double*)calloc((size_t)(w > 0 ? w : 1) * D, sizeof(double));
    c->wv = (double*)calloc((size_t)(w > 0 ? w : 1) * D, sizeof(double));
    c->cn = 0;
    c->cpos = (int64_t*)calloc((size_t)(C > 0 ? C : 1), sizeof(int64_t));
    c->ck = (double*)calloc((size_t)(C > 0 ? C : 1) * D, sizeof(double));
    c->cv = (double*)calloc((size_t)(C > 0 ? C : 1) * D, sizeof(double));
    c->cscore = (double*)calloc((size_t)(C > 0 ? C : 1), sizeof(double));
    c->n_folded = 0;
}

static void chain_free(lo_chain* c)
{
    free(c->H); free(c->s); free(c->wpos); free(c->wk); free(c->wv);
    free(c->cpos); free(c->ck); free(c->cv); free(c->cscore);
}

static void chain_copy(lo_chain* dst, const lo_chain* src, const lo_cfg* cfg)
{
    int F = 2 * cfg->feat_half, D = cfg->head_dim;
    int w = cfg->window > 0 ? cfg->window : 1, C = cfg->cache_cap > 0 ? cfg->cache_cap : 1;
    memcpy(dst->H, src->H, sizeof(double) * (size_t)F * D);
    memcpy(dst->s, src->s, sizeof(double) * (size_t)F);
    dst->wn = src->wn;
    memcpy(dst->wpos, src->wpos, sizeof(int64_t) * (size_t)w);
    memcpy(dst->wk, src->wk, sizeof(double) * (size_t)w * D);
    memcpy(dst->wv, src->wv, sizeof(double) * (size_t)w * D);
    dst->cn = src->cn;
    memcpy(dst->cpos, src->cpos, sizeof(int64_t) * (size_t)C);
    memcpy(dst->ck, src->ck, sizeof(double) * (size_t)C * D);
    memcpy(dst->cv, src->cv, sizeof(double) * (size_t)C * D);
    memcpy(dst->cscore, src->cscore, sizeof(double) * (size_t)C);
    dst->n_folded = src->n_folded;
}

lo_state* lo_create(const lo_cfg* cfg, int B, const double* W)
{
    if (!cfg || B <= 0 || cfg->n_kv_heads <= 0 || cfg->n_q_heads % cfg->n_kv_heads != 0 ||
        cfg->head_dim <= 0 || cfg->feat_half <= 0 || cfg->window < 0 || cfg->cache_cap < 0 ||
        cfg->chunk < 1 || cfg->policy < LO_SRE || cfg->policy > LO_KERR)
        return NULL;
    lo_state* st = (lo_state*)calloc(1, sizeof(lo_state));
    st->cfg = *cfg;
    if (st->cfg.scale <= 0.0) st->cfg.scale = 1.0 / sqrt((double)cfg->head_dim);
    st->B = B;
    size_t wsz = (size_t)cfg->n_kv_heads * cfg->feat_half * cfg->head_dim;
    st->W = (double*)malloc(sizeof(double) * wsz);
    memcpy(st->W, W, sizeof(double) * wsz);
    st->t0 = (int64_t*)calloc((size_t)B, sizeof(int64_t));
    st->ch = (lo_chain*)calloc((size_t)B * cfg->n_kv_heads, sizeof(lo_chain));
    for (int i = 0; i < B * cfg->n_kv_heads; ++i) chain_alloc(&st->ch[i], cfg);
    return st;
}

lo_state* lo_clone(const lo_state* src)
{
    lo_state* st = lo_create(&src->cfg, src->B, src->W);
    if (!st) return NULL;
    memcpy(st->t0, src->t0, sizeof(int64_t) * (size_t)src->B);
    for (int i = 0; i < src->B * src->cfg.n_kv_heads; ++i) chain_copy(&st->ch[i], &src->ch[i], &src->cfg);
    return st;
}

void lo_destroy(lo_state* st)
{
    if (!st) return;
    for (int i = 0; i < st->B * st->cfg.n_kv_heads; ++i) chain_free(&st->ch[i]);
    free(st->ch); free(st->t0); free(st->W); free(st);
}

int64_t lo_tokens_seen(const lo_state* st, int b) { return st->t0[b]; }

/* Copy out one chain: H [F][D], s [F], cache sorted by ascending position
 * (pos, k, v; -1 padded to C), window (pos, k, v ascending), folded count.
 * Any output pointer may be NULL. */
void lo_get_chain(const lo_state* st, int b, int g, double* H, double* s,
                  int32_t* cache_n, int64_t* cache_pos, double* cache_k, double* cache_v,
                  int32_t* win_n, int64_t* win_pos, double* win_k, double* win_v, int64_t* n_folded)
{
    const lo_cfg* cfg = &st->cfg;
    const lo_chain* c = &st->ch[(size_t)b * cfg->n_kv_heads + g];
    int F = 2 * cfg->feat_half, D = cfg->head_dim, C = cfg->cache_cap;
    if (H) memcpy(H, c->H, sizeof(double) * (size_t)F * D);
    if (s) memcpy(s, c->s, sizeof(double) * (size_t)F);
    if (cache_n) *cache_n = c->cn;
    if (cache_pos || cache_k || cache_v) {
        /* selection sort by position: plain and obviously ordered */
        int* idx = (int*)malloc(sizeof(int) * (size_t)(c->cn > 0 ? c->cn : 1));
        for (int i = 0; i < c->cn; ++i) idx[i] = i;
        for (int i = 0; i < c->cn; ++i)
            for (int j = i + 1; j < c->cn; ++j)
                if (c->cpos[idx[j]] < c->cpos[idx[i]]) { int t = idx[i]; idx[i] = idx[j]; idx[j] = t; }
        for (int i = 0; i < C; ++i) {
            if (i < c->cn) {
                if (cache_pos) cache_pos[i] = c->cpos[idx[i]];
                if (cache_k) memcpy(cache_k + (size_t)i * D, c->ck + (size_t)idx[i] * D, sizeof(double) * D);
                if (cache_v) memcpy(cache_v + (size_t)i * D, c->cv + (size_t)idx[i] * D, sizeof(double) * D);
            } else if (cache_pos) {
                cache_pos[i] = -1;
            }
        }
        free(idx);
    }
    if (win_n) *win_n = c->wn;
    for (int i = 0; i < c->wn; ++i) {
        if (win_pos) win_pos[i] = c->wpos[i];
        if (win_k) memcpy(win_k + (size_t)i * D, c->wk + (size_t)i * D, sizeof(double) * D);
        if (win_v) memcpy(win_v + (size_t)i * D, c->wv + (size_t)i * D, sizeof(double) * D);
    }
    if (n_folded) *n_folded = c->n_folded;
}

/* ------------------------------------------------------------------ */
/* one update interval of one chain                                    */
/* ------------------------------------------------------------------ */

typedef struct {
    int idx;     /* index into the candidate list */
    double e;
    int64_t pos;
} cand_t;

/* reading: keep order is (SRE descending, position ascending) -- the older pair
 * wins an exact tie, as a min-heap that keeps what it holds would. */
static int cand_cmp(const void* pa, const void* pb)
{
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->e > b->e) return -1;
    if (a->e < b->e) return 1;
    if (a->pos < b->pos) return -1;
    if (a->pos > b->pos) return 1;
    return 0;
}

typedef struct {
    lo_state* st;
    int n;                 /* tokens in this call */
    const double *q, *k, *v;
    double* out;
    const int64_t* forced; /* [B][Hkv][NI][C] or NULL */
    const lo_log* log;
    const uint8_t* chain_mask; /* [B][Hkv] or NULL */
    const uint8_t* row_mask;   /* [n] or NULL */
    int NI;
    int nthreads, tid;
    int status;
} run_job;

/* Process interval `ci` = [a, e) of chain (b, g).  Returns 0 or a negative code. */
static int run_interval(run_job* jb, int b, int g, int ci, int64_t t0c, int64_t a, int64_t e)
{
    lo_state* st = jb->st;
    const lo_cfg* cfg = &st->cfg;
    const int Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads, D = cfg->head_dim, Fh = cfg->feat_half;
    const int F = 2 * Fh, w = cfg->window, C = cfg->cache_cap, G = Hq / Hkv;
    const int n = jb->n;
    const double tau = cfg->scale;
    const double* Wg = st->W + (size_t)g * Fh * D;
    lo_chain* c = &st->ch[(size_t)b * Hkv + g];

    /* R: the recent keys -- the window as it stands at the interval start,
     * followed by this interval's tokens, in ascending position. */
    int len = (int)(e - a);
    int nR = c->wn + len;
    int64_t* Rpos = (int64_t*)malloc(sizeof(int64_t) * (size_t)nR);
    const double** Rk = (const double**)malloc(sizeof(double*) * (size_t)nR);
    const double** Rv = (const double**)malloc(sizeof(double*) * (size_t)nR);
    double* Rphi = (double*)malloc(sizeof(double) * (size_t)nR * F);
    for (int i = 0; i < c->wn; ++i) {
        Rpos[i] = c->wpos[i];
        Rk[i] = c->wk + (size_t)i * D;
        Rv[i] = c->wv + (size_t)i * D;
    }
    for (int i = 0; i < len; ++i) {
        int64_t t = a + i;
        size_t row = ((size_t)b * n + (size_t)(t - t0c)) * Hkv + g;
        Rpos[c->wn + i] = t;
        Rk[c->wn + i] = jb->k + row * D;
        Rv[c->wn + i] = jb->v + row * D;
    }
    for (int i = 0; i < nR; ++i) lo_phi(Wg, Fh, D, Rk[i], Rphi + (size_t)i * F);

    /* ---------------- read (interval-start memories) ---------------- */
    if (jb->out) {
        double* phq = (double*)malloc(sizeof(double) * F);
        double* N = (double*)malloc(sizeof(double) * D);
        double* lin = (double*)malloc(sizeof(double) * D);
        double* lg = (double*)malloc(sizeof(double) * (size_t)(nR + C + 1));
        for (int64_t t = a; t < e; ++t) {
            if (jb->row_mask && !jb->row_mask[t - t0c]) continue;
            for (int h = g * G; h < (g + 1) * G; ++h) {
                const double* qv = jb->q + (((size_t)b * n + (size_t)(t - t0c)) * Hq + h) * D;
                lo_phi(Wg, Fh, D, qv, phq);
                /* softmax keys: window of t (reading: last w tokens, t included) and the cache */
                double m = -INFINITY;
                int nl = 0;
                for (int i = 0; i < nR; ++i) {
                    if (Rpos[i] > t || Rpos[i] < t - w + 1) continue;
                    double dot = 0.0;
                    for (int j = 0; j < D; ++j) dot += qv[j] * Rk[i][j];
                    lg[nl] = tau * dot;
                    if (lg[nl] > m) m = lg[nl];
                    ++nl;
                }
                for (int i = 0; i < c->cn; ++i) {
                    double dot = 0.0;
                    for (int j = 0; j < D; ++j) dot += qv[j] * c->ck[(size_t)i * D + j];
                    lg[nl] = tau * dot;
                    if (lg[nl] > m) m = lg[nl];
                    ++nl;
                }
                if (nl == 0) m = 0.0;
                for (int j = 0; j < D; ++j) N[j] = 0.0;
                double Z = 0.0;
                nl = 0;
                for (int i = 0; i < nR; ++i) {
                    if (Rpos[i] > t || Rpos[i] < t - w + 1) continue;
                    double wgt = exp(lg[nl++] - m);
                    for (int j = 0; j < D; ++j) N[j] += wgt * Rv[i][j];
                    Z += wgt;
                }
                for (int i = 0; i < c->cn; ++i) {
                    double wgt = exp(lg[nl++] - m);
                    for (int j = 0; j < D; ++j) N[j] += wgt * c->cv[(size_t)i * D + j];
                    Z += wgt;
                }
                /* linear keys: the state, then the pending keys that left the
                 * window earlier in this interval (reading: they are linear
                 * until the interval end manages them) */
                double zl = 0.0;
                for (int j = 0; j < D; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < F; ++i) acc += phq[i] * c->H[(size_t)i * D + j];
                    lin[j] = acc;
                }
                for (int i = 0; i < F; ++i) zl += phq[i] * c->s[i];
                for (int i = 0; i < nR; ++i) {
                    if (Rpos[i] > t - w) continue;
                    double kap = 0.0;
                    for (int f = 0; f < F; ++f) kap += phq[f] * Rphi[(size_t)i * F + f];
                    for (int j = 0; j < D; ++j) lin[j] += kap * Rv[i][j];
                    zl += kap;
                }
                /* reading: one shared denominator, unit weights on every memory */
                double sc = exp(-m);
                double* o = jb->out + (((size_t)b * n + (size_t)(t - t0c)) * Hq + h) * D;
                Z += sc * zl;
                for (int j = 0; j < D; ++j) o[j] = (N[j] + sc * lin[j]) / Z;
            }
        }
        free(phq); free(N); free(lin); free(lg);
    }

    /* ---------------- manage at the interval end ---------------- */
    /* E: keys that left the window during [a, e): positions <= e-1-w.  They
     * form a prefix of R. */
    int nE = 0;
    while (nE < nR && Rpos[nE] <= e - 1 - w) ++nE;
    int nU = c->cn + nE;
    double* Uphi = (double*)malloc(sizeof(double) * (size_t)(nU > 0 ? nU : 1) * F);
    const double** Uk = (const double**)malloc(sizeof(double*) * (size_t)(nU > 0 ? nU : 1));
    const double** Uv = (const double**)malloc(sizeof(double*) * (size_t)(nU > 0 ? nU : 1));
    int64_t* Upos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nU > 0 ? nU : 1));
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nU > 0 ? nU : 1));
    for (int i = 0; i < c->cn; ++i) {
        Uk[i] = c->ck + (size_t)i * D;
        Uv[i] = c->cv + (size_t)i * D;
        Upos[i] = c->cpos[i];
        lo_phi(Wg, Fh, D, Uk[i], Uphi + (size_t)i * F);
    }
    for (int i = 0; i < nE; ++i) {
        Uk[c->cn + i] = Rk[i];
        Uv[c->cn + i] = Rv[i];
        Upos[c->cn + i] = Rpos[i];
        memcpy(Uphi + (size_t)(c->cn + i) * F, Rphi + (size_t)i * F, sizeof(double) * F);
    }
    /* score every candidate (reading: SRE against the interval-start state) */
    for (int u = 0; u < nU; ++u) {
        cand[u].idx = u;
        cand[u].pos = Upos[u];
        cand[u].e = lo_sre(F, D, c->H, c->s, Uphi + (size_t)u * F, Uv[u]);
    }
    if (cfg->policy == LO_SRE_STALE) {
        /* a cached pair keeps the score it was kept with */
        for (int u = 0; u < c->cn; ++u) cand[u].e = c->cscore[u];
    } else if (cfg->policy == LO_FIFO) {
        for (int u = 0; u < nU; ++u) cand[u].e = (double)Upos[u];
    } else if ((cfg->policy == LO_ATTN || cfg->policy == LO_KERR) && nU > 0) {
        /* the interval's last query, every query head of this KV head */
        const int64_t tl = e - 1;
        double* lgt = (double*)malloc(sizeof(double) * (size_t)nU);
        double* kap = (double*)malloc(sizeof(double) * (size_t)nU);
        double* phq = (double*)malloc(sizeof(double) * F);
        for (int u = 0; u < nU; ++u) cand[u].e = 0.0;
        for (int h = g * G; h < (g + 1) * G; ++h) {
            const double* qv = jb->q + (((size_t)b * n + (size_t)(tl - t0c)) * Hq + h) * D;
            double mx = -INFINITY, zs = 0.0, ks = 0.0;
            for (int u = 0; u < nU; ++u) {
                double dot = 0.0;
                for (int j = 0; j < D; ++j) dot += qv[j] * Uk[u][j];
                lgt[u] = tau * dot;
                if (lgt[u] > mx) mx = lgt[u];
            }
            for (int u = 0; u < nU; ++u) zs += exp(lgt[u] - mx);
            if (cfg->policy == LO_KERR) {
                lo_phi(Wg, Fh, D, qv, phq);
                for (int u = 0; u < nU; ++u) {
                    double kk = 0.0;
                    for (int f = 0; f < F; ++f) kk += phq[f] * Uphi[(size_t)u * F + f];
                    kap[u] = kk;
                    ks += kk;
                }
            }
            for (int u = 0; u < nU; ++u) {
                const double p = exp(lgt[u] - mx) / zs;
                cand[u].e += cfg->policy == LO_ATTN ? p : fabs(p - kap[u] / ks);
            }
        }
        free(lgt); free(kap); free(phq);
    }
    const lo_log* lg = jb->log;
    size_t li = ((size_t)b * Hkv + g) * (size_t)(lg ? lg->max_intervals : 0) + (size_t)ci;
    if (lg) {
        if (lg->n_cand) lg->n_cand[li] = nU;
        for (int u = 0; u < nU && u < lg->max_cand; ++u) {
            if (lg->cand_pos) lg->cand_pos[li * lg->max_cand + u] = Upos[u];
            if (lg->cand_sre) lg->cand_sre[li * lg->max_cand + u] = cand[u].e;
        }
    }
    /* keep: if everything fits, keep all (reading); else the C highest */
    uint8_t* keep = (uint8_t*)calloc((size_t)(nU > 0 ? nU : 1), 1);
    int nkeep = nU <= C ? nU : C;
    int bad_forced = 0;
    {
        cand_t* sorted = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nU > 0 ? nU : 1));
        memcpy(sorted, cand, sizeof(cand_t) * (size_t)nU);
        qsort(sorted, (size_t)nU, sizeof(cand_t), cand_cmp);
        if (lg && lg->own_kept)
            for (int i = 0; i < C; ++i)
                lg->own_kept[li * C + i] = i < nkeep ? sorted[i].pos : -1;
        if (jb->forced) {
            /* adopt a selection made elsewhere (the interval-stepped parity
             * harness); it must name nkeep distinct candidates of U */
            const int64_t* fs = jb->forced + (((size_t)b * Hkv + g) * jb->NI + ci) * (size_t)C;
            int nf = 0;
            for (int i = 0; i < C && !bad_forced; ++i) {
                if (fs[i] < 0) continue;
                int found = -1;
                for (int u = 0; u < nU; ++u)
                    if (Upos[u] == fs[i]) found = u;
                if (found < 0 || keep[found]) bad_forced = 1;
                else { keep[found] = 1; ++nf; }
            }
            if (nf != nkeep) bad_forced = 1;
        } else {
            for (int i = 0; i < nkeep; ++i) keep[sorted[i].idx] = 1;
        }
        free(sorted);
    }
    if (bad_forced) {
        free(keep); free(cand); free(Upos); free(Uv); free(Uk); free(Uphi);
        free(Rpos); free(Rk); free(Rv); free(Rphi);
        return -2; /* forced set is not a valid selection of this interval */
    }
    /* fold the rest: H += phi(k) v^T, s += phi(k) (outer-product update) */
    for (int u = 0; u < nU; ++u) {
        if (keep[u]) continue;
        const double* ph = Uphi + (size_t)u * F;
        for (int i = 0; i < F; ++i) {
            for (int j = 0; j < D; ++j) c->H[(size_t)i * D + j] += ph[i] * Uv[u][j];
            c->s[i] += ph[i];
        }
        c->n_folded += 1;
    }
    /* new cache = kept candidates; new window = R entries at positions >= e-w */
    int64_t* npos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(C > 0 ? C : 1));
    double* nk = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1) * D);
    double* nv = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1) * D);
    double* nsc = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    int cn = 0;
    for (int u = 0; u < nU; ++u) {
        if (!keep[u]) continue;
        nsc[cn] = cand[u].e;
        npos[cn] = Upos[u];
        memcpy(nk + (size_t)cn * D, Uk[u], sizeof(double) * D);
        memcpy(nv + (size_t)cn * D, Uv[u], sizeof(double) * D);
        ++cn;
    }
    int64_t* wpos2 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(w > 0 ? w : 1));
    double* wk2 = (double*)malloc(sizeof(double) * (size_t)(w > 0 ? w : 1) * D);
    double* wv2 = (double*)malloc(sizeof(double) * (size_t)(w > 0 ? w : 1) * D);
    int wn = 0;
    for (int i = 0; i < nR; ++i) {
        if (Rpos[i] < e - w) continue;
        wpos2[wn] = Rpos[i];
        memcpy(wk2 + (size_t)wn * D, Rk[i], sizeof(double) * D);
        memcpy(wv2 + (size_t)wn * D, Rv[i], sizeof(double) * D);
        ++wn;
    }
    c->cn = cn;
    memcpy(c->cpos, npos, sizeof(int64_t) * (size_t)cn);
    memcpy(c->ck, nk, sizeof(double) * (size_t)cn * D);
    memcpy(c->cv, nv, sizeof(double) * (size_t)cn * D);
    memcpy(c->cscore, nsc, sizeof(double) * (size_t)cn);
    c->wn = wn;
    memcpy(c->wpos, wpos2, sizeof(int64_t) * (size_t)wn);
    memcpy(c->wk, wk2, sizeof(double) * (size_t)wn * D);
    memcpy(c->wv, wv2, sizeof(double) * (size_t)wn * D);

    free(npos); free(nk); free(nv); free(nsc); free(wpos2); free(wk2); free(wv2);
    free(keep); free(cand); free(Upos); free(Uv); free(Uk); free(Uphi);
    free(Rpos); free(Rk); free(Rv); free(Rphi);
    return 0;
}

/* ------------------------------------------------------------------ */
/* driver                                                              */
/* ------------------------------------------------------------------ */

static void* run_worker(void* arg)
{
    run_job* jb = (run_job*)arg;
    lo_state* st = jb->st;
    const int Hkv = st->cfg.n_kv_heads, L = st->cfg.chunk;
    int idx = 0;
    for (int b = 0; b < st->B; ++b) {
        for (int g = 0; g < Hkv; ++g, ++idx) {
            if (idx % jb->nthreads != jb->tid) continue;
            if (jb->chain_mask && !jb->chain_mask[(size_t)b * Hkv + g]) continue;
            int64_t t0c = st->t0[b];
            /* reading: each call starts its own interval grid at its first token */
            for (int ci = 0; ci < jb->NI; ++ci) {
                int64_t a = t0c + (int64_t)ci * L;
                int64_t e = a + L;
                if (e > t0c + jb->n) e = t0c + jb->n;
                int rc = run_interval(jb, b, g, ci, t0c, a, e);
                if (rc != 0) { jb->status = rc; return NULL; }
            }
        }
    }
    return NULL;
}

/* Process n tokens of every sequence as consecutive intervals of `chunk`
 * tokens (the last may be shorter), starting at the current position.
 *   q   [B][n][Hq][D],  k, v [B][n][Hkv][D]
 *   out [B][n][Hq][D] or NULL (state only: no read is computed)
 *   forced      [B][Hkv][NI][C] kept positions per interval (-1 padded) or NULL
 *   log         optional per-interval log (NI must equal ceil(n / chunk))
 *   chain_mask  [B][Hkv] or NULL: chains left out are not advanced at all
 *   row_mask    [n] or NULL: outputs are only computed for rows with a 1
 * Returns 0, -1 on bad arguments, -2 when a forced set is not a valid choice.
 * Chains are independent; they are spread over `nthreads` threads. */
int lo_run(lo_state* st, int n, const double* q, const double* k, const double* v, double* out,
           const int64_t* forced, const lo_log* log, const uint8_t* chain_mask,
           const uint8_t* row_mask, int nthreads)
{
    if (!st || n <= 0 || !k || !v || (out && !q)) return -1;
    if ((st->cfg.policy == LO_ATTN || st->cfg.policy == LO_KERR) && !q) return -1; /* they score with q */
    int NI = (n + st->cfg.chunk - 1) / st->cfg.chunk;
    if (log && (log->max_intervals < NI || log->max_cand < st->cfg.cache_cap + st->cfg.chunk)) return -1;
    if (nthreads < 1) nthreads = 1;
    run_job* jobs = (run_job*)calloc((size_t)nthreads, sizeof(run_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int i = 0; i < nthreads; ++i) {
        jobs[i].st = st; jobs[i].n = n; jobs[i].q = q; jobs[i].k = k; jobs[i].v = v;
        jobs[i].out = out; jobs[i].forced = forced; jobs[i].log = log;
        jobs[i].chain_mask = chain_mask; jobs[i].row_mask = row_mask;
        jobs[i].NI = NI; jobs[i].nthreads = nthreads; jobs[i].tid = i; jobs[i].status = 0;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, run_worker, &jobs[i]);
    run_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    int status = 0;
    for (int i = 0; i < nthreads; ++i)
        if (jobs[i].status != 0) status = jobs[i].status;
    free(jobs); free(th);
    if (status == 0)
        for (int b = 0; b < st->B; ++b) st->t0[b] += n;
    return status;
}
