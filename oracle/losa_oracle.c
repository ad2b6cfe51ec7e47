/*
 * LoSA per-denoising-step attention -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * Sources (LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion
 * Language Models, arXiv 2604.12056, as described on these pages):
 *   [T]  agifrontier tutorial, sections "LoSA workflow" (深入机制：LoSA的工作流拆解)
 *        and "limitations" (局限与未来);
 *   [PT] gist.science summary (pt), section "3. Metodologia", steps 1-4;
 *   [JA] gist.science summary (ja), section "2. 提案手法", "LoSA のアルゴリズム";
 *   [FR] gist.science summary (fr), section "3. Méthodologie";
 *   [AB] hf.space abstract.
 * The pages name QUEST as the sparse selector but do not spell it out.  The
 * reading used here: per 16-token page, the element-wise minimum and maximum
 * of its keys; a query's bound for a page is sum_i max(q_i*min_i, q_i*max_i);
 * each active query keeps the budget/16 pages of largest bound.
 *
 * Precision.  Every quantity that decides an index (the locality score, the
 * page bound) is an fp32 chain taken left to right over i = 0..d-1, each
 * product rounded to fp32 and then added with one more fp32 rounding (no fused
 * multiply-add: build with -ffp-contract=off).  Attention, the log-normaliser
 * and the merge are computed in double.  Outputs are rounded to the storage
 * type (bf16: round-to-nearest-even) at the very end.
 *
 * Indexing.  Queries q_t, q_prev and outputs: [n_seq][B][H_q][d].  Block keys
 * and values: [n_seq][B][H_kv][d].  Prefix cache: [H_kv][T][d], sequence s
 * holding tokens kv_off[s] .. kv_off[s]+L_s-1 (kv_off a multiple of the page
 * size).  Page metadata: [H_kv][T/P][d] indexed by the global page
 * kv_off[s]/P + p.  Prefix statistics: o_p [n_seq][H_q][B][d] and
 * L_p [n_seq][H_q][B], both double.  Page indices that leave the oracle are
 * local to their sequence (0 .. ceil(L_s/P)-1).  GQA: query head h reads KV
 * head h / G, G = H_q / H_kv; stacked row r of KV head g is query head
 * g*G + r / |A| at active slot r % |A|.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_seq, block, n_qhead, n_kvhead, head_dim, page_size, budget_tokens, n_active;
    int32_t out_bf16;      /* 1: round outputs to bf16, 0: to fp32 */
    int32_t union_cap;     /* capacity of each union list in the debug output */
    int64_t kv_tokens;     /* T */
    double softmax_scale;  /* 0 => 1/sqrt(d) */
    int32_t flags;         /* readings of three points the pages leave open (below); 0: the
                              plain reading */
    int32_t pad_;
} oracle_shape;

/* Variants of readings the pages leave open (0 = the plain reading):
 *  ROW_MASK: each active query attends only over the pages it selected itself,
 *    not over the whole union of its KV head (QUEST's own per-query selection;
 *    the union still decides what is loaded) [FR "Réduction de l'Union KV"].
 *  SHARED_ACTIVE: one active set per sequence, shared by all query heads: the
 *    locality score of a token is the sum over query heads (ascending) of its
 *    per-head scores, an fp32 chain; the |A| largest are active, equal sums to
 *    the lower token [the tutorial's overhead estimate is per head; a
 *    per-layer score is the other reading].
 *  NO_WRITEBACK: a sparse step does not store the active tokens' new (o_p,
 *    L_p): they serve that step's output only, and the cache keeps the
 *    statistics of the block's dense first step [T "LoSA workflow": the cached
 *    statistics are reused from the last full computation]. */
#define ORACLE_ROW_MASK 1
#define ORACLE_SHARED_ACTIVE 2
#define ORACLE_NO_WRITEBACK 4

static double scale_of(const oracle_shape *sh) {
    return sh->softmax_scale > 0 ? sh->softmax_scale : 1.0 / sqrt((double)sh->head_dim);
}

static int64_t n_pages_of(const oracle_shape *sh, int32_t len) {
    return ((int64_t)len + sh->page_size - 1) / sh->page_size;
}

/* Round a double to the nearest bf16 value (ties to even), returned as float. */
static float round_to_bf16(double x) {
    if (x == 0.0 || isnan(x) || isinf(x)) return (float)x;
    double ax = fabs(x);
    int e;
    frexp(ax, &e);                       /* ax = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                       /* 8 significant bits */
    if (q < -133) q = -133;              /* subnormal quantum 2^-133 */
    double r = ldexp(nearbyint(ldexp(ax, -q)), q);
    if (r >= 0x1p128) r = INFINITY;      /* rounded past the largest bf16 */
    return (float)(x < 0 ? -r : r);
}

static float store_out(const oracle_shape *sh, double x) {
    return sh->out_bf16 ? round_to_bf16(x) : (float)x;
}

/* ------------------------------------------------------------------------ */
/* Page metadata: element-wise min and max of the keys of each page (QUEST
 * reading above).  Only the tokens below the sequence's prefix length count. */
void oracle_page_meta(const oracle_shape *sh, const float *k_cache, const int32_t *kv_off,
                      const int32_t *prefix_len, float *kmin, float *kmax) {
    const int d = sh->head_dim, P = sh->page_size;
    const int64_t T = sh->kv_tokens, TP = T / P;
    for (int g = 0; g < sh->n_kvhead; ++g)
        for (int s = 0; s < sh->n_seq; ++s) {
            int64_t np_ = n_pages_of(sh, prefix_len[s]);
            for (int64_t p = 0; p < np_; ++p) {
                int64_t gp = kv_off[s] / P + p;
                float *mn = kmin + ((int64_t)g * TP + gp) * d;
                float *mx = kmax + ((int64_t)g * TP + gp) * d;
                int64_t t0 = p * P, t1 = (p + 1) * P;
                if (t1 > prefix_len[s]) t1 = prefix_len[s];
                for (int i = 0; i < d; ++i) {
                    float lo = INFINITY, hi = -INFINITY;
                    for (int64_t t = t0; t < t1; ++t) {
                        float v = k_cache[((int64_t)g * T + kv_off[s] + t) * d + i];
                        if (v < lo) lo = v;
                        if (v > hi) hi = v;
                    }
                    mn[i] = lo;
                    mx[i] = hi;
                }
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Locality score [PT step 1; FR "Pruning par Localité"; JA 局所性プルーニング]:
 * the mean squared difference between a token's query at this step and at the
 * previous step, per query head.  score = (chain sum of (q_t-q_prev)^2) / d. */
void oracle_locality(const oracle_shape *sh, const float *q_t, const float *q_prev, float *score) {
    const int B = sh->block, H = sh->n_qhead, d = sh->head_dim;
    for (int s = 0; s < sh->n_seq; ++s)
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < B; ++t) {
                const float *a = q_t + (((int64_t)s * B + t) * H + h) * d;
                const float *b = q_prev + (((int64_t)s * B + t) * H + h) * d;
                float acc = 0.0f;
                for (int i = 0; i < d; ++i) {
                    float delta = a[i] - b[i];
                    float sq = delta * delta;
                    acc = acc + sq;
                }
                score[((int64_t)s * H + h) * B + t] = acc / (float)d;
            }
}

/* Active set [PT step 1; FR "Sélection des Tokens Actifs"]: the |A| tokens of
 * largest score, per query head; equal scores go to the lower token.  Output
 * sorted ascending, [n_seq][H_q][|A|]. */
void oracle_active_set(const oracle_shape *sh, const float *score, int32_t *active) {
    const int B = sh->block, H = sh->n_qhead, A = sh->n_active;
    char taken[4096];
    if (B > 4096) return;
    for (int s = 0; s < sh->n_seq; ++s)
        for (int h = 0; h < H; ++h) {
            const float *sc = score + ((int64_t)s * H + h) * B;
            int32_t *out = active + ((int64_t)s * H + h) * A;
            memset(taken, 0, sizeof taken);
            for (int a = 0; a < A; ++a) {
                int best = -1;
                for (int t = 0; t < B; ++t)
                    if (!taken[t] && (best < 0 || sc[t] > sc[best])) best = t;
                taken[best] = 1;
            }
            int n = 0;
            for (int t = 0; t < B; ++t)
                if (taken[t]) out[n++] = t;
        }
}

/* Shared active set (SHARED_ACTIVE): per sequence, the sum over query heads in
 * ascending order of each token's per-head score (fp32 chain), then the |A|
 * largest as in oracle_active_set, the same list written for every head. */
void oracle_shared_active_set(const oracle_shape *sh, const float *score, float *total,
                              int32_t *active) {
    const int B = sh->block, H = sh->n_qhead, A = sh->n_active;
    char taken[4096];
    if (B > 4096) return;
    for (int s = 0; s < sh->n_seq; ++s) {
        float *tot = total + (int64_t)s * B;
        for (int t = 0; t < B; ++t) {
            float acc = 0.0f;
            for (int h = 0; h < H; ++h) acc = acc + score[((int64_t)s * H + h) * B + t];
            tot[t] = acc;
        }
        memset(taken, 0, sizeof taken);
        for (int a = 0; a < A; ++a) {
            int best = -1;
            for (int t = 0; t < B; ++t)
                if (!taken[t] && (best < 0 || tot[t] > tot[best])) best = t;
            taken[best] = 1;
        }
        for (int h = 0; h < H; ++h) {
            int32_t *out = active + ((int64_t)s * H + h) * A;
            int n = 0;
            for (int t = 0; t < B; ++t)
                if (taken[t]) out[n++] = t;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* QUEST page bound for one query and one page (reading above): the sum over
 * dimensions of max(q_i*min_i, q_i*max_i), i.e. q_i times max_i when q_i is
 * not negative and times min_i otherwise, as an fp32 chain. */
float oracle_page_bound(const float *q, const float *mn, const float *mx, int d) {
    float acc = 0.0f;
    for (int i = 0; i < d; ++i) {
        float sel = q[i] >= 0.0f ? mx[i] : mn[i];
        float prod = q[i] * sel;
        acc = acc + prod;
    }
    return acc;
}

/* Top-k pages of one row: k largest bounds, equal bounds to the lower page,
 * written ascending.  k >= n selects every page.  Returns the count written. */
static int64_t topk_pages(const float *U, int64_t n, int64_t k, char *taken, int32_t *out) {
    if (k >= n) {
        for (int64_t p = 0; p < n; ++p) out[p] = (int32_t)p;
        return n;
    }
    memset(taken, 0, (size_t)n);
    for (int64_t a = 0; a < k; ++a) {
        int64_t best = -1;
        for (int64_t p = 0; p < n; ++p)
            if (!taken[p] && (best < 0 || U[p] > U[best])) best = p;
        taken[best] = 1;
    }
    int64_t c = 0;
    for (int64_t p = 0; p < n; ++p)
        if (taken[p]) out[c++] = (int32_t)p;
    return c;
}

/* Page selection for the active rows only [PT step 3; FR "Calcul Sparse pour
 * les Tokens Actifs"], then the union over a KV head's stacked rows [FR: the
 * union is taken over the active set only].
 *   page_sel  [n_seq][H_q][|A|][k]  (entries past the sequence's page count: -1)
 *   union_idx [n_seq][H_kv][union_cap], union_cnt [n_seq][H_kv]
 *   bounds    optional, [n_seq][H_kv][G*|A|][max_pages] of every row's bounds. */
void oracle_select_pages(const oracle_shape *sh, const float *q_t, const float *kmin,
                         const float *kmax, const int32_t *kv_off, const int32_t *prefix_len,
                         const int32_t *active, int32_t *page_sel, int32_t *union_idx,
                         int32_t *union_cnt, float *bounds, int64_t bounds_stride) {
    const int B = sh->block, H = sh->n_qhead, Hk = sh->n_kvhead, d = sh->head_dim;
    const int A = sh->n_active, G = H / Hk, P = sh->page_size;
    const int64_t k = sh->budget_tokens / P, TP = sh->kv_tokens / P;
    for (int s = 0; s < sh->n_seq; ++s) {
        const int64_t np_ = n_pages_of(sh, prefix_len[s]);
        float *U = (float *)malloc(sizeof(float) * (size_t)(np_ + 1));
        char *taken = (char *)malloc((size_t)np_ + 1);
        char *in_union = (char *)malloc((size_t)np_ + 1);
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(np_ + 1));
        for (int g = 0; g < Hk; ++g) {
            memset(in_union, 0, (size_t)np_ + 1);
            for (int r = 0; r < G * A; ++r) {
                const int h = g * G + r / A, a = r % A;
                const int t = active[((int64_t)s * H + h) * A + a];
                const float *q = q_t + (((int64_t)s * B + t) * H + h) * d;
                for (int64_t p = 0; p < np_; ++p) {
                    const int64_t gp = kv_off[s] / P + p;
                    U[p] = oracle_page_bound(q, kmin + ((int64_t)g * TP + gp) * d,
                                             kmax + ((int64_t)g * TP + gp) * d, d);
                    if (bounds)
                        bounds[(((int64_t)s * Hk + g) * G * A + r) * bounds_stride + p] = U[p];
                }
                int64_t c = topk_pages(U, np_, k, taken, sel);
                for (int64_t i = 0; i < c; ++i) in_union[sel[i]] = 1;
                if (page_sel) {
                    int32_t *dst = page_sel + (((int64_t)s * H + h) * A + a) * k;
                    for (int64_t i = 0; i < k; ++i) dst[i] = i < c ? sel[i] : -1;
                }
            }
            int32_t cnt = 0;
            for (int64_t p = 0; p < np_; ++p)
                if (in_union[p]) {
                    if (union_idx && cnt < sh->union_cap)
                        union_idx[((int64_t)s * Hk + g) * sh->union_cap + cnt] = (int32_t)p;
                    ++cnt;
                }
            if (union_cnt) union_cnt[(int64_t)s * Hk + g] = cnt;
        }
        free(U); free(taken); free(in_union); free(sel);
    }
}

/* ------------------------------------------------------------------------ */
/* Softmax attention of one query over n keys/values given by row pointers, in
 * double: o = sum_j softmax(s)_j v_j with s_j = scale*(q.k_j), and the
 * log-normaliser lse = log sum_j exp(s_j) (natural log).  n = 0 gives o = 0 and
 * lse = -inf.  These are the (o_p, L_p) / (o_s, L_s) statistics of the online
 * softmax decomposition [T "LoSA workflow"; PT step 4; JA オンライン Softmax]. */
static void attend(const float *q, const float *const *keys, const float *const *vals, int64_t n,
                   int d, double scale, double *s_buf, double *o, double *lse) {
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    if (n == 0) { *lse = -INFINITY; return; }
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += (double)q[i] * (double)keys[j][i];
        s_buf[j] = scale * dot;
        if (s_buf[j] > m) m = s_buf[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(s_buf[j] - m);
        sum += w;
        for (int i = 0; i < d; ++i) o[i] += w * (double)vals[j][i];
    }
    for (int i = 0; i < d; ++i) o[i] /= sum;
    *lse = m + log(sum);
}

/* Merge of prefix and suffix statistics into one softmax [T "LoSA workflow";
 * PT step 4]: L = log(e^Lp + e^Ls), O = e^(Lp-L) o_p + e^(Ls-L) o_s. */
static void merge(const double *op, double lp, const double *os, double ls, int d, double *o) {
    if (lp == -INFINITY) { for (int i = 0; i < d; ++i) o[i] = os[i]; return; }
    if (ls == -INFINITY) { for (int i = 0; i < d; ++i) o[i] = op[i]; return; }
    double m = lp > ls ? lp : ls;
    double L = m + log(exp(lp - m) + exp(ls - m));
    double wp = exp(lp - L), ws = exp(ls - L);
    for (int i = 0; i < d; ++i) o[i] = wp * op[i] + ws * os[i];
}

/* Dense in-block (suffix) attention for every block token [T: the block is
 * short, so it is attended densely; FR "Fusion"], then the merge with the
 * prefix statistics held in the cache, then the output in the storage type. */
static void suffix_and_merge(const oracle_shape *sh, const float *q_t, const float *k_blk,
                             const float *v_blk, const double *op_cache, const double *lp_cache,
                             float *out) {
    const int B = sh->block, H = sh->n_qhead, Hk = sh->n_kvhead, d = sh->head_dim;
    const int G = H / Hk;
    const double scale = scale_of(sh);
    const float **keys = (const float **)malloc(sizeof(float *) * (size_t)B);
    const float **vals = (const float **)malloc(sizeof(float *) * (size_t)B);
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)B);
    double *os = (double *)malloc(sizeof(double) * (size_t)d);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    for (int s = 0; s < sh->n_seq; ++s)
        for (int h = 0; h < H; ++h) {
            const int g = h / G;
            for (int u = 0; u < B; ++u) {
                keys[u] = k_blk + (((int64_t)s * B + u) * Hk + g) * d;
                vals[u] = v_blk + (((int64_t)s * B + u) * Hk + g) * d;
            }
            for (int t = 0; t < B; ++t) {
                const float *q = q_t + (((int64_t)s * B + t) * H + h) * d;
                double ls;
                attend(q, keys, vals, B, d, scale, s_buf, os, &ls);
                const int64_t row = ((int64_t)s * H + h) * B + t;
                merge(op_cache + row * d, lp_cache[row], os, ls, d, o);
                float *dst = out + (((int64_t)s * B + t) * H + h) * d;
                for (int i = 0; i < d; ++i) dst[i] = store_out(sh, o[i]);
            }
        }
    free(keys); free(vals); free(s_buf); free(os); free(o);
}

/* Prefix attention of one query over an explicit list of local pages of
 * sequence s, masking positions at or past the prefix length. */
static void prefix_attend(const oracle_shape *sh, int s, int g, const float *q,
                          const float *k_cache, const float *v_cache, const int32_t *kv_off,
                          const int32_t *prefix_len, const int32_t *pages, int64_t n_pages,
                          double *o, double *lse) {
    const int d = sh->head_dim, P = sh->page_size;
    const int64_t T = sh->kv_tokens;
    int64_t n = 0;
    const float **keys = (const float **)malloc(sizeof(float *) * (size_t)(n_pages * P + 1));
    const float **vals = (const float **)malloc(sizeof(float *) * (size_t)(n_pages * P + 1));
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)(n_pages * P + 1));
    for (int64_t i = 0; i < n_pages; ++i)
        for (int j = 0; j < P; ++j) {
            int64_t t = (int64_t)pages[i] * P + j;
            if (t >= prefix_len[s]) break;
            keys[n] = k_cache + ((int64_t)g * T + kv_off[s] + t) * d;
            vals[n] = v_cache + ((int64_t)g * T + kv_off[s] + t) * d;
            ++n;
        }
    attend(q, keys, vals, n, d, scale_of(sh), s_buf, o, lse);
    free(keys); free(vals); free(s_buf);
}

/* ------------------------------------------------------------------------ */
/* One LoSA step [PT steps 1-4; FR "Fonctionnement de l'algorithme"; JA
 * "LoSA のアルゴリズム"]:
 *   1. locality score per (query head, token); 2. the |A| most-changed tokens;
 *   3. page selection for those tokens only; 4. the union per KV head;
 *   5. prefix attention of each active token over every page of the union,
 *      its (o_p, L_p) overwriting the cache; 6. stable tokens keep the cached
 *      (o_p, L_p) untouched [PT step 2]; 7. dense in-block attention for all
 *      tokens; 8. merge; the cache keeps the new statistics for the next step
 *      [PT step 4].
 * Debug outputs may be NULL. */
void oracle_step(const oracle_shape *sh, const float *q_t, const float *q_prev, const float *k_blk,
                 const float *v_blk, const float *k_cache, const float *v_cache, const float *kmin,
                 const float *kmax, const int32_t *kv_off, const int32_t *prefix_len,
                 double *op_cache, double *lp_cache, float *out, float *locality,
                 int32_t *active_out, int32_t *page_sel, int32_t *union_idx, int32_t *union_cnt) {
    const int B = sh->block, H = sh->n_qhead, Hk = sh->n_kvhead, d = sh->head_dim;
    const int A = sh->n_active, G = H / Hk;
    const int64_t nsh = (int64_t)sh->n_seq * H;
    float *score = (float *)malloc(sizeof(float) * (size_t)(nsh * B));
    int32_t *active = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nsh * A + 1));
    oracle_locality(sh, q_t, q_prev, score);
    if (sh->flags & ORACLE_SHARED_ACTIVE) {
        float *total = (float *)malloc(sizeof(float) * (size_t)(sh->n_seq * B));
        oracle_shared_active_set(sh, score, total, active);
        free(total);
    } else {
        oracle_active_set(sh, score, active);
    }

    oracle_shape full = *sh;
    int32_t max_pages = 0;
    for (int s = 0; s < sh->n_seq; ++s)
        if (n_pages_of(sh, prefix_len[s]) > max_pages) max_pages = (int32_t)n_pages_of(sh, prefix_len[s]);
    full.union_cap = max_pages;
    int32_t *uidx = (int32_t *)malloc(sizeof(int32_t) * (size_t)((int64_t)sh->n_seq * Hk * max_pages + 1));
    int32_t *ucnt = (int32_t *)malloc(sizeof(int32_t) * (size_t)(sh->n_seq * Hk));
    const int64_t k = sh->budget_tokens / sh->page_size;
    int32_t *psel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nsh * A * k + 1));
    oracle_select_pages(&full, q_t, kmin, kmax, kv_off, prefix_len, active, psel, uidx, ucnt,
                        NULL, 0);
    if (page_sel) memcpy(page_sel, psel, sizeof(int32_t) * (size_t)(nsh * A * k));

    /* the statistics this step merges: the cache itself, or (NO_WRITEBACK) a copy */
    double *op_use = op_cache, *lp_use = lp_cache;
    if (sh->flags & ORACLE_NO_WRITEBACK) {
        op_use = (double *)malloc(sizeof(double) * (size_t)(nsh * B * d));
        lp_use = (double *)malloc(sizeof(double) * (size_t)(nsh * B));
        memcpy(op_use, op_cache, sizeof(double) * (size_t)(nsh * B * d));
        memcpy(lp_use, lp_cache, sizeof(double) * (size_t)(nsh * B));
    }
    int32_t *own = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k + 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    for (int s = 0; s < sh->n_seq; ++s)
        for (int h = 0; h < H; ++h) {
            const int g = h / G;
            for (int a = 0; a < A; ++a) {
                const int t = active[((int64_t)s * H + h) * A + a];
                const float *q = q_t + (((int64_t)s * B + t) * H + h) * d;
                double lse;
                if (sh->flags & ORACLE_ROW_MASK) {
                    /* the row's own pages (page_sel lists them ascending, -1 past the end) */
                    int64_t n_own = 0;
                    for (int64_t e = 0; e < k; ++e) {
                        const int32_t pg = psel[(((int64_t)s * H + h) * A + a) * k + e];
                        if (pg >= 0) own[n_own++] = pg;
                    }
                    prefix_attend(sh, s, g, q, k_cache, v_cache, kv_off, prefix_len, own, n_own,
                                  o, &lse);
                } else {
                    prefix_attend(sh, s, g, q, k_cache, v_cache, kv_off, prefix_len,
                                  uidx + ((int64_t)s * Hk + g) * max_pages, ucnt[s * Hk + g], o,
                                  &lse);
                }
                const int64_t row = ((int64_t)s * H + h) * B + t;
                memcpy(op_use + row * d, o, sizeof(double) * (size_t)d);
                lp_use[row] = lse;
            }
        }
    suffix_and_merge(sh, q_t, k_blk, v_blk, op_use, lp_use, out);
    if (op_use != op_cache) {
        free(op_use);
        free(lp_use);
    }
    free(own);
    free(psel);

    if (locality) memcpy(locality, score, sizeof(float) * (size_t)(nsh * B));
    if (active_out) memcpy(active_out, active, sizeof(int32_t) * (size_t)(nsh * A));
    for (int s = 0; s < sh->n_seq; ++s)
        for (int g = 0; g < Hk; ++g) {
            if (union_cnt) union_cnt[s * Hk + g] = ucnt[s * Hk + g];
            if (union_idx)
                for (int i = 0; i < ucnt[s * Hk + g] && i < sh->union_cap; ++i)
                    union_idx[((int64_t)s * Hk + g) * sh->union_cap + i] =
                        uidx[((int64_t)s * Hk + g) * max_pages + i];
        }
    free(score); free(active); free(uidx); free(ucnt); free(o);
}

/* The first step of a block [T "limitations": the first denoising iteration
 * of each block is a forced dense pass]: every block token attends densely to
 * the whole prefix, its (o_p, L_p) fill the cache, then suffix and merge. */
void oracle_dense_first_step(const oracle_shape *sh, const float *q_t, const float *k_blk,
                             const float *v_blk, const float *k_cache, const float *v_cache,
                             const int32_t *kv_off, const int32_t *prefix_len, double *op_cache,
                             double *lp_cache, float *out) {
    const int B = sh->block, H = sh->n_qhead, Hk = sh->n_kvhead, d = sh->head_dim;
    const int G = H / Hk;
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    for (int s = 0; s < sh->n_seq; ++s) {
        const int64_t np_ = n_pages_of(sh, prefix_len[s]);
        int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(np_ + 1));
        for (int64_t p = 0; p < np_; ++p) all[p] = (int32_t)p;
        for (int h = 0; h < H; ++h)
            for (int t = 0; t < B; ++t) {
                const float *q = q_t + (((int64_t)s * B + t) * H + h) * d;
                double lse;
                prefix_attend(sh, s, h / G, q, k_cache, v_cache, kv_off, prefix_len, all, np_, o,
                              &lse);
                const int64_t row = ((int64_t)s * H + h) * B + t;
                memcpy(op_cache + row * d, o, sizeof(double) * (size_t)d);
                lp_cache[row] = lse;
            }
        free(all);
    }
    free(o);
    (void)Hk;
    suffix_and_merge(sh, q_t, k_blk, v_blk, op_cache, lp_cache, out);
}

/* Naive per-query sparse attention (the KV-inflation baseline [T "KV
 * inflation"; PT section 1]): every block token selects its own top-k pages
 * and attends over those pages only, with no reuse; then suffix and merge.
 * Writes the per-token (o_p, L_p) into the given cache arrays. */
void oracle_naive_sparse_step(const oracle_shape *sh, const float *q_t, const float *k_blk,
                              const float *v_blk, const float *k_cache, const float *v_cache,
                              const float *kmin, const float *kmax, const int32_t *kv_off,
                              const int32_t *prefix_len, double *op_cache, double *lp_cache,
                              float *out) {
    const int B = sh->block, H = sh->n_qhead, Hk = sh->n_kvhead, d = sh->head_dim;
    const int G = H / Hk, P = sh->page_size;
    const int64_t k = sh->budget_tokens / P, TP = sh->kv_tokens / P;
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    for (int s = 0; s < sh->n_seq; ++s) {
        const int64_t np_ = n_pages_of(sh, prefix_len[s]);
        float *U = (float *)malloc(sizeof(float) * (size_t)(np_ + 1));
        char *taken = (char *)malloc((size_t)np_ + 1);
        int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(np_ + 1));
        for (int h = 0; h < H; ++h) {
            const int g = h / G;
            for (int t = 0; t < B; ++t) {
                const float *q = q_t + (((int64_t)s * B + t) * H + h) * d;
                for (int64_t p = 0; p < np_; ++p) {
                    const int64_t gp = kv_off[s] / P + p;
                    U[p] = oracle_page_bound(q, kmin + ((int64_t)g * TP + gp) * d,
                                             kmax + ((int64_t)g * TP + gp) * d, d);
                }
                int64_t c = topk_pages(U, np_, k, taken, sel);
                double lse;
                prefix_attend(sh, s, g, q, k_cache, v_cache, kv_off, prefix_len, sel, c, o, &lse);
                const int64_t row = ((int64_t)s * H + h) * B + t;
                memcpy(op_cache + row * d, o, sizeof(double) * (size_t)d);
                lp_cache[row] = lse;
            }
        }
        free(U); free(taken); free(sel);
    }
    free(o);
    suffix_and_merge(sh, q_t, k_blk, v_blk, op_cache, lp_cache, out);
}

/* One row of the dense first step, for sampled checks at sizes where the full
 * step is slow: (o_p, L_p) of query head h, token t of sequence s over its
 * whole prefix, then that row's dense in-block attention and merge. */
void oracle_dense_row(const oracle_shape *sh, int s, int h, int t, const float *q_t,
                      const float *k_blk, const float *v_blk, const float *k_cache,
                      const float *v_cache, const int32_t *kv_off, const int32_t *prefix_len,
                      double *op, double *lp, float *out_row) {
    const int B = sh->block, H = sh->n_qhead, Hk = sh->n_kvhead, d = sh->head_dim;
    const int G = H / Hk, g = h / G;
    const int64_t np_ = n_pages_of(sh, prefix_len[s]);
    int32_t *all = (int32_t *)malloc(sizeof(int32_t) * (size_t)(np_ + 1));
    for (int64_t p = 0; p < np_; ++p) all[p] = (int32_t)p;
    const float *q = q_t + (((int64_t)s * B + t) * H + h) * d;
    prefix_attend(sh, s, g, q, k_cache, v_cache, kv_off, prefix_len, all, np_, op, lp);
    free(all);
    const float **keys = (const float **)malloc(sizeof(float *) * (size_t)B);
    const float **vals = (const float **)malloc(sizeof(float *) * (size_t)B);
    double *s_buf = (double *)malloc(sizeof(double) * (size_t)B);
    double *os = (double *)malloc(sizeof(double) * (size_t)d);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    for (int u = 0; u < B; ++u) {
        keys[u] = k_blk + (((int64_t)s * B + u) * Hk + g) * d;
        vals[u] = v_blk + (((int64_t)s * B + u) * Hk + g) * d;
    }
    double ls;
    attend(q, keys, vals, B, d, scale_of(sh), s_buf, os, &ls);
    merge(op, *lp, os, ls, d, o);
    for (int i = 0; i < d; ++i) out_row[i] = store_out(sh, o[i]);
    free(keys); free(vals); free(s_buf); free(os); free(o);
}
