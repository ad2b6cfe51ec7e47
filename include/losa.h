/*
 * losa.h -- C ABI of liblosa.so: LoSA per-denoising-step attention on MI355X.
 *
 * LoSA (Locality Aware Sparse Attention for Block-Wise Diffusion Language
 * Models, arXiv 2604.12056) runs, at each denoising step of a block of B
 * tokens and for one attention layer:
 *   1. a locality score per block token: the mean squared change of its
 *      query since the previous step (gist.science pt summary, section
 *      "3. Metodologia", step 1; fr summary, "Pruning par Localité");
 *   2. the |A| most-changed tokens form the active set, the rest are stable
 *      (same passages);
 *   3. QUEST page selection for the active tokens only (pt step 3; fr
 *      "Calcul Sparse pour les Tokens Actifs");
 *   4. the union of their selected pages, the only prefix KV that is read
 *      (fr "Réduction de l'Union KV"; hf.space abstract);
 *   5. prefix attention of the active tokens over that union, giving the
 *      prefix output o_p and log-normaliser L_p (agifrontier tutorial,
 *      section on the LoSA workflow);
 *   6. stable tokens reuse the cached (o_p, L_p) (pt step 2);
 *   7. dense attention of all block tokens over the block itself (tutorial,
 *      workflow section; pt step 4);
 *   8. an online-softmax (log-sum-exp) merge of prefix and block parts, the
 *      new statistics kept for the next step (pt step 4);
 *   and the first step of every block is a forced dense prefix pass
 *   (tutorial, section on limitations).
 *
 * Reading of what the pages leave open (QUEST is named, not defined there):
 * pages are 16 consecutive tokens of one KV head; a page's metadata is the
 * element-wise min and max of its keys; a query's bound for a page is
 * sum_i max(q_i*min_i, q_i*max_i); every active query keeps the
 * budget_tokens/16 pages of largest bound (all pages when that covers the
 * prefix); the union is taken per KV head over the G*|A| active rows of its
 * query-head group (G = n_qhead / n_kvhead); every active row attends over
 * the whole union; scores are per (query head, token), so each query head
 * has its own active set.
 *
 * Canonical index arithmetic (reproduced bit for bit; see each call):
 *   locality e = fp32 chain over i ascending of fl(acc + fl(d_i*d_i)),
 *     d_i = fl(q_t,i - q_prev,i), acc from +0; reported score = e / d;
 *   active set: |A| largest e, equal scores to the lower token, ascending;
 *   page bound U = fp32 chain over i ascending of fl(acc + fl(q_i*s_i)),
 *     s_i = max_i if q_i >= 0 else min_i, acc from +0 (for bf16 inputs every
 *     product is exact, so a fused multiply-add gives the same bits);
 *   top-k: k largest U, -0 equal to +0, equal bounds to the lower page;
 *   page indices are local to their sequence and lists are ascending.
 * Values (o_p, L_p, outputs) are fp32 arithmetic on the device: scores,
 * exponentials, the log-sum-exp merge; bf16 outputs are rounded to nearest
 * even.  The natural logarithm is used for L_p.
 *
 * Memory.  Every array argument is a device pointer (hipMalloc or
 * equivalent) owned by the caller, 16-byte aligned.  The library allocates,
 * frees and synchronises nothing and keeps no state between calls (except
 * losa_step_noalloc's static scratch, below); the workspace is scratch owned
 * by the caller and must not be shared by calls that may run concurrently.  All work is enqueued on `stream` (a
 * hipStream_t; NULL is the default stream).  Calls return after enqueueing.
 *
 * Layouts (row-major, innermost last; T = kv_tokens):
 *   q_t, q_prev, out       [n_seq][B][n_qhead][head_dim]      dtype
 *   k_blk, v_blk           [n_seq][B][n_kvhead][head_dim]     dtype
 *   k_cache, v_cache       [n_kvhead][T][head_dim]            dtype
 *       the cache rows of every KV head are grouped in physical pages of 16
 *       tokens (page e: rows 16e .. 16e+15).  A sequence's prefix lies either
 *       contiguously -- sequence s holds tokens kv_off[s] .. kv_off[s] +
 *       prefix_len[s] - 1, kv_off[s] a multiple of page_size, sequences not
 *       overlapping -- or, with a page table, in any pages of the pool: the
 *       sequence's page p (its tokens 16p .. 16p+15) is physical page
 *       page_table[s][p] (a paged KV pool: ragged sequences need no
 *       contiguous room, and pages may be shared between sequences).
 *   kv_off, prefix_len     [n_seq] int32 (device); kv_off may be NULL with a page table
 *   page_table             NULL, or [n_seq][max(1, ceil(max_prefix_len / 16))] int32
 *                          (device): physical pages in [0, T/16); entries at or
 *                          past a sequence's page count are not used.  A page
 *                          shared by sequences must hold the same valid tokens in
 *                          each (whole pages, as shared prefixes give).
 *   op_cache               [n_seq][n_qhead][B][head_dim]      fp32 (o_p)
 *   lp_cache               [n_seq][n_qhead][B]                fp32 (L_p)
 *   page_meta              opaque, losa_page_meta_bytes() bytes, kept per (sequence,
 *                          page of the sequence): at the page's cache position in
 *                          the contiguous layout, from s * ceil(max_prefix_len / 16)
 *                          for sequence s with a page table
 *
 * Errors.  Arguments are checked on the host before anything is enqueued;
 * a failed check returns its status and enqueues nothing.  A failed launch
 * returns LOSA_ERR_HIP.  Asynchronous device faults surface at the caller's
 * next synchronisation.  prefix_len[s] must lie in [0, max_prefix_len] and
 * kv_off[s] + prefix_len[s] <= kv_tokens (page-table entries in [0, T/16));
 * kernels clamp out-of-range values into the cache instead of reading past
 * it, so the results for such a sequence are unspecified but memory-safe.
 * Inputs must be finite.
 */
#ifndef LOSA_H_
#define LOSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum losa_status {
    LOSA_OK = 0,
    LOSA_ERR_INVALID_ARG = 1, /* a null/misaligned pointer or an inconsistent shape */
    LOSA_ERR_UNSUPPORTED = 2, /* a legal shape this build has no kernel for */
    LOSA_ERR_WORKSPACE = 3,   /* workspace smaller than losa_workspace_bytes() */
    LOSA_ERR_HIP = 4,         /* a HIP launch failed */
    LOSA_ERR_SCRATCH = 5      /* losa_step_noalloc: the shape needs more than its static scratch */
} losa_status;

typedef enum losa_dtype { LOSA_F32 = 0, LOSA_BF16 = 1 } losa_dtype;

typedef struct losa_shape {
    int32_t n_seq;          /* sequences in the batch, >= 1 */
    int32_t block;          /* B: tokens per block, 1..64 */
    int32_t n_qhead;        /* query heads, a multiple of n_kvhead */
    int32_t n_kvhead;       /* KV heads, >= 1 */
    int32_t head_dim;       /* 64 or 128 */
    int32_t page_size;      /* 16 */
    int32_t budget_tokens;  /* per-query prefix budget in tokens, a positive multiple of page_size */
    int32_t n_active;       /* |A|: active tokens per query head, 0..block */
    int32_t max_prefix_len; /* upper bound of prefix_len[], 0..kv_tokens; sizes the grids */
    int32_t dtype;          /* losa_dtype of q, k, v and out */
    int64_t kv_tokens;      /* T: tokens per KV head in k_cache/v_cache, a multiple of page_size */
    float softmax_scale;    /* > 0, or 0 for 1/sqrt(head_dim) */
    uint32_t flags;         /* 0 (the plain reading) or an OR of the losa_flags below */
} losa_shape;

/*
 * Readings of three points the pages leave open; 0 selects the plain reading
 * (every active row attends the whole union of its KV head; one active set per
 * query head; the sparse statistics are written back to the cache).
 *   LOSA_FLAG_ROW_MASK: each active row attends only the pages it selected
 *     itself; the union still decides what is loaded (fr summary, "Réduction de
 *     l'Union KV").  Needs at most 64 stacked rows per KV head (G * n_active),
 *     else LOSA_ERR_UNSUPPORTED.
 *   LOSA_FLAG_SHARED_ACTIVE: one active set per sequence, shared by all query
 *     heads: a token's locality is the sum over query heads, in ascending head
 *     order, of its per-head mean squared change (an fp32 chain); the n_active
 *     largest sums are active, equal sums to the lower token.
 *   LOSA_FLAG_NO_WRITEBACK: a sparse step does not store the active tokens' new
 *     (o_p, L_p); they serve that step's output, and the caches keep what the
 *     block's dense first step wrote (agifrontier tutorial, workflow section:
 *     statistics are reused from the last full computation).
 * losa_dense_first_step ignores the flags.
 */
typedef enum losa_flags {
    LOSA_FLAG_ROW_MASK = 1,
    LOSA_FLAG_SHARED_ACTIVE = 2,
    LOSA_FLAG_NO_WRITEBACK = 4
} losa_flags;

/* Number of events in losa_debug.stage_events. */
#define LOSA_STAGE_EVENTS 6

/* Optional outputs of losa_step / losa_dense_first_step (each pointer may be
 * NULL; the dense call uses only stage_events). */
typedef struct losa_debug {
    float *locality;     /* [n_seq][n_qhead][B] locality score e/d */
    int32_t *active;     /* [n_seq][n_qhead][n_active] active tokens, ascending */
    int32_t *page_sel;   /* [n_seq][n_qhead][n_active][k], k = budget_tokens/page_size:
                            each active row's pages, ascending, -1 past the prefix's pages */
    int32_t *union_idx;  /* [n_seq][n_kvhead][union_cap] union of a KV head's pages, ascending */
    int32_t *union_cnt;  /* [n_seq][n_kvhead] union sizes */
    int32_t union_cap;   /* capacity of each union_idx row; >= losa_union_capacity() */
    void **stage_events; /* profiling: LOSA_STAGE_EVENTS caller-created hipEvent_t, recorded
                            on the stream before the first kernel (0) and after the
                            prepare (1), page-scoring (2), page-selection (3),
                            prefix-attention (4) and finishing (5) kernels; a skipped
                            stage records at the same point as the one before it */
} losa_debug;

/* Human-readable name of a status code (static string). */
const char *losa_status_string(int status);

/* Bytes of the page metadata for this shape (0 if the shape is invalid): per
 * KV head and metadata page -- max(kv_tokens / 16, n_seq * ceil(max_prefix_len
 * / 16)) of them, enough for either layout -- the page's per-dimension min and
 * max twice (two layouts: one for scoring, one for the exact bounds of
 * selection), 4 * head_dim element sizes, plus one fp32 (the largest |key|). */
size_t losa_page_meta_bytes(const losa_shape *shape);

/* Workspace bytes that losa_step and losa_dense_first_step need (0 if invalid). */
size_t losa_workspace_bytes(const losa_shape *shape);

/* Largest possible union per (sequence, KV head): min(pages of the longest
 * prefix, G * n_active * budget_tokens/page_size); -1 if the shape is invalid. */
int32_t losa_union_capacity(const losa_shape *shape);

/*
 * Page metadata for QUEST selection (reading above): for every page of every
 * sequence and KV head, the element-wise minimum and maximum of the keys of
 * its tokens that lie below prefix_len[s].  Run once per committed block
 * (the prefix does not change between the denoising steps of a block).
 * Writes page_meta (losa_page_meta_bytes(shape) bytes, library layout) per
 * (sequence, page): with a page table the keys are read through it and a page
 * shared by sequences gets its metadata once per sequence, so the metadata of
 * a sequence's consecutive pages stays contiguous however the table scatters
 * them.  Metadata must be built and used with the same layout (page table or
 * not).
 */
int losa_build_page_meta(const losa_shape *shape, const void *k_cache, const int32_t *kv_off,
                         const int32_t *prefix_len, const int32_t *page_table, void *page_meta,
                         void *stream);

/*
 * Block commit: when the tokens first_token[s] .. prefix_len[s] - 1 of each
 * sequence have joined its prefix (a committed block; the cache already holds
 * their keys), rewrites the metadata of the pages holding them -- the same
 * bytes losa_build_page_meta would write for those pages -- and nothing else.
 * The pages before them keep their metadata (their keys do not change).
 *   first_token: device int32 [n_seq], the first new token of each sequence
 *                (a sequence with first_token[s] >= prefix_len[s] is left as is)
 *   max_new_tokens: host bound on prefix_len[s] - first_token[s] over the
 *                sequences (sizes the launch; pages past it are not rewritten)
 *   prefix_len: the new prefix lengths; shape->max_prefix_len bounds them.
 * Errors: LOSA_ERR_INVALID_ARG for null or misaligned pointers or
 * max_new_tokens outside 0 .. max_prefix_len; nothing is enqueued then.
 * The pages' tokens themselves are read from k_cache as in
 * losa_build_page_meta (reading used for QUEST: per-page element-wise min and
 * max, gist.science pt summary, "3. Metodologia", step 3).
 */
int losa_update_page_meta(const losa_shape *shape, const void *k_cache, const int32_t *kv_off,
                          const int32_t *prefix_len, const int32_t *page_table,
                          const int32_t *first_token, int32_t max_new_tokens, void *page_meta,
                          void *stream);

/*
 * Forced dense first step of a block (agifrontier tutorial, limitations
 * section): every block token of every query head attends over its whole
 * prefix; (o_p, L_p) of every token are written to op_cache/lp_cache
 * (prefix_len 0 gives o_p = 0, L_p = -inf); then dense in-block attention
 * and the merge write `out`.
 */
int losa_dense_first_step(const losa_shape *shape, const void *q_t, const void *k_blk,
                          const void *v_blk, const void *k_cache, const void *v_cache,
                          const int32_t *kv_off, const int32_t *prefix_len,
                          const int32_t *page_table, float *op_cache, float *lp_cache, void *out,
                          const losa_debug *debug, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * One LoSA step (steps 1-8 above).  q_prev is the previous step's q_t.  Only
 * the (o_p, L_p) of active (query head, token) rows are recomputed, over the
 * union of their KV head's selected pages, and overwrite the cache; stable
 * rows read the cache unchanged.  `out` is written for every token.
 * n_active = 0 reads no prefix KV at all.  debug may be NULL.
 */
int losa_step(const losa_shape *shape, const void *q_t, const void *q_prev, const void *k_blk,
              const void *v_blk, const void *k_cache, const void *v_cache, const void *page_meta,
              const int32_t *kv_off, const int32_t *prefix_len, const int32_t *page_table,
              float *op_cache, float *lp_cache, void *out, const losa_debug *debug,
              void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the static scratch that losa_step_noalloc uses on each GPU. */
#define LOSA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * losa_step for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as losa_step, minus
 * the workspace: the step's scratch (stacked query rows, page bounds, selected
 * pages, split-K partials) lives in a static device array of
 * LOSA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held until
 * the process ends.  The first call on a device, with that device current,
 * looks up that device's copy (hipGetSymbolAddress); no call allocates or
 * frees anything.  A shape whose scratch need exceeds the limit (it is at most
 * losa_workspace_bytes(shape)) returns LOSA_ERR_SCRATCH with nothing enqueued;
 * the headline shapes (64K or 128K prefix, B = 16, 32/8 heads, d = 128,
 * budget <= 256) fit.  Every call on a GPU uses the same array, which keeps
 * the last call's contents (nothing in it needs to start at zero): calls that
 * may overlap on one GPU -- concurrent streams, or host threads -- race and
 * must be serialised by the caller.
 */
int losa_step_noalloc(const losa_shape *shape, const void *q_t, const void *q_prev,
                      const void *k_blk, const void *v_blk, const void *k_cache,
                      const void *v_cache, const void *page_meta, const int32_t *kv_off,
                      const int32_t *prefix_len, const int32_t *page_table, float *op_cache,
                      float *lp_cache, void *out, const losa_debug *debug, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LOSA_H_ */
