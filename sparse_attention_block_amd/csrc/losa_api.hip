// C-ABI entry points of liblosa.so: argument checks (host only, before any HIP
// call), workspace carve-up and the launch sequence of each call.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "losa_internal.h"

using namespace losa;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxPagesSupported = kMaxBitmapWords * 32;  // LDS bitmap of the union (32 KiB)

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const losa_shape *sh) {
    if (!sh) return LOSA_ERR_INVALID_ARG;
    if (sh->n_seq < 1 || sh->block < 1 || sh->n_qhead < 1 || sh->n_kvhead < 1)
        return LOSA_ERR_INVALID_ARG;
    if (sh->n_qhead % sh->n_kvhead) return LOSA_ERR_INVALID_ARG;
    if (sh->page_size <= 0 || sh->head_dim <= 0) return LOSA_ERR_INVALID_ARG;
    if (sh->dtype != LOSA_F32 && sh->dtype != LOSA_BF16) return LOSA_ERR_INVALID_ARG;
    if (sh->budget_tokens < sh->page_size || sh->budget_tokens % sh->page_size)
        return LOSA_ERR_INVALID_ARG;
    if (sh->n_active < 0 || sh->n_active > sh->block) return LOSA_ERR_INVALID_ARG;
    if (sh->kv_tokens < sh->page_size || sh->kv_tokens % sh->page_size) return LOSA_ERR_INVALID_ARG;
    if (sh->max_prefix_len < 0 || sh->max_prefix_len > sh->kv_tokens) return LOSA_ERR_INVALID_ARG;
    if (!(sh->softmax_scale >= 0.0f) || isinf(sh->softmax_scale)) return LOSA_ERR_INVALID_ARG;
    if (sh->flags & ~(uint32_t)(LOSA_FLAG_ROW_MASK | LOSA_FLAG_SHARED_ACTIVE | LOSA_FLAG_NO_WRITEBACK))
        return LOSA_ERR_INVALID_ARG;
    if (sh->page_size != kPage) return LOSA_ERR_UNSUPPORTED;
    if (sh->head_dim != 64 && sh->head_dim != 128) return LOSA_ERR_UNSUPPORTED;
    if (sh->block > 64) return LOSA_ERR_UNSUPPORTED;
    if ((int64_t)(sh->n_qhead / sh->n_kvhead) * sh->block > kMaxRows) return LOSA_ERR_UNSUPPORTED;
    if ((sh->flags & LOSA_FLAG_ROW_MASK) &&
        (int64_t)(sh->n_qhead / sh->n_kvhead) * sh->n_active > kMaxMaskRows)
        return LOSA_ERR_UNSUPPORTED;
    if ((sh->max_prefix_len + kPage - 1) / kPage > kMaxPagesSupported) return LOSA_ERR_UNSUPPORTED;
    if (sh->kv_tokens / kPage > (int64_t)1 << 30) return LOSA_ERR_UNSUPPORTED;
    return LOSA_OK;
}

size_t meta_main_bytes(const Dims &D) {
    const size_t sT = D.bf16 ? 2 : 4;
    return (size_t)D.Hk * D.n_tiles_total * kTile * D.d * 2 * sT;
}

Dims make_dims(const losa_shape *sh) {
    Dims D;
    D.S = sh->n_seq;
    D.B = sh->block;
    D.Hq = sh->n_qhead;
    D.Hk = sh->n_kvhead;
    D.G = D.Hq / D.Hk;
    D.d = sh->head_dim;
    D.A = sh->n_active;
    D.k = sh->budget_tokens / kPage;
    D.bf16 = sh->dtype == LOSA_BF16;
    D.flags = static_cast<int>(sh->flags);
    D.max_pages = (sh->max_prefix_len + kPage - 1) / kPage;
    D.hb_stride = (std::max(D.max_pages, 1) + 3) / 4 * 4;
    D.T = sh->kv_tokens;
    // metadata pages per KV head: the cache's pages (contiguous layout) or
    // max_pages per sequence (page table), whichever is more
    const int64_t meta_pages = std::max<int64_t>(D.T / kPage, (int64_t)D.S * D.max_pages);
    D.n_tiles_total = (meta_pages + kTile - 1) / kTile;
    D.meta_main_bytes = static_cast<int64_t>(meta_main_bytes(D));
    D.meta_pm_off = D.meta_main_bytes + D.Hk * D.n_tiles_total * kTile * 4;
    D.n_tiles_grid = std::max(1, (D.max_pages + kTile - 1) / kTile);
    D.R = D.G * D.A;
    D.Rs16 = (D.R + 15) / 16 * 16;
    D.Rd = D.G * D.B;
    D.R16 = (D.Rd + 15) / 16 * 16;
    const int64_t rk = (int64_t)D.R * D.k;
    int64_t cap = rk < D.max_pages ? rk : D.max_pages;
    D.union_cap = cap > 0 ? static_cast<int>(cap) : 1;
    // Split-K sizes.  Dense pass: the largest chunk (up to 64 pages) that still
    // gives kDenseTargetGroups workgroups.  Sparse pass: one page per wave unless
    // the union capacity would give more than kSparseTargetGroups workgroups;
    // then larger chunks, which also write fewer partial results.
    const int64_t sgc = (int64_t)D.S * D.Hk;
    auto chunks = [](int n, int c) { return (n + c - 1) / c; };
    D.dense_chunk = kMaxDenseChunk;
    while (D.dense_chunk > kMinDenseChunk &&
           sgc * chunks(D.max_pages, D.dense_chunk) < kDenseTargetGroups)
        D.dense_chunk /= 2;
    D.sparse_chunk = kMinSparseChunk;
    while (D.sparse_chunk < kMaxSparseChunk &&
           sgc * chunks(D.union_cap, 2 * D.sparse_chunk) >= kSparseTargetGroups)
        D.sparse_chunk *= 2;
    D.n_chunks_sparse = chunks(D.union_cap, D.sparse_chunk);
    D.n_chunks_dense = D.max_pages > 0 ? chunks(D.max_pages, D.dense_chunk) : 1;
    const float scale = sh->softmax_scale > 0.0f ? sh->softmax_scale
                                                 : 1.0f / sqrtf(static_cast<float>(D.d));
    D.scale_log2 = scale * 1.44269504088896340736f;
    D.page_table = nullptr;
    return D;
}

// Carve the workspace; with base == nullptr only the total size is computed.
// sparse_only: the layout losa_step alone needs (no dense first-step partials).
size_t carve(const Dims &D, char *base, Work *W, bool sparse_only = false) {
    const size_t sT = D.bf16 ? 2 : 4;
    const size_t SG = (size_t)D.S * D.Hk;
    const size_t R1 = D.R > 0 ? D.R : 1;
    const size_t A1 = D.A > 0 ? D.A : 1;
    const size_t part_rows =
        sparse_only ? (size_t)D.n_chunks_sparse * R1
                    : std::max((size_t)D.n_chunks_sparse * R1, (size_t)D.n_chunks_dense * D.Rd);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base ? base + off : nullptr;
        off += align_up(bytes);
        return p;
    };
    Work w;
    w.active = reinterpret_cast<int32_t *>(take((size_t)D.S * D.Hq * A1 * 4));
    w.qrows = take(SG * D.R16 * D.d * sT);
    w.qsel16 = reinterpret_cast<uint32_t *>(take(SG * D.Rs16 * D.d * 4));
    w.qsel32 = reinterpret_cast<float *>(take(SG * R1 * D.d * 8));
    w.qabs = reinterpret_cast<float *>(take(SG * R1 * 4));
    w.hbound = reinterpret_cast<float *>(take(SG * R1 * D.hb_stride * 4));
    w.tmax = reinterpret_cast<float *>(take(SG * R1 * D.n_tiles_grid * 4));
    w.psel = reinterpret_cast<int32_t *>(take(SG * R1 * D.k * 4));
    w.union_cnt = reinterpret_cast<int32_t *>(take(SG * 4));
    w.part_acc = reinterpret_cast<float *>(take(SG * part_rows * D.d * 4));
    w.part_ml = reinterpret_cast<float *>(take(SG * part_rows * 2 * 4));
    w.shloc = reinterpret_cast<float *>(
        take(D.flags & LOSA_FLAG_SHARED_ACTIVE ? (size_t)D.S * D.Hq * D.B * 4 : 0));
    w.blk_o = reinterpret_cast<float *>(take((size_t)D.S * D.Hq * A1 * D.d * 4));
    w.blk_l = reinterpret_cast<float *>(take((size_t)D.S * D.Hq * A1 * 4));
    if (W) *W = w;
    return off;
}

size_t meta_bytes(const Dims &D) {
    // chunk-major min/max, largest |key| per page, page-major min/max
    return 2 * meta_main_bytes(D) + (size_t)D.Hk * D.n_tiles_total * kTile * 4;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LOSA_OK : LOSA_ERR_HIP; }

// Profiling hook: record the caller's stage event i, if any.
hipError_t mark(void **events, int i, hipStream_t s) {
    if (!events || !events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
}

// The prefix cache's layout arguments: kv_off (contiguous sequences) or a page
// table (then kv_off may be null); int32 arrays, 4-byte aligned.
bool layout_ok(const int32_t *kv_off, const int32_t *prefix_len, const int32_t *page_table) {
    if (!prefix_len || !aligned(prefix_len, 4)) return false;
    if (page_table) return aligned(page_table, 4) && (!kv_off || aligned(kv_off, 4));
    return kv_off && aligned(kv_off, 4);
}

// Checks of losa_step's arguments (host only); fills the dims and the debug copy.
int check_step_args(const losa_shape *shape, const void *const (&p16)[10], const int32_t *kv_off,
                    const int32_t *prefix_len, const int32_t *page_table, const float *lp_cache,
                    const losa_debug *debug, Dims *D, losa_debug *dbg) {
    int st = check_shape(shape);
    if (st != LOSA_OK) return st;
    for (const void *p : p16)
        if (!p || !aligned(p, 16)) return LOSA_ERR_INVALID_ARG;
    if (!layout_ok(kv_off, prefix_len, page_table) || !lp_cache || !aligned(lp_cache, 4))
        return LOSA_ERR_INVALID_ARG;
    *D = make_dims(shape);
    D->page_table = page_table;
    memset(dbg, 0, sizeof *dbg);
    if (debug) {
        *dbg = *debug;
        const void *pd[] = {dbg->locality, dbg->active, dbg->page_sel, dbg->union_idx,
                            dbg->union_cnt};
        for (const void *p : pd)
            if (p && !aligned(p, 4)) return LOSA_ERR_INVALID_ARG;
        if (dbg->union_idx && dbg->union_cap < D->union_cap) return LOSA_ERR_INVALID_ARG;
    }
    if (D->R > 0 && select_lds_bytes(*D) > 60 * 1024) return LOSA_ERR_UNSUPPORTED;
    if (D->R > 0 && D->k > kMaxK && D->k < D->max_pages) return LOSA_ERR_UNSUPPORTED;
    return LOSA_OK;
}

// The launches of one LoSA step on an already carved workspace.
hipError_t launch_step(const Dims &D, const void *q_t, const void *q_prev, const void *k_blk,
                       const void *v_blk, const void *k_cache, const void *v_cache,
                       const void *page_meta, const int32_t *kv_off, const int32_t *prefix_len,
                       float *op_cache, float *lp_cache, void *out, const losa_debug &dbg,
                       const Work &W, hipStream_t s) {
    void **ev = dbg.stage_events;
    hipError_t e = mark(ev, 0, s);
    if ((D.flags & LOSA_FLAG_SHARED_ACTIVE) && e == hipSuccess)
        e = launch_shared_locality(D, q_t, q_prev, W, dbg.locality, s);
    if (score_prep_fits(D)) {
        // preparation and page scoring in one kernel (its time shows as scoring)
        if (e == hipSuccess) e = mark(ev, 1, s);
        if (e == hipSuccess)
            e = launch_score_prep(D, q_t, q_prev, page_meta, kv_off, prefix_len, W, dbg.locality,
                                  dbg.active, dbg.union_cnt, s);
    } else {
        if (e == hipSuccess)
            e = launch_prepare(D, false, q_t, q_prev, W, dbg.locality, dbg.active, dbg.union_cnt,
                               s);
        if (e == hipSuccess) e = mark(ev, 1, s);
        if (D.R > 0 && e == hipSuccess) e = launch_score(D, page_meta, kv_off, prefix_len, W, s);
    }
    if (e == hipSuccess) e = mark(ev, 2, s);
    // selection (active rows) and the in-block attention of every token
    const BlockArgs blk{q_t, k_blk, v_blk, op_cache, lp_cache, out};
    if (e == hipSuccess)
        e = launch_select(D, page_meta, kv_off, prefix_len, W, dbg.page_sel, blk, s);
    if (e == hipSuccess) e = mark(ev, 3, s);
    if (D.R > 0 && e == hipSuccess)
        e = launch_prefix(D, false, q_t, k_cache, v_cache, kv_off, prefix_len, W, dbg.union_idx,
                          dbg.union_cnt, dbg.union_cap, s);
    if (e == hipSuccess) e = mark(ev, 4, s);
    if (D.R > 0 && e == hipSuccess) e = launch_finish_active(D, W, op_cache, lp_cache, out, s);
    if (e == hipSuccess) e = mark(ev, 5, s);
    return e;
}

// ---------------------------------------------------------------------------
// Static scratch of losa_step_noalloc, for callers that cannot allocate.  In
// host code `scratch` names a host-side stand-in, never device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[LOSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

hipError_t scratch_of_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char *losa_status_string(int status) {
    switch (status) {
        case LOSA_OK: return "ok";
        case LOSA_ERR_INVALID_ARG: return "invalid argument";
        case LOSA_ERR_UNSUPPORTED: return "unsupported shape";
        case LOSA_ERR_WORKSPACE: return "workspace too small";
        case LOSA_ERR_HIP: return "HIP launch failed";
        case LOSA_ERR_SCRATCH:
            return "shape needs more than the static scratch of losa_step_noalloc";
        default: return "unknown status";
    }
}

size_t losa_page_meta_bytes(const losa_shape *shape) {
    if (check_shape(shape) != LOSA_OK) return 0;
    return meta_bytes(make_dims(shape));
}

size_t losa_workspace_bytes(const losa_shape *shape) {
    if (check_shape(shape) != LOSA_OK) return 0;
    return carve(make_dims(shape), nullptr, nullptr);
}

int32_t losa_union_capacity(const losa_shape *shape) {
    if (check_shape(shape) != LOSA_OK) return -1;
    return make_dims(shape).union_cap;
}

int losa_build_page_meta(const losa_shape *shape, const void *k_cache, const int32_t *kv_off,
                         const int32_t *prefix_len, const int32_t *page_table, void *page_meta,
                         void *stream) {
    int st = check_shape(shape);
    if (st != LOSA_OK) return st;
    if (!k_cache || !page_meta || !layout_ok(kv_off, prefix_len, page_table))
        return LOSA_ERR_INVALID_ARG;
    if (!aligned(k_cache, 16) || !aligned(page_meta, 16)) return LOSA_ERR_INVALID_ARG;
    Dims D = make_dims(shape);
    D.page_table = page_table;
    return hip_status(launch_page_meta(D, k_cache, kv_off, prefix_len, nullptr, 0, page_meta,
                                       static_cast<hipStream_t>(stream)));
}

int losa_update_page_meta(const losa_shape *shape, const void *k_cache, const int32_t *kv_off,
                          const int32_t *prefix_len, const int32_t *page_table,
                          const int32_t *first_token, int32_t max_new_tokens, void *page_meta,
                          void *stream) {
    int st = check_shape(shape);
    if (st != LOSA_OK) return st;
    if (!k_cache || !first_token || !page_meta || !layout_ok(kv_off, prefix_len, page_table))
        return LOSA_ERR_INVALID_ARG;
    if (!aligned(k_cache, 16) || !aligned(page_meta, 16) || !aligned(first_token, 4))
        return LOSA_ERR_INVALID_ARG;
    if (max_new_tokens < 0 || max_new_tokens > shape->max_prefix_len) return LOSA_ERR_INVALID_ARG;
    Dims D = make_dims(shape);
    D.page_table = page_table;
    return hip_status(launch_page_meta(D, k_cache, kv_off, prefix_len, first_token, max_new_tokens,
                                       page_meta, static_cast<hipStream_t>(stream)));
}

int losa_dense_first_step(const losa_shape *shape, const void *q_t, const void *k_blk,
                          const void *v_blk, const void *k_cache, const void *v_cache,
                          const int32_t *kv_off, const int32_t *prefix_len,
                          const int32_t *page_table, float *op_cache, float *lp_cache, void *out,
                          const losa_debug *debug, void *workspace, size_t workspace_bytes,
                          void *stream) {
    int st = check_shape(shape);
    if (st != LOSA_OK) return st;
    const void *p16[] = {q_t, k_blk, v_blk, k_cache, v_cache, op_cache, out, workspace};
    for (const void *p : p16)
        if (!p || !aligned(p, 16)) return LOSA_ERR_INVALID_ARG;
    if (!layout_ok(kv_off, prefix_len, page_table) || !lp_cache || !aligned(lp_cache, 4))
        return LOSA_ERR_INVALID_ARG;
    Dims D = make_dims(shape);
    D.page_table = page_table;
    D.flags = 0;  // the dense first step has no reading variants
    Work W;
    const size_t need = carve(D, static_cast<char *>(workspace), &W);
    if (workspace_bytes < need) return LOSA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void **ev = debug ? debug->stage_events : nullptr;
    hipError_t e = mark(ev, 0, s);
    // (the bf16 dense pass reads its query rows from q_t; fp32 reads stacked rows)
    if (!D.bf16 && e == hipSuccess)
        e = launch_prepare(D, true, q_t, nullptr, W, nullptr, nullptr, nullptr, s);
    if (e == hipSuccess) e = mark(ev, 1, s);
    if (e == hipSuccess) e = mark(ev, 2, s);
    if (e == hipSuccess) e = mark(ev, 3, s);
    if (e == hipSuccess)
        e = launch_prefix(D, true, q_t, k_cache, v_cache, kv_off, prefix_len, W, nullptr, nullptr, 0,
                          s);
    if (e == hipSuccess) e = mark(ev, 4, s);
    if (e == hipSuccess)
        e = launch_finish(D, q_t, k_blk, v_blk, kv_off, prefix_len, W, op_cache, lp_cache, out, s);
    if (e == hipSuccess) e = mark(ev, 5, s);
    return hip_status(e);
}

int losa_step(const losa_shape *shape, const void *q_t, const void *q_prev, const void *k_blk,
              const void *v_blk, const void *k_cache, const void *v_cache, const void *page_meta,
              const int32_t *kv_off, const int32_t *prefix_len, const int32_t *page_table,
              float *op_cache, float *lp_cache, void *out, const losa_debug *debug,
              void *workspace, size_t workspace_bytes, void *stream) {
    const void *const p16[10] = {q_t,      q_prev,   k_blk, v_blk, k_cache,
                                 v_cache,  page_meta, op_cache, out, workspace};
    Dims D;
    losa_debug dbg;
    int st = check_step_args(shape, p16, kv_off, prefix_len, page_table, lp_cache, debug, &D, &dbg);
    if (st != LOSA_OK) return st;
    Work W;
    const size_t need = carve(D, static_cast<char *>(workspace), &W);
    if (workspace_bytes < need) return LOSA_ERR_WORKSPACE;
    return hip_status(launch_step(D, q_t, q_prev, k_blk, v_blk, k_cache, v_cache, page_meta, kv_off,
                                  prefix_len, op_cache, lp_cache, out, dbg, W,
                                  static_cast<hipStream_t>(stream)));
}

int losa_step_noalloc(const losa_shape *shape, const void *q_t, const void *q_prev,
                      const void *k_blk, const void *v_blk, const void *k_cache,
                      const void *v_cache, const void *page_meta, const int32_t *kv_off,
                      const int32_t *prefix_len, const int32_t *page_table, float *op_cache,
                      float *lp_cache, void *out, const losa_debug *debug, void *stream) {
    // (the scratch pointer stands in for the workspace in the pointer checks)
    const void *const p16[10] = {q_t,     q_prev,    k_blk,    v_blk, k_cache,
                                 v_cache, page_meta, op_cache, out,   q_t};
    Dims D;
    losa_debug dbg;
    int st = check_step_args(shape, p16, kv_off, prefix_len, page_table, lp_cache, debug, &D, &dbg);
    if (st != LOSA_OK) return st;
    if (carve(D, nullptr, nullptr, true) > LOSA_NOALLOC_SCRATCH_BYTES) return LOSA_ERR_SCRATCH;
    void *ws = nullptr;
    if (scratch_of_current_device(&ws) != hipSuccess) return LOSA_ERR_HIP;
    Work W;
    carve(D, static_cast<char *>(ws), &W, true);
    return hip_status(launch_step(D, q_t, q_prev, k_blk, v_blk, k_cache, v_cache, page_meta, kv_off,
                                  prefix_len, op_cache, lp_cache, out, dbg, W,
                                  static_cast<hipStream_t>(stream)));
}

}  // extern "C"
