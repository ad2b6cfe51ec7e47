// Internal declarations of liblosa.so: problem dimensions, the carve-up of the
// caller's workspace, kernel launchers and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "losa.h"

namespace losa {

constexpr int kPage = 16;         // tokens per page
constexpr int kTile = 64;         // pages per metadata tile: one page per lane of a wave
constexpr int kMinSparseChunk = 4;   // union pages per prefix workgroup (sparse step): 1 per wave
constexpr int kMaxSparseChunk = 64;  // ... at most (one page per lane of a wave)
constexpr int kMaxBitmapWords = 8192;  // union bitmap in LDS: 262144 pages
constexpr int kMinDenseChunk = 16;  // prefix pages per prefix workgroup (dense first step) ...
constexpr int kMaxDenseChunk = 64;  // ... chosen between these so the grid covers the chip
constexpr int kDenseTargetGroups = 512;   // workgroups a dense pass should have at least
constexpr int kSparseTargetGroups = 1024; // workgroups a sparse pass may keep at most (by capacity)
constexpr int kMaxRows = 256;     // G * B stacked rows per KV head at most
constexpr int kMaxK = 64;         // pages per row the exact selection keeps in one register
constexpr int kMaxMaskRows = 64;  // stacked rows per KV head with per-row page masks (bits)
constexpr int kMaxSharedPrep = 1024;  // query heads x block tokens staged in LDS by the
                                      // folded preparation for a shared active set

// Relative error bound between the MFMA-accumulated page bound and the exact
// fp32 chain (both sides together), and an absolute floor for flushed
// subnormal products: |U_mfma - U_chain| <= kBoundRel * sum_i |q_i| * max|k| + kBoundAbs.
constexpr float kBoundRel = 1.0f / 4096.0f;
constexpr float kBoundAbs = 1.0e-30f;

// Everything a kernel needs to know about the problem, by value.
struct Dims {
    int S, B, Hq, Hk, G, d, A, k;     // k = budget pages per row
    int bf16;                         // 1: bf16 storage, 0: fp32
    int flags;                        // losa_flags of the shape
    int max_pages;                    // pages of the longest prefix
    int hb_stride;                    // row stride of the upper-bound buffer (max_pages, 4-aligned)
    int64_t T;                        // kv_tokens
    int64_t n_tiles_total;            // metadata tiles per KV head over the whole cache
    int64_t meta_main_bytes;          // bytes of the min/max part of the page metadata
    int64_t meta_pm_off;              // byte offset of its page-major copy
    int n_tiles_grid;                 // 64-page groups of the longest sequence (from its first page)
    int union_cap;                    // min(max_pages, G*A*k)
    int R;                            // stacked active rows per KV head = G*A
    int Rs16;                         // R rounded up to 16 (selection MFMA row tiles)
    int Rd;                           // stacked dense rows per KV head = G*B
    int R16;                          // Rd rounded up to 16
    int sparse_chunk, dense_chunk;    // pages per prefix workgroup
    int n_chunks_sparse, n_chunks_dense;
    float scale_log2;                 // softmax scale * log2(e)
    const int32_t *page_table;        // [S][max(max_pages,1)] physical page of each page of a
                                      // sequence, or null: pages contiguous from kv_off[s]
};

// Device views into the workspace (all carved from one caller buffer).
struct Work {
    int32_t *active;     // [S][Hq][max(A,1)]
    void *qrows;         // [S][Hk][R16][d] storage type: stacked query rows (attention)
    uint32_t *qsel16;    // [S][Hk][Rs16][d] bf16 pairs (max(q,0) | min(q,0) << 16): MFMA operand
    float *qsel32;       // [S][Hk][max(R,1)][d][2] fp32 (max(q,0), min(q,0)): exact chain operand
    float *qabs;         // [S][Hk][max(R,1)] upper bound of sum_i |q_i|
    float *hbound;       // [S][Hk][max(R,1)][hb_stride] upper bound of each page's exact bound
    float *tmax;         // [S][Hk][max(R,1)][n_tiles_grid] per page group: max lower bound
    int32_t *psel;       // [S][Hk][max(R,1)][k] each active row's selected pages
    int32_t *union_cnt;  // [S][Hk] union size, written by the sparse prefix kernel
    float *part_acc;     // [S][Hk][n_chunks][rows][d]
    float *part_ml;      // [S][Hk][n_chunks][rows][2] (running max in log2 units, sum)
    float *shloc;        // [S][Hq][B] per-head locality / d (shared active set only)
    float *blk_o;        // [S][Hq][max(A,1)][d] in-block attention output of each active row
    float *blk_l;        // [S][Hq][max(A,1)] its log-normaliser (log2 units)
};

// Launchers (one per translation unit); each returns the hipGetLastError code.
hipError_t launch_page_meta(const Dims &D, const void *k_cache, const int32_t *kv_off,
                            const int32_t *prefix_len, const int32_t *first_token,
                            int max_new_tokens, void *meta, hipStream_t st);
// Per-head locality of every (query head, token) for the shared active set.
hipError_t launch_shared_locality(const Dims &D, const void *q_t, const void *q_prev, const Work &W,
                                  float *dbg_loc, hipStream_t st);
hipError_t launch_prepare(const Dims &D, bool dense, const void *q_t, const void *q_prev,
                          const Work &W, float *dbg_locality, int32_t *dbg_active,
                          int32_t *dbg_union_cnt, hipStream_t st);
hipError_t launch_score(const Dims &D, const void *meta, const int32_t *kv_off,
                        const int32_t *prefix_len, const Work &W, hipStream_t st);
// The sparse step's preparation folded into page scoring (bf16, the group's
// block queries fit in LDS); replaces launch_prepare + launch_score.
constexpr int kPrepVecs = 8;  // 16-byte query vectors per thread in the folded preparation
bool score_prep_fits(const Dims &D);
hipError_t launch_score_prep(const Dims &D, const void *q_t, const void *q_prev, const void *meta,
                             const int32_t *kv_off, const int32_t *prefix_len, const Work &W,
                             float *dbg_loc, int32_t *dbg_act, int32_t *dbg_ucnt, hipStream_t st);
// The step's in-block attention runs in extra one-wave workgroups of the
// selection launch (they need no selection result): stable tokens' outputs are
// final there, active tokens' (o_s, L_s) go to the workspace.
struct BlockArgs {
    const void *q_t, *k_blk, *v_blk;
    const float *op_cache, *lp_cache;
    void *out;
};
hipError_t launch_select(const Dims &D, const void *meta, const int32_t *kv_off,
                         const int32_t *prefix_len, const Work &W, int32_t *dbg_page_sel,
                         const BlockArgs &blk, hipStream_t st);
size_t select_lds_bytes(const Dims &D);  // dynamic LDS of the exact-selection kernel
// Sparse step: the union of the rows' pages is built here (the dbg_union_*
// outputs are optional).
// Dense bf16: the Q operands come straight from q_t (no stacked rows needed).
hipError_t launch_prefix(const Dims &D, bool dense, const void *q_t, const void *k_cache,
                         const void *v_cache, const int32_t *kv_off, const int32_t *prefix_len,
                         const Work &W, int32_t *dbg_union_idx, int32_t *dbg_union_cnt,
                         int dbg_union_cap, hipStream_t st);
// Dense first step: every row's prefix partials, the block attention and the merge.
hipError_t launch_finish(const Dims &D, const void *q_t, const void *k_blk, const void *v_blk,
                         const int32_t *kv_off, const int32_t *prefix_len, const Work &W,
                         float *op_cache, float *lp_cache, void *out, hipStream_t st);
// Sparse step: the active rows' prefix partials merged with their block part.
hipError_t launch_finish_active(const Dims &D, const Work &W, float *op_cache, float *lp_cache,
                                void *out, hipStream_t st);

// ---------------------------------------------------------------------------
// Device helpers.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even bf16 (finite inputs; NaN maps to a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Order-preserving map of an fp32 value to uint32 (-0 treated as +0); 0 is
// below every finite value and serves as "no candidate".
__device__ __forceinline__ uint32_t ord_key(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Values of partner lanes without an LDS round trip: l^1 and l^2 (DPP quad
// permutes), l^7 and l^15 inside each row of 16 lanes (DPP row half-mirror
// and mirror), l^16 and l^32 (v_permlane16_swap / v_permlane32_swap of a
// register with itself: in every lane its two results are the values of the
// lane's pair of rows, or of wave halves, and the partner's is the one that
// is not the lane's own).  In a butterfly over a value already equal across
// lane bits 0-1, l^7 stands for l^4; equal across bits 0-2, l^15 for l^8.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_f32<0xb1>(v); }    // quad_perm [1,0,3,2]
__device__ __forceinline__ float lane_xor2(float v) { return dpp_f32<0x4e>(v); }    // quad_perm [2,3,0,1]
__device__ __forceinline__ float lane_xor7(float v) { return dpp_f32<0x141>(v); }   // row_half_mirror
__device__ __forceinline__ float lane_xor15(float v) { return dpp_f32<0x140>(v); }  // row_mirror
__device__ __forceinline__ float lane_xor16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((__lane_id() & 16) ? a[0] : a[1]);
}
__device__ __forceinline__ float lane_xor32(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((__lane_id() & 32) ? a[0] : a[1]);
}

// Workgroup barrier for LDS exchanges only: this wave's LDS (and scalar)
// operations complete, then s_barrier.  Unlike __syncthreads, whose fences
// also wait for the wave's global stores and loads to complete, it lets
// stores for later kernels stay in flight.  (The memory clobber keeps the
// compiler from moving memory accesses across it.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Sequence geometry with out-of-range values clamped into the cache.
struct SeqGeom {
    int64_t off;        // first cache token (contiguous layout)
    int len;            // prefix tokens
    int pages;          // ceil(len / 16)
    int64_t gp0;        // first global page (contiguous layout)
    int64_t mp0;        // first metadata page of the sequence
    const int32_t *pt;  // the sequence's row of the page table, or null
    int64_t n_phys;     // pages in the cache (page-table entries are clamped below it)
};

// The geometry with the layout fixed at compile time (the hot kernels are
// built for both layouts, so the contiguous layout's code is free of the
// page table), and the runtime choice for the others.
template <bool PAGED>
__device__ __forceinline__ SeqGeom seq_geom_t(const Dims &D, const int32_t *kv_off,
                                              const int32_t *prefix_len, int s) {
    SeqGeom g;
    g.n_phys = D.T / kPage;
    if constexpr (PAGED) {
        int len = prefix_len[s];
        if (len < 0) len = 0;
        if (len > D.max_pages * kPage) len = D.max_pages * kPage;
        g.off = 0;
        g.gp0 = 0;
        g.mp0 = (int64_t)s * (D.max_pages > 0 ? D.max_pages : 1);
        g.pt = D.page_table + (size_t)s * (D.max_pages > 0 ? D.max_pages : 1);
        g.len = len;
    } else {
        int64_t off = kv_off[s];
        int len = prefix_len[s];
        if (off < 0) off = 0;
        off = off / kPage * kPage;
        if (off > D.T) off = D.T;
        if (len < 0) len = 0;
        if (len > D.max_pages * kPage) len = D.max_pages * kPage;
        if (off + len > D.T) len = static_cast<int>(D.T - off);
        g.off = off;
        g.gp0 = off / kPage;
        g.mp0 = g.gp0;
        g.pt = nullptr;
        g.len = len;
    }
    g.pages = (g.len + kPage - 1) / kPage;
    return g;
}

__device__ __forceinline__ SeqGeom seq_geom(const Dims &D, const int32_t *kv_off,
                                            const int32_t *prefix_len, int s) {
    return D.page_table ? seq_geom_t<true>(D, kv_off, prefix_len, s)
                        : seq_geom_t<false>(D, kv_off, prefix_len, s);
}

// Global (physical) page of the sequence's page p: the page-table entry, with
// p clamped into the sequence's pages and the entry into the cache, or the
// contiguous layout's first page + p.  Token t of a page is cache row
// 16 * phys_page + t of every KV head.
__device__ __forceinline__ int64_t phys_page(const SeqGeom &g, int p) {
    if (g.pt) {
        const int64_t e = g.pt[min(max(p, 0), max(g.pages - 1, 0))];
        return e < 0 ? 0 : (e >= g.n_phys ? g.n_phys - 1 : e);
    }
    return g.gp0 + p;
}
// Metadata page of the sequence's page p.  Page metadata is kept per
// (sequence, page): at the page's cache position in the contiguous layout,
// from s * max_pages for sequence s with a page table -- so the metadata of a
// run of a sequence's pages lies side by side in either layout, however the
// table scatters the pages themselves.
__device__ __forceinline__ int64_t meta_page(const SeqGeom &g, int p) { return g.mp0 + p; }

// The same with the layout fixed at compile time (the hot kernels are built
// for both, so the contiguous layout's code carries no page-table branch).
template <bool PAGED>
__device__ __forceinline__ int64_t phys_page_t(const SeqGeom &g, int p) {
    if constexpr (PAGED) {
        const int64_t e = g.pt[min(max(p, 0), max(g.pages - 1, 0))];
        return e < 0 ? 0 : (e >= g.n_phys ? g.n_phys - 1 : e);
    } else {
        return g.gp0 + p;
    }
}

}  // namespace losa
