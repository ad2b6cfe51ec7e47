// QUEST page selection for the active rows only, and the union per KV head.
//
// LoSA applies the sparse selector (QUEST) to the active tokens alone, so the
// union of the pages they select -- the only prefix KV the step reads -- is
// taken over |A| rows instead of B (gist.science pt summary, "3. Metodologia",
// step 3; fr summary, "Calcul Sparse pour les Tokens Actifs" and "Réduction de
// l'Union KV").  Reading used for QUEST: page bound
// U = sum_i max(q_i*min_i, q_i*max_i); each row keeps its k = budget/16 pages
// of largest U, equal bounds going to the lower page.  The bound that decides
// the selection is the fp32 chain over dimensions in ascending order (the
// contract of include/losa.h), reproduced bit for bit in two phases:
//
// Phase 1 (k_score), one wave per (sequence, KV head, 64-page tile): every
// row's bound for every page of the tile with v_mfma_f32_16x16x32_bf16 -- the
// row operand holds bf16 pairs (max(q,0), min(q,0)), the page operand the
// (max, min) metadata pairs, so one k-slot pair adds q*max or q*min.  MFMA
// accumulation order is not the chain's, so each value U' is widened to the
// interval [U' - E, U' + E] with E = 2^-12 * sum|q| * max|k| + 1e-30, which
// contains the exact chain's value (both errors are at most a few hundred
// units of 2^-24 relative to sum|q_i * k_i| <= sum|q| * max|k|).  The upper
// ends go to the workspace, with the largest lower end of every tile.
//
// Phase 2 (k_select), one one-wave workgroup per (sequence, KV head, active
// row): the k-th largest tile maximum of the lower ends is at most the k-th
// largest exact bound, so every page of the exact top-k has an upper end at or
// above it; those candidate pages (typically a little more than k) get the
// exact fp32 chain -- one IEEE fused multiply-add per dimension with max_i or
// min_i chosen by the sign of q_i, the same value as the pair q+ * max then
// q- * min (one of them an exact zero, the products exact for bf16) -- and the
// exact top-k is taken on keys (score bits, page).  Each row's pages go to the
// workspace; the prefix kernel builds their union.  The same launch carries
// one more one-wave workgroup per (sequence, query head, block token) for the
// step's in-block attention (block_attn.h), which needs no selection result.
#include <algorithm>
#include <type_traits>

#include "block_attn.h"
#include "losa_internal.h"

namespace losa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// wave reductions with DPP (row shifts, then row broadcasts 15 and 31)

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_step_max(uint32_t v) {
    return max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                      static_cast<int>(v), static_cast<int>(v), CTRL, ROW_MASK, 0xf, false)));
}

// maximum over the 64 lanes, returned to every lane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_step_max<0x111, 0xf>(v);  // row_shr:1
    v = dpp_step_max<0x112, 0xf>(v);  // row_shr:2
    v = dpp_step_max<0x114, 0xf>(v);  // row_shr:4
    v = dpp_step_max<0x118, 0xf>(v);  // row_shr:8
    v = dpp_step_max<0x142, 0xa>(v);  // row_bcast:15
    v = dpp_step_max<0x143, 0xc>(v);  // row_bcast:31
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// maximum over each row of 16 lanes, valid in the row's last lane (15, 31, 47, 63)
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = dpp_step_max<0x111, 0xf>(v);
    v = dpp_step_max<0x112, 0xf>(v);
    v = dpp_step_max<0x114, 0xf>(v);
    v = dpp_step_max<0x118, 0xf>(v);
    return v;
}

__device__ __forceinline__ float ord_to_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

// Page groups: the pages of a sequence are bounded in groups of 64 counted
// from its first page (group x: pages 64x .. 64x + 63), whatever their place
// in the metadata tiles, so a 64K prefix has exactly 64 groups.  Metadata
// page gp's chunk c (of nch per page) in the tile layout of KV head g, and
// the page's largest |key|; gp is clamped into the metadata.
__device__ __forceinline__ const uint4 *meta_chunk(const uint4 *meta, const Dims &D, int g,
                                                   int64_t gp, int c, int nch) {
    gp = min(gp, D.n_tiles_total * kTile - 1);
    return meta + ((size_t)g * D.n_tiles_total + gp / kTile) * nch * kTile + (size_t)c * kTile +
           gp % kTile;
}
__device__ __forceinline__ float meta_amax(const uint4 *meta, const Dims &D, int g, int64_t gp) {
    gp = min(gp, D.n_tiles_total * kTile - 1);
    return reinterpret_cast<const float *>(reinterpret_cast<const char *>(meta) +
                                           D.meta_main_bytes)[(size_t)g * D.n_tiles_total * kTile + gp];
}

// ---------------------------------------------------------------------------
// Phase 1: bounds of every (row, page) of one tile, as an interval.

// Bounds of row tile rt (rows rt*16 .. +15) against the wave's 64-page tile
// with v_mfma_f32_16x16x32_bf16: aop = the lane's row operand (row rt*16 + l16,
// dims 16*kk + 4*lg .. +3 as (q+, q-) pairs), bop = the page operands (page
// cb*16 + l16, chunk 4*kk + lg), qa = sum |q| bounds of rows rt*16 + 4*lg + j.
// Writes each (row, page) upper end and each row's largest lower end of the tile.
template <int DIM>
__device__ __forceinline__ void bound_rowtile(const Dims &D, int rt, const uint4 (&aop)[DIM / 16],
                                              const float (&qa)[4], const uint4 (&bop)[DIM / 16][4],
                                              const float (&amax)[4], const int (&pl)[4], int pages,
                                              int bx, int l16, int lg, float *hb, float *tm,
                                              bool tile_full) {
    constexpr int KS = DIM / 16;
    const int R = D.R;
    float4_t acc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, aop[kk]), __builtin_bit_cast(bf16x8_t, bop[kk][cb]),
                acc[cb], 0, 0, 0);
    // lane holds rows rt*16 + 4*lg + j of pages cb*16 + l16
    if (tile_full && (rt + 1) * 16 <= R) {
        // every page of the tile and every row of the tile is live (uniform):
        // no per-element guards; the pages of a row are pl[0] + 16*cb (one
        // address per row, constant offsets); the row's maximum lower end as a
        // float, then its order key (monotone, -0 and +0 alike), reduced over
        // the 16 lanes of the row for the 4 rows together
        float *h0 = hb + (size_t)(rt * 16 + 4 * lg) * D.hb_stride + pl[0];
        uint32_t lk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float *hr = h0 + (size_t)j * D.hb_stride;
            const float qe = kBoundRel * qa[j];
            float lm = -__builtin_huge_valf();
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const float e = qe * amax[cb] + kBoundAbs;
                const float u = acc[cb][j];
                hr[16 * cb] = u + e;
                lm = fmaxf(lm, u - e);
            }
            lk[j] = ord_key(lm);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) lk[j] = dpp_step_max<0x111, 0xf>(lk[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) lk[j] = dpp_step_max<0x112, 0xf>(lk[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) lk[j] = dpp_step_max<0x114, 0xf>(lk[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) lk[j] = dpp_step_max<0x118, 0xf>(lk[j]);
        if (l16 == 15) {
            float *t0 = tm + (size_t)(rt * 16 + 4 * lg) * D.n_tiles_grid + bx;
#pragma unroll
            for (int j = 0; j < 4; ++j) t0[(size_t)j * D.n_tiles_grid] = ord_to_f32(lk[j]);
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = rt * 16 + 4 * lg + j;
        const float qa_j = r < R ? qa[j] : 0.0f;
        uint32_t lmax = 0u;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const bool valid = r < R && pl[cb] >= 0 && pl[cb] < pages;
            const float e = kBoundRel * qa_j * amax[cb] + kBoundAbs;
            const float u = acc[cb][j];
            if (valid) {
                hb[(size_t)r * D.hb_stride + pl[cb]] = u + e;
                lmax = max(lmax, ord_key(u - e));
            }
        }
        lmax = row16_max_u32(lmax);
        if (l16 == 15 && r < R) tm[(size_t)r * D.n_tiles_grid + bx] = ord_to_f32(lmax);
    }
}


template <int DIM, bool BF>
__global__ __launch_bounds__(256) void k_score(Dims D, const uint4 *__restrict__ meta,
                                               const int32_t *__restrict__ kv_off,
                                               const int32_t *__restrict__ prefix_len, Work W) {
    constexpr int DPC = BF ? 4 : 2;
    constexpr int NCH = DIM / DPC;
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int bx = (blockIdx.x / ng) * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    if (D.k >= sg.pages) return;  // every page is selected; nothing to score
    const int n_t = (sg.pages + kTile - 1) / kTile;  // page groups of the sequence
    if (bx >= n_t) return;
    const bool tile_full = (bx + 1) * kTile <= sg.pages;
    const int R = D.R, R1 = R > 0 ? R : 1;
    float *hb = W.hbound + (size_t)sgi * R1 * D.hb_stride;
    float *tm = W.tmax + (size_t)sgi * R1 * D.n_tiles_grid;
    const float *qabs = W.qabs + (size_t)sgi * R1;

    if constexpr (BF) {
        const int l16 = lane & 15, lg = lane >> 4;
        float amax[4];
        int pl[4];
        int64_t gpl[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            pl[cb] = bx * kTile + cb * 16 + l16;
            gpl[cb] = meta_page(sg, pl[cb]);
            amax[cb] = meta_amax(meta, D, g, gpl[cb]);
        }
        const uint32_t *q16 = W.qsel16 + (size_t)sgi * D.Rs16 * DIM;
        constexpr int KS = DIM / 16;
        // row operands of row tile rt (row rt*16 + l16, dims 16*kk + 4*lg .. +3 as
        // (q+, q-) pairs) and the sum |q| bounds of the lane's output rows;
        // clamped indexes, masked where used
        uint4 aop[KS];
        float qa[4];
        auto load_rows = [&](int rt) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                aop[kk] = *reinterpret_cast<const uint4 *>(q16 + (size_t)(rt * 16 + l16) * DIM +
                                                           16 * kk + 4 * lg);
#pragma unroll
            for (int j = 0; j < 4; ++j) qa[j] = qabs[min(rt * 16 + 4 * lg + j, R1 - 1)];
        };
        load_rows(0);
        // the whole tile's page operands, requested at once:
        // page cb*16 + l16, metadata chunk 4*kk + lg (dims 16kk + 4lg .. +3)
        uint4 bop[KS][4];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) bop[kk][cb] = *meta_chunk(meta, D, g, gpl[cb], 4 * kk + lg, NCH);
        __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
        const int n_rt = D.Rs16 / 16;
        for (int rt = 0; rt < n_rt; ++rt) {
            float qcur[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) qcur[j] = qa[j];
            uint4 acur[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) acur[kk] = aop[kk];
            if (rt + 1 < n_rt) load_rows(rt + 1);  // in flight during this tile's epilogue
            bound_rowtile<DIM>(D, rt, acur, qcur, bop, amax, pl, sg.pages, bx, l16, lg, hb, tm,
                               tile_full);
        }
    } else {
        // fp32 storage: lane = page, any summation order (the interval absorbs it)
        const int p = bx * kTile + lane;
        const bool valid = p < sg.pages;
        const int64_t gp = meta_page(sg, p);
        const float am = meta_amax(meta, D, g, gp);
        const uint4 *mt = meta_chunk(meta, D, g, gp, 0, NCH);  // chunk c at mt[c * kTile]
        const float *q32 = W.qsel32 + (size_t)sgi * R1 * DIM * 2;
        for (int r = 0; r < R; ++r) {
            float u = 0.0f;
            const float *q = q32 + (size_t)r * DIM * 2;
#pragma unroll 4
            for (int c = 0; c < NCH; ++c) {
                const uint4 m4 = mt[(size_t)c * kTile];
                u = fmaf(q[4 * c + 0], __uint_as_float(m4.x), u);
                u = fmaf(q[4 * c + 1], __uint_as_float(m4.y), u);
                u = fmaf(q[4 * c + 2], __uint_as_float(m4.z), u);
                u = fmaf(q[4 * c + 3], __uint_as_float(m4.w), u);
            }
            const float e = kBoundRel * qabs[r] * am + kBoundAbs;
            if (valid) hb[(size_t)r * D.hb_stride + p] = u + e;
            const uint32_t lmax = wave_max_u32(valid ? ord_key(u - e) : 0u);
            if (lane == 0) tm[(size_t)r * D.n_tiles_grid + bx] = ord_to_f32(lmax);
        }
    }
}

// ---------------------------------------------------------------------------
// Phase 1 with the step's preparation folded in (bf16, the group's block
// queries fit in LDS).  One workgroup per (sequence, KV head) and TPW
// consecutive 64-page tiles, four waves per tile, each wave bounding 16 pages,
// so the metadata stream is spread over the whole chip.  Every workgroup of a
// (sequence, KV head) repeats the preparation from the same inputs -- locality
// chain, active set, stacked rows -- so all of them agree, and builds its MFMA
// row operands from LDS; the workgroup of the first tiles also writes the
// active list and the stacked rows for the later kernels and resets the union
// size.  The locality chain is the one of prepare.hip: each rounded square
// added in ascending dimension order.  Each thread holds matching 16-byte
// vectors of both steps, so all threads compute the rounded squares (into
// LDS), and one thread per row adds them.  The query rows reuse the squares'
// LDS once the chains are done.  Barriers wait for LDS traffic only, so the
// bounds' stores stay in flight.

constexpr int kPrepPad = 4;  // words of padding per LDS row (bank spread)
#ifndef LOSA_SCORE_TPW
#define LOSA_SCORE_TPW 2
#endif
constexpr int kScoreTilesPerGroup = LOSA_SCORE_TPW;  // 64-page tiles per scoring workgroup

template <int DIM, bool SHARED, int TPW, bool PAGED>
__global__ __launch_bounds__(256 * TPW) void k_score_prep(Dims D, const uint16_t *__restrict__ q_t,
                                                          const uint16_t *__restrict__ q_prev,
                                                          const uint4 *__restrict__ meta,
                                                          const int32_t *__restrict__ kv_off,
                                                          const int32_t *__restrict__ prefix_len,
                                                          Work W, float *__restrict__ dbg_loc,
                                                          int32_t *__restrict__ dbg_act,
                                                          int32_t *__restrict__ dbg_ucnt) {
    constexpr int NT = 256 * TPW;            // threads
    constexpr int KS = DIM / 16, NCH = DIM / 4;
    constexpr int RWS = DIM + kPrepPad;      // words per LDS row of squares
    constexpr int VPR = DIM / 8;             // 16-byte vectors per row
    constexpr int NV = kPrepVecs / 2 / TPW;  // vectors per thread and step
    constexpr int OPS = DIM / 4 + 1;         // 16-byte chunks per LDS operand row (one of padding)
    extern __shared__ uint32_t qsm[];        // [G*B][RWS] fp32 squares, then [Rs16][OPS] operand rows
    // localities as rank keys: the fp32 bits (localities are >= +0, so their
    // bits order as the values) above ~token, so that "greater key" is
    // "larger locality, or equal and earlier token"
    __shared__ uint64_t ek_s[kMaxRows];
    __shared__ int sel_s[kMaxRows];
    __shared__ int act_s[kMaxRows];
    __shared__ int rmap_s[kMaxRows];         // query row j*B + t: its stacked row, or -1
    __shared__ float qabs_s[kMaxRows];
    __shared__ uint32_t tmk_s[4 * TPW][16];   // per wave and row of a row tile: lower-end maxima
    __shared__ float shl_s[SHARED ? kMaxSharedPrep : 1];  // per-head localities [Hq][B]
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng, bx = blockIdx.x / ng;  // tiles TPW*bx .. of the sequence
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = TPW * bx + w / 4;  // the wave's tile, counted in the sequence
    const int G = D.G, B = D.B, A = D.A, GB = G * B, R = D.R, Hq = D.Hq;
    const bool writer = bx == 0;

    // 1. the group's query rows of both steps (clamped 16-byte vectors; a thread
    //    holds the same vectors of q_t and q_prev)
    const int nvec = GB * VPR;
    static_assert(NV * 2 * TPW == kPrepVecs, "vectors per thread");
    auto qaddr = [&](const uint16_t *base, int i) {
        const int v = min(tid + NT * i, nvec - 1);
        const int row = v / VPR, c = v % VPR;
        return reinterpret_cast<const uint4 *>(
            base + ((size_t)(s * B + row % B) * Hq + g * G + row / B) * DIM + c * 8);
    };
    uint4 qa_v[NV], qb_v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) qa_v[i] = *qaddr(q_t, i);
    if constexpr (!SHARED) {
#pragma unroll
        for (int i = 0; i < NV; ++i) qb_v[i] = *qaddr(q_prev, i);
    }
    // shared active set: the sequence's per-head localities (clamped reads)
    constexpr int kShl = SHARED ? (kMaxSharedPrep + NT - 1) / NT : 1;
    float shl[kShl];
    if constexpr (SHARED) {
        const float *e = W.shloc + (size_t)s * Hq * B;
#pragma unroll
        for (int i = 0; i < kShl; ++i) shl[i] = e[min(tid + NT * i, Hq * B - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);  // the query vectors are requested first
    // 2. the metadata of the wave's 16 pages: chunk 4*kk + lg of page
    //    16*(w%4) + l16 of the wave's page group (clamped into the metadata
    //    where the sequence has no such page, so that no load sits in a branch)
    const SeqGeom sg = seq_geom_t<PAGED>(D, kv_off, prefix_len, s);
    const int n_t = (sg.pages + kTile - 1) / kTile;       // page groups of the sequence
    const bool wg_ok = D.k < sg.pages && TPW * bx < n_t;  // uniform over the workgroup
    const bool wave_ok = D.k < sg.pages && wt < n_t;      // uniform over the wave
    const bool tile_full = (wt + 1) * kTile <= sg.pages;   // every page of the group is live
    const int R1 = R > 0 ? R : 1;
    const int l16 = lane & 15, lg = lane >> 4;
    const int pl = wt * kTile + 16 * (w % 4) + l16;  // the lane's page in the sequence
    uint4 bop[KS];
    const int64_t gpl = meta_page(sg, pl);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) bop[kk] = *meta_chunk(meta, D, g, gpl, 4 * kk + lg, NCH);
    const float amax = meta_amax(meta, D, g, gpl);
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
    if constexpr (SHARED) {
#pragma unroll
        for (int i = 0; i < kShl; ++i)
            if (tid + NT * i < kMaxSharedPrep) shl_s[tid + NT * i] = shl[i];
    } else {
        // rounded squares of the change, dimensions c*8 .. c*8+7 of a row
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = min(tid + NT * i, nvec - 1);
            const uint32_t aw[4] = {qa_v[i].x, qa_v[i].y, qa_v[i].z, qa_v[i].w};
            const uint32_t bw[4] = {qb_v[i].x, qb_v[i].y, qb_v[i].z, qb_v[i].w};
            float sv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d0 = bf16_lo(aw[e]) - bf16_lo(bw[e]);
                sv[2 * e] = d0 * d0;
                const float d1 = bf16_hi(aw[e]) - bf16_hi(bw[e]);
                sv[2 * e + 1] = d1 * d1;
            }
            float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(qsm) +
                                                     (v / VPR) * RWS + (v % VPR) * 8);
            dst[0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
            dst[1] = make_float4(sv[4], sv[5], sv[6], sv[7]);
        }
    }
    lds_barrier();

    // 3. locality chain per (query head, token), then the active set; with a
    //    shared active set, the sum of the per-head localities over the query
    //    heads in ascending order, then one set for all of the group's heads
    if constexpr (SHARED) {
        if (tid < B) {
            float acc = 0.0f;
            for (int h = 0; h < Hq; ++h) acc = acc + shl_s[h * B + tid];
            ek_s[tid] = (static_cast<uint64_t>(__float_as_uint(acc)) << 32) | static_cast<uint32_t>(~tid);
        }
        lds_barrier();
        if (tid < B) {
            const uint64_t kt = ek_s[tid];
            int rank = 0;
            for (int u = 0; u < B; ++u) rank += ek_s[u] > kt;
            sel_s[tid] = rank < A;
        }
        lds_barrier();
        if (tid < B) {
            int pos = 0;
            for (int u = 0; u < tid; ++u) pos += sel_s[u];
            for (int j = 0; j < G; ++j) {
                if (sel_s[tid]) act_s[j * A + pos] = tid;
                rmap_s[j * B + tid] = sel_s[tid] ? j * A + pos : -1;
            }
        }
    } else {
        if (tid < GB) {
            const float4 *sr = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(qsm) +
                                                                tid * RWS);
            float acc = 0.0f;
            // 16-byte reads in batches of RB, the next batch requested before
            // the adds of this one
            constexpr int RB = 8, NB = DIM / 4 / RB;
            float4 x[2][RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) x[0][i] = sr[i];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b + 1 < NB) {
#pragma unroll
                    for (int i = 0; i < RB; ++i) x[(b + 1) & 1][i] = sr[(b + 1) * RB + i];
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    acc = acc + x[b & 1][i].x;
                    acc = acc + x[b & 1][i].y;
                    acc = acc + x[b & 1][i].z;
                    acc = acc + x[b & 1][i].w;
                }
            }
            ek_s[tid] = (static_cast<uint64_t>(__float_as_uint(acc)) << 32) |
                        static_cast<uint32_t>(~(tid % B));
            if (writer && dbg_loc)
                dbg_loc[((size_t)s * Hq + g * G + tid / B) * B + tid % B] = acc / static_cast<float>(DIM);
        }
        lds_barrier();
        // rank inside the row's head (score desc, token asc); the |A| best are
        // active, listed in ascending token order
        const int j = tid / B, t = tid % B;
        bool sel = false;
        if (tid < GB) {
            const uint64_t kt = ek_s[tid];
            int rank = 0;
#pragma unroll 16
            for (int u = 0; u < B; ++u) rank += ek_s[j * B + u] > kt;
            sel = rank < A;
        }
        int pos = 0;
        if (64 % B == 0) {
            // a head's B rows are B consecutive lanes of one wave: the position
            // is the count of selected lanes of the head below this one
            const uint64_t bal = __ballot(sel);
            const uint64_t below = (1ull << lane) - 1ull, before_head = (1ull << (lane - t)) - 1ull;
            pos = __popcll(bal & below & ~before_head);
        } else {
            if (tid < GB) sel_s[tid] = sel;
            lds_barrier();
            if (sel)
                for (int u = 0; u < t; ++u) pos += sel_s[j * B + u];
        }
        if (sel) act_s[j * A + pos] = t;
        if (tid < GB) rmap_s[tid] = sel ? j * A + pos : -1;
    }
    lds_barrier();  // the squares have been read: their LDS takes the operand rows
    // 4. the stacked rows' MFMA operands, built once for all waves: the (q+, q-)
    //    pairs of dims 4c .. 4c+3 as 16-byte chunk c of row r (a bf16 value goes
    //    to the low half of its word when its sign bit is clear, else to the
    //    high half, so -0 sits in the q- slot: a zero product either way), from
    //    the query vectors each thread still holds (the writer stores the rows
    //    themselves, bf16, for the later kernels at its end)
    uint4 *opb = reinterpret_cast<uint4 *>(qsm);  // [Rs16][OPS]
    uint16_t *qr = static_cast<uint16_t *>(W.qrows) + (size_t)sgi * D.R16 * DIM;
    auto split = [](uint32_t x) {
        const uint32_t ml = static_cast<uint32_t>(static_cast<int32_t>(x << 16) >> 31);  // sign of low
        const uint32_t mh = static_cast<uint32_t>(static_cast<int32_t>(x) >> 31);        // sign of high
        return make_uint2(__builtin_amdgcn_perm(x, x, (ml & 0x01000c0cu) | (~ml & 0x0c0c0100u)),
                          __builtin_amdgcn_perm(x, x, (mh & 0x03020c0cu) | (~mh & 0x0c0c0302u)));
    };
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int v = tid + NT * i;
        const int r = v < nvec ? rmap_s[v / VPR] : -1;
        if (r >= 0) {
            const int c = v % VPR;  // dims 8c .. 8c+7: operand chunks 2c, 2c+1
            const uint2 a = split(qa_v[i].x), b = split(qa_v[i].y);
            const uint2 c2 = split(qa_v[i].z), d2 = split(qa_v[i].w);
            opb[r * OPS + 2 * c] = make_uint4(a.x, a.y, b.x, b.y);
            opb[r * OPS + 2 * c + 1] = make_uint4(c2.x, c2.y, d2.x, d2.y);
        }
    }
    // padding rows of the last row tile: zero operands (their bounds are not stored)
    for (int i = tid; i < (D.Rs16 - R) * (DIM / 4); i += NT)
        opb[(R + i / (DIM / 4)) * OPS + i % (DIM / 4)] = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();

    // sum |q| bounds of the stacked rows: 16 lanes per row, each summing DIM/16
    // values; any order (an upper bound with 1/256 of margin); a row's (q+, q-)
    // pairs hold each value once and a zero
    for (int r0 = 0; r0 < R; r0 += NT / 16) {
        const int r = r0 + tid / 16, part = tid % 16;
        float ab = 0.0f;
        if (r < R) {
            const uint32_t *a = reinterpret_cast<const uint32_t *>(&opb[r * OPS]) + part * (DIM / 16);
#pragma unroll
            for (int w2 = 0; w2 < DIM / 16; ++w2) ab += fabsf(bf16_lo(a[w2])) + fabsf(bf16_hi(a[w2]));
        }
        ab += lane_xor1(ab);  // then l^2, l^4, l^8: the row's sum in each of its lanes
        ab += lane_xor2(ab);
        ab += lane_xor7(ab);
        ab += lane_xor15(ab);
        if (r < R && part == 0) qabs_s[r] = ab * (1.0f + 1.0f / 256.0f);
    }
    lds_barrier();
    // The writer's stores for the later kernels -- the active list, the sum |q|
    // bounds, the stacked rows with their zero padding and a zero union count,
    // which the sparse prefix kernel overwrites -- go out after the bounds (or
    // before an early return): a wait for the metadata would wait for them too.
    auto writer_stores = [&]() {
        if (!writer) return;
        if (tid == 0) {
            W.union_cnt[sgi] = 0;
            if (dbg_ucnt) dbg_ucnt[sgi] = 0;
        }
        int32_t *act = W.active + ((size_t)s * Hq + g * G) * A;  // [G][A], rows j*A + a
        for (int i = tid; i < R; i += NT) {
            act[i] = act_s[i];
            W.qabs[(size_t)sgi * R1 + i] = qabs_s[i];  // for the selection's short-sequence threshold
            if (dbg_act) dbg_act[((size_t)s * Hq + g * G) * A + i] = act_s[i];
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + NT * i;
            const int r = v < nvec ? rmap_s[v / VPR] : -1;
            if (r >= 0) *reinterpret_cast<uint4 *>(qr + (size_t)r * DIM + (v % VPR) * 8) = qa_v[i];
        }
        for (int i = tid; i < (D.Rs16 - R) * VPR; i += NT)
            *reinterpret_cast<uint4 *>(qr + (size_t)(R + i / VPR) * DIM + (i % VPR) * 8) =
                make_uint4(0u, 0u, 0u, 0u);
    };
    if (!wg_ok) {
        writer_stores();
        return;
    }

    // 5. the wave's 16 pages, row tile by row tile: each (row, page) upper end,
    //    and each row's largest lower end over each tile's 64 pages (the four
    //    waves' maxima meet in LDS); waves past the sequence's tiles store nothing
    float *hb = W.hbound + (size_t)sgi * R1 * D.hb_stride;
    float *tm = W.tmax + (size_t)sgi * R1 * D.n_tiles_grid;
    const bool page_ok = wave_ok && pl < sg.pages;
    for (int rt = 0; rt < D.Rs16 / 16; ++rt) {
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, opb[(rt * 16 + l16) * OPS + 4 * kk + lg]),
                __builtin_bit_cast(bf16x8_t, bop[kk]), acc, 0, 0, 0);
        // lane holds rows rt*16 + 4*lg + j of page pl
        uint32_t lk[4];
        if (tile_full && (rt + 1) * 16 <= R) {
            // every page of the tile and every row of the tile is live (uniform
            // over the wave): no per-element guards
            float *hr = hb + (size_t)(rt * 16 + 4 * lg) * D.hb_stride + pl;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e = kBoundRel * qabs_s[rt * 16 + 4 * lg + j] * amax + kBoundAbs;
                hr[(size_t)j * D.hb_stride] = acc[j] + e;
                lk[j] = ord_key(acc[j] - e);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = rt * 16 + 4 * lg + j;
                const float e = kBoundRel * qabs_s[min(r, R1 - 1)] * amax + kBoundAbs;
                lk[j] = 0u;
                if (r < R && page_ok) {
                    hb[(size_t)r * D.hb_stride + pl] = acc[j] + e;
                    lk[j] = ord_key(acc[j] - e);
                }
            }
        }
        // the rows' maxima over the wave's 16 pages (lanes 16*lg + 15), then over
        // each tile's four waves
#pragma unroll
        for (int j = 0; j < 4; ++j) lk[j] = row16_max_u32(lk[j]);
        if (l16 == 15) {
#pragma unroll
            for (int j = 0; j < 4; ++j) tmk_s[w][4 * lg + j] = lk[j];
        }
        lds_barrier();
        if (tid < 16 * TPW) {
            const int tt = tid / 16, rr = rt * 16 + tid % 16;  // the tile of the workgroup, the row
            if (rr < R && TPW * bx + tt < n_t) {
                const uint32_t m = max(max(tmk_s[4 * tt][tid % 16], tmk_s[4 * tt + 1][tid % 16]),
                                       max(tmk_s[4 * tt + 2][tid % 16], tmk_s[4 * tt + 3][tid % 16]));
                tm[(size_t)rr * D.n_tiles_grid + TPW * bx + tt] = ord_to_f32(m);
            }
        }
        lds_barrier();  // tmk_s is rewritten by the next row tile
    }
    writer_stores();
}

// ---------------------------------------------------------------------------
// Phase 2: exact top-k per row over the candidates.

struct SelectDbg {
    int32_t *page_sel;   // [S][Hq][A][k]
};

// The selection workgroup is one wave: its LDS writes are seen by its later
// LDS reads once they have completed, so it needs the wait and no s_barrier
// (which is not free even for a lone wave).
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The exact chain for metadata page gp (contract of include/losa.h), computed
// by a group of LPC consecutive lanes: lane j of the group loads chunks
// j*NCH/LPC .. of the page's metadata (from the page-major copy) before the
// chain starts, and the chain runs through the group in LPC phases -- in phase
// p lane p carries on from lane p-1's value (a quad permute) over its own
// chunks -- so the group's last lane ends with the one ascending chain, while
// each lane holds only 1/LPC of the page.  bf16: qw holds the row's query
// values as fp32 (DIM words), then per dimension the byte selector that turns
// the metadata word (max | min << 16) into the fp32 bits of max_i (q >= 0, -0
// included) or of min_i (q < 0); per dimension one fused multiply-add with
// that value -- the same value as the pair q+ * max then q- * min, whose
// other product is an exact zero.  fp32: qw holds (max(q,0), min(q,0)) per
// dimension, each product rounded, then added.
constexpr uint32_t kSelMax = 0x01000c0cu;  // v_perm_b32: bytes 1,0 of the word to 3,2; zeros below
constexpr uint32_t kSelMin = 0x03020c0cu;  // bytes 3,2 to 3,2; zeros below
template <bool BF>
constexpr int chain_lanes() { return BF ? 2 : 4; }  // 16 chunks (64 VGPRs) per lane at d = 128
constexpr int kPendRing = 128;  // candidate pages waiting for their chains (a ring in LDS)

template <int DIM, bool BF>
__device__ __forceinline__ float exact_bound(const uint4 *meta, const Dims &D, int g, int64_t gp,
                                             const uint32_t *qw, int lane) {
    constexpr int DPC = BF ? 4 : 2;  // dimensions per 16-byte chunk
    constexpr int NCH = DIM / DPC;
    constexpr int LPC = chain_lanes<BF>();
    constexpr int NQ = NCH / LPC;    // chunks per lane
    const int j = lane % LPC;
    const uint4 *m =
        reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(meta) + D.meta_pm_off) +
        ((size_t)g * D.n_tiles_total * kTile + gp) * NCH + j * NQ;
    uint4 mv[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) mv[c] = m[c];
    float acc = 0.0f;
#pragma unroll 1
    for (int ph = 0; ph < LPC; ++ph) {
        // lane j of each quad takes lane j-1's value (lane 0 its own): in
        // phase ph the value of lane ph is the chain up to its chunks
        if (ph > 0) acc = dpp_f32<0x90>(acc);  // quad_perm [0,0,1,2]
        int cq = j * NQ;                // the lane's first chunk, opaque to the
        asm volatile("" : "+v"(cq));   // compiler so that the query reads stay in the loop
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const uint4 m4 = mv[c];
            const int cc = cq + c;
            if constexpr (BF) {
                const float4 q4 = *reinterpret_cast<const float4 *>(qw + 4 * cc);
                const uint4 sl = *reinterpret_cast<const uint4 *>(qw + DIM + 4 * cc);
                const float qd[4] = {q4.x, q4.y, q4.z, q4.w};
                const uint32_t wd[4] = {m4.x, m4.y, m4.z, m4.w}, sd[4] = {sl.x, sl.y, sl.z, sl.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_fmaf(qd[e], __uint_as_float(__builtin_amdgcn_perm(0u, wd[e], sd[e])),
                                         acc);
            } else {
                const float4 q4 = *reinterpret_cast<const float4 *>(qw + 4 * cc);
                const float p0 = q4.x * __uint_as_float(m4.x);
                acc = acc + p0;
                const float p1 = q4.y * __uint_as_float(m4.y);
                acc = acc + p1;
                const float p2 = q4.z * __uint_as_float(m4.z);
                acc = acc + p2;
                const float p3 = q4.w * __uint_as_float(m4.w);
                acc = acc + p3;
            }
        }
    }
    return acc;
}

// MAXB: the block-size bound of the in-block attention workgroups (16, 32 or
// 64), a template parameter so that the larger blocks' registers do not lower
// the occupancy of launches with small blocks.
template <int DIM, bool BF, int MAXB, bool PAGED>
__global__ __launch_bounds__(64) void k_select(Dims D, const uint4 *__restrict__ meta,
                                               const int32_t *__restrict__ kv_off,
                                               const int32_t *__restrict__ prefix_len, Work W,
                                               const void *__restrict__ qrows,
                                               const float *__restrict__ qsel32,
                                               const float *__restrict__ hbound,
                                               const float *__restrict__ tmax, SelectDbg dbg,
                                               BlockArgs blk) {
    extern __shared__ uint32_t smem[];
    const int ng = D.S * D.Hk;
    if (blockIdx.x >= ng * D.R) {
        // in-block attention of kBlockTPW tokens: workgroup ng*R + u*ng +
        // (s*Hk + g) for tokens kBlockTPW*(u % ntg) .. of head g*G + u / ntg, so
        // that a group's tokens run on the XCD of its selection and prefix
        // workgroups (ng a multiple of 8)
        using T = typename std::conditional<BF, uint16_t, float>::type;
        const int ntg = (D.B + kBlockTPW - 1) / kBlockTPW;
        const int b = blockIdx.x - ng * D.R;
        const int sg2 = b % ng, u = b / ng;
        const int t = (u % ntg) * kBlockTPW, s = sg2 / D.Hk, h = (sg2 % D.Hk) * D.G + u / ntg;
        const T *q = static_cast<const T *>(blk.q_t), *kb = static_cast<const T *>(blk.k_blk),
                *vb = static_cast<const T *>(blk.v_blk);
        T *o = static_cast<T *>(blk.out);
        block_token<T, DIM, MAXB>(D, q, kb, vb, W, blk.op_cache, blk.lp_cache, o, smem, s, h, t);
        return;
    }
    const int sgi = blockIdx.x % ng;
    const int r = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int lane = threadIdx.x;
    const int R = D.R, R1 = R > 0 ? R : 1, k = D.k;
    const int h = g * D.G + r / D.A, a = r % D.A;
    uint64_t *mk = reinterpret_cast<uint64_t *>(smem);  // [128] keys being merged
    uint32_t *qw = smem + 256;                           // [2*DIM] the row's chain operands
    int32_t *pend = reinterpret_cast<int32_t *>(smem + 256 + 2 * DIM);  // [kPendRing] candidate pages
    int32_t *psel = W.psel + ((size_t)sgi * R1 + r) * k;
    const float *tm = tmax + ((size_t)sgi * R1 + r) * D.n_tiles_grid;
    const float *hb = hbound + ((size_t)sgi * R1 + r) * D.hb_stride;
    // Requested together, before the sequence's geometry is read (the
    // addresses need only the grid's shape, so no load waits for it): the
    // row's chain operands, the tile maxima of the first 256 tiles and the
    // first 4096 upper ends.  Indexes are clamped into the buffers; entries
    // past the sequence's pages are masked where the values are used, and a
    // row whose budget covers every page does not use them.
    constexpr int QPL = BF ? DIM / 128 : 2 * DIM / 64;  // operand words per lane (0: half a wave)
    uint32_t qv[QPL > 0 ? QPL : 1];
    if constexpr (BF) {
        const uint32_t *qg = reinterpret_cast<const uint32_t *>(
            static_cast<const uint16_t *>(qrows) + ((size_t)sgi * D.R16 + r) * DIM);
        qv[0] = qg[lane % (DIM / 2)];
    } else {
        const float *qg = qsel32 + ((size_t)sgi * R1 + r) * DIM * 2;
#pragma unroll
        for (int i = 0; i < QPL; ++i) qv[i] = __float_as_uint(qg[lane + 64 * i]);
    }
    constexpr int TMR = 4;
    float tmv[TMR];
#pragma unroll
    for (int i = 0; i < TMR; ++i) tmv[i] = tm[min(lane + 64 * i, D.n_tiles_grid - 1)];
    // upper ends of pages base + 256*jj + 4*lane + e, jj < 16, e < 4
    // (the lane's offset is recomputed per call, opaque to the compiler:
    // else the 16 offsets stay in registers through the whole selection)
    auto load_h = [&](int base, float4 (&hv)[16]) {
        int o = base + 4 * lane;
        asm volatile("" : "+v"(o));
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
            hv[jj] = *reinterpret_cast<const float4 *>(hb + min(o + 256 * jj, D.hb_stride - 4));
    };
    float4 hv0[16];
    load_h(0, hv0);
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
    const SeqGeom sg = seq_geom_t<PAGED>(D, kv_off, prefix_len, s);
    const bool all_pages = k >= sg.pages;

    if (all_pages) {
        // (the values loaded above are used on this path too, so that the
        // compiler does not move their loads into the other path, behind the
        // read of the sequence's geometry)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) asm volatile("" ::"v"(hv0[jj].x));
#pragma unroll
        for (int i = 0; i < TMR; ++i) asm volatile("" ::"v"(tmv[i]));
#pragma unroll
        for (int i = 0; i < (QPL > 0 ? QPL : 1); ++i) asm volatile("" ::"v"(qv[i]));
        if (dbg.page_sel)
            for (int e = lane; e < k; e += 64)
                dbg.page_sel[(((size_t)s * D.Hq + h) * D.A + a) * k + e] = e < sg.pages ? e : -1;
    } else {
        const int n_t = (sg.pages + kTile - 1) / kTile;  // page groups of the sequence
        if constexpr (BF) {
            // every lane stores (lanes past DIM/2 repeat a word with its own value),
            // so that the query word's load is not sunk into a branch
            const int wl = lane % (DIM / 2);
            const float q0 = bf16_lo(qv[0]), q1 = bf16_hi(qv[0]);
            *reinterpret_cast<float2 *>(qw + 2 * wl) = make_float2(q0, q1);
            *reinterpret_cast<uint2 *>(qw + DIM + 2 * wl) =
                make_uint2(q0 >= 0.0f ? kSelMax : kSelMin, q1 >= 0.0f ? kSelMax : kSelMin);
        } else {
#pragma unroll
            for (int i = 0; i < QPL; ++i) qw[lane + 64 * i] = qv[i];
        }
        // 1. threshold: each lane's maximum over its tiles (lane, lane + 64, ...)
        // of the lower ends; the k-th largest of these 64 values is reached by
        // k distinct pages, so it is at most the k-th largest exact bound.
        uint32_t gm = 0u;
#pragma unroll
        for (int i = 0; i < TMR; ++i)
            if (lane + 64 * i < n_t) gm = max(gm, ord_key(tmv[i]));
        for (int x = lane + 64 * TMR; x < n_t; x += 64) gm = max(gm, ord_key(tm[x]));
        // Any lower value serves as well (more candidates, the same result):
        // the threshold is the largest key with 16 low zero bits that at least
        // k lanes reach, found bit by bit with ballots -- the k-th largest key
        // with its low 16 bits cleared (within 2^-7 of it as a float).
        // A sequence with fewer tiles than k (fewer than 4096 pages, so every
        // page is in the first batch) takes each lane's maximum over its pages
        // of a lower end formed from the upper end: u + e rounded is hx, so u - e
        // >= hx - 2e - (|hx| + 2e) * 2^-21 whatever the roundings, with e the
        // scoring kernel's bound recomputed from the same operands (the row's
        // sum |q| and the page's max |k|).  Each lane's maximum is reached by a
        // page of its own, so the k-th largest of them is again a valid
        // threshold.  (Lanes without pages keep key 0.)
        const bool short_seq = min(n_t, 64) < k && sg.pages >= 4 * k;  // uniform
        if (short_seq) {
            const float qa = W.qabs[(size_t)sgi * R1 + r];
            float lmax = -__builtin_huge_valf();
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                if (256 * jj < sg.pages) {  // uniform
                    const float hx[4] = {hv0[jj].x, hv0[jj].y, hv0[jj].z, hv0[jj].w};
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const int p = 256 * jj + 4 * lane + e4;
                        const float e =
                            kBoundRel * qa * meta_amax(meta, D, g, meta_page(sg, min(p, sg.pages - 1))) + kBoundAbs;
                        const float lo = (hx[e4] - 2.0f * e) - (fabsf(hx[e4]) + 2.0f * e) * (1.0f / 2097152.0f);
                        if (p < sg.pages) lmax = fmaxf(lmax, lo);
                    }
                }
            }
            gm = lmax == -__builtin_huge_valf() ? 0u : ord_key(lmax);
        }
        uint32_t lam = 0u;  // below every finite key: all pages qualify
        if (min(n_t, 64) >= k || short_seq) {
#pragma unroll
            for (int b = 31; b >= 16; --b) {
                const uint32_t c = lam | (1u << b);
                if (__popcll(__ballot(gm >= c)) >= k) lam = c;
            }
        }
        wave_lds_fence();  // qw visible to the chains
        // 2. candidates: upper end >= threshold; exact chains, CPP at a time
        uint64_t lst = 0ull;  // lane e < k: e-th best (score key << 32 | ~page)
        // the threshold as a float: ord_key preserves the order of floats (-0
        // and +0 alike), so ord_key(x) >= lam is x >= lamf; key 0 (every page
        // qualifies) is below every finite value
        const float lamf = lam == 0u ? -__builtin_huge_valf() : ord_to_f32(lam);
        // Exact chains of the pending pages c0 .. c0 + n - 1 of the ring, n <=
        // CPP, one per group of LPC lanes (candidate i on lanes LPC*i ..; its
        // value on the group's last lane), merged into the list: a key's rank
        // is the number of greater keys among the chains' and the list's
        // (lanes < nlst), read lane by lane into scalar registers (keys are
        // distinct: one per page); the key of rank e < k goes to lane e
        // through LDS.
        constexpr int LPC = chain_lanes<BF>(), CPP = 64 / LPC;
        auto chains = [&](int c0, int n) {
            const int pc = pend[(c0 + min(lane / LPC, n - 1)) & (kPendRing - 1)];
            // (lanes past the groups stay idle: a load's cost grows with its active lanes)
            float u = 0.0f;
            if (lane < LPC * n)
                u = exact_bound<DIM, BF>(meta, D, g, meta_page(sg, pc), qw, lane);
            const bool mine = lane % LPC == LPC - 1 && lane / LPC < n;
            const uint64_t cand = mine ? (static_cast<uint64_t>(ord_key(u)) << 32) |
                                             static_cast<uint32_t>(~static_cast<uint32_t>(pc))
                                       : 0ull;
            const int nlst = __popcll(__ballot(lane < k && lst != 0ull));
            auto lane_key = [](uint64_t v, int i) {
                const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), i);
                const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), i);
                return (static_cast<uint64_t>(hi) << 32) | lo;
            };
            int rc = 0, rl = 0;
            for (int i = 0; i < n; ++i) {
                const uint64_t y = lane_key(cand, LPC * i + LPC - 1);
                rc += y > cand;
                rl += y > lst;
            }
            for (int e = 0; e < nlst; ++e) {
                const uint64_t y = lane_key(lst, e);
                rc += y > cand;
                rl += y > lst;
            }
            wave_lds_fence();  // the previous list has been read from mk
            if (mine && rc < k) mk[rc] = cand;
            if (lane < nlst && rl < k) mk[rl] = lst;
            wave_lds_fence();
            lst = lane < min(n + nlst, k) ? mk[lane] : 0ull;
        };
        // The largest float below lamf: hx >= lamf is then lamb - hx < 0, the
        // sign bit of one subtraction (exact in sign: denormals are kept).
        // lam == 0: -inf, below every finite upper end.
        const uint32_t lb = __float_as_uint(lamf);
        const float lamb = lam == 0u ? -__builtin_huge_valf()
                                     : __uint_as_float(lb == 0u ? 0x80000001u
                                                                : ((lb & 0x80000000u) ? lb + 1u : lb - 1u));
        // Pending candidates: ring entries done .. listed - 1 (at most CPP - 1
        // left after each listing round, plus the round's 64 new ones)
        static_assert(CPP - 1 + 64 <= kPendRing, "candidate ring");
        int listed = 0, done = 0;
        // One batch of 4096 pages.  Candidate bits: element i = 4*jj + e4 (page
        // base + 256*jj + 4*lane + e4) at bit 31 - i%32 of cm[i/32], shifted in
        // with v_alignbit (two instructions per upper end, no branch).  Each
        // lane then lists its candidates, lowest bit first, while any lane has
        // some; whenever CPP are pending their chains run.  The first batch
        // uses the upper ends requested above; later ones load theirs.
        auto batch = [&](int base, const float4 (&hv)[16]) {
            uint32_t cm[2] = {0u, 0u};
            if (sg.pages - base >= 4096) {  // uniform: every page of the batch is in the sequence
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const float hx[4] = {hv[jj].x, hv[jj].y, hv[jj].z, hv[jj].w};
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
                        cm[jj >> 3] = __builtin_amdgcn_alignbit(cm[jj >> 3], __float_as_uint(lamb - hx[e4]), 31);
                }
            } else {
                int lim = sg.pages - base - 4 * lane;  // in the sequence: 256*jj + e4 < lim
                asm volatile("" : "+v"(lim));
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const float hx[4] = {hv[jj].x, hv[jj].y, hv[jj].z, hv[jj].w};
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
                        cm[jj >> 3] = (cm[jj >> 3] << 1) |
                                      static_cast<uint32_t>((256 * jj + e4 < lim) & (hx[e4] >= lamf));
                }
            }
            uint64_t cmask = (static_cast<uint64_t>(cm[1]) << 32) | cm[0];
            for (;;) {
                const bool c = cmask != 0ull;
                const uint64_t bal = __ballot(c);
                if (bal == 0ull) break;
                if (c) {
                    const int b = __ffsll(static_cast<unsigned long long>(cmask)) - 1;
                    const int e = (b & 32) + 31 - (b & 31);  // the element
                    pend[(listed + lanes_below(bal, lane)) & (kPendRing - 1)] =
                        base + 256 * (e >> 2) + 4 * lane + (e & 3);
                    cmask &= cmask - 1ull;
                }
                listed += __popcll(bal);
                if (listed - done >= CPP) {  // uniform
                    wave_lds_fence();  // the listed pages visible to every lane
                    do {
                        chains(done, CPP);
                        done += CPP;
                    } while (listed - done >= CPP);
                }
            }
        };
        batch(0, hv0);
        for (int base = 4096; base < sg.pages; base += 4096) {
            float4 hv[16];
            load_h(base, hv);
            batch(base, hv);
        }
        if (listed > done) {
            wave_lds_fence();
            chains(done, listed - done);
        }
        // 3. the row's pages (k of them: every page of the exact top-k is a candidate)
        const bool has = lane < k && lst != 0ull;
        const int page = has ? static_cast<int>(~static_cast<uint32_t>(lst)) : 0x7fffffff;
        if (lane < k) psel[lane] = has ? page : -1;
        if (dbg.page_sel) {
            int rank = 0;
            for (int e = 0; e < k; ++e) rank += __builtin_amdgcn_readlane(page, e) < page;
            int32_t *dst = dbg.page_sel + (((size_t)s * D.Hq + h) * D.A + a) * k;
            if (lane < k) dst[rank] = has ? page : -1;
        }
    }
}

size_t select_lds_bytes(const Dims &D) { return (256 + 2 * (size_t)D.d + kPendRing) * 4; }

hipError_t launch_score(const Dims &D, const void *meta, const int32_t *kv_off,
                        const int32_t *prefix_len, const Work &W, hipStream_t st) {
    const int ng = D.S * D.Hk;
    const dim3 grid(((D.n_tiles_grid + 3) / 4) * ng);
    auto *m = static_cast<const uint4 *>(meta);
#define LAUNCH_S(DIMV, BFV)                                                                     \
    hipLaunchKernelGGL((k_score<DIMV, BFV>), grid, dim3(256), 0, st, D, m, kv_off, prefix_len, W)
    if (D.bf16) {
        if (D.d == 128) LAUNCH_S(128, true);
        else LAUNCH_S(64, true);
    } else {
        if (D.d == 128) LAUNCH_S(128, false);
        else LAUNCH_S(64, false);
    }
#undef LAUNCH_S
    return hipGetLastError();
}

size_t score_prep_lds_bytes(const Dims &D) {
    // the squares, then (in the same place) the stacked rows' MFMA operands
    const size_t rows = (size_t)D.G * D.B;
    const size_t squares = (D.flags & LOSA_FLAG_SHARED_ACTIVE) ? 0 : rows * (D.d + kPrepPad) * 4;
    return std::max((size_t)D.Rs16 * (D.d + 4) * 4, squares);
}

bool score_prep_fits(const Dims &D) {
    return D.bf16 && D.R > 0 && 2 * D.G * D.B * D.d / 8 <= kPrepVecs * 256 &&
           score_prep_lds_bytes(D) <= 56 * 1024 &&
           (!(D.flags & LOSA_FLAG_SHARED_ACTIVE) || D.Hq * D.B <= kMaxSharedPrep);
}

hipError_t launch_score_prep(const Dims &D, const void *q_t, const void *q_prev, const void *meta,
                             const int32_t *kv_off, const int32_t *prefix_len, const Work &W,
                             float *dbg_loc, int32_t *dbg_act, int32_t *dbg_ucnt, hipStream_t st) {
    const int ng = D.S * D.Hk;
    constexpr int TPW = kScoreTilesPerGroup;
    const dim3 grid(((D.n_tiles_grid + TPW - 1) / TPW) * ng);
    const size_t lds = score_prep_lds_bytes(D);
    auto *a = static_cast<const uint16_t *>(q_t);
    auto *b = static_cast<const uint16_t *>(q_prev);
    auto *m = static_cast<const uint4 *>(meta);
#define LAUNCH_P(DIMV, SH)                                                                       \
    do {                                                                                         \
        if (D.page_table)                                                                        \
            hipLaunchKernelGGL((k_score_prep<DIMV, SH, TPW, true>), grid, dim3(256 * TPW), lds, st, \
                               D, a, b, m, kv_off, prefix_len, W, dbg_loc, dbg_act, dbg_ucnt);   \
        else                                                                                     \
            hipLaunchKernelGGL((k_score_prep<DIMV, SH, TPW, false>), grid, dim3(256 * TPW), lds,   \
                               st, D, a, b, m, kv_off, prefix_len, W, dbg_loc, dbg_act, dbg_ucnt); \
    } while (0)
    const bool shared = D.flags & LOSA_FLAG_SHARED_ACTIVE;
    if (D.d == 128) {
        if (shared) LAUNCH_P(128, true);
        else LAUNCH_P(128, false);
    } else {
        if (shared) LAUNCH_P(64, true);
        else LAUNCH_P(64, false);
    }
#undef LAUNCH_P
    return hipGetLastError();
}

hipError_t launch_select(const Dims &D, const void *meta, const int32_t *kv_off,
                         const int32_t *prefix_len, const Work &W, int32_t *dbg_page_sel,
                         const BlockArgs &blk, hipStream_t st) {
    const int ng = D.S * D.Hk;
    const int maxb = D.B <= 16 ? 16 : (D.B <= 32 ? 32 : 64);
    const size_t blk_lds = maxb == 16   ? block_lds_bytes<16>(D.d, D.bf16)
                           : maxb == 32 ? block_lds_bytes<32>(D.d, D.bf16)
                                        : block_lds_bytes<64>(D.d, D.bf16);
    const size_t lds = std::max(D.R > 0 ? select_lds_bytes(D) : 0, blk_lds);
    const int ntg = (D.B + kBlockTPW - 1) / kBlockTPW;
    const dim3 grid(ng * D.R + D.S * D.Hq * ntg);  // selection rows, then block token groups
    SelectDbg dbg{dbg_page_sel};
    auto *m = static_cast<const uint4 *>(meta);
#define LAUNCH_S(DIMV, BFV, MB)                                                                  \
    do {                                                                                         \
        if (D.page_table)                                                                        \
            hipLaunchKernelGGL((k_select<DIMV, BFV, MB, true>), grid, dim3(64), lds, st, D, m,      \
                               kv_off, prefix_len, W, W.qrows, W.qsel32, W.hbound, W.tmax, dbg,  \
                               blk);                                                             \
        else                                                                                     \
            hipLaunchKernelGGL((k_select<DIMV, BFV, MB, false>), grid, dim3(64), lds, st, D, m,     \
                               kv_off, prefix_len, W, W.qrows, W.qsel32, W.hbound, W.tmax, dbg,  \
                               blk);                                                             \
    } while (0)
#define PICK_S(DIMV, BFV)                           \
    do {                                            \
        if (maxb == 16) LAUNCH_S(DIMV, BFV, 16);    \
        else if (maxb == 32) LAUNCH_S(DIMV, BFV, 32); \
        else LAUNCH_S(DIMV, BFV, 64);               \
    } while (0)
    if (D.bf16) {
        if (D.d == 128) PICK_S(128, true);
        else PICK_S(64, true);
    } else {
        if (D.d == 128) PICK_S(128, false);
        else PICK_S(64, false);
    }
#undef PICK_S
#undef LAUNCH_S
    return hipGetLastError();
}

}  // namespace losa
