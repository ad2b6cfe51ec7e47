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
// Phase 2 (k_select), one workgroup per (sequence, KV head), one wave per row:
// the k-th largest tile maximum of the lower ends is at most the k-th largest
// exact bound, so every page of the exact top-k has an upper end at or above
// it; those candidate pages (typically a little more than k) get the exact
// fp32 chain -- two IEEE fused multiply-adds per dimension, q+ * max then
// q- * min, one of them an exact zero and the products exact for bf16 -- and
// the exact top-k is taken on keys (score bits, page).  The union is a bitmap
// in LDS compacted into an ascending list.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    const uint32_t hi = wave_max_u32(static_cast<uint32_t>(v >> 32));
    const uint32_t lo =
        wave_max_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ float ord_to_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {
    return __popcll(mask & ((1ull << lane) - 1ull));
}

// ---------------------------------------------------------------------------
// Phase 1: bounds of every (row, page) of one tile, as an interval.

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
    const int64_t tile0 = sg.gp0 / kTile;
    const int n_t = static_cast<int>((sg.gp0 + sg.pages - 1) / kTile - tile0 + 1);
    if (bx >= n_t) return;
    const int64_t tile = tile0 + bx;
    const int R = D.R, R1 = R > 0 ? R : 1;
    const float *aux = reinterpret_cast<const float *>(reinterpret_cast<const char *>(meta) +
                                                       D.meta_main_bytes) +
                       (size_t)g * D.n_tiles_total * kTile + tile * kTile;
    const uint4 *mt = meta + (size_t)(g * D.n_tiles_total + tile) * NCH * kTile;
    float *hb = W.hbound + (size_t)sgi * R1 * D.hb_stride;
    float *tm = W.tmax + (size_t)sgi * R1 * D.n_tiles_grid;
    const float *qabs = W.qabs + (size_t)sgi * R1;

    if constexpr (BF) {
        const int l16 = lane & 15, lg = lane >> 4;
        float amax[4];
        int pl[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int in_tile = cb * 16 + l16;
            pl[cb] = static_cast<int>(tile * kTile + in_tile - sg.gp0);
            amax[cb] = aux[in_tile];
        }
        const uint32_t *q16 = W.qsel16 + (size_t)sgi * D.Rs16 * DIM;
        // the whole tile's page operands, requested at once:
        // page cb*16 + l16, metadata chunk 4*kk + lg (dims 16kk + 4lg .. +3)
        constexpr int KS = DIM / 16;
        uint4 bop[KS][4];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) bop[kk][cb] = mt[(size_t)(4 * kk + lg) * kTile + cb * 16 + l16];
        for (int rt = 0; rt < D.Rs16 / 16; ++rt) {
            // row operands: row rt*16 + l16, dims 16*kk + 4*lg .. +3 as (q+, q-) pairs
            uint4 aop[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                aop[kk] = *reinterpret_cast<const uint4 *>(q16 + (size_t)(rt * 16 + l16) * DIM +
                                                           16 * kk + 4 * lg);
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
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = rt * 16 + 4 * lg + j;
                const float qa = r < R ? qabs[r] : 0.0f;
                uint32_t lmax = 0u;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const bool valid = r < R && pl[cb] >= 0 && pl[cb] < sg.pages;
                    const float e = kBoundRel * qa * amax[cb] + kBoundAbs;
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
    } else {
        // fp32 storage: lane = page, any summation order (the interval absorbs it)
        const int p = static_cast<int>(tile * kTile + lane - sg.gp0);
        const bool valid = p >= 0 && p < sg.pages;
        const float am = aux[lane];
        const float *q32 = W.qsel32 + (size_t)sgi * R1 * DIM * 2;
        for (int r = 0; r < R; ++r) {
            float u = 0.0f;
            const float *q = q32 + (size_t)r * DIM * 2;
#pragma unroll 4
            for (int c = 0; c < NCH; ++c) {
                const uint4 m4 = mt[(size_t)c * kTile + lane];
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
// Phase 2: exact top-k per row over the candidates, and the union.

struct SelectDbg {
    int32_t *page_sel;   // [S][Hq][A][k]
    int32_t *union_idx;  // [S][Hk][cap]
    int32_t *union_cnt;  // [S][Hk]
    int cap;
};

// The exact chain for global page gp (contract of include/losa.h); the page's
// metadata chunks are loaded before the chain starts.
template <int DIM, bool BF>
__device__ __forceinline__ float exact_bound(const uint4 *meta, const Dims &D, int g, int64_t gp,
                                             const float *q) {
    constexpr int DPC = BF ? 4 : 2;
    constexpr int NCH = DIM / DPC;
    const uint4 *m = meta + (size_t)(g * D.n_tiles_total + gp / kTile) * NCH * kTile + gp % kTile;
    float acc = 0.0f;
    constexpr int BATCH = NCH < 32 ? NCH : 32;
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += BATCH) {
        uint4 mv[BATCH];
#pragma unroll
        for (int c = 0; c < BATCH; ++c) mv[c] = m[(size_t)(c0 + c) * kTile];
#pragma unroll
        for (int c = 0; c < BATCH; ++c) {
            const uint4 m4 = mv[c];
            const int cc = c0 + c;
            if constexpr (BF) {
                const uint32_t wd[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = __builtin_fmaf(q[2 * (4 * cc + e)], bf16_lo(wd[e]), acc);
                    acc = __builtin_fmaf(q[2 * (4 * cc + e) + 1], bf16_hi(wd[e]), acc);
                }
            } else {
                const float p0 = q[4 * cc + 0] * __uint_as_float(m4.x);
                acc = acc + p0;
                const float p1 = q[4 * cc + 1] * __uint_as_float(m4.y);
                acc = acc + p1;
                const float p2 = q[4 * cc + 2] * __uint_as_float(m4.z);
                acc = acc + p2;
                const float p3 = q[4 * cc + 3] * __uint_as_float(m4.w);
                acc = acc + p3;
            }
        }
    }
    return acc;
}

template <int DIM, bool BF>
__global__ __launch_bounds__(64) void k_select(Dims D, const uint4 *__restrict__ meta,
                                               const int32_t *__restrict__ kv_off,
                                               const int32_t *__restrict__ prefix_len, Work W,
                                               const float *__restrict__ qsel32,
                                               const float *__restrict__ hbound,
                                               const float *__restrict__ tmax, SelectDbg dbg) {
    extern __shared__ uint32_t smem[];
    __shared__ int s_last;
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int r = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int lane = threadIdx.x;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int R = D.R, R1 = R > 0 ? R : 1, k = D.k;
    const int h = g * D.G + r / D.A, a = r % D.A;
    const bool all_pages = k >= sg.pages;
    const int bm_words = (D.max_pages + 31) / 32;
    uint32_t *bitmap = smem;
    volatile int32_t *pend = reinterpret_cast<int32_t *>(smem + bm_words);
    float *qw = reinterpret_cast<float *>(smem + bm_words + 128);
    int32_t *psel = W.psel + ((size_t)sgi * R1 + r) * k;

    if (all_pages) {
        if (dbg.page_sel)
            for (int e = lane; e < k; e += 64)
                dbg.page_sel[(((size_t)s * D.Hq + h) * D.A + a) * k + e] = e < sg.pages ? e : -1;
    } else {
        const int64_t tile0 = sg.gp0 / kTile;
        const int n_t = static_cast<int>((sg.gp0 + sg.pages - 1) / kTile - tile0 + 1);
        const float *tm = tmax + ((size_t)sgi * R1 + r) * D.n_tiles_grid;
        const float *hb = hbound + ((size_t)sgi * R1 + r) * D.hb_stride;
        const float *qg = qsel32 + ((size_t)sgi * R1 + r) * DIM * 2;
        // the row's chain operands, staged in LDS (read as broadcasts)
        for (int i = lane; i < 2 * DIM; i += 64) qw[i] = qg[i];
        const float *q = qw;
        // loads of the tile maxima (up to 4 per lane) and of the first 4096 upper
        // ends are issued together
        constexpr int TMR = 4;
        uint32_t tmk[TMR];
#pragma unroll
        for (int i = 0; i < TMR; ++i) {
            const int x = lane + 64 * i;
            tmk[i] = x < n_t ? ord_key(tm[x]) : 0u;
        }
        float4 hv[16];
        // upper ends of pages base + 256*jj + 4*lane + e, jj < 16, e < 4
        auto load_h = [&](int base) {
            const int lim = sg.pages - base - 4 * lane;  // valid while 256*jj + e < lim
            const float *hp = hb + base + 4 * lane;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                if (256 * jj + 3 < lim) {
                    hv[jj] = *reinterpret_cast<const float4 *>(hp + 256 * jj);
                } else {
                    hv[jj].x = 256 * jj + 0 < lim ? hp[256 * jj + 0] : -__builtin_huge_valf();
                    hv[jj].y = 256 * jj + 1 < lim ? hp[256 * jj + 1] : -__builtin_huge_valf();
                    hv[jj].z = 256 * jj + 2 < lim ? hp[256 * jj + 2] : -__builtin_huge_valf();
                    hv[jj].w = 256 * jj + 3 < lim ? hp[256 * jj + 3] : -__builtin_huge_valf();
                }
            }
        };
        load_h(0);
        // 1. threshold: the k-th largest tile maximum of the lower ends
        uint32_t lam = 0u;  // below every finite key: all pages qualify
        if (n_t >= k) {
            uint64_t taken = 0ull;  // per lane: which of its tiles were extracted
            for (int e = 0; e < k; ++e) {
                uint32_t best = 0u;
                int bi = -1;
                for (int i = 0, x = lane; x < n_t; ++i, x += 64) {
                    const uint32_t v = i < TMR ? tmk[i] : ord_key(tm[x]);
                    if (!((taken >> i) & 1ull) && (bi < 0 || v > best)) {
                        best = v;
                        bi = i;
                    }
                }
                const uint32_t m = wave_max_u32(best);
                const uint64_t own = __ballot(bi >= 0 && best == m);
                if (lane == __ffsll(static_cast<unsigned long long>(own)) - 1) taken |= 1ull << bi;
                lam = m;
            }
        }
        // 2. candidates: upper end >= threshold; exact chain in batches of 64
        uint64_t lst = 0ull;  // lane e < k: e-th best (score key << 32 | ~page)
        int npend = 0;
        for (int base = 0; base < sg.pages; base += 4096) {
            if (base > 0) load_h(base);
            // bit 4*jj + e4 of cmask: page base + 256*jj + 4*lane + e4 is a candidate
            uint64_t cmask = 0ull;
            const int lim = sg.pages - base - 4 * lane;
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const float hx[4] = {hv[jj].x, hv[jj].y, hv[jj].z, hv[jj].w};
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const bool c = 256 * jj + e4 < lim && ord_key(hx[e4]) >= lam;
                    cmask |= static_cast<uint64_t>(c) << (4 * jj + e4);
                }
            }
            const bool last_batch = base + 4096 >= sg.pages;
            for (int bit = 0; bit < 64; ++bit) {
                const bool c = (cmask >> bit) & 1ull;
                const uint64_t bal = __ballot(c);
                if (c) pend[npend + lanes_below(bal, lane)] = base + 256 * (bit >> 2) + 4 * lane + (bit & 3);
                npend += __popcll(bal);
                const bool last = last_batch && bit == 63;
                while (npend >= 64 || (last && npend > 0)) {
                    __builtin_amdgcn_wave_barrier();
                    const int n = npend < 64 ? npend : 64;
                    uint64_t cand = 0ull;
                    if (lane < n) {
                        const int pc = pend[lane];
                        const float u = exact_bound<DIM, BF>(meta, D, g, sg.gp0 + pc, q);
                        cand = (static_cast<uint64_t>(ord_key(u)) << 32) |
                               static_cast<uint32_t>(~static_cast<uint32_t>(pc));
                    }
                    __builtin_amdgcn_wave_barrier();
                    const int rest = npend - n;
                    const int moved = lane < rest ? pend[lane + n] : 0;
                    __builtin_amdgcn_wave_barrier();
                    if (lane < rest) pend[lane] = moved;
                    npend = rest;
                    // merge: top-k of (candidates, current list)
                    uint64_t av = cand, bv = lane < k ? lst : 0ull, nl = 0ull;
                    for (int e = 0; e < k; ++e) {
                        const uint64_t loc = av > bv ? av : bv;
                        const uint64_t m = wave_max_u64(loc);
                        if (m == 0ull) break;
                        if (lane == e) nl = m;
                        if (av == m) av = 0ull;
                        else if (bv == m) bv = 0ull;
                    }
                    lst = nl;
                }
            }
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

    // Arrival: the last row of this (sequence, KV head) builds the union.
    __threadfence();
    __syncthreads();
    if (lane == 0) s_last = atomicAdd(&W.counters[sgi], 1) == R - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int words = (sg.pages + 31) / 32;
    for (int i = lane; i < words; i += 64) {
        if (all_pages) {
            const int rem = sg.pages - i * 32;
            bitmap[i] = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
        } else {
            bitmap[i] = 0u;
        }
    }
    __syncthreads();
    if (!all_pages) {
        const int32_t *ps = W.psel + (size_t)sgi * R1 * k;
        for (int i = lane; i < R * k; i += 64) {
            const int pg = ps[i];
            if (pg >= 0) atomicOr(&bitmap[pg >> 5], 1u << (pg & 31));
        }
    }
    __syncthreads();
    const int wpt = (words + 63) / 64;
    const int w0 = min(lane * wpt, words), w1 = min(w0 + wpt, words);
    int cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(bitmap[i]);
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    int pos = incl - cnt;
    const int total = __shfl(incl, 63);
    int32_t *uo = W.union_idx + (size_t)sgi * D.union_cap;
    for (int i = w0; i < w1; ++i) {
        uint32_t b = bitmap[i];
        while (b) {
            const int bit = __ffs(b) - 1;
            b &= b - 1;
            const int pg = i * 32 + bit;
            if (pos < D.union_cap) uo[pos] = pg;
            if (dbg.union_idx && pos < dbg.cap) dbg.union_idx[(size_t)sgi * dbg.cap + pos] = pg;
            ++pos;
        }
    }
    if (lane == 0) {
        W.union_cnt[sgi] = min(total, D.union_cap);
        if (dbg.union_cnt) dbg.union_cnt[sgi] = total;
        W.counters[sgi] = 0;  // ready for the next kernel that counts arrivals
    }
}

size_t select_lds_bytes(const Dims &D) {
    const size_t bm_words = (D.max_pages + 31) / 32;
    return (bm_words + 128 + 2 * (size_t)D.d) * 4;
}

hipError_t launch_select(const Dims &D, const void *meta, const int32_t *kv_off,
                         const int32_t *prefix_len, const Work &W, int32_t *dbg_page_sel,
                         int32_t *dbg_union_idx, int32_t *dbg_union_cnt, int dbg_union_cap,
                         hipStream_t st) {
    const int ng = D.S * D.Hk;
    const dim3 grid1(((D.n_tiles_grid + 3) / 4) * ng);
    const size_t lds = select_lds_bytes(D);
    SelectDbg dbg{dbg_page_sel, dbg_union_idx, dbg_union_cnt, dbg_union_cap};
    auto *m = static_cast<const uint4 *>(meta);
#define LAUNCH_S(DIMV, BFV)                                                                       \
    do {                                                                                          \
        hipLaunchKernelGGL((k_score<DIMV, BFV>), grid1, dim3(256), 0, st, D, m, kv_off,           \
                           prefix_len, W);                                                        \
        hipLaunchKernelGGL((k_select<DIMV, BFV>), dim3(ng * D.R), dim3(64), lds, st, D, m, kv_off, \
                           prefix_len, W, W.qsel32, W.hbound, W.tmax, dbg);                       \
    } while (0)
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

}  // namespace losa
