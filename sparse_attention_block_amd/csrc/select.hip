// QUEST page selection for the active rows only, and the union per KV head.
//
// LoSA applies the sparse selector (QUEST) to the active tokens alone, so the
// union of the pages they select -- the only prefix KV the step reads -- is
// taken over |A| rows instead of B (gist.science pt summary, "3. Metodologia",
// step 3; fr summary, "Calcul Sparse pour les Tokens Actifs" and "Réduction de
// l'Union KV").  Reading used for QUEST: page bound
// U = sum_i max(q_i*min_i, q_i*max_i); each row keeps its k = budget/16 pages
// of largest U (equal bounds to the lower page).
//
// One workgroup per (sequence, KV head, 64-page tile); lane = page.  Each wave
// scores groups of RG stacked rows over its tile's pages: an fp32 chain over
// dimensions in ascending order.  The selection operand of dimension i is the
// pair (q+, q-) = (max(q,0), min(q,0)) and the page's metadata pair is
// (max_i, min_i); the chain adds q+ * max_i and then q- * min_i, one of which
// is an exact zero, so it equals the single chain acc += q_i * (q_i >= 0 ?
// max_i : min_i) up to the sign of a zero (which the ranking key ignores).
// bf16: products are exact in fp32, so each step is one IEEE fused
// multiply-add (v_dot2_f32_bf16 is not used: on gfx950 its sum is not the
// correctly rounded acc + q*x).  fp32: each product is rounded, then added.
// Each (tile, row) keeps its top min(k, 64) pages as 64-bit keys
// (order-preserving score bits << 32 | ~page); the last workgroup of a
// (sequence, KV head) to arrive merges the tile lists (a tournament over their
// sorted heads), ORs every row's k pages into a bitmap and compacts it into
// the ascending union.
#include "losa_internal.h"

namespace losa {

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(v, o)));
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    const uint32_t hi = wave_max_u32(static_cast<uint32_t>(v >> 32));
    const uint32_t lo =
        wave_max_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

struct SelectDbg {
    int32_t *page_sel;   // [S][Hq][A][k]
    int32_t *union_idx;  // [S][Hk][cap]
    int32_t *union_cnt;  // [S][Hk]
    int cap;
};

template <int DIM, int RG, bool BF>
__global__ __launch_bounds__(256) void k_select(Dims D, const uint4 *__restrict__ meta,
                                                const float *__restrict__ qsel,
                                                const int32_t *__restrict__ kv_off,
                                                const int32_t *__restrict__ prefix_len, Work W,
                                                SelectDbg dbg) {
    constexpr int DPC = BF ? 4 : 2;
    constexpr int NCH = DIM / DPC;
    extern __shared__ uint32_t smem[];
    __shared__ int s_last;
    __shared__ int s_scan[256];
    const int g = blockIdx.y, s = blockIdx.z, bx = blockIdx.x;
    const int sgi = s * D.Hk + g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int R = D.R, kk = D.kk;
    const bool all_pages = D.k >= sg.pages;
    const int64_t tile0 = sg.gp0 / kTile;
    const int n_t = sg.pages > 0 ? static_cast<int>((sg.gp0 + sg.pages - 1) / kTile - tile0 + 1) : 0;
    uint64_t *cand = W.cand + (size_t)sgi * R * D.n_tiles_grid * kk;

    if (!all_pages && bx < n_t) {
        const int64_t tile = tile0 + bx;
        const int64_t gp = tile * kTile + lane;
        const bool valid = gp >= sg.gp0 && gp < sg.gp0 + sg.pages;
        const uint4 *mp = meta + ((size_t)(g * D.n_tiles_total + tile) * NCH) * kTile + lane;
        const float *qbase = qsel + (size_t)sgi * R * DIM * 2;
        const int n_groups = (R + RG - 1) / RG;
        for (int grp = w; grp < n_groups; grp += 4) {
            const int r0 = grp * RG;
            float acc[RG];
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) acc[rr] = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const uint4 m4 = mp[(size_t)c * kTile];
                float mx[DPC], mn[DPC];
                if constexpr (BF) {
                    mx[0] = bf16_lo(m4.x); mn[0] = bf16_hi(m4.x);
                    mx[1] = bf16_lo(m4.y); mn[1] = bf16_hi(m4.y);
                    mx[2] = bf16_lo(m4.z); mn[2] = bf16_hi(m4.z);
                    mx[3] = bf16_lo(m4.w); mn[3] = bf16_hi(m4.w);
                } else {
                    mx[0] = __uint_as_float(m4.x); mn[0] = __uint_as_float(m4.y);
                    mx[1] = __uint_as_float(m4.z); mn[1] = __uint_as_float(m4.w);
                }
#pragma unroll
                for (int rr = 0; rr < RG; ++rr) {
                    // (q+, q-) pairs of dimensions c*DPC .. c*DPC+DPC-1: uniform, scalar loads
                    const float *q = qbase + ((size_t)min(r0 + rr, R - 1) * DIM + c * DPC) * 2;
#pragma unroll
                    for (int e = 0; e < DPC; ++e) {
                        if constexpr (BF) {
                            acc[rr] = __builtin_fmaf(q[2 * e], mx[e], acc[rr]);
                            acc[rr] = __builtin_fmaf(q[2 * e + 1], mn[e], acc[rr]);
                        } else {
                            const float p0 = q[2 * e] * mx[e];
                            acc[rr] = acc[rr] + p0;
                            const float p1 = q[2 * e + 1] * mn[e];
                            acc[rr] = acc[rr] + p1;
                        }
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) {
                const int r = r0 + rr;
                if (r >= R) break;
                uint32_t key = valid ? ord_key(acc[rr]) : 0u;
                uint64_t mine = 0;
                for (int e = 0; e < kk; ++e) {
                    const uint32_t m = wave_max_u32(key);
                    if (m == 0u) break;
                    const uint64_t bal = __ballot(key == m);
                    const int win = __ffsll(static_cast<unsigned long long>(bal)) - 1;
                    const uint32_t pl = static_cast<uint32_t>(tile * kTile + win - sg.gp0);
                    if (lane == e) mine = (static_cast<uint64_t>(m) << 32) | static_cast<uint32_t>(~pl);
                    if (lane == win) key = 0u;
                }
                if (lane < kk) cand[((size_t)r * D.n_tiles_grid + bx) * kk + lane] = mine;
            }
        }
    }

    // Arrival: the last workgroup of this (sequence, KV head) merges.
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&W.counters[sgi], 1) == static_cast<int>(gridDim.x) - 1;
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int words = (sg.pages + 31) / 32;
    uint32_t *bitmap = smem;
    const int bm_words = (D.max_pages + 31) / 32;
    const int k_eff = D.k < D.max_pages ? D.k : D.max_pages;
    // Per-wave list positions and winners; volatile: lanes of the wave exchange them.
    volatile uint8_t *ptrs = reinterpret_cast<uint8_t *>(smem + bm_words) + w * D.n_tiles_grid;
    volatile int32_t *wins =
        reinterpret_cast<int32_t *>(smem + bm_words + (4 * D.n_tiles_grid + 3) / 4) + w * k_eff;
    for (int i = tid; i < words; i += 256) bitmap[i] = 0u;
    __syncthreads();
    if (all_pages) {
        for (int i = tid; i < words; i += 256) {
            const int rem = sg.pages - i * 32;
            bitmap[i] = rem >= 32 ? 0xffffffffu : ((1u << rem) - 1u);
        }
        if (dbg.page_sel) {
            for (int idx = tid; idx < R * D.k; idx += 256) {
                const int r = idx / D.k, e = idx % D.k;
                const int h = g * D.G + r / D.A, a = r % D.A;
                dbg.page_sel[(((size_t)s * D.Hq + h) * D.A + a) * D.k + e] = e < sg.pages ? e : -1;
            }
        }
    } else {
        for (int r = w; r < R; r += 4) {
            for (int i = lane; i < n_t; i += 64) ptrs[i] = 0;
            __builtin_amdgcn_wave_barrier();
            const uint64_t *crow = cand + (size_t)r * D.n_tiles_grid * kk;
            int n_win = 0;
            for (int e = 0; e < D.k; ++e) {
                uint64_t best = 0;
                int x_best = -1;
                for (int x = lane; x < n_t; x += 64) {
                    const int p = ptrs[x];
                    if (p < kk) {
                        const uint64_t v = crow[(size_t)x * kk + p];
                        if (v > best) { best = v; x_best = x; }
                    }
                }
                const uint64_t m = wave_max_u64(best);
                if (m == 0) break;
                if (best == m) ptrs[x_best] = static_cast<uint8_t>(ptrs[x_best] + 1);
                const uint32_t page = ~static_cast<uint32_t>(m);
                if (lane == 0) {
                    atomicOr(&bitmap[page >> 5], 1u << (page & 31));
                    wins[e] = static_cast<int32_t>(page);
                }
                n_win = e + 1;
                __builtin_amdgcn_wave_barrier();
            }
            if (dbg.page_sel) {
                __builtin_amdgcn_wave_barrier();
                const int h = g * D.G + r / D.A, a = r % D.A;
                int32_t *dst = dbg.page_sel + (((size_t)s * D.Hq + h) * D.A + a) * D.k;
                for (int e = lane; e < D.k; e += 64) {
                    if (e < n_win) {
                        const int32_t pe = wins[e];
                        int rank = 0;
                        for (int f = 0; f < n_win; ++f) rank += wins[f] < pe;
                        dst[rank] = pe;
                    } else {
                        dst[e] = -1;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();

    // Compact the bitmap into the ascending union.
    const int wpt = (words + 255) / 256;
    const int w0 = min(tid * wpt, words), w1 = min(w0 + wpt, words);
    int cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(bitmap[i]);
    s_scan[tid] = cnt;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int v = tid >= o ? s_scan[tid - o] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    int pos = s_scan[tid] - cnt;
    const int total = s_scan[255];
    int32_t *uo = W.union_idx + (size_t)sgi * D.union_cap;
    for (int i = w0; i < w1; ++i) {
        uint32_t b = bitmap[i];
        while (b) {
            const int bit = __ffs(b) - 1;
            b &= b - 1;
            const int page = i * 32 + bit;
            if (pos < D.union_cap) uo[pos] = page;
            if (dbg.union_idx && pos < dbg.cap) dbg.union_idx[(size_t)sgi * dbg.cap + pos] = page;
            ++pos;
        }
    }
    if (tid == 0) {
        W.union_cnt[sgi] = min(total, D.union_cap);
        if (dbg.union_cnt) dbg.union_cnt[sgi] = total;
    }
}

size_t select_lds_bytes(const Dims &D) {
    const size_t bm_words = (D.max_pages + 31) / 32;
    const size_t ptr_words = (4 * (size_t)D.n_tiles_grid + 3) / 4;
    const size_t k_eff = D.k < D.max_pages ? D.k : D.max_pages;
    return (bm_words + ptr_words + 4 * k_eff) * 4;
}

template <int DIM, bool BF>
static void launch_rg(const Dims &D, dim3 grid, size_t lds, hipStream_t st, const uint4 *meta,
                      const float *qsel, const int32_t *kv_off, const int32_t *prefix_len,
                      const Work &W, SelectDbg dbg) {
    const int R = D.R;
    if (R >= 16)
        hipLaunchKernelGGL((k_select<DIM, 4, BF>), grid, dim3(256), lds, st, D, meta, qsel, kv_off,
                           prefix_len, W, dbg);
    else if (R >= 5)
        hipLaunchKernelGGL((k_select<DIM, 2, BF>), grid, dim3(256), lds, st, D, meta, qsel, kv_off,
                           prefix_len, W, dbg);
    else
        hipLaunchKernelGGL((k_select<DIM, 1, BF>), grid, dim3(256), lds, st, D, meta, qsel, kv_off,
                           prefix_len, W, dbg);
}

hipError_t launch_select(const Dims &D, const void *meta, const int32_t *kv_off,
                         const int32_t *prefix_len, const Work &W, int32_t *dbg_page_sel,
                         int32_t *dbg_union_idx, int32_t *dbg_union_cnt, int dbg_union_cap,
                         hipStream_t st) {
    dim3 grid(D.n_tiles_grid, D.Hk, D.S);
    const size_t lds = select_lds_bytes(D);
    SelectDbg dbg{dbg_page_sel, dbg_union_idx, dbg_union_cnt, dbg_union_cap};
    auto *m = static_cast<const uint4 *>(meta);
    if (D.bf16) {
        if (D.d == 128) launch_rg<128, true>(D, grid, lds, st, m, W.qsel, kv_off, prefix_len, W, dbg);
        else launch_rg<64, true>(D, grid, lds, st, m, W.qsel, kv_off, prefix_len, W, dbg);
    } else {
        if (D.d == 128) launch_rg<128, false>(D, grid, lds, st, m, W.qsel, kv_off, prefix_len, W, dbg);
        else launch_rg<64, false>(D, grid, lds, st, m, W.qsel, kv_off, prefix_len, W, dbg);
    }
    return hipGetLastError();
}

}  // namespace losa
