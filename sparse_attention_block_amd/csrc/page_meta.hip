// Page metadata for QUEST selection: element-wise min and max of each page's
// keys (the pages name QUEST as LoSA's selector for active tokens: gist.science
// pt summary, "3. Metodologia", step 3; the min/max bound is this library's
// reading of it).
//
// Layout (library-owned).  Pages are grouped per KV head into tiles of 64
// consecutive metadata pages: sequence s's page p is metadata page kv_off/16
// + p in the contiguous layout and s * max_pages + p with a page table (which
// reads the keys through the table but keeps the metadata of a sequence's
// pages side by side, so scoring reads whole tiles either way).  Inside a
// tile, the metadata of chunk c of every page's dimensions is stored for the
// 64 pages back to back, 16 bytes per page, so a wave whose lane = page reads
// one chunk with one fully coalesced 1 KiB load:
//   bf16: chunk = 4 dimensions, one dword per dimension = (max | min << 16)
//   fp32: chunk = 2 dimensions, (max_0, min_0, max_1, min_1)
// That chunk is also exactly the B operand a lane supplies to
// v_mfma_f32_16x16x32_bf16 for 8 consecutive k-slots (max_i, min_i pairs).
// After the min/max part follows, per KV head and metadata page, the largest
// |key| element of the page (fp32), which bounds the error of MFMA scoring.
// Last comes a page-major copy of the min/max part: per KV head and metadata
// page, the page's chunks 0 .. DIM/DPC - 1 back to back (DIM*2 element sizes
// contiguous), for the exact bound of selection, whose lanes each take one
// page scattered over the prefix: one page then fills whole cache lines
// instead of one 16-byte piece of a line per chunk.
#include "losa_internal.h"

namespace losa {

// One thread per (page, 16-byte column chunk of a token row): it loads that
// chunk of each of the page's 16 tokens (the lanes of a page cover a token row
// contiguously, so every load instruction reads whole rows), keeps the
// element-wise minimum and maximum in registers, and writes its metadata chunks;
// the page's largest |key| is reduced over the page's lanes.  With first_token,
// only the pages holding tokens first_token[s] .. prefix_len[s] - 1 of each
// sequence are rewritten (a committed block); page p of the launch is then page
// first_token[s] / 16 + p.
template <typename T, int DIM>
__global__ __launch_bounds__(256) void k_page_meta(Dims D, const T *__restrict__ kc,
                                                   const int32_t *__restrict__ kv_off,
                                                   const int32_t *__restrict__ prefix_len,
                                                   const int32_t *__restrict__ first_token,
                                                   uint32_t *__restrict__ meta) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte column chunk
    constexpr int CPR = DIM / EPC;        // column chunks per token row (= lanes per page)
    constexpr int PPW = 256 / CPR;        // pages per workgroup
    constexpr int DPC = BF ? 4 : 2;       // dimensions per metadata chunk
    constexpr int NCH = DIM / DPC;        // metadata chunks per page
    constexpr int MPT = EPC / DPC;        // metadata chunks per thread
    static_assert(CPR <= 64 && 64 % CPR == 0, "a page's lanes lie in one wave");
    const int g = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, cc = tid % CPR;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int p0 = first_token ? max(0, first_token[s]) / kPage : 0;
    const int pl = p0 + blockIdx.x * PPW + tid / CPR;  // local page
    const bool live = pl < sg.pages;
    const int valid = live ? min(kPage, sg.len - pl * kPage) : 0;
    // the page's 16 rows of this column chunk (clamped rows: tokens past the
    // prefix, and pages past the sequence, reread its last valid token)
    const int last = max(sg.len - 1, 0);
    // (a page past the sequence rereads its last token, which lies in its last page)
    const int plc = min(pl, max(sg.pages - 1, 0));
    const int64_t prow = phys_page(sg, plc) * kPage;
    uint4 v[kPage];
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
        const int64_t row = min(prow + min(pl * kPage + t, last) - plc * kPage, D.T - 1);  // inside the cache
        v[t] = *reinterpret_cast<const uint4 *>(kc + ((size_t)g * D.T + max(row, int64_t{0})) * DIM + cc * EPC);
    }
    __builtin_amdgcn_sched_barrier(0);
    float mn[EPC], mx[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        mn[e] = __builtin_huge_valf();
        mx[e] = -__builtin_huge_valf();
    }
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
        const uint32_t w[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
        float x[EPC];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if constexpr (BF) {
                x[2 * q] = bf16_lo(w[q]);
                x[2 * q + 1] = bf16_hi(w[q]);
            } else {
                x[q] = __uint_as_float(w[q]);
            }
        }
        if (t < valid) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                mn[e] = fminf(mn[e], x[e]);
                mx[e] = fmaxf(mx[e], x[e]);
            }
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) am = fmaxf(am, fmaxf(fabsf(mn[e]), fabsf(mx[e])));
#pragma unroll
    for (int o = 1; o < CPR; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
    if (!live) return;
    const int64_t gp = meta_page(sg, pl);
    const int64_t tile = gp / kTile;
    const int lane = static_cast<int>(gp % kTile);
#pragma unroll
    for (int m = 0; m < MPT; ++m) {
        const int c = cc * MPT + m;  // metadata chunk: dimensions c*DPC ..
        uint4 u;
        if constexpr (BF) {
            // min/max of bf16 values are bf16 values: the top 16 bits are exact
            uint32_t wd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wd[e] = (__float_as_uint(mx[4 * m + e]) >> 16) | (__float_as_uint(mn[4 * m + e]) & 0xffff0000u);
            u = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        } else {
            u = make_uint4(__float_as_uint(mx[2 * m]), __float_as_uint(mn[2 * m]),
                           __float_as_uint(mx[2 * m + 1]), __float_as_uint(mn[2 * m + 1]));
        }
        reinterpret_cast<uint4 *>(meta)[((size_t)(g * D.n_tiles_total + tile) * NCH + c) * kTile + lane] = u;
        reinterpret_cast<uint4 *>(reinterpret_cast<char *>(meta) + D.meta_pm_off)
            [((size_t)g * D.n_tiles_total * kTile + gp) * NCH + c] = u;
    }
    if (cc == 0) {
        float *aux = reinterpret_cast<float *>(reinterpret_cast<char *>(meta) + D.meta_main_bytes);
        aux[(size_t)g * D.n_tiles_total * kTile + gp] = am;
    }
}

hipError_t launch_page_meta(const Dims &D, const void *k_cache, const int32_t *kv_off,
                            const int32_t *prefix_len, const int32_t *first_token,
                            int max_new_tokens, void *meta, hipStream_t st) {
    // pages per sequence the launch covers: all of the longest prefix, or those
    // a committed block of at most max_new_tokens tokens can touch
    const int pages = first_token ? (max_new_tokens + kPage - 1) / kPage + 1 : D.max_pages;
    const int cpr = D.d * (D.bf16 ? 2 : 4) / 16, ppw = 256 / cpr;
    dim3 grid((pages + ppw - 1) / ppw, D.Hk, D.S);
    if (pages <= 0 || grid.x == 0) return hipSuccess;
    auto *m = static_cast<uint32_t *>(meta);
#define LAUNCH_M(TV, DIMV)                                                                       \
    hipLaunchKernelGGL((k_page_meta<TV, DIMV>), grid, dim3(256), 0, st, D,                       \
                       static_cast<const TV *>(k_cache), kv_off, prefix_len, first_token, m)
    if (D.bf16) {
        if (D.d == 128) LAUNCH_M(uint16_t, 128);
        else LAUNCH_M(uint16_t, 64);
    } else {
        if (D.d == 128) LAUNCH_M(float, 128);
        else LAUNCH_M(float, 64);
    }
#undef LAUNCH_M
    return hipGetLastError();
}

}  // namespace losa
