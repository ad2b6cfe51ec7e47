// Prefix attention of the stacked rows over a list of pages, split over
// workgroups by chunks of pages (split-K); each workgroup writes partial
// online-softmax statistics (running max m in log2 units, sum l, unnormalised
// output) that the finishing kernel combines in a fixed order.
//
// Sparse step: the rows are the active (query head, token) pairs of a KV
// head's group and the pages are the union of their selections, so every
// union page is read from HBM once for all of them (agifrontier tutorial,
// workflow section: only active tokens query the prefix; fr summary,
// "Réduction de l'Union KV").  Dense first step: all G*B rows over every page
// of the prefix (tutorial, limitations section).
//
// bf16 path, per wave and page (16 tokens):
//   S^T[tok][row] = K_page . Q^T  with v_mfma_f32_16x16x32_bf16
//     A = K (lane l: token l%16, 8 dims of k-block l/16), B = Q rows;
//   online softmax per row in fp32 (exp2 on log2-scaled scores);
//   O^T[dim][row] += V^T . P     with v_mfma_f32_16x16x16_bf16
//     A = V^T (lane l: dim DPL*(l%16)+e, tokens 4*(l/16)..+3, gathered from
//     four 16-byte row loads per lane), B = P in S^T's own register layout.
//   A lane's output registers then hold 4*DPL consecutive dimensions of one
//   row, written with vector stores.
// fp32 path: plain VALU through LDS.
#include "losa_internal.h"

namespace losa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float shfl_max32(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}
__device__ __forceinline__ float shfl_sum32(float v) {
    v = v + __shfl_xor(v, 16);
    v = v + __shfl_xor(v, 32);
    return v;
}

// K and V of one page in the register layouts of the two MFMAs.
template <int DIM>
struct PageRegs {
    static constexpr int KSTEPS = DIM / 32;
    static constexpr int DPL = DIM / 16;
    uint4 k[KSTEPS];         // token l%16, dims 32*kk + 8*(l/16) .. +7
    uint32_t v[4][DPL / 2];  // tokens 4*(l/16) + j, dims DPL*(l%16) .. +DPL-1
    int valid;               // tokens of the page below the prefix length

    __device__ __forceinline__ void load(const uint16_t *kc, const uint16_t *vc, size_t base,
                                         int valid_, int l16, int lg) {
        valid = valid_;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            k[kk] = *reinterpret_cast<const uint4 *>(kc + base + (size_t)l16 * DIM + 32 * kk + 8 * lg);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint16_t *src = vc + base + (size_t)(4 * lg + j) * DIM + DPL * l16;
            if constexpr (DPL == 8) {
                const uint4 v4 = *reinterpret_cast<const uint4 *>(src);
                v[j][0] = v4.x; v[j][1] = v4.y; v[j][2] = v4.z; v[j][3] = v4.w;
            } else {
                const uint2 v2 = *reinterpret_cast<const uint2 *>(src);
                v[j][0] = v2.x; v[j][1] = v2.y;
            }
        }
    }
};

// Union of the selected pages of one (sequence, KV head) -- the rows' lists
// psel[0 .. n_sel), -1 for none -- as a bitmap in LDS (bm: ceil(pages/32)
// words), compacted in ascending page order.  The pages at union positions
// [first, first + cp) go to pg_out; with dbg_idx, every position is written
// there too.  Returns the union size.  Called by all 256 threads.
__device__ int union_slice(const int32_t *__restrict__ psel, int n_sel, int pages, bool all_pages,
                           int first, int cp, uint32_t *bm, int *wsum, int *pg_out,
                           int32_t *dbg_idx, int dbg_cap) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (all_pages) {
        if (tid < cp) pg_out[tid] = first + tid;
        if (dbg_idx)
            for (int i = tid; i < min(pages, dbg_cap); i += 256) dbg_idx[i] = i;
        __syncthreads();
        return pages;
    }
    const int words = (pages + 31) / 32;
    for (int i = tid; i < words; i += 256) bm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_sel; i += 256) {
        const int pg = psel[i];
        if (pg >= 0) atomicOr(&bm[pg >> 5], 1u << (pg & 31));
    }
    __syncthreads();
    const int wpt = (words + 255) / 256;
    const int w0 = min(tid * wpt, words), w1 = min(w0 + wpt, words);
    int cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(bm[i]);
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int pos = incl - cnt, total = 0;
    for (int q = 0; q < 4; ++q) {
        if (q < w) pos += wsum[q];
        total += wsum[q];
    }
    for (int i = w0; i < w1; ++i) {
        uint32_t b = bm[i];
        while (b) {
            const int pg = i * 32 + __ffs(b) - 1;
            b &= b - 1u;
            if (pos >= first && pos < first + cp) pg_out[pos - first] = pg;
            if (dbg_idx && pos < dbg_cap) dbg_idx[pos] = pg;
            ++pos;
        }
    }
    __syncthreads();
    return total;
}

template <int DIM, int RTW, bool DENSE>
__global__ __launch_bounds__(256) void k_prefix_bf16(Dims D,
                                                     const uint16_t *__restrict__ kc,
                                                     const uint16_t *__restrict__ vc,
                                                     const int32_t *__restrict__ kv_off,
                                                     const int32_t *__restrict__ prefix_len,
                                                     Work W, int32_t *dbg_uidx, int32_t *dbg_ucnt,
                                                     int dbg_cap) {
    constexpr bool dense = DENSE;
    constexpr int KSTEPS = DIM / 32;  // QK^T k-steps of 32 dims
    constexpr int DPL = DIM / 16;     // V dims per lane = PV MFMAs per page
    constexpr int RAW = 4 * 16 * DIM > kMaxBitmapWords ? 4 * 16 * DIM : kMaxBitmapWords;
    __shared__ float s_raw[RAW];  // the union bitmap first, then the page groups' outputs
    __shared__ int s_wsum[4], s_pg[kSparseChunk];
    auto s_acc = reinterpret_cast<float (*)[16][DIM]>(s_raw);
    __shared__ float s_ml[4][16][2];

    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int chunk = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int cp = dense ? kDenseChunk : kSparseChunk;
    const int first = chunk * cp;
    const int rows = dense ? D.Rd : D.R;
    const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
    const int n_rt = (rows + 15) / 16;
    const int WPG = n_rt < 4 ? n_rt : 4;
    const int n_pg = 4 / WPG;
    const int pg = w / WPG, wr = w % WPG;

    // Q operands (B of QK^T): lane l holds row l%16, dims 32*kk + 8*(l/16) .. +7;
    // requested before the union is built.
    uint4 qop[RTW][KSTEPS];
    const uint16_t *qr = static_cast<const uint16_t *>(W.qrows) + (size_t)sgi * D.R16 * DIM;
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wr + i * WPG;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            if (rt < n_rt)
                qop[i][kk] = *reinterpret_cast<const uint4 *>(qr + (size_t)(rt * 16 + l16) * DIM +
                                                              32 * kk + 8 * lg);
            else
                qop[i][kk] = make_uint4(0, 0, 0, 0);
        }
    }
    // this chunk's pages (lane i: union position first + i)
    int n_items, my_page = first + lane;
    if (dense) {
        n_items = sg.pages;
    } else {
        const int R1 = D.R > 0 ? D.R : 1;
        n_items = union_slice(W.psel + (size_t)sgi * R1 * D.k, D.R * D.k, sg.pages, D.k >= sg.pages,
                              first, cp, reinterpret_cast<uint32_t *>(s_raw), s_wsum, s_pg,
                              chunk == 0 && dbg_uidx ? dbg_uidx + (size_t)sgi * dbg_cap : nullptr,
                              dbg_cap);
        if (chunk == 0 && tid == 0) {
            W.union_cnt[sgi] = min(n_items, D.union_cap);
            if (dbg_ucnt) dbg_ucnt[sgi] = n_items;
        }
        my_page = lane < cp ? s_pg[lane] : 0;
    }
    if (first >= n_items) return;
    const int n_here = min(cp, n_items - first);

    float4_t oacc[RTW][DPL];
    float m_run[RTW], l_run[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        m_run[i] = -__builtin_huge_valf();
        l_run[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) oacc[i][e] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    auto page_of = [&](int it) { return __builtin_amdgcn_readlane(my_page, it); };
    auto base_of = [&](int p) { return ((size_t)g * D.T + sg.off + (size_t)p * kPage) * DIM; };
    if (pg < n_pg && pg < n_here) {
        PageRegs<DIM> cur, nxt;
        {
            const int p = page_of(pg);
            cur.load(kc, vc, base_of(p), min(kPage, sg.len - p * kPage), l16, lg);
        }
        for (int it = pg; it < n_here; it += n_pg) {
            const int itn = it + n_pg;
            if (itn < n_here) {
                const int pn = page_of(itn);
                nxt.load(kc, vc, base_of(pn), min(kPage, sg.len - pn * kPage), l16, lg);
            }
            const int valid = cur.valid;
            // V^T operands: output dim DPL*m + e, tokens 4*lg .. 4*lg+3 (masked past the prefix)
            short4_t vop[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int q = e >> 1, sh = (e & 1) * 16;
                short vv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vv[j] = (4 * lg + j < valid) ? static_cast<short>(cur.v[j][q] >> sh) : short(0);
                vop[e] = short4_t{vv[0], vv[1], vv[2], vv[3]};
            }
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const int rt = wr + i * WPG;
                if (rt >= n_rt) break;
                float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk)
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, cur.k[kk]),
                        __builtin_bit_cast(bf16x8_t, qop[i][kk]), sacc, 0, 0, 0);
                float sv[4];
                float mp = -__builtin_huge_valf();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sv[j] = (4 * lg + j < valid) ? sacc[j] * D.scale_log2 : -__builtin_huge_valf();
                    mp = fmaxf(mp, sv[j]);
                }
                mp = shfl_max32(mp);
                const float mn = fmaxf(m_run[i], mp);
                const float alpha = __builtin_amdgcn_exp2f(m_run[i] - mn);
                // P in bf16 feeds the MFMA; the row sum uses the same rounded weights.
                uint16_t pb[4];
                float ls = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pb[j] = f32_to_bf16(__builtin_amdgcn_exp2f(sv[j] - mn));
                    ls += bf16_to_f32(pb[j]);
                }
                l_run[i] = l_run[i] * alpha + ls;
                m_run[i] = mn;
                const short4_t pop = short4_t{static_cast<short>(pb[0]), static_cast<short>(pb[1]),
                                              static_cast<short>(pb[2]), static_cast<short>(pb[3])};
#pragma unroll
                for (int e = 0; e < DPL; ++e) {
                    oacc[i][e] *= alpha;
                    oacc[i][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop[e], pop, oacc[i][e], 0, 0, 0);
                }
            }
            cur = nxt;
        }
    }
#pragma unroll
    for (int i = 0; i < RTW; ++i) l_run[i] = shfl_sum32(l_run[i]);

    // Lane l holds, for row l%16, dims DPL*(4*lg + j) + e.
    if (n_pg == 1) {
        if (pg >= n_pg) return;
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = wr + i * WPG;
            if (rt >= n_rt) break;
            const int r = rt * 16 + l16;
            if (r >= rows) continue;
            const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
            if (lg == 0) {
                W.part_ml[pb * 2 + 0] = m_run[i];
                W.part_ml[pb * 2 + 1] = l_run[i];
            }
            float *dst = W.part_acc + pb * DIM;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float tmp[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e) tmp[e] = oacc[i][e][j];
                float *d0 = dst + DPL * (4 * lg + j);
#pragma unroll
                for (int e = 0; e < DPL; e += 4)
                    *reinterpret_cast<float4 *>(d0 + e) = make_float4(tmp[e], tmp[e + 1], tmp[e + 2], tmp[e + 3]);
            }
        }
        return;
    }
    // Several page groups (then RTW == 1 and n_rt <= 2): combine through LDS.
    if (lg == 0) {
        s_ml[w][l16][0] = m_run[0];
        s_ml[w][l16][1] = l_run[0];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_acc[w][l16][DPL * (4 * lg + j) + e] = oacc[0][e][j];
    __syncthreads();
    for (int idx = tid; idx < n_rt * 16 * DIM; idx += 256) {
        const int rtile = idx / (16 * DIM);
        const int rr = (idx / DIM) % 16;
        const int dim = idx % DIM;
        const int r = rtile * 16 + rr;
        if (r >= rows) continue;
        float mx = -__builtin_huge_valf();
        for (int q = 0; q < n_pg; ++q) mx = fmaxf(mx, s_ml[q * WPG + rtile][rr][0]);
        float lsum = 0.0f, a = 0.0f;
        for (int q = 0; q < n_pg; ++q) {
            const int wq = q * WPG + rtile;
            const float wgt = __builtin_amdgcn_exp2f(s_ml[wq][rr][0] - mx);
            lsum += wgt * s_ml[wq][rr][1];
            a += wgt * s_acc[wq][rr][dim];
        }
        const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
        W.part_acc[pb * DIM + dim] = a;
        if (dim == 0) {
            W.part_ml[pb * 2 + 0] = mx;
            W.part_ml[pb * 2 + 1] = lsum;
        }
    }
}

template <int DIM, bool DENSE>
__global__ __launch_bounds__(256) void k_prefix_f32(Dims D, const float *__restrict__ kc,
                                                    const float *__restrict__ vc,
                                                    const int32_t *__restrict__ kv_off,
                                                    const int32_t *__restrict__ prefix_len, Work W,
                                                    int32_t *dbg_uidx, int32_t *dbg_ucnt, int dbg_cap) {
    constexpr bool dense = DENSE;
    constexpr int DPT = DIM / 16;
    __shared__ uint32_t s_bm[kMaxBitmapWords];
    __shared__ int s_wsum[4], s_pg[kSparseChunk];
    __shared__ float q_s[16][DIM];
    __shared__ float k_s[16][DIM + 1];
    __shared__ float v_s[16][DIM];
    __shared__ float s_s[16][17];
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int chunk = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int cp = dense ? kDenseChunk : kSparseChunk;
    const int first = chunk * cp;
    int n_items;
    if (dense) {
        n_items = sg.pages;
    } else {
        const int R1 = D.R > 0 ? D.R : 1;
        n_items = union_slice(W.psel + (size_t)sgi * R1 * D.k, D.R * D.k, sg.pages, D.k >= sg.pages,
                              first, cp, s_bm, s_wsum, s_pg,
                              chunk == 0 && dbg_uidx ? dbg_uidx + (size_t)sgi * dbg_cap : nullptr,
                              dbg_cap);
        if (chunk == 0 && threadIdx.x == 0) {
            W.union_cnt[sgi] = min(n_items, D.union_cap);
            if (dbg_ucnt) dbg_ucnt[sgi] = n_items;
        }
    }
    if (first >= n_items) return;
    const int n_here = min(cp, n_items - first);
    const int rows = dense ? D.Rd : D.R;
    const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
    const int n_rt = (rows + 15) / 16;
    const int tid = threadIdx.x, r16 = tid / 16, j16 = tid % 16;
    const float *qr = static_cast<const float *>(W.qrows) + (size_t)sgi * D.R16 * DIM;

    for (int rt = 0; rt < n_rt; ++rt) {
        __syncthreads();
        for (int idx = tid; idx < 16 * DIM; idx += 256) q_s[idx / DIM][idx % DIM] = qr[(size_t)rt * 16 * DIM + idx];
        float m_run = -__builtin_huge_valf(), l_run = 0.0f, acc[DPT];
#pragma unroll
        for (int x = 0; x < DPT; ++x) acc[x] = 0.0f;
        for (int it = 0; it < n_here; ++it) {
            const int pos = first + it;
            const int p = dense ? pos : s_pg[it];
            const int valid = min(kPage, sg.len - p * kPage);
            const size_t base = ((size_t)g * D.T + sg.off + (size_t)p * kPage) * DIM;
            __syncthreads();
            for (int idx = tid; idx < 16 * DIM; idx += 256) {
                const int t = idx / DIM, x = idx % DIM;
                k_s[t][x] = kc[base + idx];
                v_s[t][x] = t < valid ? vc[base + idx] : 0.0f;
            }
            __syncthreads();
            float dot = 0.0f;
            for (int x = 0; x < DIM; ++x) dot = fmaf(q_s[r16][x], k_s[j16][x], dot);
            s_s[r16][j16] = j16 < valid ? dot * D.scale_log2 : -__builtin_huge_valf();
            __syncthreads();
            float mp = -__builtin_huge_valf();
            for (int u = 0; u < 16; ++u) mp = fmaxf(mp, s_s[r16][u]);
            const float mn = fmaxf(m_run, mp);
            const float alpha = exp2f(m_run - mn);
            float pu[16], ls = 0.0f;
            for (int u = 0; u < 16; ++u) {
                pu[u] = exp2f(s_s[r16][u] - mn);
                ls += pu[u];
            }
#pragma unroll
            for (int x = 0; x < DPT; ++x) {
                float a = acc[x] * alpha;
                for (int u = 0; u < 16; ++u) a = fmaf(pu[u], v_s[u][j16 * DPT + x], a);
                acc[x] = a;
            }
            l_run = l_run * alpha + ls;
            m_run = mn;
        }
        const int r = rt * 16 + r16;
        if (r < rows) {
            const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
            if (j16 == 0) {
                W.part_ml[pb * 2 + 0] = m_run;
                W.part_ml[pb * 2 + 1] = l_run;
            }
#pragma unroll
            for (int x = 0; x < DPT; ++x) W.part_acc[pb * DIM + j16 * DPT + x] = acc[x];
        }
    }
}

hipError_t launch_prefix(const Dims &D, bool dense, const void *k_cache, const void *v_cache,
                         const int32_t *kv_off, const int32_t *prefix_len, const Work &W,
                         int32_t *dbg_uidx, int32_t *dbg_ucnt, int dbg_cap, hipStream_t st) {
    const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
    dim3 grid(nch * D.S * D.Hk);
    if (D.bf16) {
        auto *k = static_cast<const uint16_t *>(k_cache);
        auto *v = static_cast<const uint16_t *>(v_cache);
        const int rows = dense ? D.Rd : D.R;
        const int n_rt = (rows + 15) / 16;
        const int rtw = n_rt <= 4 ? 1 : (n_rt <= 8 ? 2 : 4);
#define LAUNCH_P(DIMV, RTWV, DN)                                                                 \
    hipLaunchKernelGGL((k_prefix_bf16<DIMV, RTWV, DN>), grid, dim3(256), 0, st, D, k, v, kv_off, \
                       prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap)
#define PICK_P(DIMV, DN)                         \
    do {                                         \
        if (rtw == 1) LAUNCH_P(DIMV, 1, DN);     \
        else if (rtw == 2) LAUNCH_P(DIMV, 2, DN); \
        else LAUNCH_P(DIMV, 4, DN);              \
    } while (0)
        if (D.d == 128) {
            if (dense) PICK_P(128, true);
            else PICK_P(128, false);
        } else {
            if (dense) PICK_P(64, true);
            else PICK_P(64, false);
        }
#undef PICK_P
#undef LAUNCH_P
    } else {
        auto *k = static_cast<const float *>(k_cache);
        auto *v = static_cast<const float *>(v_cache);
#define LAUNCH_F(DIMV, DN)                                                                      \
    hipLaunchKernelGGL((k_prefix_f32<DIMV, DN>), grid, dim3(256), 0, st, D, k, v, kv_off,       \
                       prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap)
        if (D.d == 128) {
            if (dense) LAUNCH_F(128, true);
            else LAUNCH_F(128, false);
        } else {
            if (dense) LAUNCH_F(64, true);
            else LAUNCH_F(64, false);
        }
#undef LAUNCH_F
    }
    return hipGetLastError();
}

}  // namespace losa
