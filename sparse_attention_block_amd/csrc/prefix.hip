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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Reductions over the lanes l, l^16, l^32, l^48 (the 4 lane rows of 16).
// v_permlane16_swap of a register with itself gives, in every lane, the
// values of its row pair (rows 0 and 1, or 2 and 3) in its two results, and
// v_permlane32_swap those of its two halves; a symmetric operation on the
// two results so combines lane l with l^16, then with l^32, in one VALU
// instruction each (no LDS round trip), the same value in all four lanes.
__device__ __forceinline__ float shfl_max32(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float shfl_sum32(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// inclusive prefix sum over the 64 lanes with DPP: row shifts 1, 2, 4, 8 sum
// inside each row of 16 lanes (a lane with no source adds 0), then row
// broadcasts 15 and 31 carry the row totals into the later rows
__device__ __forceinline__ int wave_incl_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
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


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// A row's softmax reference may trail its running maximum by this much (log2
// units): weights up to 2^8 are exact to bf16's relative precision and far
// from any overflow in the fp32 sums.
constexpr float kLazyRescale = 8.0f;

// The attention of the wave's row tiles over NP pages given the V^T operands
// in MFMA layout: vpair[n/2][e] for page pairs (NP even; the A operand of
// v_mfma_f32_16x16x32_bf16 for output block e), vop[n][e] for single pages
// (v_mfma_f32_16x16x16bf16_1k); the output layout of block e is the caller's.
// MSUM (page pairs only): the row sums of the rounded weights come from one
// more MFMA with an all-ones A operand, accumulated in l4[i] (every element
// the row's sum over all lanes' tokens; l_run is then unused), and the scale
// is applied inside the exponent's fused multiply-add -- fewer vector
// instructions per page pair.
template <int DIM, int RTW, int NP, bool MASK = false, bool MSUM = false>
__device__ __forceinline__ void attend_core(const uint4 (&kop)[NP][DIM / 32],
                                            const u32x4_t (&vpair)[NP % 2 == 0 ? NP / 2 : 1][DIM / 16],
                                            const short4_t (&vop)[NP % 2 == 0 ? 1 : NP][DIM / 16],
                                            const int (&valid)[NP],
                                            const uint4 (&qop)[RTW][DIM / 32],
                                            const bool (&rt_ok)[RTW], float scale_log2,
                                            float4_t (&oacc)[RTW][DIM / 16], float (&m_run)[RTW],
                                            float (&l_run)[RTW], int lg,
                                            const uint64_t (&rmask)[NP] = {},
                                            const int (&row0)[RTW] = {}, float4_t *l4 = nullptr) {
    constexpr int KSTEPS = DIM / 32, DPL = DIM / 16;
    static_assert(!MSUM || NP % 2 == 0, "MFMA row sums are written for page pairs");
    bool full[NP];
#pragma unroll
    for (int n = 0; n < NP; ++n) full[n] = valid[n] >= kPage;  // uniform
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        if (!rt_ok[i]) break;
        float sv[NP][4];
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, kop[n][kk]), __builtin_bit_cast(bf16x8_t, qop[i][kk]),
                    sacc, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[n][j] = MSUM ? sacc[j] : sacc[j] * scale_log2;
            if (!full[n]) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * lg + j >= valid[n]) sv[n][j] = -__builtin_huge_valf();
            }
            if constexpr (MASK) {  // rows that did not select the page attend none of it
                const int l16 = __lane_id() & 15;
                if (!((rmask[n] >> (row0[i] + l16)) & 1ull)) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) sv[n][j] = -__builtin_huge_valf();
                }
            }
        }
        float mp = -__builtin_huge_valf();
#pragma unroll
        for (int n = 0; n < NP; ++n) mp = fmaxf(mp, fmaxf(fmaxf(sv[n][0], sv[n][1]), fmaxf(sv[n][2], sv[n][3])));
        mp = shfl_max32(mp);
        if constexpr (MSUM) mp *= scale_log2;  // (a positive scale keeps the maximum)
        // Lazy reference: a row's reference m_run moves to its running maximum
        // only once a score exceeds it by more than kLazyRescale (log2 units), so
        // weights stay below 2^kLazyRescale and the output is rescaled rarely
        // (softmax does not depend on the reference; the partial keeps it).
        const float mx = fmaxf(m_run[i], mp);
        if (__ballot(mx > m_run[i] + kLazyRescale) != 0ull) {  // uniform branch
            const float mn = mx > m_run[i] + kLazyRescale ? mx : m_run[i];
            // (with masks a row's reference may still be -inf: it keeps factor 1)
            const float alpha = MASK && mn == m_run[i] ? 1.0f : __builtin_amdgcn_exp2f(m_run[i] - mn);
#pragma unroll
            for (int e = 0; e < DPL; ++e) oacc[i][e] *= alpha;
            if constexpr (MSUM) l4[i] *= alpha;
            else l_run[i] *= alpha;
            m_run[i] = mn;
        }
        // (with masks a row may have seen no score yet: its weights are zero)
        const float mn = MASK && m_run[i] == -__builtin_huge_valf() ? 0.0f : m_run[i];
        u32x2_t pw[NP];  // the lane's weights of page n (tokens 4*lg .. +3), bf16
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = MSUM ? __builtin_fmaf(sv[n][j], scale_log2, -mn) : sv[n][j] - mn;
            const bf16x2_t p01 = {static_cast<__bf16>(__builtin_amdgcn_exp2f(x[0])),
                                  static_cast<__bf16>(__builtin_amdgcn_exp2f(x[1]))};
            const bf16x2_t p23 = {static_cast<__bf16>(__builtin_amdgcn_exp2f(x[2])),
                                  static_cast<__bf16>(__builtin_amdgcn_exp2f(x[3]))};
            const uint32_t w01 = __builtin_bit_cast(uint32_t, p01), w23 = __builtin_bit_cast(uint32_t, p23);
            if constexpr (!MSUM)
                l_run[i] += (bf16_lo(w01) + bf16_hi(w01)) + (bf16_lo(w23) + bf16_hi(w23));
            pw[n] = u32x2_t{w01, w23};
        }
        if constexpr (NP % 2 == 0) {
            // pages n and n+1 in one v_mfma_f32_16x16x32_bf16: its k index
            // 8*lg + c stands for token 4*lg + c%4 of page n + c/4, in both
            // operands (the sum over k does not depend on the order)
#pragma unroll
            for (int n = 0; n < NP; n += 2) {
                const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, u32x4_t{pw[n].x, pw[n].y, pw[n + 1].x, pw[n + 1].y});
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    oacc[i][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, vpair[n / 2][e]), pop, oacc[i][e], 0, 0, 0);
                if constexpr (MSUM) {  // bf16 1.0 in every k slot: the weights' sum per row
                    constexpr uint32_t kOnes = 0x3f803f80u;
                    l4[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, u32x4_t{kOnes, kOnes, kOnes, kOnes}), pop, l4[i], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < NP; ++n) {
                const short4_t pop = __builtin_bit_cast(short4_t, pw[n]);
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    oacc[i][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop[n][e], pop, oacc[i][e], 0, 0, 0);
            }
        }
    }
}


// NP pages of 16 tokens for the wave's row tiles i (those with rt_ok[i]):
// S^T = K.Q^T with v_mfma_f32_16x16x32_bf16, online softmax in log2 units over
// the NP pages together, then O^T += V^T.P: two pages per
// v_mfma_f32_16x16x32_bf16 when NP is even, else v_mfma_f32_16x16x16bf16_1k.
// kop[n]: the lane's K operand of page n (token l%16, dims 32*kk + 8*(l/16) ..
// +7); vw[n]: V words of tokens 4*(l/16) + j for the lane's DPL dims; valid[n]:
// tokens of page n inside the prefix (0 for no page).  P is rounded to bf16 for
// the MFMA and the row sum is taken from the rounded weights.  The running
// output is rescaled only when some row's maximum passed its reference by more
// than kLazyRescale (the factor is exactly 1 for the other rows).  Several pages at once keep independent MFMA chains
// in flight and share one max reduction.
template <int DIM, int RTW, int NP, bool MASK = false>
__device__ __forceinline__ void attend_pages(const uint4 (&kop)[NP][DIM / 32],
                                             const uint32_t (&vw)[NP][4][DIM / 32],
                                             const int (&valid)[NP],
                                             const uint4 (&qop)[RTW][DIM / 32],
                                             const bool (&rt_ok)[RTW], float scale_log2,
                                             float4_t (&oacc)[RTW][DIM / 16], float (&m_run)[RTW],
                                             float (&l_run)[RTW], int lg,
                                             const uint64_t (&rmask)[NP] = {},
                                             const int (&row0)[RTW] = {}) {
    constexpr int KSTEPS = DIM / 32, DPL = DIM / 16;
    bool full[NP];
#pragma unroll
    for (int n = 0; n < NP; ++n) full[n] = valid[n] >= kPage;  // uniform
    // V^T operands: output dim DPL*(l%16) + e, tokens 4*lg .. 4*lg+3 of a
    // page, as two words (tokens 0,1 and 2,3) from byte permutes of the
    // tokens' words; for page pairs both pages' words are formed straight
    // into one 4-register operand (no register moves).  Tokens past the
    // prefix get zero values.
    constexpr int NPP = NP % 2 == 0 ? NP / 2 : 1;
    u32x4_t vpair[NPP][DPL];
    short4_t vop[NP % 2 == 0 ? 1 : NP][DPL];
    auto tok2 = [&](int n, int j, int e) {  // tokens j, j+1 of page n, dim half e&1 of word e/2
        return __builtin_amdgcn_perm(vw[n][j + 1][e >> 1], vw[n][j][e >> 1],
                                     (e & 1) ? 0x07060302u : 0x05040100u);
    };
    auto page_masks = [&](int n, uint32_t &m0, uint32_t &m1) {
        m0 = (4 * lg + 0 < valid[n] ? 0x0000ffffu : 0u) | (4 * lg + 1 < valid[n] ? 0xffff0000u : 0u);
        m1 = (4 * lg + 2 < valid[n] ? 0x0000ffffu : 0u) | (4 * lg + 3 < valid[n] ? 0xffff0000u : 0u);
    };
    if constexpr (NP % 2 == 0) {
#pragma unroll
        for (int np = 0; np < NPP; ++np) {
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                vpair[np][e] = u32x4_t{tok2(2 * np, 0, e), tok2(2 * np, 2, e), tok2(2 * np + 1, 0, e),
                                       tok2(2 * np + 1, 2, e)};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (!full[2 * np + h]) {  // uniform branch
                    uint32_t m0, m1;
                    page_masks(2 * np + h, m0, m1);
#pragma unroll
                    for (int e = 0; e < DPL; ++e) {
                        vpair[np][e][2 * h] &= m0;
                        vpair[np][e][2 * h + 1] &= m1;
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            uint32_t m0 = ~0u, m1 = ~0u;
            if (!full[n]) page_masks(n, m0, m1);
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                vop[n][e] = __builtin_bit_cast(short4_t, u32x2_t{tok2(n, 0, e) & m0, tok2(n, 2, e) & m1});
        }
    }
    attend_core<DIM, RTW, NP, MASK>(kop, vpair, vop, valid, qop, rt_ok, scale_log2, oacc, m_run, l_run,
                                    lg, rmask, row0);
}

// Union of the selected pages of one (sequence, KV head) -- the rows' lists
// psel[0 .. n_sel), -1 for none -- as a bitmap in LDS (bm: ceil(pages/32)
// words), compacted in ascending page order.  The pages at union positions
// [first, first + cp) go to pg_out, and with dbg_idx to the same positions
// there (so every workgroup reports the pages it loads).  Returns the union
// size.  Called by all 256 threads; pre0 is psel[tid] (read by the caller
// ahead of time; ignored for tid >= n_sel).
__device__ int union_slice(const int32_t *__restrict__ psel, int pre0, int n_sel, int pages,
                           bool all_pages, int first, int cp, uint32_t *bm, int *wsum, int *pg_out,
                           int32_t *dbg_idx, int dbg_cap, int k = 0, uint64_t *rmask = nullptr) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (all_pages) {
        if (tid < cp) pg_out[tid] = first + tid;
        if (rmask && tid < cp) rmask[tid] = ~0ull;  // every row selected every page
        if (dbg_idx)
            for (int i = first + tid; i < min(min(pages, dbg_cap), first + cp); i += 256)
                dbg_idx[i] = i;
        __syncthreads();
        return pages;
    }
    const int words = (pages + 31) / 32;
    for (int i = tid; i < words; i += 256) bm[i] = 0u;
    __syncthreads();
    if (tid < n_sel && pre0 >= 0) atomicOr(&bm[pre0 >> 5], 1u << (pre0 & 31));
    for (int i = tid + 256; i < n_sel; i += 256) {
        const int pg = psel[i];
        if (pg >= 0) atomicOr(&bm[pg >> 5], 1u << (pg & 31));
    }
    __syncthreads();
    const int wpt = (words + 255) / 256;
    const int w0 = min(tid * wpt, words), w1 = min(w0 + wpt, words);
    int cnt = 0;
    for (int i = w0; i < w1; ++i) cnt += __popc(bm[i]);
    const int incl = wave_incl_sum(cnt);
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
            if (pos >= first && pos < first + cp) {
                pg_out[pos - first] = pg;
                if (dbg_idx && pos < dbg_cap) dbg_idx[pos] = pg;
            }
            ++pos;
        }
    }
    __syncthreads();
    if (rmask) {
        // bit r of rmask[x]: row r (entries r*k .. of psel) selected this chunk's page x
        const int n_here = max(0, min(cp, total - first));
        for (int x = tid; x < cp; x += 256) rmask[x] = 0ull;
        __syncthreads();
        for (int e = tid; e < n_sel; e += 256) {
            const int pg = psel[e];
            if (pg < 0) continue;
            int lo = 0, hi = n_here;  // the chunk's pages ascend
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (pg_out[mid] < pg) lo = mid + 1;
                else hi = mid;
            }
            if (lo < n_here && pg_out[lo] == pg)
                atomicOr(reinterpret_cast<unsigned long long *>(&rmask[lo]), 1ull << (e / k));
        }
        __syncthreads();
    }
    return total;
}

template <int DIM, int RTW, bool DENSE, bool MASK>
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
    __shared__ __align__(16) float s_raw[RAW];  // the union bitmap, then the page groups' outputs
    __shared__ int s_wsum[4], s_pg[kMaxSparseChunk];
    __shared__ uint64_t s_rmask[MASK ? kMaxSparseChunk : 1];  // rows that selected each page
    auto s_acc = reinterpret_cast<float (*)[16][DIM]>(s_raw);
    __shared__ float s_ml[4][16][2];
    __shared__ __align__(16) float s_wt[4][16][4];  // each row's page-group weights (combine)

    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int chunk = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int cp = dense ? D.dense_chunk : D.sparse_chunk;
    const int first = chunk * cp;
    const int rows = dense ? D.Rd : D.R;
    const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
    const int n_rt = (rows + 15) / 16;
    // waves per page group: a wave takes row tiles wr, wr + WPG, ... (RTW at
    // most) of its group's pages
    const int WPG = n_rt < 4 ? n_rt : 4;
    const int n_pg = 4 / WPG;
    const int pg = w / WPG, wr = w % WPG;

    // the rows' page lists (one entry per thread, clamped), requested first
    const int32_t *psel_g = W.psel + (size_t)sgi * (D.R > 0 ? D.R : 1) * D.k;
    const int n_sel = D.R * D.k;
    const int pre0 = dense ? -1 : psel_g[min(tid, max(n_sel - 1, 0))];
    // Q operands (B of QK^T): lane l holds row l%16, dims 32*kk + 8*(l/16) .. +7;
    // requested before the union is built.
    uint4 qop[RTW][KSTEPS];
    const uint16_t *qr = static_cast<const uint16_t *>(W.qrows) + (size_t)sgi * D.R16 * DIM;
    // (row tiles past the rows read the last tile -- the buffer holds whole
    // tiles -- and are zeroed: no load is conditional)
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wr + i * WPG, rtc = min(rt, max(n_rt - 1, 0));
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qr + (size_t)(rtc * 16 + l16) * DIM +
                                                             32 * kk + 8 * lg);
            qop[i][kk] = rt < n_rt ? v : make_uint4(0, 0, 0, 0);
        }
    }
    // this chunk's pages (lane i: union position first + i)
    int n_items, my_page = first + lane;
    if (dense) {
        n_items = sg.pages;
    } else {
        n_items = union_slice(psel_g, pre0, n_sel, sg.pages, D.k >= sg.pages,
                              first, cp, reinterpret_cast<uint32_t *>(s_raw), s_wsum, s_pg,
                              dbg_uidx ? dbg_uidx + (size_t)sgi * dbg_cap : nullptr,
                              dbg_cap, D.k, MASK ? s_rmask : nullptr);
        my_page = lane < cp ? s_pg[lane] : 0;
    }
    // The union size, for the finishing kernel: stored once the page loads are
    // out (a wait for the pages would otherwise wait for this store too).
    auto store_count = [&]() {
        if (!dense && chunk == 0 && tid == 0) {
            W.union_cnt[sgi] = min(n_items, D.union_cap);
            if (dbg_ucnt) dbg_ucnt[sgi] = n_items;
        }
    };
    if (first >= n_items) {
        store_count();
        return;
    }
    const int n_here = min(cp, n_items - first);
    int row0[RTW];  // first row of each of the wave's row tiles
#pragma unroll
    for (int i = 0; i < RTW; ++i) row0[i] = (wr + i * WPG) * 16;

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
    auto base_of = [&](int p) { return ((size_t)g * D.T + (size_t)phys_page(sg, p) * kPage) * DIM; };
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
            bool rt_ok[RTW];
#pragma unroll
            for (int i = 0; i < RTW; ++i) rt_ok[i] = wr + i * WPG < n_rt;
            const int vld[1] = {cur.valid};
            const uint64_t rm[1] = {MASK ? s_rmask[it] : 0ull};
            attend_pages<DIM, RTW, 1, MASK>(reinterpret_cast<const uint4(&)[1][KSTEPS]>(cur.k),
                                            reinterpret_cast<const uint32_t(&)[1][4][DPL / 2]>(cur.v),
                                            vld, qop, rt_ok, D.scale_log2, oacc, m_run, l_run, lg,
                                            rm, row0);
            cur = nxt;
        }
    }
    store_count();
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
    // Several page groups: combine them through LDS, RTW rounds of one row
    // tile per wave (round i: the waves hold row tiles i*WPG .. i*WPG + WPG-1).
    // Per row, one thread forms the groups' weights (and the row's m, l); then
    // every thread combines 4 dimensions of a row, groups in ascending order.
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        if (i * WPG >= n_rt) break;  // uniform
        if (i > 0) __syncthreads();  // the previous round has read s_acc and s_wt
        if (lg == 0) {
            s_ml[w][l16][0] = m_run[i];
            s_ml[w][l16][1] = l_run[i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < DPL; ++e) s_acc[w][l16][DPL * (4 * lg + j) + e] = oacc[i][e][j];
        __syncthreads();
        if (tid < WPG * 16) {
            const int rtile = tid / 16, rr = tid % 16;
            const int r = (i * WPG + rtile) * 16 + rr;
            float mq[4], wq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) mq[q] = s_ml[min(q * WPG + rtile, 3)][rr][0];
            float mx = -__builtin_huge_valf();
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < n_pg) mx = fmaxf(mx, mq[q]);
            // (with masks a row may have no page in any group: zero weights)
            const float mref = MASK && mx == -__builtin_huge_valf() ? 0.0f : mx;
            float lsum = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wq[q] = q < n_pg ? __builtin_amdgcn_exp2f(mq[q] - mref) : 0.0f;
                if (q < n_pg) lsum += wq[q] * s_ml[q * WPG + rtile][rr][1];
            }
            *reinterpret_cast<float4 *>(&s_wt[rtile][rr][0]) = make_float4(wq[0], wq[1], wq[2], wq[3]);
            if (r < rows) {
                const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
                *reinterpret_cast<float2 *>(&W.part_ml[pb * 2]) = make_float2(mx, lsum);
            }
        }
        __syncthreads();
        constexpr int D4 = DIM / 4;
        for (int idx = tid; idx < WPG * 16 * D4; idx += 256) {
            const int rtile = idx / (16 * D4);
            const int rr = (idx / D4) % 16;
            const int d4 = idx % D4;
            const int r = (i * WPG + rtile) * 16 + rr;
            if (r >= rows) continue;
            const float4 wv = *reinterpret_cast<const float4 *>(&s_wt[rtile][rr][0]);
            const float wq[4] = {wv.x, wv.y, wv.z, wv.w};
            float4 av[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                av[q] = *reinterpret_cast<const float4 *>(&s_acc[min(q * WPG + rtile, 3)][rr][4 * d4]);
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q < n_pg) {  // uniform
                    a0 += wq[q] * av[q].x;
                    a1 += wq[q] * av[q].y;
                    a2 += wq[q] * av[q].z;
                    a3 += wq[q] * av[q].w;
                }
            }
            const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
            *reinterpret_cast<float4 *>(&W.part_acc[pb * DIM + 4 * d4]) = make_float4(a0, a1, a2, a3);
        }
    }
}

// Sparse prefix, bf16, head_dim 128, chunks of 4 union pages and at most RTW
// row tiles of stacked rows.  Wave w reads the keys of the chunk's page w and
// forms its scores (S^T = K.Q^T, as in attend_pages); the scores of the 4
// pages meet in LDS.  Each wave then takes the softmax of its rows over all 4
// pages and multiplies the weights by its quarter of the output dimensions of
// V, read for all 4 pages.  So K and V are each read once, and the waves need
// no combine of outputs: each writes its dimensions of the chunk's partial,
// wave 0 the (m, l).  The union slice, the arithmetic (log2-unit scores,
// weights rounded to bf16, row sums of the rounded weights) and the partial
// layout are those of k_prefix_bf16; the row sums come from an MFMA, so they
// are added in another order.  Token masks (a prefix's partial last page, the
// union's last chunk) sit behind a uniform branch.
template <int DIM, int RTW, bool MASK, bool PAGED>
__global__ __launch_bounds__(256) void k_prefix_quarter_bf16(Dims D,
                                                             const uint16_t *__restrict__ kc,
                                                             const uint16_t *__restrict__ vc,
                                                             const int32_t *__restrict__ kv_off,
                                                             const int32_t *__restrict__ prefix_len,
                                                             Work W, int32_t *dbg_uidx,
                                                             int32_t *dbg_ucnt, int dbg_cap) {
    constexpr int KSTEPS = DIM / 32;
    constexpr int DQ = DIM / 4;    // output dimensions per wave
    constexpr int DPLQ = DQ / 16;  // PV products per page pair: 16 dimensions each
    constexpr int NP = 4;          // the chunk's pages: one per wave
    static_assert(DPLQ == 2, "one 32-bit V word per token and lane");
    __shared__ uint32_t s_bm[kMaxBitmapWords];
    __shared__ int s_wsum[4], s_pg[kMaxSparseChunk];
    __shared__ uint64_t s_rmask[MASK ? kMaxSparseChunk : 1];  // rows that selected each page
    __shared__ float4 s_sc[RTW][NP][64];                       // scores, in the MFMA's lane layout

    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int chunk = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const SeqGeom sg = seq_geom_t<PAGED>(D, kv_off, prefix_len, s);
    const int cp = D.sparse_chunk, first = chunk * cp;  // cp == NP
    const int rows = D.R, nch = D.n_chunks_sparse;
    const int n_rt = (rows + 15) / 16;

    // the rows' page lists (one entry per thread, clamped) and the Q operands,
    // requested first.  Row tiles past the rows read the last one again: their
    // scores go to LDS slots that are never read, so no load is conditional
    // (a zeroing select would be compiled as a branch around each load, with a
    // wait for all loads in flight before it)
    const int32_t *psel_g = W.psel + (size_t)sgi * rows * D.k;
    const int n_sel = rows * D.k;
    const int pre0 = psel_g[min(tid, max(n_sel - 1, 0))];
    uint4 qop[RTW][KSTEPS];
    const uint16_t *qr = static_cast<const uint16_t *>(W.qrows) + (size_t)sgi * D.R16 * DIM;
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rtc = min(i, max(n_rt - 1, 0));
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            qop[i][kk] = *reinterpret_cast<const uint4 *>(qr + (size_t)(rtc * 16 + l16) * DIM +
                                                          32 * kk + 8 * lg);
    }
    const int n_items = union_slice(psel_g, pre0, n_sel, sg.pages, D.k >= sg.pages, first, cp,
                                    s_bm, s_wsum, s_pg,
                                    dbg_uidx ? dbg_uidx + (size_t)sgi * dbg_cap : nullptr,
                                    dbg_cap, D.k, MASK ? s_rmask : nullptr);
    auto store_count = [&]() {
        if (chunk == 0 && tid == 0) {
            W.union_cnt[sgi] = min(n_items, D.union_cap);
            if (dbg_ucnt) dbg_ucnt[sgi] = n_items;
        }
    };
    if (first >= n_items) {
        store_count();
        return;
    }
    const int n_here = min(cp, n_items - first);
    const int my_page = lane < cp ? s_pg[min(lane, n_here - 1)] : 0;

    // K of page w (token l%16, dims 32*kk + 8*(l/16) ..), then this wave's
    // quarter of V for every page (tokens 4*(l/16) + j, dims DQ*w + 2*(l%16), +1);
    // slots past the chunk repeat its last page and count no token
    int valid[NP];
    size_t base[NP];
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        const int p = __builtin_amdgcn_readlane(my_page, min(n, n_here - 1));
        base[n] = ((size_t)g * D.T + (size_t)phys_page_t<PAGED>(sg, p) * kPage) * DIM;
        valid[n] = n < n_here ? min(kPage, sg.len - p * kPage) : 0;
    }
    const size_t kbase = base[min(w, n_here - 1)];
    const int kvalid = w < n_here ? valid[min(w, NP - 1)] : 0;
    // every slot a whole page (uniform): only a prefix's last page is partial,
    // and only the union's last chunk has fewer than NP pages
    const bool full = n_here == NP && valid[NP - 1] >= kPage;
    uint4 kop[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
        kop[kk] = *reinterpret_cast<const uint4 *>(kc + kbase + (size_t)l16 * DIM + 32 * kk + 8 * lg);
    uint32_t vw[NP][4];
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            vw[n][j] = *reinterpret_cast<const uint32_t *>(vc + base[n] + (size_t)(4 * lg + j) * DIM +
                                                           DQ * w + DPLQ * l16);
    __builtin_amdgcn_sched_barrier(0);  // K and V are requested together, before any is used

    // scores of page w, log2 units; tokens past the prefix (and, with row
    // masks, rows that did not select the page) get -inf
    const uint64_t rmw = MASK ? s_rmask[min(w, NP - 1)] : 0ull;
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[kk]),
                                                           __builtin_bit_cast(bf16x8_t, qop[i][kk]),
                                                           sacc, 0, 0, 0);
        float sv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[j] = sacc[j] * D.scale_log2;
        if (!full) {  // uniform branch
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * lg + j >= kvalid) sv[j] = -__builtin_huge_valf();
        }
        if constexpr (MASK) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!((rmw >> (i * 16 + l16)) & 1ull)) sv[j] = -__builtin_huge_valf();
        }
        s_sc[i][w][lane] = make_float4(sv[0], sv[1], sv[2], sv[3]);
    }
    // (the V words are held to be in use here: else the compiler issues their
    // loads only behind the barrier, a second round trip)
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(vw[n][j]));
    __syncthreads();

    // V^T operands of the wave's quarter: dim 2*(l%16) + e, tokens 4*lg .. +3,
    // one byte permute per pair of tokens (tokens past the prefix zeroed, behind
    // a uniform branch)
    u32x2_t vop2[NP][DPLQ];
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int e = 0; e < DPLQ; ++e) {
            const uint32_t sel = e ? 0x07060302u : 0x05040100u;
            vop2[n][e] = u32x2_t{__builtin_amdgcn_perm(vw[n][1], vw[n][0], sel),
                                 __builtin_amdgcn_perm(vw[n][3], vw[n][2], sel)};
        }
    if (!full) {  // uniform branch
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const uint32_t m0 = (4 * lg + 0 < valid[n] ? 0x0000ffffu : 0u) | (4 * lg + 1 < valid[n] ? 0xffff0000u : 0u);
            const uint32_t m1 = (4 * lg + 2 < valid[n] ? 0x0000ffffu : 0u) | (4 * lg + 3 < valid[n] ? 0xffff0000u : 0u);
#pragma unroll
            for (int e = 0; e < DPLQ; ++e) {
                vop2[n][e][0] &= m0;
                vop2[n][e][1] &= m1;
            }
        }
    }
    short4_t vop[NP][DPLQ];
#pragma unroll
    for (int n = 0; n < NP; ++n)
#pragma unroll
        for (int e = 0; e < DPLQ; ++e) vop[n][e] = __builtin_bit_cast(short4_t, vop2[n][e]);
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        if (i >= n_rt) break;
        float sv[NP][4];
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const float4 x = s_sc[i][n][lane];
            sv[n][0] = x.x; sv[n][1] = x.y; sv[n][2] = x.z; sv[n][3] = x.w;
        }
        float mp = -__builtin_huge_valf();
#pragma unroll
        for (int n = 0; n < NP; ++n) mp = fmaxf(mp, fmaxf(fmaxf(sv[n][0], sv[n][1]), fmaxf(sv[n][2], sv[n][3])));
        mp = shfl_max32(mp);
        // (with row masks a row may have no score in the chunk: zero weights)
        const float mref = MASK && mp == -__builtin_huge_valf() ? 0.0f : mp;
        uint2 pw[NP];
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const bf16x2_t p01 = {static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[n][0] - mref)),
                                  static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[n][1] - mref))};
            const bf16x2_t p23 = {static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[n][2] - mref)),
                                  static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[n][3] - mref))};
            pw[n] = make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
        }
        // O^T += V^T.P, pages n and n+1 in one v_mfma_f32_16x16x32_bf16 (its k
        // index 8*lg + c: token 4*lg + c%4 of page n + c/4, in both operands);
        // wave 0, which stores the (m, l), takes the rows' sums of the rounded
        // weights with one more MFMA against an all-ones operand: every output
        // row of it is the row sum, in the output's lane layout
        float4_t oacc[DPLQ], lacc = {0.f, 0.f, 0.f, 0.f};
        const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u,
                                                                      0x3f803f80u, 0x3f803f80u));
#pragma unroll
        for (int e = 0; e < DPLQ; ++e) oacc[e] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NP; n += 2) {
            const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, make_uint4(pw[n].x, pw[n].y, pw[n + 1].x, pw[n + 1].y));
            if (w == 0) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop, lacc, 0, 0, 0);  // uniform
#pragma unroll
            for (int e = 0; e < DPLQ; ++e) {
                const uint2 v0 = __builtin_bit_cast(uint2, vop[n][e]), v1 = __builtin_bit_cast(uint2, vop[n + 1][e]);
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
                oacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pop, oacc[e], 0, 0, 0);
            }
        }
        // lane l holds, for row 16*i + l%16, dims DQ*w + 2*(4*lg + j) + e: 8
        // consecutive dimensions
        const int r = i * 16 + l16;
        if (r < rows) {
            const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
            if (w == 0 && lg == 0) *reinterpret_cast<float2 *>(&W.part_ml[pb * 2]) = make_float2(mp, lacc[0]);
            float *dst = W.part_acc + pb * DIM + DQ * w + DPLQ * 4 * lg;
            *reinterpret_cast<float4 *>(dst) = make_float4(oacc[0][0], oacc[1][0], oacc[0][1], oacc[1][1]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(oacc[0][2], oacc[1][2], oacc[0][3], oacc[1][3]);
        }
    }
    store_count();  // after the waits for the pages, which would wait for it too
}

// Prefix pass over a page list streamed through LDS, bf16: the dense first
// step's chunk of consecutive pages, or (SPARSE) a sparse step's slice of the
// group's union with the stacked active rows as queries, optionally with row
// masks.  Each page of the workgroup's list is read
// from HBM once, straight into a ring of NS LDS page slots with
// global_load_lds_dwordx4 (no register staging), so NS - 2*kDenseGroup
// pages stay in flight while a group is attended.  The NW waves (row tiles w,
// w + NW, ...) read their K and V^T operands from LDS and attend kDenseGroup
// pages together.  Chunks of 8 elements are XOR-swizzled per token row (for
// d = 128, V's chunk pairs, for the transposing reads), which makes the
// operand reads free of bank conflicts; a direct load writes lane i's 16 bytes
// to LDS position i, so each lane fetches the global chunk that belongs at its
// swizzled position.  The arithmetic is k_prefix_bf16's (log2-unit scores,
// weights rounded to bf16, row sums of the rounded weights); for d = 128 the
// row sums come from an MFMA, so they are added in another order.
// LDS page slots per workgroup (ring): 6 with 4 waves (measured 2-3% faster
// than 8 or 10 on the 64K layer), 10 with 8 waves (one load per thread and page)
template <int NW>
constexpr int dense_slots() { return NW == 4 ? 6 : 10; }
constexpr int kDenseGroup = 2;   // pages attended together (independent MFMA chains)

template <int DIM>
__device__ __forceinline__ int swz(int t, int c) {
    constexpr int CPT = DIM / 8;  // 16-byte chunks per token row
    return t * CPT + (c ^ (t & (CPT - 1)));
}

// The K and V operands of two adjacent LDS page slots in one block of
// ds_read_b128: ak[kk] / av[j] are the lane's byte addresses of K chunk kk and
// V chunk j in the ring's first slot, and the pair starts SB bytes into the
// ring (an immediate offset, so no address arithmetic per pair).  Written as one asm block that
// waits for its own reads, so that the compiler, which cannot tell the ring's
// slots apart, does not make the reads wait for every direct load in flight.
// (The low 32 bits of a generic pointer into LDS are its LDS address.)
template <int DIM>
struct GroupReads;

template <>
struct GroupReads<128> {
    template <uint32_t SB>
    static __device__ __forceinline__ void read(const uint32_t (&ak)[4], const uint32_t (&av)[4],
                                                u32x4_t (&k)[2][4], u32x4_t (&v)[2][4]) {
        asm volatile(
            "ds_read_b128 %0, %16 offset:%24\n\tds_read_b128 %1, %17 offset:%24\n\t"
            "ds_read_b128 %2, %18 offset:%24\n\tds_read_b128 %3, %19 offset:%24\n\t"
            "ds_read_b128 %4, %16 offset:%25\n\tds_read_b128 %5, %17 offset:%25\n\t"
            "ds_read_b128 %6, %18 offset:%25\n\tds_read_b128 %7, %19 offset:%25\n\t"
            "ds_read_b128 %8, %20 offset:%24\n\tds_read_b128 %9, %21 offset:%24\n\t"
            "ds_read_b128 %10, %22 offset:%24\n\tds_read_b128 %11, %23 offset:%24\n\t"
            "ds_read_b128 %12, %20 offset:%25\n\tds_read_b128 %13, %21 offset:%25\n\t"
            "ds_read_b128 %14, %22 offset:%25\n\tds_read_b128 %15, %23 offset:%25\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[0][2]), "=&v"(k[0][3]),
              "=&v"(k[1][0]), "=&v"(k[1][1]), "=&v"(k[1][2]), "=&v"(k[1][3]),
              "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]),
              "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
            : "v"(ak[0]), "v"(ak[1]), "v"(ak[2]), "v"(ak[3]),
              "v"(av[0]), "v"(av[1]), "v"(av[2]), "v"(av[3]), "i"(SB), "i"(SB + 8192u)
            : "memory");
    }
};

// The K operands of two LDS page slots as GroupReads<128> reads them, and
// the V^T operands with gfx950's transposing read ds_read_b64_tr_b16: in each
// group of 16 lanes, lane a + 4k points at 4 consecutive dims of row k of the
// group's 4 token rows, and lane 4a + e receives dim e of the vectors of lanes
// a, a + 4, a + 8, a + 12.  So lane l gets one dim of tokens 4*(l/16) .. +3,
// the A operand of the PV product for its output dims: no byte permutes.
// av[f]: the lane's byte address for output block f (dims 16 f ..) in the
// ring's first slot; the pair's slots start SB and SB + 8192 bytes on.
struct GroupReadsTr128 {
    template <uint32_t SB>
    static __device__ __forceinline__ void read(const uint32_t (&ak)[4], const uint32_t (&av)[8],
                                                u32x4_t (&k)[2][4], u32x2_t (&v)[2][8]) {
        asm volatile(
            "ds_read_b128 %0, %24 offset:%36\n\t"
            "ds_read_b128 %1, %25 offset:%36\n\t"
            "ds_read_b128 %2, %26 offset:%36\n\t"
            "ds_read_b128 %3, %27 offset:%36\n\t"
            "ds_read_b128 %4, %24 offset:%37\n\t"
            "ds_read_b128 %5, %25 offset:%37\n\t"
            "ds_read_b128 %6, %26 offset:%37\n\t"
            "ds_read_b128 %7, %27 offset:%37\n\t"
            "ds_read_b64_tr_b16 %8, %28 offset:%36\n\t"
            "ds_read_b64_tr_b16 %9, %29 offset:%36\n\t"
            "ds_read_b64_tr_b16 %10, %30 offset:%36\n\t"
            "ds_read_b64_tr_b16 %11, %31 offset:%36\n\t"
            "ds_read_b64_tr_b16 %12, %32 offset:%36\n\t"
            "ds_read_b64_tr_b16 %13, %33 offset:%36\n\t"
            "ds_read_b64_tr_b16 %14, %34 offset:%36\n\t"
            "ds_read_b64_tr_b16 %15, %35 offset:%36\n\t"
            "ds_read_b64_tr_b16 %16, %28 offset:%37\n\t"
            "ds_read_b64_tr_b16 %17, %29 offset:%37\n\t"
            "ds_read_b64_tr_b16 %18, %30 offset:%37\n\t"
            "ds_read_b64_tr_b16 %19, %31 offset:%37\n\t"
            "ds_read_b64_tr_b16 %20, %32 offset:%37\n\t"
            "ds_read_b64_tr_b16 %21, %33 offset:%37\n\t"
            "ds_read_b64_tr_b16 %22, %34 offset:%37\n\t"
            "ds_read_b64_tr_b16 %23, %35 offset:%37\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[0][2]), "=&v"(k[0][3]),
              "=&v"(k[1][0]), "=&v"(k[1][1]), "=&v"(k[1][2]), "=&v"(k[1][3]),
              "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]),
              "=&v"(v[0][4]), "=&v"(v[0][5]), "=&v"(v[0][6]), "=&v"(v[0][7]),
              "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3]),
              "=&v"(v[1][4]), "=&v"(v[1][5]), "=&v"(v[1][6]), "=&v"(v[1][7])
            : "v"(ak[0]), "v"(ak[1]), "v"(ak[2]), "v"(ak[3]),
              "v"(av[0]), "v"(av[1]), "v"(av[2]), "v"(av[3]), "v"(av[4]), "v"(av[5]), "v"(av[6]), "v"(av[7]),
              "i"(SB), "i"(SB + 8192u)
            : "memory");
    }
};

template <>
struct GroupReads<64> {
    template <uint32_t SB>
    static __device__ __forceinline__ void read(const uint32_t (&ak)[2], const uint32_t (&av)[4],
                                                u32x4_t (&k)[2][2], u32x4_t (&v)[2][4]) {
        asm volatile(
            "ds_read_b128 %0, %12 offset:%18\n\tds_read_b128 %1, %13 offset:%18\n\t"
            "ds_read_b128 %2, %12 offset:%19\n\tds_read_b128 %3, %13 offset:%19\n\t"
            "ds_read_b128 %4, %14 offset:%18\n\tds_read_b128 %5, %15 offset:%18\n\t"
            "ds_read_b128 %6, %16 offset:%18\n\tds_read_b128 %7, %17 offset:%18\n\t"
            "ds_read_b128 %8, %14 offset:%19\n\tds_read_b128 %9, %15 offset:%19\n\t"
            "ds_read_b128 %10, %16 offset:%19\n\tds_read_b128 %11, %17 offset:%19\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[1][0]), "=&v"(k[1][1]),
              "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[0][3]),
              "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[1][2]), "=&v"(v[1][3])
            : "v"(ak[0]), "v"(ak[1]), "v"(av[0]), "v"(av[1]), "v"(av[2]), "v"(av[3]), "i"(SB),
              "i"(SB + 4096u)
            : "memory");
    }
};

// f(IntC<I>{}) for I = 0, 1, .., N - 1 while f returns true (a loop body
// that needs I as a constant)
template <int I>
struct IntC {
    static constexpr int value = I;
};
template <int I, int N, typename F>
__device__ __forceinline__ void static_while(F &&f) {
    if constexpr (I < N) {
        if (f(IntC<I>{})) static_while<I + 1, N>(f);
    }
}

// s_waitcnt with only the vector-memory counter: at most N loads in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int DIM, int RTW, int NW, bool SPARSE, bool MASK, bool PAGED>
__global__ __launch_bounds__(64 * NW) void k_prefix_ring_bf16(Dims D, const uint16_t *__restrict__ q_t,
                                                              const uint16_t *__restrict__ kc,
                                                              const uint16_t *__restrict__ vc,
                                                              const int32_t *__restrict__ kv_off,
                                                              const int32_t *__restrict__ prefix_len,
                                                              Work W, int32_t *dbg_uidx,
                                                              int32_t *dbg_ucnt, int dbg_cap) {
    constexpr int KSTEPS = DIM / 32, DPL = DIM / 16, CPT = DIM / 8;
    constexpr bool TR = DIM == 128;          // V^T operands by transposing LDS reads
    constexpr int NCK = 16 * CPT;            // 16-byte chunks per page and tensor
    constexpr int NT = 64 * NW;              // threads
    constexpr int LPT = 2 * NCK / NT;        // direct loads per thread per page (K and V)
    static_assert(LPT >= 1 && LPT * NT == 2 * NCK, "whole wave loads per page");
    constexpr int NS = dense_slots<NW>(), NG = kDenseGroup;
    static_assert(NS % NG == 0 && NS >= 2 * NG, "the ring holds whole groups");
    // loads each thread may leave in flight when a group must have landed: the
    // pages of the groups after it that have been issued
    constexpr int kAhead = LPT * (NS - 2 * NG);
    static_assert(!SPARSE || NW == 4, "the union slice is built by 256 threads");
    static_assert(!MASK || (SPARSE && RTW == 1), "row masks: sparse pass, at most 64 rows");
    __shared__ uint4 s_page[NS][2 * NCK];  // [slot][K chunks, then V chunks], swizzled
    // the union bitmap (sparse pass) lives in the ring where it fits: the ring
    // is first written after the union slice's last barrier
    constexpr bool kBmInRing = sizeof(uint4) * NS * 2 * NCK >= 4 * kMaxBitmapWords;
    __shared__ uint32_t s_bm[SPARSE && !kBmInRing ? kMaxBitmapWords : 1];
    __shared__ int s_wsum[4], s_pg[SPARSE ? kMaxSparseChunk : 1];
    __shared__ uint64_t s_rmask[MASK ? kMaxSparseChunk : 1];  // rows that selected each page
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int chunk = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lg = lane >> 4;
    const SeqGeom sg = seq_geom_t<PAGED>(D, kv_off, prefix_len, s);
    const int cp = SPARSE ? D.sparse_chunk : D.dense_chunk;
    const int first = chunk * cp;
    if (!SPARSE && first >= sg.pages) return;
    const int rows = SPARSE ? D.R : D.Rd, nch = SPARSE ? D.n_chunks_sparse : D.n_chunks_dense;
    const int n_rt = (rows + 15) / 16;

    // Sparse pass: the rows' page lists (one entry per thread, clamped),
    // requested first, for the union slice below
    const int32_t *psel_g = W.psel + (size_t)sgi * (rows > 0 ? rows : 1) * D.k;
    const int n_sel = rows * D.k;
    const int pre0 = SPARSE ? psel_g[min(tid, max(n_sel - 1, 0))] : 0;
    // Q operands (B of QK^T) of row tiles w + NW*i.  Dense pass: straight from
    // the block queries, row r = j*B + t of the group being head g*G + j, token
    // t (rows past the group read its last row; their outputs are not stored).
    // Sparse pass: the stacked active rows of the group, zero-padded to whole
    // tiles.  Lane l holds row l%16, dims 32*kk + 8*(l/16) .. +7.  Issued
    // before any page so that waiting for them never waits for a page.
    uint4 qop[RTW][KSTEPS];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = min(w + NW * i, n_rt - 1);
        const uint16_t *qrow;
        if constexpr (SPARSE) {
            qrow = static_cast<const uint16_t *>(W.qrows) + ((size_t)sgi * D.R16 + rt * 16 + l16) * DIM;
        } else {
            const int r = min(rt * 16 + l16, rows - 1);
            qrow = q_t + ((size_t)(s * D.B + r % D.B) * D.Hq + g * D.G + r / D.B) * DIM;
        }
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
            qop[i][kk] = *reinterpret_cast<const uint4 *>(qrow + 32 * kk + 8 * lg);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the chunk's pages: the dense pass's consecutive ones, or the sparse
    // pass's slice of the group's union (chunk 0 records the union size)
    int n_items = sg.pages;
    if constexpr (SPARSE) {
        uint32_t *bm = kBmInRing ? reinterpret_cast<uint32_t *>(&s_page[0][0]) : s_bm;
        n_items = union_slice(psel_g, pre0, n_sel, sg.pages, D.k >= sg.pages, first, cp, bm, s_wsum,
                              s_pg, dbg_uidx ? dbg_uidx + (size_t)sgi * dbg_cap : nullptr, dbg_cap, D.k,
                              MASK ? s_rmask : nullptr);
        if (chunk == 0 && tid == 0) {
            W.union_cnt[sgi] = min(n_items, D.union_cap);
            if (dbg_ucnt) dbg_ucnt[sgi] = n_items;
        }
        if (first >= n_items) return;
    }
    const int n_here = min(cp, n_items - first);

    // Direct load h of a page: wave w writes LDS chunks (h*NW + w)*64 .. +63 of
    // the slot; lane i's chunk L holds token t = (L % NCK) / CPT, swizzled column
    // c' = (L % NCK) % CPT, i.e. global column c' ^ (t & (CPT-1)) of K (L < NCK) or V.
    const uint16_t *src_h[LPT];
#pragma unroll
    for (int h = 0; h < LPT; ++h) {
        const int L = (h * NW + w) * 64 + lane, cq = L % NCK;
        // K: chunks XOR-swizzled by the token row; V with the transposing
        // reads (d = 128): chunk pairs (32 bytes) XOR-swizzled by the row's
        // low 3 bits
        const int t = cq / CPT;
        const int c = (L < NCK || !TR) ? (cq % CPT) ^ (t & (CPT - 1)) : (cq % CPT) ^ ((t & 7) << 1);
        src_h[h] = (L < NCK ? kc : vc) + (size_t)g * D.T * DIM + t * DIM + c * 8;
    }
    // the sequence page and the cache row of each page of the chunk: lane i
    // holds the chunk's page i (clamped to its last page; a page table is read
    // once here)
    const int my_page = SPARSE ? s_pg[min(lane, n_here - 1)] : first + min(lane, n_here - 1);
    const int64_t prow_lane = phys_page_t<PAGED>(sg, my_page) * kPage;
    auto seq_page = [&](int q) {  // the chunk's page q (uniform)
        return SPARSE ? __builtin_amdgcn_readlane(my_page, q) : first + q;
    };
    // (the builtin's arguments are passed as plain void pointers: with typed or
    // const ones the host pass silently drops the kernel's launch stub)
    // Workgroups take their chunk's pages in a rotated order, starting at page
    // blockIdx.x mod n_here, so that the many streams in flight at once do
    // not walk the same offsets of their regions in step (measured 1 us faster
    // on the 64K layer); attention over a set of pages does not depend on
    // their order beyond rounding.
    const int rot = static_cast<int>(blockIdx.x % static_cast<unsigned>(n_here));
    auto rp = [&](int p) { return p + rot < n_here ? p + rot : p + rot - n_here; };  // p < n_here
    auto issue = [&](int p, int slot) {  // page p of the chunk (clamped) into a slot
        const int pc = rp(min(p, n_here - 1));
        const int64_t prow = static_cast<int64_t>(
            (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                 static_cast<int>(prow_lane >> 32), pc))) << 32) |
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(prow_lane), pc)));
        const size_t off = (size_t)prow * DIM;
#pragma unroll
        for (int h = 0; h < LPT; ++h)
            __builtin_amdgcn_global_load_lds(static_cast<void *>(const_cast<uint16_t *>(src_h[h] + off)),
                                             static_cast<void *>(&s_page[slot][(h * NW + w) * 64]),
                                             16, 0, 0);
    };
#pragma unroll
    for (int p = 0; p < NS; ++p) issue(p, p);
    // the Q operands have landed; the ring's loads may still be in flight
    wait_vmcnt<LPT * NS>();

    float4_t oacc[RTW][DPL];
    float m_run[RTW], l_run[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        m_run[i] = -__builtin_huge_valf();
        l_run[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) oacc[i][e] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    bool rt_ok[RTW];
#pragma unroll
    for (int i = 0; i < RTW; ++i) rt_ok[i] = w + NW * i < n_rt;
    float4_t l4[RTW];  // (transposing reads) the rows' weight sums from the MFMA
#pragma unroll
    for (int i = 0; i < RTW; ++i) l4[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    // the lane's operand chunks inside a slot (bytes): K chunk (token l%16,
    // dims 32*kk + 8*(l/16) ..) and V chunk (token 4*(l/16) + j, dims DPL*(l%16) ..)
    static_assert(NG == 2, "operand reads are written for page pairs");
    constexpr int SLOT_BYTES = 2 * NCK * 16;
    const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&s_page[0][0]));
    uint32_t ak[KSTEPS], av[4];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) ak[kk] = ring + 16u * swz<DIM>(l16, 4 * kk + lg);
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = ring + 16u * (NCK + swz<DIM>(4 * lg + j, (DPL * l16) / 8));
    // (transposing reads) the lane's V address per output block f: token row
    // 4*lg + l16/4, dims 16 f + 4*(l16 % 4) .. +3, in the pair-swizzled layout
    uint32_t avt[TR ? 8 : 1];
    if constexpr (TR) {
        const int t = 4 * lg + (l16 >> 2), a = l16 & 3;
#pragma unroll
        for (int f = 0; f < 8; ++f)
            avt[f] = ring + 16u * NCK + 256u * t + 32u * static_cast<uint32_t>(f ^ (t & 7)) + 8u * a;
    }

    // Group at pages pi .. pi+NG-1 (slots pi % NS ..): loads are issued in page
    // order and complete in order, and when the group is due the pages issued
    // after it are at most NS - 2*NG (the prologue's NS pages, then NG per group
    // from the second on), so once at most kAhead of this thread's loads are in
    // flight the group's pieces of this thread have landed.  The barrier then
    // covers every thread's pieces, and tells that the previous group's slots
    // are no longer read, so they are refilled with the pages NS ahead (clamped
    // to the chunk's last page: slots past the chunk are never attended).
    // The ring holds NSG groups; the loop body is unrolled over them, so that
    // each group's slots are a constant offset in its LDS reads.
    constexpr int NSG = NS / NG;
    auto group = [&](auto sgc, int pi) {
        constexpr int SG = decltype(sgc)::value;  // pages pi.. sit in slots SG*NG ..
        // the pair's byte offset in the ring; LDS offsets have 16 bits, so a
        // pair that ends past 64 KiB (10 slots of d = 128) adds 64 KiB to the
        // addresses instead
        constexpr uint32_t HI = SG * NG * SLOT_BYTES + NG * SLOT_BYTES > 0x10000u ? 0x10000u : 0u;
        constexpr uint32_t SB = SG * NG * SLOT_BYTES - HI;
        uint32_t akh[KSTEPS], avh[TR ? 8 : 4];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) akh[kk] = ak[kk] + HI;
        if constexpr (TR) {
#pragma unroll
            for (int f = 0; f < 8; ++f) avh[f] = avt[f] + HI;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) avh[j] = av[j] + HI;
        }
        wait_vmcnt<kAhead>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (pi > 0) {  // (the first group waits for a little more than it needs)
#pragma unroll
            for (int n = 0; n < NG; ++n) issue(pi - NG + n + NS, ((SG + NSG - 1) % NSG) * NG + n);
        }
        __builtin_amdgcn_sched_barrier(0);
        // (row masks) the rows that selected each page of the pair, and the
        // first row of the wave's row tile
        uint64_t rm[NG];
#pragma unroll
        for (int n = 0; n < NG; ++n) rm[n] = MASK && pi + n < n_here ? s_rmask[rp(pi + n)] : 0ull;
        int row0[RTW];
#pragma unroll
        for (int i = 0; i < RTW; ++i) row0[i] = (w + NW * i) * 16;
        if constexpr (TR) {
            u32x4_t kraw[NG][KSTEPS];
            u32x2_t vtr[NG][8];
            GroupReadsTr128::read<SB>(akh, avh, kraw, vtr);
            uint4 kop[NG][KSTEPS];
            int valid[NG];
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                valid[n] = pi + n < n_here ? min(kPage, sg.len - seq_page(rp(pi + n)) * kPage) : 0;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) kop[n][kk] = __builtin_bit_cast(uint4, kraw[n][kk]);
            }
            // the PV operand of block f: page pi's tokens, then page pi + 1's
            u32x4_t vpair[1][DPL];
#pragma unroll
            for (int f = 0; f < DPL; ++f)
                vpair[0][f] = u32x4_t{vtr[0][f].x, vtr[0][f].y, vtr[1][f].x, vtr[1][f].y};
            if (valid[0] < kPage || valid[1] < kPage) {  // uniform; only a prefix's last pages
                // (the empty asm keeps this rare masking behind the branch
                // instead of turning it into selects on every page pair)
                asm volatile("");
                u32x4_t vm;  // tokens 4*lg .. +3 of each page past the prefix zeroed
#pragma unroll
                for (int n = 0; n < NG; ++n) {
                    vm[2 * n] = (4 * lg + 0 < valid[n] ? 0x0000ffffu : 0u) | (4 * lg + 1 < valid[n] ? 0xffff0000u : 0u);
                    vm[2 * n + 1] = (4 * lg + 2 < valid[n] ? 0x0000ffffu : 0u) | (4 * lg + 3 < valid[n] ? 0xffff0000u : 0u);
                }
#pragma unroll
                for (int f = 0; f < DPL; ++f) vpair[0][f] &= vm;
            }
            short4_t vop_none[1][DPL];
            attend_core<DIM, RTW, NG, MASK, true>(kop, vpair, vop_none, valid, qop, rt_ok, D.scale_log2,
                                                  oacc, m_run, l_run, lg, rm, row0, l4);
        } else {
            u32x4_t kraw[NG][KSTEPS], vraw[NG][4];
            GroupReads<DIM>::template read<SB>(akh, avh, kraw, vraw);

            uint4 kop[NG][KSTEPS];
            uint32_t vw[NG][4][DPL / 2];
            int valid[NG];
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                // a page past the chunk (odd count) attends nothing
                valid[n] = pi + n < n_here ? min(kPage, sg.len - seq_page(rp(pi + n)) * kPage) : 0;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk) kop[n][kk] = __builtin_bit_cast(uint4, kraw[n][kk]);
                // V words of tokens 4*lg + j for the lane's dims DPL*l16 .. +DPL-1
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4_t c4 = vraw[n][j];
                    if constexpr (DPL == 8) {
                        vw[n][j][0] = c4[0]; vw[n][j][1] = c4[1]; vw[n][j][2] = c4[2]; vw[n][j][3] = c4[3];
                    } else {
                        const bool hi = (l16 & 1) != 0;
                        vw[n][j][0] = hi ? c4[2] : c4[0];
                        vw[n][j][1] = hi ? c4[3] : c4[1];
                    }
                }
            }
            attend_pages<DIM, RTW, NG, MASK>(kop, vw, valid, qop, rt_ok, D.scale_log2, oacc, m_run, l_run,
                                             lg, rm, row0);
        }
    };
    for (int p0 = 0; p0 < n_here; p0 += NS)
        static_while<0, NSG>([&](auto sgc) {
            const int pi = p0 + decltype(sgc)::value * NG;
            if (pi >= n_here) return false;
            group(sgc, pi);
            return true;
        });
    // no direct load may still be writing LDS when the workgroup ends
    wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < RTW; ++i) l_run[i] = TR ? l4[i][0] : shfl_sum32(l_run[i]);

    // Lane l holds, for row l%16, dims DPL*(4*lg + j) + e (transposing reads:
    // dims 16 e + 4*lg + j).  The dense pass stores its partials
    // non-temporally: every workgroup stores at about the same time, at the
    // end, and stores that skip the L2 leave no dirty lines for the kernel's
    // end to write back (measured 2.4 us shorter on the 64K layer; the
    // finishing kernel then reads them 0.4 us more slowly).  The sparse pass's
    // few partials are read sooner from the L2 (its finish took 0.9 us longer
    // with non-temporal stores).
    auto st4 = [](float *p, float a, float b, float c, float d) {
        if constexpr (SPARSE) *reinterpret_cast<float4_t *>(p) = float4_t{a, b, c, d};
        else __builtin_nontemporal_store(float4_t{a, b, c, d}, reinterpret_cast<float4_t *>(p));
    };
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = w + NW * i;
        if (rt >= n_rt) break;
        const int r = rt * 16 + l16;
        if (r >= rows) continue;
        const size_t pb = ((size_t)sgi * nch + chunk) * rows + r;
        if (lg == 0) {
            if constexpr (SPARSE) {
                W.part_ml[pb * 2 + 0] = m_run[i];
                W.part_ml[pb * 2 + 1] = l_run[i];
            } else {
                __builtin_nontemporal_store(m_run[i], &W.part_ml[pb * 2 + 0]);
                __builtin_nontemporal_store(l_run[i], &W.part_ml[pb * 2 + 1]);
            }
        }
        float *dst = W.part_acc + pb * DIM;
        if constexpr (TR) {
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                st4(dst + 16 * e + 4 * lg, oacc[i][e][0], oacc[i][e][1], oacc[i][e][2], oacc[i][e][3]);
            continue;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float tmp[DPL];
#pragma unroll
            for (int e = 0; e < DPL; ++e) tmp[e] = oacc[i][e][j];
            float *d0 = dst + DPL * (4 * lg + j);
#pragma unroll
            for (int e = 0; e < DPL; e += 4) st4(d0 + e, tmp[e], tmp[e + 1], tmp[e + 2], tmp[e + 3]);
        }
    }
}

template <int DIM, bool DENSE, bool MASK>
__global__ __launch_bounds__(256) void k_prefix_f32(Dims D, const float *__restrict__ kc,
                                                    const float *__restrict__ vc,
                                                    const int32_t *__restrict__ kv_off,
                                                    const int32_t *__restrict__ prefix_len, Work W,
                                                    int32_t *dbg_uidx, int32_t *dbg_ucnt, int dbg_cap) {
    constexpr bool dense = DENSE;
    constexpr int DPT = DIM / 16;
    __shared__ uint32_t s_bm[kMaxBitmapWords];
    __shared__ int s_wsum[4], s_pg[kMaxSparseChunk];
    __shared__ uint64_t s_rmask[MASK ? kMaxSparseChunk : 1];  // rows that selected each page
    __shared__ float q_s[16][DIM];
    __shared__ float k_s[16][DIM + 1];
    __shared__ float v_s[16][DIM];
    __shared__ float s_s[16][17];
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng;
    const int chunk = blockIdx.x / ng;
    const int s = sgi / D.Hk, g = sgi % D.Hk;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    const int cp = dense ? D.dense_chunk : D.sparse_chunk;
    const int first = chunk * cp;
    int n_items;
    if (dense) {
        n_items = sg.pages;
    } else {
        const int32_t *psel_g = W.psel + (size_t)sgi * (D.R > 0 ? D.R : 1) * D.k;
        const int n_sel = D.R * D.k;
        const int pre0 = psel_g[min(static_cast<int>(threadIdx.x), max(n_sel - 1, 0))];
        n_items = union_slice(psel_g, pre0, n_sel, sg.pages, D.k >= sg.pages,
                              first, cp, s_bm, s_wsum, s_pg,
                              dbg_uidx ? dbg_uidx + (size_t)sgi * dbg_cap : nullptr,
                              dbg_cap, D.k, MASK ? s_rmask : nullptr);
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
            const size_t base = ((size_t)g * D.T + (size_t)phys_page(sg, p) * kPage) * DIM;
            __syncthreads();
            for (int idx = tid; idx < 16 * DIM; idx += 256) {
                const int t = idx / DIM, x = idx % DIM;
                k_s[t][x] = kc[base + idx];
                v_s[t][x] = t < valid ? vc[base + idx] : 0.0f;
            }
            __syncthreads();
            float dot = 0.0f;
            for (int x = 0; x < DIM; ++x) dot = fmaf(q_s[r16][x], k_s[j16][x], dot);
            bool keep = j16 < valid;
            if constexpr (MASK) keep = keep && ((s_rmask[it] >> (rt * 16 + r16)) & 1ull);
            s_s[r16][j16] = keep ? dot * D.scale_log2 : -__builtin_huge_valf();
            __syncthreads();
            float mp = -__builtin_huge_valf();
            for (int u = 0; u < 16; ++u) mp = fmaxf(mp, s_s[r16][u]);
            const float mn = fmaxf(m_run, mp);
            // (with masks a row may have seen no score yet: its weights are zero)
            const float mref = MASK && mn == -__builtin_huge_valf() ? 0.0f : mn;
            const float alpha = exp2f(m_run - mref);
            float pu[16], ls = 0.0f;
            for (int u = 0; u < 16; ++u) {
                pu[u] = exp2f(s_s[r16][u] - mref);
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

hipError_t launch_prefix(const Dims &D, bool dense, const void *q_t, const void *k_cache,
                         const void *v_cache, const int32_t *kv_off, const int32_t *prefix_len,
                         const Work &W, int32_t *dbg_uidx, int32_t *dbg_ucnt, int dbg_cap,
                         hipStream_t st) {
    const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
    dim3 grid(nch * D.S * D.Hk);
    const bool paged = D.page_table != nullptr;
    if (D.bf16) {
        auto *k = static_cast<const uint16_t *>(k_cache);
        auto *v = static_cast<const uint16_t *>(v_cache);
        const int rows = dense ? D.Rd : D.R;
        const int n_rt = (rows + 15) / 16;
        const int rtw = n_rt <= 4 ? 1 : (n_rt <= 8 ? 2 : 4);
#define LAUNCH_P(DIMV, RTWV, DN, MK)                                                              \
    hipLaunchKernelGGL((k_prefix_bf16<DIMV, RTWV, DN, MK>), grid, dim3(256), 0, st, D, k, v, kv_off, \
                       prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap)
        // row masks: at most 64 rows, so one row tile per wave
#define PICK_P(DIMV, DN)                                     \
    do {                                                     \
        if (D.flags & LOSA_FLAG_ROW_MASK) LAUNCH_P(DIMV, 1, DN, true); \
        else if (rtw == 1) LAUNCH_P(DIMV, 1, DN, false);     \
        else if (rtw == 2) LAUNCH_P(DIMV, 2, DN, false);     \
        else LAUNCH_P(DIMV, 4, DN, false);                   \
    } while (0)
#define LAUNCH_R(DIMV, RTWV, NWV, SP, MK)                                                         \
    do {                                                                                          \
        if (paged)                                                                                \
            hipLaunchKernelGGL((k_prefix_ring_bf16<DIMV, RTWV, NWV, SP, MK, true>), grid,           \
                               dim3(64 * NWV), 0, st, D, static_cast<const uint16_t *>(q_t), k, v, \
                               kv_off, prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap);             \
        else                                                                                      \
            hipLaunchKernelGGL((k_prefix_ring_bf16<DIMV, RTWV, NWV, SP, MK, false>), grid,          \
                               dim3(64 * NWV), 0, st, D, static_cast<const uint16_t *>(q_t), k, v, \
                               kv_off, prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap);             \
    } while (0)
#define LAUNCH_D(DIMV, RTWV, NWV) LAUNCH_R(DIMV, RTWV, NWV, false, false)
        // dense pass: wave w of NW takes row tiles w, w + NW, ...; head_dim 128
        // with up to 8 row tiles takes 4 waves of two row tiles each (two
        // independent chains per wave at 210 VGPRs, two workgroups per CU,
        // where 8 waves of one row tile at 164 VGPRs fit one per CU: the ragged
        // batch's dense first step takes 409 us instead of 496), beyond that 8
        // waves of two (one page of K and V is one 16-byte piece per thread)
        if (D.d == 128) {
            if (dense) {
                if (n_rt <= 4) LAUNCH_D(128, 1, 4);
                else if (n_rt <= 8) LAUNCH_D(128, 2, 4);
                else LAUNCH_D(128, 2, 8);
            } else if (D.sparse_chunk == 4 && n_rt <= 2) {
                // chunks of 4 pages, at most 32 rows: waves split the dimensions
                const bool mk = D.flags & LOSA_FLAG_ROW_MASK;
#define LAUNCH_Q(RTWV, MK)                                                                          \
    do {                                                                                            \
        if (paged)                                                                                  \
            hipLaunchKernelGGL((k_prefix_quarter_bf16<128, RTWV, MK, true>), grid, dim3(256), 0, st, \
                               D, k, v, kv_off, prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap);      \
        else                                                                                        \
            hipLaunchKernelGGL((k_prefix_quarter_bf16<128, RTWV, MK, false>), grid, dim3(256), 0,   \
                               st, D, k, v, kv_off, prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap);  \
    } while (0)
                if (n_rt == 1) {
                    if (mk) LAUNCH_Q(1, true);
                    else LAUNCH_Q(1, false);
                } else {
                    if (mk) LAUNCH_Q(2, true);
                    else LAUNCH_Q(2, false);
                }
#undef LAUNCH_Q
            } else if (D.flags & LOSA_FLAG_ROW_MASK ? n_rt <= 4 : n_rt <= 8) {
                // larger union slices stream through the dense pass's LDS ring
                if (D.flags & LOSA_FLAG_ROW_MASK) LAUNCH_R(128, 1, 4, true, true);
                else if (n_rt <= 4) LAUNCH_R(128, 1, 4, true, false);
                else LAUNCH_R(128, 2, 4, true, false);
            } else {
                PICK_P(128, false);
            }
        } else {
            if (dense) {
                if (n_rt <= 4) LAUNCH_D(64, 1, 4);
                else if (n_rt <= 8) LAUNCH_D(64, 2, 4);
                else LAUNCH_D(64, 4, 4);
            } else if (D.flags & LOSA_FLAG_ROW_MASK ? n_rt <= 4 : n_rt <= 8) {
                if (D.flags & LOSA_FLAG_ROW_MASK) LAUNCH_R(64, 1, 4, true, true);
                else if (n_rt <= 4) LAUNCH_R(64, 1, 4, true, false);
                else LAUNCH_R(64, 2, 4, true, false);
            } else {
                PICK_P(64, false);
            }
        }
#undef LAUNCH_D
#undef LAUNCH_R
#undef PICK_P
#undef LAUNCH_P
    } else {
        auto *k = static_cast<const float *>(k_cache);
        auto *v = static_cast<const float *>(v_cache);
#define LAUNCH_F(DIMV, DN, MK)                                                                  \
    hipLaunchKernelGGL((k_prefix_f32<DIMV, DN, MK>), grid, dim3(256), 0, st, D, k, v, kv_off,   \
                       prefix_len, W, dbg_uidx, dbg_ucnt, dbg_cap)
        const bool mask = !dense && (D.flags & LOSA_FLAG_ROW_MASK);
        if (D.d == 128) {
            if (dense) LAUNCH_F(128, true, false);
            else if (mask) LAUNCH_F(128, false, true);
            else LAUNCH_F(128, false, false);
        } else {
            if (dense) LAUNCH_F(64, true, false);
            else if (mask) LAUNCH_F(64, false, true);
            else LAUNCH_F(64, false, false);
        }
#undef LAUNCH_F
    }
    return hipGetLastError();
}

}  // namespace losa
