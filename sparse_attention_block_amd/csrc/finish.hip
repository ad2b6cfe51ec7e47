// Finishing kernel, one workgroup per (sequence, query head, group of block
// tokens):
//  * active rows (every row on a dense first step): combine the prefix
//    workgroups' partial statistics in chunk order into (o_p, L_p) and
//    overwrite the cache entry -- "updated statistics are stored for the next
//    step" (gist.science pt summary, "3. Metodologia", step 4);
//  * stable rows: read the cached (o_p, L_p) unchanged (pt step 2);
//  * dense attention of the tokens over the B in-block keys/values, giving
//    (o_s, L_s) (agifrontier tutorial, workflow section: the block is short
//    and attended densely);
//  * the online-softmax merge L = log(e^L_p + e^L_s),
//    out = e^(L_p-L) o_p + e^(L_s-L) o_s, rounded to the storage type.
// The reads that depend on no other read (block keys, queries, the active
// list, the union size) are requested together; one wave per candidate row
// reduces the partial maxima and sums, and the partial outputs and block
// values are read in unrolled batches.  All arithmetic is fp32; scores and
// log-normalisers are in log2 units inside.
#include "losa_internal.h"

namespace losa {

template <typename T>
__device__ __forceinline__ float ldv(const T *p, size_t i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else return reinterpret_cast<const float *>(p)[i];
}

constexpr int kFinishThreads = 512;
constexpr int kFinishWaves = kFinishThreads / 64;

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T, int DIM>
__global__ __launch_bounds__(kFinishThreads) void k_finish(
    Dims D, int dense, int TG, const T *__restrict__ q_t, const T *__restrict__ k_blk,
    const T *__restrict__ v_blk, const int32_t *__restrict__ kv_off,
    const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ active,
    const int32_t *__restrict__ union_cnt, const float *__restrict__ part_ml,
    const float *__restrict__ part_acc, float *__restrict__ op_cache,
    float *__restrict__ lp_cache, T *__restrict__ out) {
    constexpr float kLn2 = 0.69314718055994530942f;
    constexpr float kLog2e = 1.44269504088896340736f;
    extern __shared__ float sm[];
    const int B = D.B, G = D.G;
    const int t0 = blockIdx.x * TG, h = blockIdx.y, s = blockIdx.z;
    const int nt = min(TG, B - t0);
    const int g = h / G, j = h % G;
    const int sgi = s * D.Hk + g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
    const int rows = dense ? D.Rd : D.R;
    // candidate prefix rows: the |A| stacked rows of this head (sparse) or this
    // group's tokens (dense); rho indexes them
    const int NR = dense ? nt : D.A;
    const int row0 = dense ? j * B + t0 : j * D.A;

    // LDS: at most 64*129 + 16*128 + 16*64 + 16 + 4*64 words (< 48 KiB)
    float *kb = sm;                        // [B][DIM + 1]
    float *qs = kb + B * (DIM + 1);        // [TG][DIM]
    float *ps = qs + TG * DIM;             // [TG][B] scores, then softmax weights
    float *ls2 = ps + TG * B;              // [TG] L_s (log2 units)
    float *rst = ls2 + TG;                 // [NR][3] per candidate row: max, 1/sum, L_p (log2)
    int *act = reinterpret_cast<int *>(rst + 3 * NR);  // [NR] token of candidate row (sparse)

    // the number of prefix chunks that wrote partials (uniform scalar load,
    // requested before the block loads so that its latency overlaps them)
    int nchu;
    {
        const int cp = dense ? kDenseChunk : kSparseChunk;
        int n_items;
        if (dense) n_items = seq_geom(D, kv_off, prefix_len, s).pages;
        else n_items = union_cnt[sgi];
        nchu = (n_items + cp - 1) / cp;
    }
    for (int idx = tid; idx < B * DIM; idx += blockDim.x) {
        const int u = idx / DIM, x = idx % DIM;
        kb[u * (DIM + 1) + x] = ldv(k_blk, ((size_t)(s * B + u) * D.Hk + g) * DIM + x);
    }
    for (int idx = tid; idx < nt * DIM; idx += blockDim.x) {
        const int t = idx / DIM, x = idx % DIM;
        qs[t * DIM + x] = ldv(q_t, ((size_t)(s * B + t0 + t) * D.Hq + h) * DIM + x);
    }
    if (!dense && tid < NR) act[tid] = active[((size_t)s * D.Hq + h) * D.A + tid];
    // per candidate row, one wave reduces the chunk maxima and sums
    for (int rho = wave; rho < NR; rho += kFinishWaves) {
        const float *ml = part_ml + ((size_t)sgi * nch * rows + row0 + rho) * 2;
        const size_t cs = (size_t)rows * 2;
        float mx = -__builtin_huge_valf();
        for (int c = lane; c < nchu; c += 64) mx = fmaxf(mx, ml[c * cs]);
        mx = wave_max_f(mx);
        float ls = 0.0f;
        for (int c = lane; c < nchu; c += 64)
            ls = fmaf(__builtin_amdgcn_exp2f(ml[c * cs] - mx), ml[c * cs + 1], ls);
        ls = wave_sum_f(ls);
        if (lane == 0) {
            rst[3 * rho] = mx;
            rst[3 * rho + 1] = nchu > 0 ? 1.0f / ls : 0.0f;
            rst[3 * rho + 2] = nchu > 0 ? mx + __log2f(ls) : -__builtin_huge_valf();
        }
    }
    __syncthreads();

    // block scores q.k (scaled, log2 units)
    for (int pr = tid; pr < nt * B; pr += blockDim.x) {
        const int t = pr / B, u = pr % B;
        float dot = 0.0f;
#pragma unroll 8
        for (int x = 0; x < DIM; ++x) dot = fmaf(qs[t * DIM + x], kb[u * (DIM + 1) + x], dot);
        ps[t * B + u] = dot * D.scale_log2;
    }
    __syncthreads();
    if (tid < nt) {
        float m = -__builtin_huge_valf();
        for (int u = 0; u < B; ++u) m = fmaxf(m, ps[tid * B + u]);
        float l = 0.0f;
        for (int u = 0; u < B; ++u) {
            const float p = __builtin_amdgcn_exp2f(ps[tid * B + u] - m);
            ps[tid * B + u] = p;
            l += p;
        }
        const float inv = 1.0f / l;
        for (int u = 0; u < B; ++u) ps[tid * B + u] *= inv;
        ls2[tid] = m + __log2f(l);
    }
    __syncthreads();

    // outputs: one thread per (token, dimension)
    for (int item = tid; item < nt * DIM; item += blockDim.x) {
        const int t = item / DIM, x = item % DIM;
        const int tok = t0 + t;
        const size_t crow = ((size_t)s * D.Hq + h) * B + tok;
        int rho = -1;
        if (dense) {
            rho = t;
        } else {
            for (int a = 0; a < NR; ++a)
                if (act[a] == tok) rho = a;
        }
        float op, lp2;
        if (rho >= 0) {
            // chunk weights exp2(m_c - max) / sum, applied to the partial outputs
            const float mx = rst[3 * rho], inv = rst[3 * rho + 1];
            lp2 = rst[3 * rho + 2];
            const float *acc = part_acc + ((size_t)sgi * nch * rows + row0 + rho) * DIM + x;
            const float *ml = part_ml + ((size_t)sgi * nch * rows + row0 + rho) * 2;
            const size_t as = (size_t)rows * DIM, cs = (size_t)rows * 2;
            op = 0.0f;
#pragma unroll 16
            for (int c = 0; c < nchu; ++c)
                op = fmaf(__builtin_amdgcn_exp2f(ml[c * cs] - mx), acc[c * as], op);
            op *= inv;
            op_cache[crow * DIM + x] = op;
            if (x == 0) lp_cache[crow] = lp2 * kLn2;
        } else {
            op = op_cache[crow * DIM + x];
            lp2 = lp_cache[crow] * kLog2e;
        }
        const T *vcol = v_blk + ((size_t)s * B * D.Hk + g) * DIM + x;
        const size_t vs = (size_t)D.Hk * DIM;
        float os = 0.0f;
#pragma unroll 16
        for (int u = 0; u < B; ++u) os = fmaf(ps[t * B + u], ldv(vcol, u * vs), os);
        float v;
        if (lp2 == -__builtin_huge_valf()) {
            v = os;
        } else {
            const float M = fmaxf(lp2, ls2[t]);
            const float ep = __builtin_amdgcn_exp2f(lp2 - M), es = __builtin_amdgcn_exp2f(ls2[t] - M);
            v = (ep * op + es * os) / (ep + es);
        }
        T *o = out + ((size_t)(s * B + tok) * D.Hq + h) * DIM + x;
        if constexpr (sizeof(T) == 2) *reinterpret_cast<uint16_t *>(o) = f32_to_bf16(v);
        else *reinterpret_cast<float *>(o) = v;
    }
}

size_t finish_lds_bytes(const Dims &D, bool dense, int TG) {
    const int NR = dense ? TG : D.A;
    return ((size_t)D.B * (D.d + 1) + (size_t)TG * D.d + (size_t)TG * D.B + TG + 4 * (size_t)NR) * 4;
}

int finish_group(const Dims &D, bool dense) {
    // tokens per workgroup: on the dense step every row combines one partial
    // per prefix chunk, so the groups are small
    return dense ? (D.B < 2 ? D.B : 2) : (D.B < 16 ? D.B : 16);
}

hipError_t launch_finish(const Dims &D, bool dense, const void *q_t, const void *k_blk,
                         const void *v_blk, const int32_t *kv_off, const int32_t *prefix_len,
                         const Work &W, float *op_cache, float *lp_cache, void *out,
                         hipStream_t st) {
    const int TG = finish_group(D, dense);
    dim3 grid((D.B + TG - 1) / TG, D.Hq, D.S);
    const size_t lds = finish_lds_bytes(D, dense, TG);
    const int dn = dense ? 1 : 0;
#define LAUNCH_F(T, DIMV)                                                                        \
    hipLaunchKernelGGL((k_finish<T, DIMV>), grid, dim3(kFinishThreads), lds, st, D, dn, TG,      \
                       static_cast<const T *>(q_t), static_cast<const T *>(k_blk),               \
                       static_cast<const T *>(v_blk), kv_off, prefix_len, W.active, W.union_cnt, \
                       W.part_ml, W.part_acc, op_cache, lp_cache, static_cast<T *>(out))
    if (D.bf16) {
        if (D.d == 128) LAUNCH_F(uint16_t, 128);
        else LAUNCH_F(uint16_t, 64);
    } else {
        if (D.d == 128) LAUNCH_F(float, 128);
        else LAUNCH_F(float, 64);
    }
#undef LAUNCH_F
    return hipGetLastError();
}

}  // namespace losa
