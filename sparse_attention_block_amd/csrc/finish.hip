// Finishing kernel, one wave per (sequence, query head, block token):
//  * active rows (every row on a dense first step): combine the prefix
//    workgroups' partial statistics in chunk order into (o_p, L_p) and
//    overwrite the cache entry -- "updated statistics are stored for the next
//    step" (gist.science pt summary, "3. Metodologia", step 4);
//  * stable rows: read the cached (o_p, L_p) unchanged (pt step 2);
//  * dense attention of the token over the B in-block keys/values, giving
//    (o_s, L_s) (agifrontier tutorial, workflow section: the block is short
//    and attended densely);
//  * the online-softmax merge L = log(e^L_p + e^L_s),
//    out = e^(L_p-L) o_p + e^(L_s-L) o_s, rounded to the storage type.
#include "losa_internal.h"

namespace losa {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <typename T, int DIM>
__device__ __forceinline__ void load_dims(const T *p, int lane, float (&x)[DIM / 64]) {
    constexpr int DPT = DIM / 64;
    if constexpr (sizeof(T) == 2) {
        const uint16_t *q = reinterpret_cast<const uint16_t *>(p) + lane * DPT;
        if constexpr (DPT == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(q);
            x[0] = bf16_lo(w);
            x[1] = bf16_hi(w);
        } else {
            x[0] = bf16_to_f32(q[0]);
        }
    } else {
        const float *q = reinterpret_cast<const float *>(p) + lane * DPT;
#pragma unroll
        for (int i = 0; i < DPT; ++i) x[i] = q[i];
    }
}

template <typename T, int DIM>
__global__ __launch_bounds__(64) void k_finish(Dims D, int dense, const T *__restrict__ q_t,
                                               const T *__restrict__ k_blk,
                                               const T *__restrict__ v_blk,
                                               const int32_t *__restrict__ kv_off,
                                               const int32_t *__restrict__ prefix_len, Work W,
                                               float *__restrict__ op_cache,
                                               float *__restrict__ lp_cache, T *__restrict__ out) {
    constexpr int DPT = DIM / 64;
    constexpr float kLn2 = 0.69314718055994530942f;
    constexpr float kLog2e = 1.44269504088896340736f;
    const int t = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int lane = threadIdx.x;
    const int G = D.G, B = D.B;
    const int g = h / G, j = h % G;
    const int sgi = s * D.Hk + g;

    int r = -1;
    if (dense) {
        r = j * B + t;
    } else {
        const int32_t *act = W.active + ((size_t)s * D.Hq + h) * D.A;
        for (int a = 0; a < D.A; ++a)
            if (act[a] == t) r = j * D.A + a;
    }
    const size_t crow = ((size_t)s * D.Hq + h) * B + t;
    float op[DPT], lp2;  // L_p kept in log2 units here
    if (r >= 0) {
        const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
        const int cp = dense ? kDenseChunk : kSparseChunk;
        const int n_items = dense ? sg.pages : W.union_cnt[sgi];
        const int nchu = (n_items + cp - 1) / cp;
        const int nch = dense ? D.n_chunks_dense : D.n_chunks_sparse;
        const int rows = dense ? D.Rd : D.R;
#pragma unroll
        for (int i = 0; i < DPT; ++i) op[i] = 0.0f;
        if (nchu == 0) {
            lp2 = -__builtin_huge_valf();
        } else {
            const float *ml = W.part_ml + ((size_t)sgi * nch * rows + r) * 2;
            const size_t cstride = (size_t)rows * 2;
            float mx = -__builtin_huge_valf();
            for (int c = lane; c < nchu; c += 64) mx = fmaxf(mx, ml[c * cstride]);
            mx = wave_maxf(mx);
            float lsum = 0.0f;
            for (int c = lane; c < nchu; c += 64)
                lsum += __builtin_amdgcn_exp2f(ml[c * cstride] - mx) * ml[c * cstride + 1];
            lsum = wave_sum(lsum);
            const float *acc = W.part_acc + ((size_t)sgi * nch * rows + r) * DIM + lane * DPT;
            const size_t astride = (size_t)rows * DIM;
            for (int c = 0; c < nchu; ++c) {
                const float wgt = __builtin_amdgcn_exp2f(ml[c * cstride] - mx);
#pragma unroll
                for (int i = 0; i < DPT; ++i) op[i] += wgt * acc[c * astride + i];
            }
            const float inv = 1.0f / lsum;
#pragma unroll
            for (int i = 0; i < DPT; ++i) op[i] *= inv;
            lp2 = mx + __log2f(lsum);
        }
        float *dst = op_cache + crow * DIM + lane * DPT;
#pragma unroll
        for (int i = 0; i < DPT; ++i) dst[i] = op[i];
        if (lane == 0) lp_cache[crow] = lp2 * kLn2;
    } else {
        const float *src = op_cache + crow * DIM + lane * DPT;
#pragma unroll
        for (int i = 0; i < DPT; ++i) op[i] = src[i];
        lp2 = lp_cache[crow] * kLog2e;
    }

    // Dense in-block attention over the B block keys of KV head g.
    float q[DPT];
    load_dims<T, DIM>(q_t + ((size_t)(s * B + t) * D.Hq + h) * DIM, lane, q);
    float su = -__builtin_huge_valf();  // lane u keeps score u (log2 units)
    for (int u = 0; u < B; ++u) {
        float kx[DPT];
        load_dims<T, DIM>(k_blk + ((size_t)(s * B + u) * D.Hk + g) * DIM, lane, kx);
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < DPT; ++i) part = fmaf(q[i], kx[i], part);
        const float dot = wave_sum(part);
        if (lane == u) su = dot * D.scale_log2;
    }
    const float ms = wave_maxf(su);
    const float pu = lane < B ? __builtin_amdgcn_exp2f(su - ms) : 0.0f;
    const float ls = wave_sum(pu);
    float os[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) os[i] = 0.0f;
    for (int u = 0; u < B; ++u) {
        const float w = __shfl(pu, u);
        float vx[DPT];
        load_dims<T, DIM>(v_blk + ((size_t)(s * B + u) * D.Hk + g) * DIM, lane, vx);
#pragma unroll
        for (int i = 0; i < DPT; ++i) os[i] = fmaf(w, vx[i], os[i]);
    }
    const float ls2 = ms + __log2f(ls);
    const float inv_ls = 1.0f / ls;

    // Merge.
    float wp, ws;
    if (lp2 == -__builtin_huge_valf()) {
        wp = 0.0f;
        ws = 1.0f;
    } else {
        const float M = fmaxf(lp2, ls2);
        const float ep = __builtin_amdgcn_exp2f(lp2 - M), es = __builtin_amdgcn_exp2f(ls2 - M);
        wp = ep / (ep + es);
        ws = es / (ep + es);
    }
    T *o = out + ((size_t)(s * B + t) * D.Hq + h) * DIM;
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
        const float v = wp * op[i] + ws * (os[i] * inv_ls);
        if constexpr (sizeof(T) == 2)
            reinterpret_cast<uint16_t *>(o)[lane * DPT + i] = f32_to_bf16(v);
        else
            reinterpret_cast<float *>(o)[lane * DPT + i] = v;
    }
}

hipError_t launch_finish(const Dims &D, bool dense, const void *q_t, const void *k_blk,
                         const void *v_blk, const int32_t *kv_off, const int32_t *prefix_len,
                         const Work &W, float *op_cache, float *lp_cache, void *out,
                         hipStream_t st) {
    dim3 grid(D.B, D.Hq, D.S);
    const int dn = dense ? 1 : 0;
#define LAUNCH_F(T, DIMV)                                                                          \
    hipLaunchKernelGGL((k_finish<T, DIMV>), grid, dim3(64), 0, st, D, dn,                          \
                       static_cast<const T *>(q_t), static_cast<const T *>(k_blk),                 \
                       static_cast<const T *>(v_blk), kv_off, prefix_len, W, op_cache, lp_cache,   \
                       static_cast<T *>(out))
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
