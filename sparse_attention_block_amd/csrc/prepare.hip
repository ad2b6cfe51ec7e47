// Per-step preparation, one workgroup per (sequence, KV head):
//  * locality score of every (query head, token) of the KV head's group: the
//    squared change of the token's query since the previous step, summed in
//    fp32 over dimensions in ascending order, each square rounded before the
//    add (gist.science pt summary, "3. Metodologia", step 1: MSE between the
//    step's queries and the previous step's);
//  * the |A| largest scores per query head form the active set, equal scores
//    going to the lower token (same passage; fr summary, "Sélection des
//    Tokens Actifs");
//  * the active rows' queries, stacked per KV head (row r = j*|A| + a for
//    query head j of the group and active slot a) so a KV page is read once
//    for all of them, in the storage type for attention and as the fp32
//    selection operands (max(q,0), min(q,0)) of the page bound;
//  * the dense first step stacks all G*B rows instead (r = j*B + t).
// The module is compiled with -ffp-contract=off, so a*b+c stays two roundings.
#include "losa_internal.h"

namespace losa {

template <typename T>
__device__ __forceinline__ float ld(const T *p, int i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else return reinterpret_cast<const float *>(p)[i];
}

template <typename T, int DIM>
__global__ __launch_bounds__(256) void k_prepare(Dims D, int dense, const T *__restrict__ q_t,
                                                 const T *__restrict__ q_prev, Work W,
                                                 float *__restrict__ dbg_loc,
                                                 int32_t *__restrict__ dbg_act,
                                                 int32_t *__restrict__ dbg_ucnt) {
    constexpr bool BF = sizeof(T) == 2;
    __shared__ float e_s[kMaxRows];
    __shared__ int sel_s[kMaxRows];
    __shared__ int act_s[kMaxRows];
    const int g = blockIdx.x, s = blockIdx.y;
    const int G = D.G, B = D.B, A = D.A, Hq = D.Hq;
    const int sg = s * D.Hk + g;
    if (threadIdx.x == 0) {
        W.counters[sg] = 0;
        W.union_cnt[sg] = 0;
        if (dbg_ucnt) dbg_ucnt[sg] = 0;  // the selection kernel overwrites it when |A| > 0
    }
    int rows;
    if (!dense) {
        for (int i = threadIdx.x; i < G * B; i += blockDim.x) {
            const int j = i / B, t = i % B, h = g * G + j;
            const T *a = q_t + ((size_t)(s * B + t) * Hq + h) * DIM;
            const T *b = q_prev + ((size_t)(s * B + t) * Hq + h) * DIM;
            float acc = 0.0f;
#pragma unroll 8
            for (int x = 0; x < DIM; ++x) {
                const float dl = ld(a, x) - ld(b, x);
                const float sq = dl * dl;
                acc = acc + sq;
            }
            e_s[i] = acc;
            if (dbg_loc) dbg_loc[((size_t)s * Hq + h) * B + t] = acc / static_cast<float>(DIM);
        }
        __syncthreads();
        for (int i = threadIdx.x; i < G * B; i += blockDim.x) {
            const int j = i / B, t = i % B;
            const float et = e_s[i];
            int rank = 0;
            for (int u = 0; u < B; ++u) {
                const float eu = e_s[j * B + u];
                rank += (eu > et) || (eu == et && u < t);
            }
            sel_s[i] = rank < A;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < G * B; i += blockDim.x) {
            if (!sel_s[i]) continue;
            const int j = i / B, t = i % B, h = g * G + j;
            int pos = 0;
            for (int u = 0; u < t; ++u) pos += sel_s[j * B + u];
            act_s[j * A + pos] = t;
            W.active[((size_t)s * Hq + h) * A + pos] = t;
            if (dbg_act) dbg_act[((size_t)s * Hq + h) * A + pos] = t;
        }
        __syncthreads();
        rows = G * A;
    } else {
        rows = G * B;
    }
    // Stacked query rows.
    T *qr = static_cast<T *>(W.qrows) + (size_t)sg * D.R16 * DIM;
    float *qs = W.qsel + (size_t)sg * (D.R > 0 ? D.R : 1) * DIM * 2;
    for (int idx = threadIdx.x; idx < D.R16 * DIM; idx += blockDim.x) {
        const int r = idx / DIM, x = idx % DIM;
        if (r >= rows) {
            if constexpr (BF) reinterpret_cast<uint16_t *>(qr)[idx] = 0;
            else reinterpret_cast<float *>(qr)[idx] = 0.0f;
            continue;
        }
        int j, t;
        if (dense) { j = r / B; t = r % B; }
        else { j = r / A; t = act_s[r]; }
        const int h = g * G + j;
        const T *src = q_t + ((size_t)(s * B + t) * Hq + h) * DIM + x;
        qr[idx] = *src;
        if (!dense) {
            // Selection operands (q+, q-): q+ = q, q- = 0 when q >= 0 (also for -0),
            // else q+ = 0, q- = q.
            const float q = ld(src, 0);
            const bool pos = q >= 0.0f;
            qs[2 * idx] = pos ? q : 0.0f;
            qs[2 * idx + 1] = pos ? 0.0f : q;
        }
    }
}

hipError_t launch_prepare(const Dims &D, bool dense, const void *q_t, const void *q_prev,
                          const Work &W, float *dbg_loc, int32_t *dbg_act, int32_t *dbg_ucnt,
                          hipStream_t st) {
    dim3 grid(D.Hk, D.S);
    const int dn = dense ? 1 : 0;
    if (D.bf16) {
        auto *a = static_cast<const uint16_t *>(q_t);
        auto *b = static_cast<const uint16_t *>(q_prev);
        if (D.d == 128)
            hipLaunchKernelGGL((k_prepare<uint16_t, 128>), grid, dim3(256), 0, st, D, dn, a, b, W,
                               dbg_loc, dbg_act, dbg_ucnt);
        else
            hipLaunchKernelGGL((k_prepare<uint16_t, 64>), grid, dim3(256), 0, st, D, dn, a, b, W,
                               dbg_loc, dbg_act, dbg_ucnt);
    } else {
        auto *a = static_cast<const float *>(q_t);
        auto *b = static_cast<const float *>(q_prev);
        if (D.d == 128)
            hipLaunchKernelGGL((k_prepare<float, 128>), grid, dim3(256), 0, st, D, dn, a, b, W,
                               dbg_loc, dbg_act, dbg_ucnt);
        else
            hipLaunchKernelGGL((k_prepare<float, 64>), grid, dim3(256), 0, st, D, dn, a, b, W,
                               dbg_loc, dbg_act, dbg_ucnt);
    }
    return hipGetLastError();
}

}  // namespace losa
