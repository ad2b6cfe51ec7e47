// Per-step preparation, one workgroup per (sequence, KV head):
//  * locality score of every (query head, token) of the KV head's group: the
//    squared change of the token's query since the previous step, summed in
//    fp32 over dimensions in ascending order, each square rounded before the
//    add (gist.science pt summary, "3. Metodologia", step 1: MSE between the
//    step's queries and the previous step's);
//  * the |A| largest scores per query head form the active set, equal scores
//    going to the lower token (same passage; fr summary, "Sélection des
//    Tokens Actifs");
//  * the active rows' queries stacked per KV head (row r = j*|A| + a for query
//    head j of the group and active slot a), so that a KV page is read once
//    for all of them: in the storage type for attention, as bf16 pairs
//    (max(q,0), min(q,0)) for the MFMA page scoring, as fp32 pairs for the
//    exact page-bound chain, and an upper bound of sum_i |q_i| per row;
//  * the dense first step stacks all G*B rows instead (r = j*B + t).
// The module is compiled with -ffp-contract=off, so a*b+c stays two roundings.
#include "losa_internal.h"

namespace losa {

template <typename T>
__device__ __forceinline__ float ld(const T *p, int i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else return reinterpret_cast<const float *>(p)[i];
}

// Squared-change chain of one (head, token) row, loads issued before the chain.
template <typename T, int DIM>
__device__ __forceinline__ float locality_chain(const T *a, const T *b) {
    float acc = 0.0f;
    if constexpr (sizeof(T) == 2) {
        constexpr int N = DIM / 8;  // uint4 = 8 bf16
        uint4 va[N], vb[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            va[i] = reinterpret_cast<const uint4 *>(a)[i];
            vb[i] = reinterpret_cast<const uint4 *>(b)[i];
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads in flight before the chain starts
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t xa[4] = {va[i].x, va[i].y, va[i].z, va[i].w};
            const uint32_t xb[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d0 = bf16_lo(xa[e]) - bf16_lo(xb[e]);
                const float s0 = d0 * d0;
                acc = acc + s0;
                const float d1 = bf16_hi(xa[e]) - bf16_hi(xb[e]);
                const float s1 = d1 * d1;
                acc = acc + s1;
            }
        }
    } else {
        constexpr int SEG = 64;  // floats per batch of loads
#pragma unroll
        for (int s0 = 0; s0 < DIM; s0 += SEG) {
            float4 va[SEG / 4], vb[SEG / 4];
#pragma unroll
            for (int i = 0; i < SEG / 4; ++i) {
                va[i] = reinterpret_cast<const float4 *>(a + s0)[i];
                vb[i] = reinterpret_cast<const float4 *>(b + s0)[i];
            }
#pragma unroll
            for (int i = 0; i < SEG / 4; ++i) {
                const float xa[4] = {va[i].x, va[i].y, va[i].z, va[i].w};
                const float xb[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dl = xa[e] - xb[e];
                    const float sq = dl * dl;
                    acc = acc + sq;
                }
            }
        }
    }
    return acc;
}

// Shared active set (LOSA_FLAG_SHARED_ACTIVE), one workgroup per sequence:
// every (query head, token) locality chain as above, divided by d; per token
// the sum over query heads in ascending order (an fp32 chain); the |A| largest
// sums are active, equal sums going to the lower token; the same ascending list
// is written for every head (the per-layer reading of the locality score).
template <typename T, int DIM>
__global__ __launch_bounds__(256) void k_shared_active(Dims D, const T *__restrict__ q_t,
                                                       const T *__restrict__ q_prev, Work W,
                                                       float *__restrict__ dbg_loc,
                                                       int32_t *__restrict__ dbg_act) {
    __shared__ float sc[kMaxSharedScores];
    __shared__ float tot[64];
    __shared__ int sel[64];
    const int s = blockIdx.x, tid = threadIdx.x;
    const int B = D.B, A = D.A, Hq = D.Hq;
    for (int i = tid; i < Hq * B; i += blockDim.x) {
        const int h = i / B, t = i % B;
        const size_t off = ((size_t)(s * B + t) * Hq + h) * DIM;
        const float e = locality_chain<T, DIM>(q_t + off, q_prev + off) / static_cast<float>(DIM);
        sc[i] = e;
        if (dbg_loc) dbg_loc[((size_t)s * Hq + h) * B + t] = e;
    }
    __syncthreads();
    if (tid < B) {
        float acc = 0.0f;
        for (int h = 0; h < Hq; ++h) acc = acc + sc[h * B + tid];
        tot[tid] = acc;
    }
    __syncthreads();
    if (tid < B) {
        const float et = tot[tid];
        int rank = 0;
        for (int u = 0; u < B; ++u) rank += (tot[u] > et) || (tot[u] == et && u < tid);
        sel[tid] = rank < A;
    }
    __syncthreads();
    if (tid < B && sel[tid]) {
        int pos = 0;
        for (int u = 0; u < tid; ++u) pos += sel[u];
        for (int h = 0; h < Hq; ++h) {
            W.active[((size_t)s * Hq + h) * A + pos] = tid;
            if (dbg_act) dbg_act[((size_t)s * Hq + h) * A + pos] = tid;
        }
    }
}

template <typename T, int DIM, bool DENSE>
__global__ __launch_bounds__(256) void k_prepare(Dims D, const T *__restrict__ q_t,
                                                 const T *__restrict__ q_prev, Work W,
                                                 float *__restrict__ dbg_loc,
                                                 int32_t *__restrict__ dbg_act,
                                                 int32_t *__restrict__ dbg_ucnt) {
    constexpr bool dense = DENSE;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int CH = 8;            // dimensions per work item when stacking rows
    constexpr int NCHK = DIM / CH;   // 8 or 16 items per row
    __shared__ float e_s[kMaxRows];
    __shared__ int sel_s[kMaxRows];
    __shared__ int act_s[kMaxRows];
    const int g = blockIdx.x, s = blockIdx.y;
    const int G = D.G, B = D.B, A = D.A, Hq = D.Hq;
    const int sg = s * D.Hk + g;
    if (threadIdx.x == 0) {
        W.union_cnt[sg] = 0;
        if (dbg_ucnt) dbg_ucnt[sg] = 0;  // the sparse prefix kernel overwrites them when |A| > 0
    }
    int rows;
    if (!dense && (D.flags & LOSA_FLAG_SHARED_ACTIVE)) {
        // the active set shared by all heads, from k_shared_active
        for (int i = threadIdx.x; i < G * A; i += blockDim.x)
            act_s[i] = W.active[((size_t)s * Hq + g * G + i / A) * A + i % A];
        __syncthreads();
        rows = G * A;
    } else if (!dense) {
        for (int i = threadIdx.x; i < G * B; i += blockDim.x) {
            const int j = i / B, t = i % B, h = g * G + j;
            const size_t off = ((size_t)(s * B + t) * Hq + h) * DIM;
            const float acc = locality_chain<T, DIM>(q_t + off, q_prev + off);
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
    // Stacked rows, CH dimensions per work item; the NCHK consecutive lanes of
    // a row reduce sum |q| with shuffles, so every pass covers whole rows.  The
    // loads of up to kPasses passes are issued before any of them is used.
    T *qr = static_cast<T *>(W.qrows) + (size_t)sg * D.R16 * DIM;
    const int R1 = D.R > 0 ? D.R : 1;
    uint32_t *q16 = W.qsel16 + (size_t)sg * D.Rs16 * DIM;
    float *q32 = W.qsel32 + (size_t)sg * R1 * DIM * 2;
    const int pad_rows = dense ? D.R16 : D.Rs16;
    const int n_items = rows > 0 ? ((pad_rows * NCHK + 255) / 256) * 256 : 0;
    constexpr int kPasses = 4;
    for (int i0 = 0; i0 < n_items; i0 += kPasses * 256) {
        // CH consecutive dimensions of one row per item, as 16-byte vectors read
        // from a clamped row (always in bounds), zeroed past the live rows
        constexpr int NV = CH * sizeof(T) / 16;
        uint4 raw[kPasses][NV];
#pragma unroll
        for (int pi = 0; pi < kPasses; ++pi) {
            const int item = i0 + pi * 256 + threadIdx.x;
            const int r = min(item / NCHK, rows - 1), c = item % NCHK;
            int j, t;
            if (dense) { j = r / B; t = r % B; }
            else { j = r / A; t = act_s[r]; }
            const uint4 *src = reinterpret_cast<const uint4 *>(
                q_t + ((size_t)(s * B + t) * Hq + g * G + j) * DIM + c * CH);
#pragma unroll
            for (int e = 0; e < NV; ++e) raw[pi][e] = src[e];
        }
        float v[kPasses][CH];
#pragma unroll
        for (int pi = 0; pi < kPasses; ++pi) {
            const int item = i0 + pi * 256 + threadIdx.x;
            const bool ok = item < n_items && item / NCHK < rows;
#pragma unroll
            for (int e = 0; e < NV; ++e) {
                const uint32_t w[4] = {raw[pi][e].x, raw[pi][e].y, raw[pi][e].z, raw[pi][e].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (BF) {
                        v[pi][e * 8 + 2 * q] = ok ? bf16_lo(w[q]) : 0.0f;
                        v[pi][e * 8 + 2 * q + 1] = ok ? bf16_hi(w[q]) : 0.0f;
                    } else {
                        v[pi][e * 4 + q] = ok ? __uint_as_float(w[q]) : 0.0f;
                    }
                }
            }
        }
#pragma unroll
        for (int pi = 0; pi < kPasses; ++pi) {
            const int item = i0 + pi * 256 + threadIdx.x;
            if (i0 + pi * 256 >= n_items) break;  // uniform over the workgroup
            const int r = item / NCHK, c = item % NCHK;
            const bool live = r < rows;
            if (r < pad_rows) {
                T *dst = qr + (size_t)r * DIM + c * CH;
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                    if constexpr (BF) reinterpret_cast<uint16_t *>(dst)[e] = f32_to_bf16(v[pi][e]);
                    else reinterpret_cast<float *>(dst)[e] = v[pi][e];
                }
            }
            if (!dense) {
                // (q+, q-): q+ = q, q- = 0 when q >= 0 (-0 included), else q+ = 0, q- = q.
                float ab = 0.0f;
                if (r < D.Rs16) {
                    uint32_t *d16 = q16 + (size_t)r * DIM + c * CH;
#pragma unroll
                    for (int e = 0; e < CH; ++e) {
                        const bool pos = v[pi][e] >= 0.0f;
                        const uint32_t hb = __float_as_uint(v[pi][e]) >> 16;  // exact for bf16 values
                        d16[e] = BF ? (pos ? hb : (hb << 16)) : 0u;
                    }
                }
                if (live) {
                    float *d32 = q32 + ((size_t)r * DIM + c * CH) * 2;
#pragma unroll
                    for (int e = 0; e < CH; ++e) {
                        const bool pos = v[pi][e] >= 0.0f;
                        d32[2 * e] = pos ? v[pi][e] : 0.0f;
                        d32[2 * e + 1] = pos ? 0.0f : v[pi][e];
                        ab += fabsf(v[pi][e]);
                    }
                }
#pragma unroll
                for (int o = 1; o < NCHK; o <<= 1) ab += __shfl_xor(ab, o);
                if (live && c == 0) W.qabs[(size_t)sg * R1 + r] = ab * (1.0f + 1.0f / 256.0f);
            }
        }
    }
}

hipError_t launch_shared_active(const Dims &D, const void *q_t, const void *q_prev, const Work &W,
                                float *dbg_loc, int32_t *dbg_act, hipStream_t st) {
#define LAUNCH_A(TV, DIMV)                                                                    \
    hipLaunchKernelGGL((k_shared_active<TV, DIMV>), dim3(D.S), dim3(256), 0, st, D,           \
                       static_cast<const TV *>(q_t), static_cast<const TV *>(q_prev), W, dbg_loc, \
                       dbg_act)
    if (D.bf16) {
        if (D.d == 128) LAUNCH_A(uint16_t, 128);
        else LAUNCH_A(uint16_t, 64);
    } else {
        if (D.d == 128) LAUNCH_A(float, 128);
        else LAUNCH_A(float, 64);
    }
#undef LAUNCH_A
    return hipGetLastError();
}

hipError_t launch_prepare(const Dims &D, bool dense, const void *q_t, const void *q_prev,
                          const Work &W, float *dbg_loc, int32_t *dbg_act, int32_t *dbg_ucnt,
                          hipStream_t st) {
    dim3 grid(D.Hk, D.S);
#define LAUNCH_Q(T, DIMV, DN)                                                                   \
    hipLaunchKernelGGL((k_prepare<T, DIMV, DN>), grid, dim3(256), 0, st, D,                    \
                       static_cast<const T *>(q_t), static_cast<const T *>(q_prev), W, dbg_loc, \
                       dbg_act, dbg_ucnt)
#define PICK_Q(T, DIMV)                      \
    do {                                     \
        if (dense) LAUNCH_Q(T, DIMV, true);  \
        else LAUNCH_Q(T, DIMV, false);       \
    } while (0)
    if (D.bf16) {
        if (D.d == 128) PICK_Q(uint16_t, 128);
        else PICK_Q(uint16_t, 64);
    } else {
        if (D.d == 128) PICK_Q(float, 128);
        else PICK_Q(float, 64);
    }
#undef PICK_Q
#undef LAUNCH_Q
    return hipGetLastError();
}

}  // namespace losa
