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

// Shared active set (LOSA_FLAG_SHARED_ACTIVE), first half: one thread per
// (sequence, token, query head) row -- consecutive threads read consecutive
// rows of the query arrays -- computes that row's locality chain as above,
// divided by d, into W.shloc[s][h][t].  The second half (the sum over query
// heads in ascending order, an fp32 chain, and the |A| largest sums, equal sums
// going to the lower token; the per-layer reading of the locality score) runs
// at the start of the kernel that stacks the rows, for all of its heads.
template <typename T, int DIM>
__global__ __launch_bounds__(64) void k_shared_locality(Dims D, const T *__restrict__ q_t,
                                                        const T *__restrict__ q_prev, Work W,
                                                        float *__restrict__ dbg_loc) {
    const int64_t n = (int64_t)D.S * D.B * D.Hq;
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (i >= n) return;
    const int h = static_cast<int>(i % D.Hq);
    const int64_t st = i / D.Hq;
    const int t = static_cast<int>(st % D.B), s = static_cast<int>(st / D.B);
    const float e = locality_chain<T, DIM>(q_t + i * DIM, q_prev + i * DIM) / static_cast<float>(DIM);
    const size_t o = ((size_t)s * D.Hq + h) * D.B + t;
    W.shloc[o] = e;
    if (dbg_loc) dbg_loc[o] = e;
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
        // the active set shared by all heads, from the per-head localities
        if (threadIdx.x < B) {
            const float *e = W.shloc + (size_t)s * Hq * B + threadIdx.x;
            float acc = 0.0f;
            for (int h = 0; h < Hq; ++h) acc = acc + e[(size_t)h * B];
            e_s[threadIdx.x] = acc;
        }
        __syncthreads();
        if (threadIdx.x < B) {
            const int t = threadIdx.x;
            const float et = e_s[t];
            int rank = 0;
            for (int u = 0; u < B; ++u) rank += (e_s[u] > et) || (e_s[u] == et && u < t);
            sel_s[t] = rank < A;
        }
        __syncthreads();
        if (threadIdx.x < B && sel_s[threadIdx.x]) {
            const int t = threadIdx.x;
            int pos = 0;
            for (int u = 0; u < t; ++u) pos += sel_s[u];
            for (int j = 0; j < G; ++j) {
                act_s[j * A + pos] = t;
                W.active[((size_t)s * Hq + g * G + j) * A + pos] = t;
                if (dbg_act) dbg_act[((size_t)s * Hq + g * G + j) * A + pos] = t;
            }
        }
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

hipError_t launch_shared_locality(const Dims &D, const void *q_t, const void *q_prev, const Work &W,
                                  float *dbg_loc, hipStream_t st) {
    const int64_t n = (int64_t)D.S * D.B * D.Hq;
    const dim3 grid(static_cast<unsigned>((n + 63) / 64));
    if (n == 0) return hipSuccess;
#define LAUNCH_A(TV, DIMV)                                                                      \
    hipLaunchKernelGGL((k_shared_locality<TV, DIMV>), grid, dim3(64), 0, st, D,                 \
                       static_cast<const TV *>(q_t), static_cast<const TV *>(q_prev), W, dbg_loc)
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
