// In-block attention of kBlockTPW consecutive tokens of a sparse step, for one
// wave (64 lanes), the block keys and values read once for all of them: each
// token's query against the B block keys and values of its KV head
// (agifrontier tutorial, workflow section: the block is short and attended
// densely), giving (o_s, L_s).  A stable token (not in its head's active list)
// takes the cached (o_p, L_p) unchanged (gist.science pt summary, "3.
// Metodologia", step 2) and its output is final here: the online-softmax merge
// of the two parts (pt step 4), rounded to the storage type.  An active token's
// (o_s, L_s) goes to the workspace for the finishing kernel, which merges it
// with the fresh prefix statistics.  All arithmetic is fp32; scores and
// log-normalisers are in log2 units.
//
// Lanes: for the scores, lane = 4 * key + quarter (16 keys per pass, a quarter
// of the dimensions each); the block values are staged in LDS and lane l owns
// output dimensions (DIM / 64) * l ...  Every global load is issued before the
// first is used; indexes are clamped so that none is conditional.
#pragma once
#include "losa_internal.h"

namespace losa {

// LDS bytes a block wave needs: the values of up to MAXB keys, then MAXB weights
template <int MAXB>
constexpr size_t block_lds_bytes(int d, bool bf16) {
    return (size_t)MAXB * d * (bf16 ? 2 : 4) + MAXB * 4;
}

constexpr int kBlockTPW = 2;  // tokens per in-block wave

template <typename T, int DIM, int MAXB>
__device__ __forceinline__ void block_token(const Dims &D, const T *__restrict__ q_t,
                                            const T *__restrict__ k_blk,
                                            const T *__restrict__ v_blk, const Work &W,
                                            const float *__restrict__ op_cache,
                                            const float *__restrict__ lp_cache,
                                            T *__restrict__ out, uint32_t *lds, int s, int h,
                                            int t0) {
    constexpr int TPW = kBlockTPW;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int QD = DIM / 4;           // dimensions per lane in the scores
    constexpr int EV = 16 / sizeof(T);    // elements per 16-byte vector
    constexpr int NVQ = QD / EV;          // vectors per lane per key
    constexpr int KG = MAXB / 16;         // key passes of 16
    constexpr int NVV = MAXB * DIM / EV / 64;  // value vectors per lane
    constexpr int OD = DIM / 64;          // output dimensions per lane
    constexpr float kLog2e = 1.44269504088896340736f;
    static_assert(NVV >= 1 && OD >= 1, "shape");
    const int lane = threadIdx.x;
    const int B = D.B, A = D.A, Hq = D.Hq, Hk = D.Hk, g = h / D.G;
    const int ku = lane >> 2, qq = lane & 3;
    T *sv = reinterpret_cast<T *>(lds);                                   // [MAXB][DIM]
    float *sp = reinterpret_cast<float *>(lds) + MAXB * DIM * sizeof(T) / 4;  // [MAXB]

    // -- loads: the tokens' query quarters, keys, values, active list, cached
    //    statistics (tokens past the block read the last one and store nothing)
    uint4 qv[TPW][NVQ];
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const T *qrow = q_t + ((size_t)(s * B + min(t0 + x, B - 1)) * Hq + h) * DIM + qq * QD;
#pragma unroll
        for (int i = 0; i < NVQ; ++i) qv[x][i] = reinterpret_cast<const uint4 *>(qrow)[i];
    }
    uint4 kv[KG][NVQ];
#pragma unroll
    for (int p = 0; p < KG; ++p) {
        const int u = min(p * 16 + ku, B - 1);  // clamped key (its score is masked)
        const uint4 *krow =
            reinterpret_cast<const uint4 *>(k_blk + ((size_t)(s * B + u) * Hk + g) * DIM + qq * QD);
#pragma unroll
        for (int i = 0; i < NVQ; ++i) kv[p][i] = krow[i];
    }
    constexpr int VPR = DIM / EV;  // vectors per value row
    const int nvec = B * VPR;
    uint4 vv[NVV];
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
        const int v = min(lane + 64 * i, nvec - 1);
        vv[i] = *reinterpret_cast<const uint4 *>(v_blk + ((size_t)(s * B + v / VPR) * Hk + g) * DIM +
                                                 (v % VPR) * EV);
    }
    const int act = A > 0 ? W.active[((size_t)s * Hq + h) * A + min(lane, A - 1)] : -1;
    float opc[TPW][OD], lpc[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const size_t crow = ((size_t)s * Hq + h) * B + min(t0 + x, B - 1);
#pragma unroll
        for (int e = 0; e < OD; ++e) opc[x][e] = op_cache[crow * DIM + OD * lane + e];
        lpc[x] = lp_cache[crow];
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used

    // -- values to LDS (clamped vectors rewrite the last one with its own value)
#pragma unroll
    for (int i = 0; i < NVV; ++i) {
        const int v = min(lane + 64 * i, nvec - 1);
        *reinterpret_cast<uint4 *>(sv + (size_t)v * EV) = vv[i];
    }

    // -- scores (log2 units): 4 lanes per key, a quarter of the dimensions each
    auto unpack = [](const uint4 &w, float *f) {
        if constexpr (BF) {
            const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = bf16_lo(a[e]);
                f[2 * e + 1] = bf16_hi(a[e]);
            }
        } else {
            f[0] = __uint_as_float(w.x);
            f[1] = __uint_as_float(w.y);
            f[2] = __uint_as_float(w.z);
            f[3] = __uint_as_float(w.w);
        }
    };
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int t = t0 + x;
        if (t >= B) break;  // uniform
        if (x > 0) __syncthreads();  // the previous token's weights have been read
        float qf[QD];
#pragma unroll
        for (int i = 0; i < NVQ; ++i) unpack(qv[x][i], qf + i * EV);
        float sc[KG];
        float m = -__builtin_huge_valf();
#pragma unroll
        for (int p = 0; p < KG; ++p) {
            float dot = 0.0f;
#pragma unroll
            for (int i = 0; i < NVQ; ++i) {
                float kf[EV];
                unpack(kv[p][i], kf);
#pragma unroll
                for (int e = 0; e < EV; ++e) dot = fmaf(qf[i * EV + e], kf[e], dot);
            }
            dot += lane_xor1(dot);
            dot += lane_xor2(dot);
            sc[p] = p * 16 + ku < B ? dot * D.scale_log2 : -__builtin_huge_valf();
            m = fmaxf(m, sc[p]);
        }
        // over the keys (lane bits 2-5; m is equal across bits 0-1): l^4, l^8, l^16, l^32
        m = fmaxf(m, lane_xor7(m));
        m = fmaxf(m, lane_xor15(m));
        m = fmaxf(m, lane_xor16(m));
        m = fmaxf(m, lane_xor32(m));
        float l = 0.0f, pw[KG];
#pragma unroll
        for (int p = 0; p < KG; ++p) {
            pw[p] = p * 16 + ku < B ? __builtin_amdgcn_exp2f(sc[p] - m) : 0.0f;
            l += pw[p];
        }
        l += lane_xor7(l);
        l += lane_xor15(l);
        l += lane_xor16(l);
        l += lane_xor32(l);
        const float ls2 = m + __log2f(l);
        // normalised weights to LDS, one lane per key
        if (qq == 0) {
#pragma unroll
            for (int p = 0; p < KG; ++p) sp[p * 16 + ku] = pw[p] / l;
        }
        __syncthreads();  // one wave per workgroup: orders the weights' LDS writes and reads

        // -- output dimensions of this lane: weights in ascending key order
        float os[OD];
#pragma unroll
        for (int e = 0; e < OD; ++e) os[e] = 0.0f;
#pragma unroll 16
        for (int u = 0; u < B; ++u) {
            const float pu = sp[u];
#pragma unroll
            for (int e = 0; e < OD; ++e) {
                float vx;
                if constexpr (BF) vx = bf16_to_f32(reinterpret_cast<const uint16_t *>(sv)[u * DIM + OD * lane + e]);
                else vx = sv[u * DIM + OD * lane + e];
                os[e] = fmaf(pu, vx, os[e]);
            }
        }

        // -- active or stable: the token's slot in its head's active list
        const uint64_t hit = __ballot(lane < A && act == t);
        if (hit != 0ull) {
            const int slot = __ffsll(static_cast<unsigned long long>(hit)) - 1;
            const size_t ar = ((size_t)s * Hq + h) * A + slot;
#pragma unroll
            for (int e = 0; e < OD; ++e) W.blk_o[ar * DIM + OD * lane + e] = os[e];
            if (lane == 0) W.blk_l[ar] = ls2;
            continue;
        }
        const float lp2 = lpc[x] * kLog2e;
        T *o = out + ((size_t)(s * B + t) * Hq + h) * DIM + OD * lane;
#pragma unroll
        for (int e = 0; e < OD; ++e) {
            float v;
            if (lp2 == -__builtin_huge_valf()) {
                v = os[e];
            } else {
                const float M = fmaxf(lp2, ls2);
                const float ep = __builtin_amdgcn_exp2f(lp2 - M), es = __builtin_amdgcn_exp2f(ls2 - M);
                v = (ep * opc[x][e] + es * os[e]) / (ep + es);
            }
            if constexpr (BF) reinterpret_cast<uint16_t *>(o)[e] = f32_to_bf16(v);
            else o[e] = v;
        }
    }
}

}  // namespace losa
