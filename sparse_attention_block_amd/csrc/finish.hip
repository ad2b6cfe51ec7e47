// Finishing kernels.
//
// k_finish (dense first step), one workgroup per (sequence, query head, group
// of block tokens), one thread per output element:
//  * every row: combine the prefix workgroups' partial statistics in chunk
//    order into (o_p, L_p) and overwrite the cache entry -- updated statistics
//    are kept for the next step (gist.science pt summary, "3. Metodologia",
//    step 4);
//  * dense attention of the tokens over the B in-block keys/values, giving
//    (o_s, L_s) (agifrontier tutorial, workflow section: the block is short
//    and attended densely);
//  * the online-softmax merge L = log(e^L_p + e^L_s),
//    out = e^(L_p-L) o_p + e^(L_s-L) o_s, rounded to the storage type.
// The reads that depend on no other read (block keys and values, queries, the
// cached statistics) are requested together with the first batch of a token's
// prefix partials, which is in flight while the block scores are computed.
//
// k_finish_active (sparse step), one workgroup per active row (sequence, query
// head, active slot), one thread per dimension: the row's partials in chunk
// order, its cache entry, and the merge with the row's (o_s, L_s) from the
// in-block attention that ran beside the selection.  Stable rows were finished
// there.  The row's partials are requested at once, chunk indexes clamped
// into the buffer and those past the union masked, so that no read waits for
// another.  All arithmetic is fp32; scores and log-normalisers are in log2
// units inside.
#include "losa_internal.h"

namespace losa {

template <typename T>
__device__ __forceinline__ float ldv(const T *p, size_t i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[i]);
    else return reinterpret_cast<const float *>(p)[i];
}

constexpr int kFinishMaxThreads = 256;
constexpr int kVReg = 16;    // block values per thread held in registers (the rest re-read)
constexpr int kActBatch = 32;  // prefix chunks per batch in the active-row finish
constexpr int kDenseBatch = 64;  // first batch of prefix chunks in the dense finish
constexpr int kPartBatch = 30;  // prefix partials per thread requested together (60
                                // loads: each wave keeps at most 63 in flight)

// running combination of prefix partials (log2 units): max, sum, weighted output
struct PartAcc {
    float mx = -__builtin_huge_valf(), ls = 0.0f, oa = 0.0f;
    // entries i < n of m, l, a
    template <int N>
    __device__ __forceinline__ void add(const float (&m)[N], const float (&l)[N], const float (&a)[N], int n) {
        float bm = -__builtin_huge_valf();
#pragma unroll
        for (int i = 0; i < N; ++i)
            if (i < n) bm = fmaxf(bm, m[i]);
        const float nm = fmaxf(mx, bm);
        if (nm == -__builtin_huge_valf()) return;
        const float sc = __builtin_amdgcn_exp2f(mx - nm);
        ls *= sc;
        oa *= sc;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if (i < n) {
                const float w = __builtin_amdgcn_exp2f(m[i] - nm);
                ls = fmaf(w, l[i], ls);
                oa = fmaf(w, a[i], oa);
            }
        }
        mx = nm;
    }
};

// online-softmax merge of a prefix part (o_p, L_p) and a block part (o_s, L_s),
// log-normalisers in log2 units; a prefix part with L_p = -inf is empty
__device__ __forceinline__ float merge_parts(float op, float lp2, float os, float ls2) {
    if (lp2 == -__builtin_huge_valf()) return os;
    const float M = fmaxf(lp2, ls2);
    const float ep = __builtin_amdgcn_exp2f(lp2 - M), es = __builtin_amdgcn_exp2f(ls2 - M);
    return (ep * op + es * os) / (ep + es);
}

template <typename T>
__device__ __forceinline__ void store_out(T *o, float v) {
    if constexpr (sizeof(T) == 2) *reinterpret_cast<uint16_t *>(o) = f32_to_bf16(v);
    else *reinterpret_cast<float *>(o) = v;
}

template <typename T, int DIM>
__global__ __launch_bounds__(kFinishMaxThreads) void k_finish(
    Dims D, int TG, const T *__restrict__ q_t, const T *__restrict__ k_blk,
    const T *__restrict__ v_blk, const int32_t *__restrict__ kv_off,
    const int32_t *__restrict__ prefix_len, const float *__restrict__ part_ml,
    const float *__restrict__ part_acc, float *__restrict__ op_cache,
    float *__restrict__ lp_cache, T *__restrict__ out) {
    constexpr float kLn2 = 0.69314718055994530942f;
    extern __shared__ float sm[];
    __shared__ float s_m0[kFinishMaxThreads / 64][kDenseBatch], s_l0[kFinishMaxThreads / 64][kDenseBatch];
    const int B = D.B, G = D.G;
    // workgroup u * (S*Hk) + (s*Hk + g) takes token group u % n_tg of head
    // g*G + u / n_tg: a group's workgroups run on the XCD that ran its prefix
    // workgroups (their partials are in that XCD's L2) when S*Hk is a multiple of 8
    const int ng = D.S * D.Hk, n_tg = (D.B + TG - 1) / TG;
    const int sg_ = blockIdx.x % ng, u_ = blockIdx.x / ng;
    const int t0 = (u_ % n_tg) * TG, h = (sg_ % D.Hk) * D.G + u_ / n_tg, s = sg_ / D.Hk;
    const int nt = min(TG, B - t0);
    const int g = h / G, j = h % G;
    const int sgi = s * D.Hk + g;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int t = tid / DIM, x = tid % DIM;  // this thread's output element
    const bool live = t < nt;
    const int tok = t0 + t;
    const int nch = D.n_chunks_dense;
    const int rows = D.Rd;
    const int row0 = j * B + t0;  // the prefix row of token t0 + t is row0 + t

    // LDS: at most 64*129 + 4*128 + 4*64 + 4 words + 64*DIM bf16 (< 49 KiB)
    constexpr bool BF = sizeof(T) == 2;
    float *kb = sm;                        // [B][DIM + 1]
    float *qs = kb + B * (DIM + 1);        // [TG][DIM]
    float *ps = qs + TG * DIM;             // [TG][B] scores, then softmax weights
    float *ls2 = ps + TG * B;              // [TG] L_s (log2 units)
    const int vb_words = (B * (DIM + 1) + TG * DIM + TG * B + TG + 3) & ~3;
    uint16_t *vb = reinterpret_cast<uint16_t *>(sm + vb_words);  // [B][DIM] (bf16), 16-byte aligned

    // -- 1. every read that depends on no other read ---------------------------
    // prefix chunks that wrote partials
    const int nchu = (seq_geom(D, kv_off, prefix_len, s).pages + D.dense_chunk - 1) / D.dense_chunk;
    // Block keys (and values, bf16) and the queries as 16-byte vectors, every
    // address clamped into its tensor so that no load is conditional: all of
    // them are in flight before the first is used.
    constexpr int EV = 16 / sizeof(T);             // elements per vector
    constexpr int KPT = 64 * DIM / EV / kFinishMaxThreads;  // vectors per thread (B <= 64)
    const int nkv = B * DIM / EV;
    uint4 kr[KPT], vr4[BF ? KPT : 1];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = min(tid + i * nthr, nkv - 1);
        const size_t off = ((size_t)(s * B + idx * EV / DIM) * D.Hk + g) * DIM + (idx * EV) % DIM;
        kr[i] = *reinterpret_cast<const uint4 *>(k_blk + off);
        if constexpr (BF) vr4[i] = *reinterpret_cast<const uint4 *>(v_blk + off);
    }
    const int nq = nt * DIM / EV;
    const int qi = min(tid, nq - 1);
    const uint4 qv4 = *reinterpret_cast<const uint4 *>(
        q_t + ((size_t)(s * B + t0 + qi * EV / DIM) * D.Hq + h) * DIM + (qi * EV) % DIM);
    // fp32 storage: this thread's column of the block values, from global memory
    const T *vcol = v_blk + ((size_t)s * B * D.Hk + g) * DIM + x;
    const size_t vs = (size_t)D.Hk * DIM;
    float vr[BF ? 1 : kVReg];
    if constexpr (!BF) {
#pragma unroll
        for (int u = 0; u < kVReg; ++u) vr[u] = ldv(vcol, min(u, B - 1) * vs);
    }
    const size_t crow = ((size_t)s * D.Hq + h) * B + tok;
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
    // LDS stores at the same clamped indexes (threads past the end rewrite the
    // last vector with its own value), so that no store -- and no load feeding
    // it -- sits in a branch
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int idx = min(tid + i * nthr, nkv - 1);
        float f[EV];
        unpack(kr[i], f);
        float *dst = kb + (idx * EV / DIM) * (DIM + 1) + (idx * EV) % DIM;
#pragma unroll
        for (int e = 0; e < EV; ++e) dst[e] = f[e];
        if constexpr (BF) *reinterpret_cast<uint4 *>(vb + idx * EV) = vr4[i];
    }
    {
        float f[EV];
        unpack(qv4, f);
#pragma unroll
        for (int e = 0; e < EV; ++e) qs[qi * EV + e] = f[e];
    }
    __syncthreads();

    // -- 2. this token's prefix row; its first batch of partials is requested
    //       before the block scores are computed -------------------------------
    // The first kDenseBatch chunks stay in flight until the merge (the
    // barriers up to it wait on LDS only): (m, l) of chunk x by thread x of
    // the token (shared through LDS), and 8-byte pieces of the chunks' outputs
    // -- lanes x and x^1 both read dimensions 2*(x/2) and 2*(x/2) + 1, lane x
    // of chunks 32*(x%2) .. + 31, and swap one sum at the end -- so that a
    // thread has 33 loads in flight (a wave tracks at most 63: 65 loads would
    // hold the last ones back a round trip).  Chunk indexes are clamped, so
    // that no load is conditional; entries past the chunk count are ignored.
    // Later chunks (long prefixes) are read in batches of kPartBatch.
    const int rho = live ? t : -1;
    const size_t pr0 = (size_t)sgi * nch * rows + row0 + (rho < 0 ? 0 : rho);
    const float *mlp = part_ml + pr0 * 2;
    const float *acp = part_acc + pr0 * DIM + x;
    // chunk strides in elements: a row's partials span < 2^31 bytes (at most
    // 4096 chunks x 256 rows x DIM floats), so 32-bit offsets suffice
    const int cs = rows * 2, as = rows * DIM;
    const int clast = max(nchu - 1, 0);
    const int h32 = (kDenseBatch / 2) * (x & 1);  // this lane's half of the first batch
    const float2 ml0 = *reinterpret_cast<const float2 *>(mlp + min(min(x, kDenseBatch - 1), clast) * cs);
    const float *acp2 = part_acc + pr0 * DIM + (x & ~1);
    float2 av0[kDenseBatch / 2];
#pragma unroll
    for (int i = 0; i < kDenseBatch / 2; ++i)
        av0[i] = *reinterpret_cast<const float2 *>(acp2 + (size_t)min(h32 + i, clast) * as);
    __builtin_amdgcn_sched_barrier(0);  // the partials stay in flight during the block scores
    // block scores q.k (scaled, log2 units): 8 threads per (token, key) pair
    {
        constexpr int SEG = DIM / 8;
        const int n_pairs = nt * B;
        const int iters = (n_pairs * 8 + nthr - 1) / nthr;
        for (int it = 0; it < iters; ++it) {
            const int idx = it * nthr + tid;
            const int pr = idx >> 3, part = idx & 7;
            float dot = 0.0f;
            if (pr < n_pairs) {
                const int tt = pr / B, u = pr % B;
                const float *qp = qs + tt * DIM + part * SEG;
                const float *kp = kb + u * (DIM + 1) + part * SEG;
#pragma unroll
                for (int i = 0; i < SEG; ++i) dot = fmaf(qp[i], kp[i], dot);
            }
            dot += lane_xor1(dot);  // then l^2, l^4: the 8 parts of the pair
            dot += lane_xor2(dot);
            dot += lane_xor7(dot);
            if (pr < n_pairs && part == 0) ps[pr] = dot * D.scale_log2;
        }
    }
    if (x < kDenseBatch) {
        s_m0[t][x] = ml0.x;
        s_l0[t][x] = ml0.y;
    }
    lds_barrier();
    // the first batch's chunk weights, once per (token, chunk): lane c of the
    // token's first wave takes chunk c, after the batch maximum by lane
    // butterflies (published by the barriers of the block softmax below)
    __shared__ float s_w0[kFinishMaxThreads / 64][kDenseBatch], s_mx0[kFinishMaxThreads / 64];
    static_assert(kDenseBatch == 64, "one chunk per lane of a wave");
    if (x < 64) {
        const bool v = x < min(nchu, kDenseBatch);
        const float m = v ? s_m0[t][x] : -__builtin_huge_valf();
        float bm = m;
        bm = fmaxf(bm, lane_xor1(bm));
        bm = fmaxf(bm, lane_xor2(bm));
        bm = fmaxf(bm, lane_xor7(bm));
        bm = fmaxf(bm, lane_xor15(bm));
        bm = fmaxf(bm, lane_xor16(bm));
        bm = fmaxf(bm, lane_xor32(bm));
        s_w0[t][x] = v && bm != -__builtin_huge_valf() ? __builtin_amdgcn_exp2f(m - bm) : 0.0f;
        if (x == 0) s_mx0[t] = bm;
    }
    {
        // softmax over each token's B scores: lanes (token, key) in segments of
        // Bp = B rounded up to a power of two (nt * Bp <= 256 threads)
        int Bp = 1;
        while (Bp < B) Bp <<= 1;
        const int tt = tid / Bp, u = tid % Bp;
        const bool on = tt < nt && u < B;
        const float v = on ? ps[tt * B + u] : -__builtin_huge_valf();
        // butterflies over the segment: l^1, l^2, then l^4, l^8, l^16, l^32
        // (xor 7 and 15 once the value is equal across the lower lane bits)
        auto seg_max = [&](float y) {
            if (Bp > 1) y = fmaxf(y, lane_xor1(y));
            if (Bp > 2) y = fmaxf(y, lane_xor2(y));
            if (Bp > 4) y = fmaxf(y, lane_xor7(y));
            if (Bp > 8) y = fmaxf(y, lane_xor15(y));
            if (Bp > 16) y = fmaxf(y, lane_xor16(y));
            if (Bp > 32) y = fmaxf(y, lane_xor32(y));
            return y;
        };
        auto seg_sum = [&](float y) {
            if (Bp > 1) y += lane_xor1(y);
            if (Bp > 2) y += lane_xor2(y);
            if (Bp > 4) y += lane_xor7(y);
            if (Bp > 8) y += lane_xor15(y);
            if (Bp > 16) y += lane_xor16(y);
            if (Bp > 32) y += lane_xor32(y);
            return y;
        };
        const float m = seg_max(v);
        const float p = on ? __builtin_amdgcn_exp2f(v - m) : 0.0f;
        const float l = seg_sum(p);
        lds_barrier();  // every score has been read
        if (on) ps[tt * B + u] = p / l;
        if (on && u == 0) ls2[tt] = m + __log2f(l);
    }
    lds_barrier();
    if (!live) return;

    // -- 3. output ---------------------------------------------------------------
    float os = 0.0f;
    if constexpr (BF) {
        for (int u = 0; u < B; ++u) os = fmaf(ps[t * B + u], bf16_to_f32(vb[u * DIM + x]), os);
    } else {
#pragma unroll
        for (int u = 0; u < kVReg; ++u)
            if (u < B) os = fmaf(ps[t * B + u], vr[u], os);
        for (int u = kVReg; u < B; ++u) os = fmaf(ps[t * B + u], ldv(vcol, u * vs), os);
    }
    // the row's prefix statistics, in chunk order; they overwrite the cache
    PartAcc pa;
    if (nchu > 0) {
        const int nb = min(nchu, kDenseBatch);
        float ls = 0.0f, sx = 0.0f, sy = 0.0f;
#pragma unroll
        for (int i = 0; i < kDenseBatch; ++i) ls = fmaf(s_w0[t][i], s_l0[t][i], ls);
        // this lane's half of the chunks for both dimensions of its pair, in
        // chunk order; then the sum over the other half from lane x^1
#pragma unroll
        for (int i = 0; i < kDenseBatch / 2; ++i) {
            const float w = s_w0[t][h32 + i];
            const bool on = h32 + i < nb;
            sx = fmaf(w, on ? av0[i].x : 0.0f, sx);
            sy = fmaf(w, on ? av0[i].y : 0.0f, sy);
        }
        const float other = lane_xor1((x & 1) ? sx : sy);  // lane x^1's sum for dimension x
        pa.mx = s_mx0[t];
        pa.ls = ls;
        pa.oa = ((x & 1) ? sy : sx) + other;  // (halves added in either order: the same sum)
    }
    for (int c0 = kDenseBatch; c0 < nchu; c0 += kPartBatch) {
        float mv[kPartBatch], lv[kPartBatch], av[kPartBatch];
#pragma unroll
        for (int i = 0; i < kPartBatch; ++i) {
            const int c = min(c0 + i, nchu - 1);
            const float2 v = *reinterpret_cast<const float2 *>(mlp + c * cs);
            mv[i] = v.x;
            lv[i] = v.y;
            av[i] = acp[c * as];
        }
        pa.add(mv, lv, av, min(kPartBatch, nchu - c0));
    }
    float op = 0.0f, lp2 = -__builtin_huge_valf();
    if (nchu > 0) {
        op = pa.oa / pa.ls;
        lp2 = pa.mx + __log2f(pa.ls);
    }
    op_cache[crow * DIM + x] = op;
    if (x == 0) lp_cache[crow] = lp2 * kLn2;
    T *o = out + ((size_t)(s * B + tok) * D.Hq + h) * DIM + x;
    store_out(o, merge_parts(op, lp2, os, ls2[t]));
}

template <typename T, int DIM>
__global__ __launch_bounds__(DIM) void k_finish_active(
    Dims D, const int32_t *__restrict__ active, const int32_t *__restrict__ union_cnt,
    const float *__restrict__ part_ml, const float *__restrict__ part_acc,
    const float *__restrict__ blk_o, const float *__restrict__ blk_l, float *__restrict__ op_cache,
    float *__restrict__ lp_cache, T *__restrict__ out) {
    constexpr float kLn2 = 0.69314718055994530942f;
    // workgroup u * (S*Hk) + (s*Hk + g): consecutive workgroups go to the XCDs
    // in turn, so a group's rows run on the XCD that ran its prefix workgroups
    // (whose partials are still in that XCD's L2) whenever S*Hk is a multiple of 8
    const int ng = D.S * D.Hk;
    const int sgi = blockIdx.x % ng, u = blockIdx.x / ng;
    const int A = D.A, B = D.B, j = u / A, a = u % A, x = threadIdx.x;
    const int s = sgi / D.Hk, g = sgi % D.Hk, h = g * D.G + j;
    const int nch = D.n_chunks_sparse, rows = D.R;
    const size_t ar = ((size_t)s * D.Hq + h) * A + a;
    // every read at once: the row's token, the union size, its block part and
    // its partials (chunk indexes clamped into the buffer)
    const int tok = active[ar];
    const int ucnt = union_cnt[sgi];
    const float os = blk_o[ar * DIM + x], ls2 = blk_l[ar];
    const size_t pr0 = (size_t)sgi * nch * rows + j * A + a;
    const float *mlp = part_ml + pr0 * 2;
    const float *acp = part_acc + pr0 * DIM + x;
    const int cs = rows * 2, as = rows * DIM;  // chunk strides (elements)
    // a batch of kActBatch chunks: thread c of the batch reads chunk c's (m, l);
    // wave 0 forms the batch's running maximum and each chunk's weight
    // exp2(m - max) once, shared through LDS; every thread then combines its
    // dimension of the chunks' outputs in chunk order
    __shared__ float s_w[kActBatch], s_l[kActBatch], s_scale[2];  // weights, sums; factor, max
    float av[kActBatch];
    auto load_ml = [&](int c0) {
        return *reinterpret_cast<const float2 *>(mlp + min(c0 + min(x, kActBatch - 1), nch - 1) * cs);
    };
    auto load_acc = [&](int c0) {
#pragma unroll
        for (int i = 0; i < kActBatch; ++i) av[i] = acp[min(c0 + i, nch - 1) * as];
    };
    float2 ml = load_ml(0);
    load_acc(0);
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any is used
    const int nchu = (ucnt + D.sparse_chunk - 1) / D.sparse_chunk;  // chunks that wrote partials
    float mx = -__builtin_huge_valf(), ls = 0.0f, oa = 0.0f;  // running max, sum, output
    // The first batch is always combined (with no chunk it changes nothing), so
    // that its loads are needed on every path: if they were used only when the
    // union is not empty, the compiler would move them behind the union size's
    // read, a round trip later.
    int c0 = 0;
    do {
        if (c0 > 0) {
            ml = load_ml(c0);
            load_acc(c0);
            __syncthreads();  // the previous batch's weights have been read
        }
        const int n = min(kActBatch, nchu - c0);
        {
            // every wave runs this (lanes past the batch see no chunk and store
            // nothing), so that the (m, l) loads above are not moved into a
            // branch behind the union size's read
            const bool v = x < n;
            const float m = v ? ml.x : -__builtin_huge_valf();
            float bm = m;  // maximum over the batch: butterflies over the wave
            bm = fmaxf(bm, lane_xor1(bm));
            bm = fmaxf(bm, lane_xor2(bm));
            bm = fmaxf(bm, lane_xor7(bm));
            bm = fmaxf(bm, lane_xor15(bm));
            bm = fmaxf(bm, lane_xor16(bm));
            bm = fmaxf(bm, lane_xor32(bm));
            const float nm = fmaxf(mx, bm);
            // (every chunk so far empty: zero weights, factor 1)
            const bool none = nm == -__builtin_huge_valf();
            if (x < kActBatch) {
                s_w[x] = v && !none ? __builtin_amdgcn_exp2f(m - nm) : 0.0f;
                s_l[x] = v ? ml.y : 0.0f;
            }
            if (x == 0) {
                s_scale[0] = none ? 1.0f : __builtin_amdgcn_exp2f(mx - nm);
                s_scale[1] = nm;
            }
        }
        __syncthreads();
        const float sc = s_scale[0];
        mx = s_scale[1];
        ls *= sc;
        oa *= sc;
#pragma unroll
        for (int i = 0; i < kActBatch; ++i) {
            const float w = s_w[i];
            ls = fmaf(w, s_l[i], ls);
            oa = fmaf(w, i < n ? av[i] : 0.0f, oa);  // (chunks past the batch: clamped reads)
        }
        c0 += kActBatch;
    } while (c0 < nchu);
    float op = 0.0f, lp2 = -__builtin_huge_valf();
    if (nchu > 0) {
        op = oa / ls;
        lp2 = mx + __log2f(ls);
    }
    const size_t crow = ((size_t)s * D.Hq + h) * B + tok;
    if (!(D.flags & LOSA_FLAG_NO_WRITEBACK)) {  // else the caches keep the dense statistics
        op_cache[crow * DIM + x] = op;
        if (x == 0) lp_cache[crow] = lp2 * kLn2;
    }
    T *o = out + ((size_t)(s * B + tok) * D.Hq + h) * DIM + x;
    store_out(o, merge_parts(op, lp2, os, ls2));
}

size_t finish_lds_bytes(const Dims &D, int TG) {
    const size_t words = ((size_t)D.B * (D.d + 1) + (size_t)TG * D.d + (size_t)TG * D.B + TG + 3) &
                         ~(size_t)3;
    return words * 4 + (D.bf16 ? (size_t)D.B * D.d * 2 : 0);
}

// Tokens per workgroup: one output element per thread, 256 threads; the
// workgroup count (B / TG) * Hq * S then exceeds the CU count for the shapes
// of a long-context layer.
int finish_group(const Dims &D) {
    const int tg = kFinishMaxThreads / D.d;
    return D.B < tg ? D.B : tg;
}

hipError_t launch_finish(const Dims &D, const void *q_t, const void *k_blk, const void *v_blk,
                         const int32_t *kv_off, const int32_t *prefix_len, const Work &W,
                         float *op_cache, float *lp_cache, void *out, hipStream_t st) {
    const int TG = finish_group(D);
    dim3 grid(((D.B + TG - 1) / TG) * D.Hq * D.S);
    const size_t lds = finish_lds_bytes(D, TG);
    const int threads = TG * D.d;
#define LAUNCH_F(T, DIMV)                                                                         \
    hipLaunchKernelGGL((k_finish<T, DIMV>), grid, dim3(threads), lds, st, D, TG,                 \
                       static_cast<const T *>(q_t), static_cast<const T *>(k_blk),               \
                       static_cast<const T *>(v_blk), kv_off, prefix_len, W.part_ml, W.part_acc, \
                       op_cache, lp_cache, static_cast<T *>(out))
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

hipError_t launch_finish_active(const Dims &D, const Work &W, float *op_cache, float *lp_cache,
                                void *out, hipStream_t st) {
    if (D.A == 0) return hipSuccess;
    const dim3 grid(D.S * D.Hk * D.G * D.A);  // (row of the group, group)
#define LAUNCH_A(T, DIMV)                                                                        \
    hipLaunchKernelGGL((k_finish_active<T, DIMV>), grid, dim3(DIMV), 0, st, D, W.active,         \
                       W.union_cnt, W.part_ml, W.part_acc, W.blk_o, W.blk_l, op_cache, lp_cache, \
                       static_cast<T *>(out))
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

}  // namespace losa
