// Page metadata for QUEST selection: element-wise min and max of each page's
// keys (the pages name QUEST as LoSA's selector for active tokens: gist.science
// pt summary, "3. Metodologia", step 3; the min/max bound is this library's
// reading of it).
//
// Layout (library-owned).  Pages are grouped per KV head into tiles of 64
// consecutive global pages (global page = kv_off/16 + local page).  Inside a
// tile, the metadata of chunk c of every page's dimensions is stored for the
// 64 pages back to back, 16 bytes per page, so a wave whose lane = page reads
// one chunk with one fully coalesced 1 KiB load:
//   bf16: chunk = 4 dimensions, one dword per dimension = (max | min << 16)
//   fp32: chunk = 2 dimensions, (max_0, min_0, max_1, min_1)
// That chunk is also exactly the B operand a lane supplies to
// v_mfma_f32_16x16x32_bf16 for 8 consecutive k-slots (max_i, min_i pairs).
// After the min/max part follows, per KV head and global page, the largest
// |key| element of the page (fp32), which bounds the error of MFMA scoring.
#include "losa_internal.h"

namespace losa {

template <typename T, int DIM>
__global__ __launch_bounds__(256) void k_page_meta(Dims D, const T *__restrict__ kc,
                                                   const int32_t *__restrict__ kv_off,
                                                   const int32_t *__restrict__ prefix_len,
                                                   uint32_t *__restrict__ meta) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int DPC = BF ? 4 : 2;       // dimensions per 16-byte chunk
    constexpr int NCH = DIM / DPC;
    __shared__ uint32_t s_amax[kTile];
    const int g = blockIdx.y, s = blockIdx.z;
    const SeqGeom sg = seq_geom(D, kv_off, prefix_len, s);
    if (threadIdx.x < kTile) s_amax[threadIdx.x] = 0u;
    __syncthreads();
    for (int item = threadIdx.x; item < kTile * NCH; item += blockDim.x) {
        const int pl = blockIdx.x * kTile + (item % kTile);
        const int c = item / kTile;
        if (pl >= sg.pages) continue;
        const int t0 = pl * kPage;
        const int t1 = min(t0 + kPage, sg.len);
        float mn[DPC], mx[DPC];
#pragma unroll
        for (int e = 0; e < DPC; ++e) {
            mn[e] = __builtin_huge_valf();
            mx[e] = -__builtin_huge_valf();
        }
        for (int t = t0; t < t1; ++t) {
            const T *row = kc + ((size_t)g * D.T + sg.off + t) * DIM + c * DPC;
#pragma unroll
            for (int e = 0; e < DPC; ++e) {
                float v;
                if constexpr (BF) v = bf16_to_f32(reinterpret_cast<const uint16_t *>(row)[e]);
                else v = reinterpret_cast<const float *>(row)[e];
                mn[e] = fminf(mn[e], v);
                mx[e] = fmaxf(mx[e], v);
            }
        }
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < DPC; ++e) am = fmaxf(am, fmaxf(fabsf(mn[e]), fabsf(mx[e])));
        atomicMax(&s_amax[item % kTile], __float_as_uint(am));  // non-negative: bits order as values
        const int64_t gp = sg.gp0 + pl;
        const int64_t tile = gp / kTile;
        const int lane = static_cast<int>(gp % kTile);
        uint4 u;
        if constexpr (BF) {
            // min/max of bf16 values are bf16 values: the top 16 bits are exact.
            u.x = (__float_as_uint(mx[0]) >> 16) | (__float_as_uint(mn[0]) & 0xffff0000u);
            u.y = (__float_as_uint(mx[1]) >> 16) | (__float_as_uint(mn[1]) & 0xffff0000u);
            u.z = (__float_as_uint(mx[2]) >> 16) | (__float_as_uint(mn[2]) & 0xffff0000u);
            u.w = (__float_as_uint(mx[3]) >> 16) | (__float_as_uint(mn[3]) & 0xffff0000u);
        } else {
            u.x = __float_as_uint(mx[0]);
            u.y = __float_as_uint(mn[0]);
            u.z = __float_as_uint(mx[1]);
            u.w = __float_as_uint(mn[1]);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(meta) +
                     ((size_t)(g * D.n_tiles_total + tile) * NCH + c) * kTile + lane;
        *dst = u;
    }
    __syncthreads();
    if (threadIdx.x < kTile) {
        const int pl = blockIdx.x * kTile + threadIdx.x;
        if (pl < sg.pages) {
            float *aux = reinterpret_cast<float *>(reinterpret_cast<char *>(meta) + D.meta_main_bytes);
            aux[(size_t)g * D.n_tiles_total * kTile + sg.gp0 + pl] = __uint_as_float(s_amax[threadIdx.x]);
        }
    }
}

hipError_t launch_page_meta(const Dims &D, const void *k_cache, const int32_t *kv_off,
                            const int32_t *prefix_len, void *meta, hipStream_t st) {
    dim3 grid((D.max_pages + kTile - 1) / kTile, D.Hk, D.S);
    if (grid.x == 0) return hipSuccess;
    auto *m = static_cast<uint32_t *>(meta);
    if (D.bf16) {
        if (D.d == 128)
            hipLaunchKernelGGL((k_page_meta<uint16_t, 128>), grid, dim3(256), 0, st, D,
                               static_cast<const uint16_t *>(k_cache), kv_off, prefix_len, m);
        else
            hipLaunchKernelGGL((k_page_meta<uint16_t, 64>), grid, dim3(256), 0, st, D,
                               static_cast<const uint16_t *>(k_cache), kv_off, prefix_len, m);
    } else {
        if (D.d == 128)
            hipLaunchKernelGGL((k_page_meta<float, 128>), grid, dim3(256), 0, st, D,
                               static_cast<const float *>(k_cache), kv_off, prefix_len, m);
        else
            hipLaunchKernelGGL((k_page_meta<float, 64>), grid, dim3(256), 0, st, D,
                               static_cast<const float *>(k_cache), kv_off, prefix_len, m);
    }
    return hipGetLastError();
}

}  // namespace losa
