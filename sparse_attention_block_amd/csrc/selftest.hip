// liblosa_selftest.so: checks of the hardware behaviour liblosa.so relies on,
// called only by the GPU tests (not part of the LoSA computation).
//  * one page-bound step, fma(q+, max, acc) then fma(q-, min, acc) with bf16
//    operands, must equal the IEEE round-to-nearest-even sum acc + q*sel;
//  * a plain copy kernel (HBM traffic calibration of the profiler counters),
//    a pure read kernel (the rate a short streaming read reaches), a gather
//    kernel with the sparse prefix pass's memory pattern and no arithmetic,
//    and an empty kernel (the launch floor);
//  * the operand/result lane layouts assumed for v_mfma_f32_16x16x32_bf16
//    and v_mfma_f32_16x16x16_bf16: lane l supplies row (or column) l%16 and
//    k-elements K*(l/16) .. K*(l/16)+K-1, and holds result rows
//    4*(l/16) .. +3 of column l%16.
// Every kernel reads and writes only inside the buffers sized by its caller.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__global__ void k_bound_step(const float *acc, const float *qp, const float *qn,
                             const uint32_t *meta, float *out, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const float mx = __uint_as_float(meta[i] << 16);
        const float mn = __uint_as_float(meta[i] & 0xffff0000u);
        float a = __builtin_fmaf(qp[i], mx, acc[i]);
        out[i] = __builtin_fmaf(qn[i], mn, a);
    }
}

// A: 16 x K row-major bf16, B: K x 16 row-major bf16, D: 16 x 16 row-major fp32; K = 32 or 16.
__global__ void k_mfma(int K, const uint16_t *A, const uint16_t *B, float *D) {
    const int l = threadIdx.x;
    const int r = l % 16, kb = l / 16;
    float4_t d = {0.f, 0.f, 0.f, 0.f};
    if (K == 32) {
        uint16_t a[8], b[8];
        for (int e = 0; e < 8; ++e) {
            a[e] = A[r * 32 + 8 * kb + e];
            b[e] = B[(8 * kb + e) * 16 + r];
        }
        bf16x8_t av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, d, 0, 0, 0);
    } else {
        short4_t av, bv;
        for (int e = 0; e < 4; ++e) {
            av[e] = static_cast<short>(A[r * 16 + 4 * kb + e]);
            bv[e] = static_cast<short>(B[(4 * kb + e) * 16 + r]);
        }
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, d, 0, 0, 0);
    }
    for (int j = 0; j < 4; ++j) D[(4 * kb + j) * 16 + r] = d[j];
}

// dst[i] = src[i] for n16 16-byte elements, grid-stride.
__global__ __launch_bounds__(256) void k_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                              size_t n16) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

__global__ void k_empty() {}

// Pure read of n16 16-byte elements: workgroup b reads a contiguous slice,
// each thread 8 loads in flight, and folds them with XOR; the fold is stored
// only when the caller sets `sink` (the reads must stay live), so the kernel
// moves no other bytes.  TAG (the size in MiB) only names the instantiation,
// so that a profiler's per-kernel statistics keep the sizes apart.
template <int TAG>
__global__ __launch_bounds__(256) void k_probe_read(const uint4 *__restrict__ src, size_t n16,
                                                    int sink, uint32_t *out) {
    constexpr int U = 8;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = blockIdx.x * per;
    const size_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint32_t acc = 0;
    for (size_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + (size_t)u * 256;
            v[u] = src[j < b1 ? j : b1 - 1];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (sink) out[blockIdx.x * 256 + threadIdx.x] = acc;
}

// The sparse prefix pass's memory pattern without its arithmetic: workgroup b
// (4 waves) reads its 4 page indexes from `list` (written by the kernel before
// it: one dependent round trip), wave w then reads page list[4b + w] of the
// pool (8 KiB: a page's keys and values), 8 loads of 16 bytes per lane in
// flight, folds them with XOR, and the workgroup stores as many bytes as the
// pass's split-K partial of 16 rows (16 x 130 floats).
constexpr int kGatherPageBytes = 8192;
constexpr int kGatherPartF4 = 16 * 130 / 4;
__global__ __launch_bounds__(256) void k_probe_gather(const int32_t *__restrict__ list,
                                                      const uint4 *__restrict__ pool,
                                                      float4 *__restrict__ part) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pg = list[blockIdx.x * 4 + w];
    const uint4 *src = pool + (size_t)pg * (kGatherPageBytes / 16);
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[u * 64 + lane];
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    const float f = __uint_as_float(acc & 0x3f7fffffu);  // finite
    float4 *dst = part + (size_t)blockIdx.x * kGatherPartF4;
    for (int i = threadIdx.x; i < kGatherPartF4; i += 256) dst[i] = make_float4(f, f, f, f);
}

extern "C" {

// list: 4 * blocks page indexes, each below pool_bytes / 8192 (the caller's
// guarantee: the list is device memory); part: blocks * 8320 bytes
int losa_selftest_gather(const int32_t *list, const void *pool, size_t pool_bytes, void *part,
                         int blocks, void *stream) {
    if (!list || !pool || !part || blocks <= 0 || pool_bytes < (size_t)kGatherPageBytes) return 1;
    hipLaunchKernelGGL(k_probe_gather, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       list, static_cast<const uint4 *>(pool), static_cast<float4 *>(part));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int losa_selftest_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream) {
    if (bytes % 16 || blocks <= 0) return 1;
    hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// bytes: a multiple of 16; out: blocks * 256 words when sink is set (else unused)
int losa_selftest_read(const void *src, size_t bytes, int blocks, int sink, void *out, void *stream) {
    if (bytes % 16 || bytes == 0 || blocks <= 0 || (sink && !out)) return 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint4 *p = static_cast<const uint4 *>(src);
    uint32_t *o = static_cast<uint32_t *>(out);
    const size_t n16 = bytes / 16;
#define PROBE(TAGV) hipLaunchKernelGGL(k_probe_read<TAGV>, dim3(blocks), dim3(256), 0, st, p, n16, sink, o)
    switch (bytes >> 20) {
        case 1: PROBE(1); break;
        case 8: PROBE(8); break;
        case 16: PROBE(16); break;
        case 64: PROBE(64); break;
        default: PROBE(0); break;
    }
#undef PROBE
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int losa_selftest_empty(void *stream) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int losa_selftest_bound_step(const float *acc, const float *qp, const float *qn,
                             const uint32_t *meta, float *out, int n, void *stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_bound_step, dim3((n + 255) / 256), dim3(256), 0,
                       static_cast<hipStream_t>(stream), acc, qp, qn, meta, out, n);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

int losa_selftest_mfma(int K, const uint16_t *A, const uint16_t *B, float *D, void *stream) {
    if (K != 32 && K != 16) return 1;
    hipLaunchKernelGGL(k_mfma, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), K, A, B, D);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
