// liblosa_selftest.so: checks of the hardware behaviour liblosa.so relies on,
// called only by the GPU tests (not part of the LoSA computation).
//  * one page-bound step, fma(q+, max, acc) then fma(q-, min, acc) with bf16
//    operands, must equal the IEEE round-to-nearest-even sum acc + q*sel;
//  * a plain copy kernel (HBM traffic calibration of the profiler counters,
//    and the bandwidth a short streaming kernel reaches) and an empty kernel
//    (the launch floor);
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

extern "C" {

int losa_selftest_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream) {
    if (bytes % 16 || blocks <= 0) return 1;
    hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
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
