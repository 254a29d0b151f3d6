// Measurement helper, not a step of the method: the bf16 MFMA rate this device sustains,
// the practical ceiling that the nominal dense bf16 peak is quoted beside.
//
// Every wave runs `iters` rounds of eight v_mfma_f32_32x32x16_bf16 over four independent
// accumulator chains, so an issue never waits on a result.  Workgroups are 4 waves; the
// caller picks the grid (4 workgroups per CU put 4 waves on every SIMD).  The accumulators
// are summed into `out` so that no product can be dropped.
#include "jt_internal.h"

namespace jt {

typedef __bf16 probe_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float probe_f32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_rate_kernel(int iters, float *out)
{
    const int lane = threadIdx.x & 63;
    probe_bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // lane-dependent operands: nothing folds at compile time
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    probe_f32x16_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            c[k][j] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            s += c[k][j];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

jt_status launch_mfma_rate(int iters, int blocks, float *out, hipStream_t st)
{
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, out);
    return launch_status(hipGetLastError());
}

} // namespace jt
