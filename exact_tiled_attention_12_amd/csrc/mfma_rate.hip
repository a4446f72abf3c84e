// Matrix-core rate probe for gfx950: back-to-back bf16 MFMAs on register operands, with
// shader-clock and real-time stamps.  A measurement aid for the attention kernels'
// roofline (what the matrix cores sustain at the clock the chip holds under load); it
// shares nothing with the attention kernels.
#include <hip/hip_runtime.h>

#include "../../include/mfma_rate.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(int iters, float* __restrict__ out,
                                                           unsigned long long* __restrict__ stamps)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)(lane + e));
        b[e] = (__bf16)(1.0f - 0.01f * (float)e);
    }
    // four independent accumulator chains: each product's result is needed three products later
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        stamps[4 * (size_t)blockIdx.x + 0] = t0;
        stamps[4 * (size_t)blockIdx.x + 1] = t1;
        stamps[4 * (size_t)blockIdx.x + 2] = r0;
        stamps[4 * (size_t)blockIdx.x + 3] = r1;
    }
}

}  // namespace

extern "C" int mfma_rate_probe(int workgroups, int iters, float* out, unsigned long long* stamps, void* stream)
{
    if (workgroups < 1 || iters < 1 || out == nullptr || stamps == nullptr) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, out, stamps);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
