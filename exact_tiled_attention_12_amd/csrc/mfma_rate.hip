// Matrix-core rate probe for gfx950: back-to-back bf16 MFMAs, optionally with the other
// work an attention loop puts beside them, with shader-clock and real-time stamps.  A
// measurement aid for the attention kernels' roofline (what the matrix cores sustain, and
// at what clock, under each mix of work); it shares nothing with the attention kernels.
#include <hip/hip_runtime.h>

#include "../../include/mfma_rate.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 32768;

// MIX bit 0: every MFMA's A operand is a fragment read from LDS (16 bytes per lane, one
// ds_read_b128 per MFMA, the next round's four read after this round's products); bit 1:
// per MFMA one v_exp_f32 of an FMA, one max and one add, on independent chains (about the
// VALU work per product of an online-softmax attention loop).
template <int MIX>
__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(int iters, float* __restrict__ out,
                                                           unsigned long long* __restrict__ stamps)
{
    __shared__ __attribute__((aligned(16))) char lds[(MIX & 1) ? kLdsBytes : 16];
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)(lane + e));
        b[e] = (__bf16)(1.0f - 0.01f * (float)e);
    }
    if constexpr (MIX & 1) {
        for (int i = threadIdx.x; i < kLdsBytes / 16; i += blockDim.x)
            *reinterpret_cast<u32x4*>(lds + 16 * i) = __builtin_bit_cast(u32x4, a);
        __syncthreads();
    }
    // four independent accumulator chains: each product's result is needed three products later
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    float x0 = 0.1f * lane, x1 = x0 + 0.25f, x2 = x0 + 0.5f, x3 = x0 + 0.75f;
    float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f, z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
    const int wave = threadIdx.x >> 6;
    // round i reads four 1 KB rows of the 4 KB block (wave + i) mod 8, 16 bytes per lane
    const char* lane_base = lds + 16 * lane;
    bf16x8 r0 = a, r1 = a, r2 = a, r3 = a;
    auto rd = [&](int i, int k) __attribute__((always_inline)) {
        const char* p = lane_base + 4096 * ((unsigned)(wave + i) & 7u) + 1024 * k;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
    };
    if constexpr (MIX & 1) {
        r0 = rd(0, 0); r1 = rd(0, 1); r2 = rd(0, 2); r3 = rd(0, 3);
    }
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long s0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
        if constexpr (MIX & 1) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r0, b, c0, 0, 0, 0);
            r0 = rd(i + 1, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r1, b, c1, 0, 0, 0);
            r1 = rd(i + 1, 1);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r2, b, c2, 0, 0, 0);
            r2 = rd(i + 1, 2);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r3, b, c3, 0, 0, 0);
            r3 = rd(i + 1, 3);
        } else {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
        if constexpr ((MIX & 2) != 0) {
            x0 = __builtin_amdgcn_exp2f(fmaf(x0, 0.5f, -0.75f));
            x1 = __builtin_amdgcn_exp2f(fmaf(x1, 0.5f, -0.75f));
            x2 = __builtin_amdgcn_exp2f(fmaf(x2, 0.5f, -0.75f));
            x3 = __builtin_amdgcn_exp2f(fmaf(x3, 0.5f, -0.75f));
            y0 = fmaxf(y0, x0); y1 = fmaxf(y1, x1); y2 = fmaxf(y2, x2); y3 = fmaxf(y3, x3);
            z0 += x0; z1 += x1; z2 += x2; z3 += x3;
        }
    }
    float s = x0 + x1 + x2 + x3 + y0 + y1 + y2 + y3 + z0 + z1 + z2 + z3;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long s1 = __builtin_amdgcn_s_memrealtime();
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        stamps[4 * (size_t)blockIdx.x + 0] = t0;
        stamps[4 * (size_t)blockIdx.x + 1] = t1;
        stamps[4 * (size_t)blockIdx.x + 2] = s0;
        stamps[4 * (size_t)blockIdx.x + 3] = s1;
    }
}

}  // namespace

extern "C" int mfma_rate_probe(int workgroups, int iters, int mix, float* out, unsigned long long* stamps,
                               void* stream)
{
    if (workgroups < 1 || iters < 1 || mix < 0 || mix > 3 || out == nullptr || stamps == nullptr) return 1;
    const hipStream_t st = (hipStream_t)stream;
    switch (mix) {
        case 0: hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(workgroups), dim3(256), 0, st, iters, out, stamps); break;
        case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(workgroups), dim3(256), 0, st, iters, out, stamps); break;
        case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3(workgroups), dim3(256), 0, st, iters, out, stamps); break;
        default: hipLaunchKernelGGL(mfma_rate_kernel<3>, dim3(workgroups), dim3(256), 0, st, iters, out, stamps); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
