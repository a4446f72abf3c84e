// Host-side launchers of the attention kernels (internal to libattn.so).
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

hipError_t launch_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, bool bf16_in,
                      int BH, int N, int d, float scale, int causal, hipStream_t st);

hipError_t launch_bwd_pre(const void* O, const void* dO, bool bf16_in, int BH, int N, int d,
                          float* D, float* dQacc, hipStream_t st);

hipError_t launch_bwd_main(const void* Q, const void* K, const void* V, const void* dO,
                           const float* LSE, const float* D, bool bf16_in, int BH, int N, int d,
                           float scale, int causal, float* dQacc, void* dK, void* dV,
                           bool bf16_grad, hipStream_t st);

hipError_t launch_f32_to_bf16(const float* src, void* dst, long n, hipStream_t st);

}  // namespace attn
