// Host-side launchers of the attention kernels (internal to libattn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Every launcher takes an optional block-sparse mask: bmask = uint8 [heads][T][T],
// T = ceil(N / 128), nonzero = kept (nullptr: dense); mhead = bytes between the
// masks of consecutive heads (0: one mask for every head).

hipError_t launch_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, bool bf16_in,
                      int BH, int N, int d, float scale, int causal, const uint8_t* bmask, long mhead,
                      hipStream_t st);

// D = rowsum(dO o O)
hipError_t launch_bwd_pre(const void* O, const void* dO, bool bf16_in, int BH, int N, int d, float* D,
                          hipStream_t st);

// bf16 inputs: dK, dV (one workgroup per key block) and dQ (one per query block),
// gradients written once in fp32 or bf16.
hipError_t launch_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                           const float* D, int BH, int N, int d, float scale, int causal, void* dK, void* dV,
                           bool bf16_grad, const uint8_t* bmask, long mhead, hipStream_t st);
// dQ with O == nullptr reads D; with O given it computes D = rowsum(dO o O) for its rows,
// uses it and writes it to D (for a key-side launch that follows).
hipError_t launch_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const float* LSE, float* D,
                         const void* O, int BH, int N, int d, float scale, int causal, void* dQ, bool bf16_grad,
                         const uint8_t* bmask, long mhead, hipStream_t st);

// fp32 inputs: zero dQacc, then one kernel for all three gradients (dQ by atomics).
hipError_t launch_bwd_f32(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                          const float* D, int BH, int N, int d, float scale, int causal, float* dQacc, float* dK,
                          float* dV, const uint8_t* bmask, long mhead, hipStream_t st);

// fp8 e4m3 inputs with per-tensor dequantisation factors; O in bf16 (d = 64 or 128).
hipError_t launch_fwd_fp8(const void* Q, const void* K, const void* V, float q_descale, float k_descale,
                          float v_descale, void* O, float* LSE, int BH, int N, int d, float scale, int causal,
                          hipStream_t st);

}  // namespace attn
