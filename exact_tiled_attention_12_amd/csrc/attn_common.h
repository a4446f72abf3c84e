// Device-side building blocks shared by the forward and backward kernels
// (gfx950 / CDNA4 only).
//
// MFMA operand layout used throughout (32x32 output tiles, wave64):
//   A (M x K) and B (K x N) fragments: lane l supplies row (A) / column (B)
//   l % 32 and the E contraction elements [E*(l/32), E*(l/32)+E) of the step.
//   C/D (32 x 32 fp32, 16 registers): lane l holds column l % 32 and rows
//   8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
// Only the C/D layout has to be right for correctness: the contraction index
// of A and B may be permuted freely as long as both sides use the same
// permutation, which the kernels exploit to feed accumulators straight back
// into the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Per-element-type MFMA traits.
//   E  : contraction elements one lane supplies per MFMA
//   KS : contraction length of one MFMA (= 2 E)
//   CH : elements in a 16-byte chunk (unit of global loads)
template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int E = 8, KS = 16, CH = 8;
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int E = 1, KS = 2, CH = 4;
    typedef float frag;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// 16-byte chunk of T.
template <typename T> struct Chunk { u32x4 v; };

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Lane with the same query in the other half of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Workgroup index -> logical index so that consecutive logical indices (the
// blocks of one head) run on the same XCD and share its L2.  Hardware hands
// workgroups to the 8 XCDs round-robin.
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
    if ((nb & 7) != 0) return bid;
    return (bid & 7) * (nb >> 3) + (bid >> 3);
}

}  // namespace attn
