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

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return zeros (hardware range check), which is how rows past N read as 0.
// Word 3 = 0x00020000: 32-bit data format, as untyped buffer loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// max(a, b, c) in one v_max3_f32.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Lane with the same query in the other half of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest p the forward lets a probability reach before it moves its reference
// max: 2^8 (log2 units).  Keeps fp32 sums and bf16 probabilities far from overflow.
constexpr float kLazyLog2 = 8.0f;

// Sum of the two bf16 halves of x added to acc (v_dot2_f32_bf16 against ones).
__device__ __forceinline__ float sum2_bf16(uint32_t x, float acc)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x), ones, acc, false);
}

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
