// fp8 forward: O = softmax(scale (sq Q8) (sk K8)^T) (sv V8), O in bf16, LSE in fp32.
//
// What it follows: the forward of the bf16 kernel (FlashAttention-2 review,
// 'core algorithm' answer, section 2 (1)-(2): tiles of K and V streamed past a
// block of queries with the running max and sum, one final division), fed with
// fp8 operands -- the review's research-directions answer names FP8 support as
// the missing piece for newer hardware.  Q, K and V arrive as OCP fp8 e4m3 bytes
// with one dequantisation factor per tensor (real Q = sq * Q8, ...).
//
// gfx950 mapping (workgroup = 4 waves, 32 queries per wave, 64-key tiles):
//   * S^T = K8 Q8^T with v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
//     fp8 x fp8 products are exact in the fp32 accumulator.  Every accumulator
//     lane holds one query and 32 of the tile's 64 keys, as in the bf16 kernel.
//   * P = exp2(S c - m) is rounded to fp8 e4m3 (RNE) and the 32 bytes of a lane
//     are the B operand of O^T += V8^T P^T with no data movement: the K = 64
//     contraction is permuted to the accumulator's key order and V^T is read
//     with the same permutation by ds_read_b64_tr_b8 (lane layout measured on
//     gfx950: in each group of 16 lanes, lane i receives byte i%8 of the 8-byte
//     reads of lanes 2k + (i >= 8), k = 0..7).
//   * The row sum l is one more MFMA against an all-ones A operand, so it sums
//     exactly the fp8 probabilities the numerator uses.
//   * Reference max: moved only when a tile's max exceeds it by more than 2^8
//     (log2 units), and then set 7 below the new max, so every P <= 2^8 < 448
//     (the e4m3 maximum) while the largest P of a row is >= 2^7, which keeps
//     small probabilities above the e4m3 subnormal floor relative to the row.
//   * K and V tiles go straight from HBM to LDS (direct-to-LDS loads) in rows of
//     128 bytes, 16-byte chunk c of row r in slot c ^ f(r) with f moving row bits
//     (2, 1, 3) to slot bits (0, 1, 2): conflict-free for both the 16-byte row
//     reads of K and the 8-byte transpose reads of V.
#include "../../include/attn.h"
#include "attn_common.h"
#include "attn_launch.h"
#include "attn_tuning.h"

namespace attn {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kFp8Headroom = 7.0f;          // log2 distance of a new reference below the row max
constexpr int kFp8One4 = 0x38383838;          // four e4m3 1.0

__device__ __forceinline__ int f8_swz(int r) { return ((r >> 2) & 1) | (r & 2) | ((r >> 1) & 4); }

template <int D, int BN_ = 64>
struct Fp8Cfg {
    static constexpr int BM = 128, BN = BN_, NKT = BN / 32, NPV = BN / 64, RB = 128;
    static constexpr int NS = D / 64;          // 64-byte contraction steps of S
    static constexpr int NDT = D / 32;         // 32-row tiles of O^T
    static constexpr int T_BYTES = BN * RB;
};

// Direct-to-LDS copy of `rows` rows of an fp8 [*, D] array into 128-byte swizzled
// rows, by one wave (8 rows per instruction).  Rows past the resource read as zeros;
// chunks past D are filled with zeros.
template <int D>
__device__ __forceinline__ void dma_rows8(__amdgpu_buffer_rsrc_t r, char* tile, int row0, int rows, int lane)
{
    constexpr int CPR = D / 16;
    for (int base = row0; base < row0 + rows; base += 8) {
        const int row = base + (lane >> 3);
        const int c = (lane & 7) ^ f8_swz(row);
        const uint32_t off = c < CPR ? (uint32_t)(row * D + c * 16) : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(tile + base * 128), 16,
                                                 off, 0, 0, 0);
    }
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(u32x4 a, u32x4 b)
{
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <int D, bool CAUSAL, int BN = 64>
__global__ __launch_bounds__(256, 2) void fwd_kernel_fp8(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                         const uint8_t* __restrict__ V, bf16* __restrict__ O,
                                                         float* __restrict__ LSE, int N, int nqblk, float c,
                                                         float v_scale, int negate_q, int slots)
{
    using C = Fp8Cfg<D, BN>;
    constexpr float NEG_INF = -__builtin_inff();
    __shared__ __attribute__((aligned(1024))) char sK0[C::T_BYTES], sK1[C::T_BYTES];
    __shared__ __attribute__((aligned(1024))) char sV0[C::T_BYTES], sV1[C::T_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    int head, qb;
    block_coords<CAUSAL, true>(blockIdx.x, gridDim.x, nqblk, slots, head, qb);
    const int q0 = qb * C::BM;
    const int q0w = q0 + 32 * wave;
    const int myq = q0w + l32;
    const size_t hoff = (size_t)head * (size_t)N * D;
    const uint8_t* __restrict__ Kh = K + hoff;
    const uint8_t* __restrict__ Vh = V + hoff;

    // Q fragments (B operand of S^T = K Q^T): bytes [64 s + 32 h, +32) of this lane's query row
    i32x8 qf[C::NS];
    {
        const auto rq = make_rsrc(Q + hoff, (uint32_t)N * D);
        const uint32_t ro = (uint32_t)myq * D + 32 * h;
        const uint32_t flip = negate_q ? 0x80808080u : 0u;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            const u32x4 a = buf_ld16(rq, ro + 64 * s) ^ flip, b = buf_ld16(rq, ro + 64 * s + 16) ^ flip;
            qf[s] = cat8(a, b);
        }
    }
    // per-lane LDS offsets: K rows (two 16-byte chunks per fragment) and V^T transpose reads
    int ko[C::NS][2], vo[C::NDT];
    {
        const int fr = f8_swz(l32);
#pragma unroll
        for (int s = 0; s < C::NS; ++s)
#pragma unroll
            for (int x = 0; x < 2; ++x) ko[s][x] = l32 * 128 + 16 * ((4 * s + 2 * h + x) ^ fr);
        const int g = lane >> 4, j = (lane & 15) >> 1, e = lane & 1;
        const int rl = 8 * (j >> 2) + 4 * h + (j & 3);       // key row this lane addresses (+16 per read)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) vo[dt] = rl * 128 + 16 * ((2 * dt + (g & 1)) ^ f8_swz(rl)) + 8 * e;
    }

    f32x16 oacc[C::NDT], lacc;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
    float mc = NEG_INF;
    const i32x8 ones = {kFp8One4, kFp8One4, kFp8One4, kFp8One4, kFp8One4, kFp8One4, kFp8One4, kFp8One4};

    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + C::BN - 1) / C::BN;

    auto issue_tile = [&](int j, char* sK, char* sV) __attribute__((always_inline)) {
        const int kv0 = j * C::BN;
        const uint32_t bytes = (uint32_t)(N - kv0) * D;          // rows past N read as zeros
        dma_rows8<D>(make_rsrc(Kh + (size_t)kv0 * D, bytes), sK, wave * (C::BN / 4), C::BN / 4, lane);
        dma_rows8<D>(make_rsrc(Vh + (size_t)kv0 * D, bytes), sV, wave * (C::BN / 4), C::BN / 4, lane);
    };

    auto tile_body = [&](int j, const char* sK, const char* sV) __attribute__((always_inline)) {
        const int kv0 = j * C::BN;
        f32x16 sacc[C::NKT];
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
            for (int s = 0; s < C::NS; ++s) {
                const i32x8 a = cat8(ld16(sK + kt * 32 * 128 + ko[s][0]), ld16(sK + kt * 32 * 128 + ko[s][1]));
                sacc[kt] = mfma_fp8(a, qf[s], sacc[kt]);
            }
        }
        // lane: query myq, keys kv0 + 32 kt + 8 (r/4) + 4 h + r%4
        const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > q0w) || (kv0 + C::BN > N);
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
                    if ((CAUSAL && key > myq) || key >= N) sacc[kt][r] = NEG_INF;
                }
        }
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx4[r >> 2] = max3f(mx4[r >> 2], sacc[kt][r], sacc[kt][r + 1]);
        float mx = max3f(mx4[0], mx4[1], fmaxf(mx4[2], mx4[3]));
        mx = fmaxf(mx, xor32(mx));
        const float mxc = (mx == NEG_INF) ? NEG_INF : mx * c;
        if (__builtin_amdgcn_ballot_w64(mxc > mc + kLazyLog2) != 0) {
            const float mnew = fmaxf(mc, mxc - kFp8Headroom);
            const float alpha = (mnew == NEG_INF) ? 1.f : fast_exp2(mc - mnew);   // 0 on the first tile
            lacc[0] *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            mc = mnew;
        }
        // P in fp8, bytes in (kt, r) order, 64 keys per contraction step: the B operands of
        // the P V and row-sum products
#pragma unroll
        for (int ks = 0; ks < C::NPV; ++ks) {
            int pw[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                float p[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sv = sacc[2 * ks + (w >> 2)][4 * (w & 3) + e];
                    p[e] = need_mask && sv == NEG_INF ? 0.f : fast_exp2(fmaf(sv, c, -mc));
                }
                int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], x, true);
            }
            const i32x8 pf = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
            lacc = mfma_fp8(ones, pf, lacc);
            // O^T += V^T P^T: four 8-byte transpose reads per 32-row tile of V^T
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                i32x2 t[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    t[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sV + ks * 64 * 128 + vo[dt] + i * 2048));
                const i32x8 a = {t[0][0], t[0][1], t[1][0], t[1][1], t[2][0], t[2][1], t[3][0], t[3][1]};
                oacc[dt] = mfma_fp8(a, pf, oacc[dt]);
            }
        }
    };

    auto step = [&](int j, const char* kc, const char* vc, char* kn, char* vn) __attribute__((always_inline)) {
        wait_vmem_all();                                // this wave's loads of tile j landed
        __syncthreads();                                // everyone's; tile j-1 fully read
        if (j + 1 < ntiles) issue_tile(j + 1, kn, vn);
        if (!(CAUSAL && j * C::BN > q0w + 31))          // else every key follows this wave's rows
            tile_body(j, kc, vc);
    };

    issue_tile(0, sK0, sV0);
    int j = 0;
    for (; j + 1 < ntiles; j += 2) {
        step(j, sK0, sV0, sK1, sV1);
        step(j + 1, sK1, sV1, sK0, sV0);
    }
    if (j < ntiles) step(j, sK0, sV0, sK1, sV1);

    // epilogue: one division by l (the sum of exactly the fp8 P), O (bf16) and LSE written once
    const float lt = lacc[0];
    const float inv = v_scale / lt;
    if (myq < N) {
        bf16* dst = O + (size_t)head * N * D + (size_t)myq * D;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * dt + 8 * g + 4 * h;
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = to_bf16(oacc[dt][4 * g + e] * inv);
                *reinterpret_cast<bf16x4*>(dst + d0) = v;
            }
        if (h == 0) LSE[(size_t)head * N + myq] = (mc + __log2f(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_fp8_dc(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH, int N,
                                float c, float v_scale, int negq, hipStream_t st)
{
    const int nqblk = (N + Fp8Cfg<D>::BM - 1) / Fp8Cfg<D>::BM;
    const TuneEntry t = tune_lookup(kTuneFwdFp8, D, CAUSAL, N);
    if (t.key_tile == 128)
        hipLaunchKernelGGL((fwd_kernel_fp8<D, CAUSAL, 128>), dim3(nqblk * BH), dim3(256), 0, st, (const uint8_t*)Q,
                           (const uint8_t*)K, (const uint8_t*)V, (bf16*)O, LSE, N, nqblk, c, v_scale, negq, t.slots);
    else
        hipLaunchKernelGGL((fwd_kernel_fp8<D, CAUSAL, 64>), dim3(nqblk * BH), dim3(256), 0, st, (const uint8_t*)Q,
                           (const uint8_t*)K, (const uint8_t*)V, (bf16*)O, LSE, N, nqblk, c, v_scale, negq, t.slots);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(const void* Q, const void* K, const void* V, float q_descale, float k_descale,
                          float v_descale, void* O, float* LSE, int BH, int N, int d, float scale, int causal,
                          hipStream_t st)
{
    const float sqk = scale * q_descale * k_descale;
    const float c = fabsf(sqk) * kLog2e;
    const int negq = sqk < 0.f;
    switch (d) {
        case 64:
            return causal ? launch_fp8_dc<64, true>(Q, K, V, O, LSE, BH, N, c, v_descale, negq, st)
                          : launch_fp8_dc<64, false>(Q, K, V, O, LSE, BH, N, c, v_descale, negq, st);
        case 128:
            return causal ? launch_fp8_dc<128, true>(Q, K, V, O, LSE, BH, N, c, v_descale, negq, st)
                          : launch_fp8_dc<128, false>(Q, K, V, O, LSE, BH, N, c, v_descale, negq, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
