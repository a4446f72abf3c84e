// Backward kernels: D = rowsum(dO o O), then dQ, dK, dV by recomputation.
//
// What it follows: FlashAttention-2 review, 'core algorithm' answer, section 2
// (3) Backward Pass -- recompute S and P from the saved statistics instead of
// storing them, then dS, dQ = dS K, dK = dS^T Q, dV = P^T dO (read as the
// softmax Jacobian dS = P o (dP - D) with D_i = dO_i . O_i, and with the
// chain-rule factor `scale` on dQ and dK); '[LLM] Flash Attention' blog,
// "Recomputation" (more FLOPs, fewer HBM accesses).  The loop order (one
// workgroup per block of keys, iterating over query blocks, so dK and dV are
// reduced on chip and written once) follows the FlashAttention-2 review's
// point that the backward parallelises over the sequence with little
// synchronisation between blocks (results answer, section 3 (2)).
//
// gfx950 mapping.  Every kernel puts ONE key (key-side products) or ONE query
// (query-side products) on each accumulator lane, which is exactly the operand
// layout the following product needs:
//   * key side: S = Q K^T and dP = dO V^T with keys on lanes feed dV^T += dO^T P
//     and dK^T += Q^T dS, accumulated over all query blocks and written once;
//   * query side: S^T and dP^T with queries on lanes feed dQ^T += K^T dS^T;
//   * P = exp2(S * scale * log2e - LSE * log2e): no max and no sum are needed.
// bf16 inputs (the hot path): a key-side kernel (dK, dV) and a separate
// query-side kernel (dQ), both written once, no atomics, deterministic; K/V and
// Q/dO tiles go straight to swizzled LDS (direct-to-LDS loads) and transposed
// operands come from ds_read_b64_tr_b16.  fp32 inputs: one fused kernel with
// K and V fragments resident in registers, Q^T/dO^T staged transposed in LDS,
// and dQ added into a zero-filled fp32 accumulator with float atomics.
// Causal: query blocks entirely before a workgroup's keys are never visited;
// waves whose keys all follow a block's queries get P = 0 (or skip the block).
#include "attn_common.h"
#include "attn_launch.h"
#include "attn_tuning.h"

namespace attn {

// ----------------------------------------------------------------------------
// Preprocess: D_i = sum_k dO_ik O_ik (fp32).  Memory bound: 8 lanes per row,
// 32 rows per 256-thread block, 16-byte loads; a grid-stride loop over row
// groups, so the grid stays small for any number of rows.
// ----------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      float* __restrict__ Dout, long rows)
{
    constexpr int CH = Mma<T>::CH, CPR = D / CH, LPR = 8;
    const int u = threadIdx.x % LPR;
    for (long row = (long)blockIdx.x * (256 / LPR) + (threadIdx.x / LPR); row - (threadIdx.x / LPR) < rows;
         row += (long)gridDim.x * (256 / LPR)) {
        float acc = 0.f;
        if (row < rows) {
            const T* o = O + row * D;
            const T* g = dO + row * D;
            for (int cidx = u; cidx < CPR; cidx += LPR) {
                const u32x4 a = ld16(o + cidx * CH), b = ld16(g + cidx * CH);
                if constexpr (sizeof(T) == 2) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc = fmaf((float)av[e], (float)bv[e], acc);
                } else {
                    const f32x4 av = __builtin_bit_cast(f32x4, a), bv = __builtin_bit_cast(f32x4, b);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = fmaf(av[e], bv[e], acc);
                }
            }
        }
        // every lane of the wave takes part in the shuffles (the loop condition is uniform per block)
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (row < rows && u == 0) Dout[row] = acc;
    }
}

// Zero fill (a kernel rather than a memset, so callers may capture it in a graph); grid-stride.
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, long n4)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) st16(p + 4 * i, zero4());
}

// Blocks of an elementwise grid-stride launch: enough to fill the GPU several times over,
// never more than the work needs.
static inline unsigned stride_grid(long work_blocks)
{
    const long cap = 256L * 64;
    return (unsigned)(work_blocks < 1 ? 1 : work_blocks < cap ? work_blocks : cap);
}

// ----------------------------------------------------------------------------
// fp32 backward (all three gradients in one kernel, dQ by fp32 atomics into a
// zero-filled accumulator).  Used for fp32 inputs, where rows are twice as wide
// and the bf16 tile layouts below do not apply.
// ----------------------------------------------------------------------------
template <typename T, int D>
struct BwdCfg {
    static_assert(sizeof(T) == 4, "the fused kernel serves fp32 inputs");
    static constexpr int THREADS = 256;
    static constexpr int BN = 128;                       // keys per workgroup (32 per wave)
    static constexpr int BM = 32;                        // query rows per iteration
    static constexpr int NQT = BM / 32;
    static constexpr int DP = (D + 31) / 32 * 32;
    static constexpr int NDT = DP / 32;
    static constexpr int E = Mma<T>::E, KS = Mma<T>::KS, CH = Mma<T>::CH;
    static constexpr int NKS = D / KS;                   // steps over the head dim
    static constexpr int CPR = D / CH;
    static constexpr int QPITCH = D + 4;                          // Qs, dOs  [BM][QPITCH]
    static constexpr int TPITCH = BM + 4;                         // Qt, dOt  [DP][TPITCH]
    static constexpr int SPITCH = BN + 4;                         // dS       [BM][SPITCH]
    static constexpr int KTPITCH = BN + 4;                        // Kt       [DP][KTPITCH]
    static constexpr int OFF_QS = 0;
    static constexpr int OFF_DOS = OFF_QS + BM * QPITCH;
    static constexpr int OFF_QT = OFF_DOS + BM * QPITCH;
    static constexpr int OFF_DOT = OFF_QT + DP * TPITCH;
    static constexpr int OFF_DS = OFF_DOT + DP * TPITCH;
    static constexpr int OFF_KT = OFF_DS + BM * SPITCH;
    static constexpr int ELEMS = OFF_KT + DP * KTPITCH;
    static constexpr int BYTES = ELEMS * sizeof(T) + 2 * BM * sizeof(float);
    static constexpr int QGROUPS = (BM / 4) * CPR;       // 4 rows x 1 chunk per group
    static constexpr int QLD = (QGROUPS + THREADS - 1) / THREADS;
    static constexpr int KGROUPS = (BN / 4) * CPR;
    static constexpr int DQ_TILES = NQT * NDT;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(D % KS == 0 && D % CH == 0, "head dim");
};

// Transposed store of a 4-row x 1-chunk group (fp32): for each of the chunk's 4
// columns, the 4 rows' values are written contiguously at dst[col][row0..row0+3].
__device__ __forceinline__ void store_transposed4(float* base, int pitch, int col0, int row0, const u32x4 (&v)[4])
{
#pragma unroll
    for (int x = 0; x < 4; ++x)
        st16(base + (col0 + x) * pitch + row0, u32x4{v[0][x], v[1][x], v[2][x], v[3][x]});
}

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256) void bwd_kernel_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, const float* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      const float* __restrict__ Dg,
                                                      float* __restrict__ dQacc, float* __restrict__ dK,
                                                      float* __restrict__ dV, int N, int nkblk, float scale,
                                                      const uint8_t* __restrict__ bmask, long mhead, int slots)
{
    typedef float T;
    using C = BwdCfg<T, D>;
    static_assert(kMaskBlock == C::BN && kMaskBlock % C::BM == 0, "mask block = key block");
    using M = Mma<T>;
    typedef typename M::frag frag;

    __shared__ __attribute__((aligned(16))) char smem_raw[C::BYTES];
    T* smem = reinterpret_cast<T*>(smem_raw);
    T* Qs = smem + C::OFF_QS;
    T* dOs = smem + C::OFF_DOS;
    T* Qt = smem + C::OFF_QT;
    T* dOt = smem + C::OFF_DOT;
    T* dSl = smem + C::OFF_DS;
    T* Kt = smem + C::OFF_KT;
    float* lse_l = reinterpret_cast<float*>(smem_raw + C::ELEMS * sizeof(T));
    float* d_l = lse_l + C::BM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;

    int head, kb;
    block_coords<CAUSAL, false>(blockIdx.x, gridDim.x, nkblk, slots, head, kb);
    const int k0 = kb * C::BN;
    const int k0w = k0 + 32 * wave;            // this wave's first key
    const int mykey = k0w + l32;
    const size_t hoff = (size_t)head * (size_t)N * D;
    const T* __restrict__ Qh = Q + hoff;
    const T* __restrict__ Kh = K + hoff;
    const T* __restrict__ Vh = V + hoff;
    const T* __restrict__ dOh = dO + hoff;
    const float* __restrict__ LSEh = LSE + (size_t)head * N;
    const float* __restrict__ Dh = Dg + (size_t)head * N;
    float* __restrict__ dQh = dQacc + hoff;

    const float c2 = scale * kLog2e;

    // ---- resident K, V fragments (B operands of S = Q K^T and dP = dO V^T) ----
    frag kf[C::NKS], vf[C::NKS];
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) {
        const bool ok = mykey < N;
        kf[s] = ok ? Kh[(size_t)mykey * D + s * C::KS + h] : 0.f;
        vf[s] = ok ? Vh[(size_t)mykey * D + s * C::KS + h] : 0.f;
    }

    // ---- K^T of the workgroup's keys in LDS (B operand of dQ = dS K); pad rows zeroed ----
    for (int f = tid; f < C::KGROUPS; f += C::THREADS) {
        const int g = f / C::CPR, col = f - g * C::CPR;
        u32x4 v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = k0 + 4 * g + e;
            v[e] = key < N ? ld16(Kh + (size_t)key * D + col * C::CH) : zero4();
        }
        store_transposed4(Kt, C::KTPITCH, col * C::CH, 4 * g, v);
    }
    if constexpr (C::DP > D) {
        for (int x = tid; x < (C::DP - D) * C::KTPITCH; x += C::THREADS) Kt[D * C::KTPITCH + x] = from_f32<T>(0.f);
        for (int x = tid; x < (C::DP - D) * C::TPITCH; x += C::THREADS) {
            Qt[D * C::TPITCH + x] = from_f32<T>(0.f);
            dOt[D * C::TPITCH + x] = from_f32<T>(0.f);
        }
    }

    f32x16 dvacc[C::NDT], dkacc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[dt][r] = 0.f; dkacc[dt][r] = 0.f; }

    const int nq = (N + C::BM - 1) / C::BM;
    const int i0 = CAUSAL ? (k0 / C::BM) : 0;

    // ---- staging of one query block: Q, dO (4-row groups), LSE*log2e, D ----
    u32x4 qst[C::QLD][4], gst[C::QLD][4];
    float lst = 0.f, dst_ = 0.f;
    auto load_q = [&](int i) {
        const int q0 = i * C::BM;
#pragma unroll
        for (int it = 0; it < C::QLD; ++it) {
            const int f = tid + C::THREADS * it;
            if (f < C::QGROUPS) {
                const int g = f / C::CPR, col = f - g * C::CPR;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = q0 + 4 * g + e;
                    const bool ok = q < N;
                    qst[it][e] = ok ? ld16(Qh + (size_t)q * D + col * C::CH) : zero4();
                    gst[it][e] = ok ? ld16(dOh + (size_t)q * D + col * C::CH) : zero4();
                }
            }
        }
        if (tid < C::BM) {
            const int q = q0 + tid;
            lst = q < N ? LSEh[q] * kLog2e : __builtin_inff();
            dst_ = q < N ? Dh[q] : 0.f;
        }
    };
    auto store_q = [&]() {
#pragma unroll
        for (int it = 0; it < C::QLD; ++it) {
            const int f = tid + C::THREADS * it;
            if (f < C::QGROUPS) {
                const int g = f / C::CPR, col = f - g * C::CPR;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    st16(Qs + (4 * g + e) * C::QPITCH + col * C::CH, qst[it][e]);
                    st16(dOs + (4 * g + e) * C::QPITCH + col * C::CH, gst[it][e]);
                }
                store_transposed4(Qt, C::TPITCH, col * C::CH, 4 * g, qst[it]);
                store_transposed4(dOt, C::TPITCH, col * C::CH, 4 * g, gst[it]);
            }
        }
        if (tid < C::BM) { lse_l[tid] = lst; d_l[tid] = dst_; }
    };

    // the query blocks to visit: all from i0 on, or (block-sparse) those of kept mask rows
    // (kMaskBlock / BM query blocks per mask block); this workgroup's keys are mask column kb
    MaskWalk mw;
    constexpr int U = kMaskBlock / C::BM;
    if constexpr (SPARSE) {
        const int nmb = (N + kMaskBlock - 1) / kMaskBlock;
        mw.init(bmask + head * mhead + kb, nmb, nmb, lane);
    }
    auto next_block = [&](int i) __attribute__((always_inline)) {
        if constexpr (SPARSE) return mw.next_unit(i, nq, U, lane);
        else return i;
    };
    int i = next_block(i0);
    if (i < nq) load_q(i);
    for (int in; i < nq; i = in) {
        in = next_block(i + 1);
        const int q0 = i * C::BM;
        __syncthreads();                 // previous iteration's LDS readers are done
        store_q();
        __syncthreads();
        if (in < nq) load_q(in);

        const bool skip = CAUSAL && (k0w > q0 + C::BM - 1);   // all of this wave's keys after the block
        if (skip) {
            // contribute zeros to the dS tile the dQ product reads
            for (int x = lane; x < C::BM; x += 64) {
                T* row = dSl + x * C::SPITCH + 32 * wave;
#pragma unroll
                for (int y = 0; y < 32; ++y) row[y] = from_f32<T>(0.f);
            }
        } else {
            const bool need_mask = (CAUSAL && q0 < k0w + 31) || (q0 + C::BM > N) || (k0w + 32 > N);
            f32x16 sacc[C::NQT], pacc[C::NQT];
#pragma unroll
            for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
                for (int r = 0; r < 16; ++r) { sacc[qt][r] = 0.f; pacc[qt][r] = 0.f; }
            // S = Q K^T, dP = dO V^T
#pragma unroll
            for (int s = 0; s < C::NKS; ++s) {
#pragma unroll
                for (int qt = 0; qt < C::NQT; ++qt) {
                    const int off = (32 * qt + l32) * C::QPITCH + s * C::KS + C::E * h;
                    const frag a = Qs[off], g = dOs[off];
                    sacc[qt] = M::mma(a, kf[s], sacc[qt]);
                    pacc[qt] = M::mma(g, vf[s], pacc[qt]);
                }
            }
            // P = exp2(S c2 - LSE log2e); dS = P o (dP - D)   (sacc <- P, pacc <- dS)
#pragma unroll
            for (int qt = 0; qt < C::NQT; ++qt) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int qo = 32 * qt + 8 * g4 + 4 * h;
                    const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lse_l + qo);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(d_l + qo);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * g4 + e;
                        float p = fast_exp2(fmaf(sacc[qt][r], c2, -lse4[e]));
                        if (need_mask) {
                            const int q = q0 + qo + e;
                            if ((CAUSAL && mykey > q) || mykey >= N) p = 0.f;
                        }
                        sacc[qt][r] = p;
                        pacc[qt][r] = p * (pacc[qt][r] - d4[e]);
                    }
                }
            }
            // dV^T += dO^T P ;  dK^T += Q^T dS   (contraction over the block's queries)
#pragma unroll
            for (int qt = 0; qt < C::NQT; ++qt) {
#pragma unroll
                for (int s2 = 0; s2 < 32 / C::KS; ++s2) {
                    const frag bp = sacc[qt][s2], bs = pacc[qt][s2];
#pragma unroll
                    for (int dt = 0; dt < C::NDT; ++dt) {
                        const int rowoff = (32 * dt + l32) * C::TPITCH + 32 * qt;
                        const int o = rowoff + 8 * (s2 >> 2) + 4 * h + (s2 & 3);
                        const frag ag = dOt[o], aq = Qt[o];
                        dvacc[dt] = M::mma(ag, bp, dvacc[dt]);
                        dkacc[dt] = M::mma(aq, bs, dkacc[dt]);
                    }
                }
            }
            // dS -> LDS as [query][key] for the dQ product
#pragma unroll
            for (int qt = 0; qt < C::NQT; ++qt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qo = 32 * qt + 8 * (r >> 2) + 4 * h + (r & 3);
                    dSl[qo * C::SPITCH + 32 * wave + l32] = from_f32<T>(pacc[qt][r]);
                }
        }
        __syncthreads();
        // dQ[q][d] += scale * sum_key dS[q][key] K[key][d]  (tiles of 32 q x 32 d)
        for (int tile = wave; tile < C::DQ_TILES; tile += 4) {
            const int qt = tile % C::NQT, dt = tile / C::NQT;
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < C::BN / C::KS; ++s) {
                const T* pa = dSl + (32 * qt + l32) * C::SPITCH + s * C::KS + C::E * h;
                const T* pb = Kt + (32 * dt + l32) * C::KTPITCH + s * C::KS + C::E * h;
                acc = M::mma(*pa, *pb, acc);
            }
            const int dcol = 32 * dt + l32;
            if (dcol < D) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = q0 + 32 * qt + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (q < N) unsafeAtomicAdd(dQh + (size_t)q * D + dcol, acc[r] * scale);
                }
            }
        }
    }

    // ---- dK = scale * dK^T acc, dV = dV^T acc, written once ----
    if (mykey < N) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * dt + 8 * g4 + 4 * h;
                if (d0 < D) {
                    f32x4 a, b;
#pragma unroll
                    for (int e = 0; e < 4; ++e) { a[e] = dkacc[dt][4 * g4 + e] * scale; b[e] = dvacc[dt][4 * g4 + e]; }
                    *reinterpret_cast<f32x4*>(dK + hoff + (size_t)mykey * D + d0) = a;
                    *reinterpret_cast<f32x4*>(dV + hoff + (size_t)mykey * D + d0) = b;
                }
            }
    }
}

// ----------------------------------------------------------------------------
// bf16 backward, part 1: dK and dV.  One workgroup of 8 waves per BN = 128 keys,
// iterating over query blocks of BM = 64 rows.  Wave w owns the 32 keys of group
// w % 4 and the 32 query rows w / 4 of each block, so two waves share every key
// group and each keeps its own partial dK, dV (summed through LDS at the end).
// That keeps a wave under 256 registers: two waves per SIMD, one's VALU work
// overlapping the other's MFMAs.
//   S = Q K^T, dP = dO V^T       (accumulator lane = one key, rows = queries)
//   P = exp2(S c2 - LSE log2 e), dS = P o (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS   (contraction over queries; dO^T and Q^T
//                                      come from transpose reads of row tiles)
// LDS: sQ*/sG* hold the Q and dO rows of the current and next block (direct-to-LDS
// loads into swizzled rows); sK, sV the workgroup's K and V rows (row reads give
// the B operands of S and dP).  Separate __shared__ objects and a loop unrolled by
// two let the compiler see that the in-flight loads never alias the tiles read.
// ----------------------------------------------------------------------------
template <int D>
struct BwdKVCfg {
    static constexpr int BN = 128, BM = 64, WAVES = 8;
    static constexpr int RB = D == 64 ? 128 : 256;        // LDS bytes per row
    static constexpr int DP = (D + 31) / 32 * 32, NDT = DP / 32;
    static constexpr int NKS = D / 16;
    static constexpr int Q_BYTES = BM * RB, K_BYTES = BN * RB;
    static_assert(4 * Q_BYTES + 2 * K_BYTES + 4 * BM * 4 <= 160 * 1024, "LDS budget");
    // the end-of-kernel reduction parks one wave's dK (dV) partial, NDT*16 floats
    // per lane, in a Q/dO buffer (a K/V tile holds two of them)
    static_assert(NDT * 16 * 64 * 4 <= Q_BYTES, "dK partial fits a Q/dO buffer");
};

template <int D, bool CAUSAL, typename G, bool SPARSE>
__global__ __launch_bounds__(512) void bwd_dkdv_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                     const bf16* __restrict__ V, const bf16* __restrict__ dO,
                                                     const float* __restrict__ LSE, const float* __restrict__ Dg,
                                                     G* __restrict__ dK, G* __restrict__ dV, int N, int nkblk,
                                                     float scale, const uint8_t* __restrict__ bmask, long mhead,
                                                     int slots, int nitems)
{
    using C = BwdKVCfg<D>;
    static_assert(kMaskBlock == C::BN && kMaskBlock == 2 * C::BM, "mask block = key block");
    constexpr int RB = C::RB;
    constexpr uint32_t ROWB = D * 2;                    // global bytes per row
    __shared__ __attribute__((aligned(1024))) char sQ0[C::Q_BYTES], sQ1[C::Q_BYTES];
    __shared__ __attribute__((aligned(1024))) char sG0[C::Q_BYTES], sG1[C::Q_BYTES];
    __shared__ __attribute__((aligned(1024))) char sK[C::K_BYTES], sV[C::K_BYTES];
    __shared__ __attribute__((aligned(16))) float sL0[C::BM], sL1[C::BM], sD0[C::BM], sD1[C::BM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3, qh = wave >> 2;            // key group, query half
    const int l32 = lane & 31, h = lane >> 5;

    // persistent grid (one workgroup per CU) over the nitems (head, key block) items
    ItemWalk walk;
    walk.init(blockIdx.x, gridDim.x, nitems, items_split<CAUSAL>(nitems, nkblk));
    for (int t = 0;; ++t) {
    const int item = walk.item(t);
    if (item < 0) break;
    int head, kb;
    block_coords<CAUSAL, false>(item, nitems, nkblk, slots, head, kb);
    const int k0 = kb * C::BN;
    const int k0w = k0 + 32 * kg;
    const int mykey = k0w + l32;
    const size_t hoff = (size_t)head * (size_t)N * D;
    const bf16* __restrict__ Qh = Q + hoff;
    const bf16* __restrict__ dOh = dO + hoff;
    const float c2 = scale * kLog2e;
    // fragment offsets of this wave's own row bands: keys 32 kg.. of K/V, queries 32 qh.. of Q/dO
    TileLane<RB, C::NKS, C::NDT, false> tlk, tlq;
    tlk.init(lane, 32 * kg);
    tlq.init(lane, 32 * qh);

    // the workgroup's K and V rows to LDS (16 rows per wave each); after the first item
    // the previous item's epilogue has already issued them
    auto issue_kv = [&](size_t ho, int kk0) {
        const uint32_t bytes = (uint32_t)(N - kk0) * ROWB;
        int lane_k = lane;                              // opaque: offsets computed here, not held in registers
        asm volatile("" : "+v"(lane_k));
        dma_rows<D, RB, false>(make_rsrc(K + ho + (size_t)kk0 * D, bytes), sK, wave * (C::BN / 8), C::BN / 8, lane_k);
        dma_rows<D, RB, false>(make_rsrc(V + ho + (size_t)kk0 * D, bytes), sV, wave * (C::BN / 8), C::BN / 8, lane_k);
    };
    if (t == 0) issue_kv(hoff, k0);

    f32x16 dvacc[C::NDT], dkacc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[dt][r] = 0.f; dkacc[dt][r] = 0.f; }

    const int nq = (N + C::BM - 1) / C::BM;
    const int i0 = CAUSAL ? (k0 / C::BM) : 0;

    float lreg = 0.f;
    auto issue_block = [&](int i, char* sQ, char* sG) {
        const int q0 = i * C::BM;
        const uint32_t bytes = (uint32_t)(N - q0) * ROWB;         // rows past N read as zeros
        dma_rows<D, RB, false>(make_rsrc(Qh + (size_t)q0 * D, bytes), sQ, wave * (C::BM / 8), C::BM / 8, lane);
        dma_rows<D, RB, false>(make_rsrc(dOh + (size_t)q0 * D, bytes), sG, wave * (C::BM / 8), C::BM / 8, lane);
        // raw values: scaling here would make wave 0 wait for every load in flight, the block's
        // Q/dO rows included, right after issuing them (the step top scales LSE after its wait)
        if (wave == 0) lreg = buf_ld4f(make_rsrc(LSE + (size_t)head * N + q0, (uint32_t)(N - q0) * 4), lane * 4);
        if (wave == 1) lreg = buf_ld4f(make_rsrc(Dg + (size_t)head * N + q0, (uint32_t)(N - q0) * 4), lane * 4);
    };

    // One query block, ordered so that each wave's VALU work overlaps its own MFMAs:
    //   S = Q K^T;  dP = dO V^T while P = exp2(S c2 - LSE log2 e) is computed (in place);
    //   dV^T += dO^T P while dS = P o (dP - D) is computed;  dK^T += Q^T dS.
    // Fragments are read PF MFMAs ahead through small rings; sched_barrier keeps each
    // MFMA next to its slice of VALU work.
    // `loads` issues the next block's direct-to-LDS loads; it runs after the fourth score product,
    // so that the step's loads do not all queue at the address unit while the waves wait
    auto block_body = [&](int i, const char* sQ, const char* sG, const float* sL, const float* sD, auto&& loads) {
        const int q0 = i * C::BM;
        // the two waves of a SIMD run the same block; priority 3, 2, 1, 0 over its four products
        // gives the wave that is behind the issue slots (else the older wave always wins them,
        // finishes first and idles at the next barrier while the other runs alone)
        __builtin_amdgcn_s_setprio(3);
        constexpr int PF = 4, NKS = C::NKS, NDT = C::NDT;
        f32x16 sacc, pacc;
        {
            constexpr int NF = 2 * NKS;                 // f: s = f / 2; A (Q rows), then B (K rows)
            static_assert(NF >= 8, "the loads go out after the fourth product");
            auto frag = [&](int f) __attribute__((always_inline)) {
                return (f & 1) ? tlk.row(sK, 0, f >> 1) : tlq.row(sQ, 0, f >> 1);
            };
            bf16x8 ring[PF];
#pragma unroll
            for (int f = 0; f < PF; ++f) ring[f] = frag(f);
#pragma unroll
            for (int f = 0; f < NF; f += 2) {
                const bf16x8 a = ring[f % PF], b = ring[(f + 1) % PF];
                if (f + PF < NF) {
                    ring[f % PF] = frag(f + PF);
                    ring[(f + 1) % PF] = frag(f + PF + 1);
                }
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, f == 0 ? f32x16{} : sacc, 0, 0, 0);
                if (f == 6) loads();                      // NF >= 8 for every head dim
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(2);
        {
            constexpr int NF = 2 * NKS;                 // dO rows (A), V rows (B)
            auto frag = [&](int f) __attribute__((always_inline)) {
                return (f & 1) ? tlk.row(sV, 0, f >> 1) : tlq.row(sG, 0, f >> 1);
            };
            bf16x8 ring[PF];
#pragma unroll
            for (int f = 0; f < PF; ++f) ring[f] = frag(f);
            f32x4 l4[2];
            l4[0] = *reinterpret_cast<const f32x4*>(sL + 32 * qh + 4 * h);
#pragma unroll
            for (int f = 0; f < NF; f += 2) {
                const int s = f >> 1;
                const bf16x8 a = ring[f % PF], b = ring[(f + 1) % PF];
                if (f + PF < NF) {
                    ring[f % PF] = frag(f + PF);
                    ring[(f + 1) % PF] = frag(f + PF + 1);
                }
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, f == 0 ? f32x16{} : pacc, 0, 0, 0);
                // P of score elements [16 s / NKS, 16 (s + 1) / NKS), in place; row group g4 = r / 4
#pragma unroll
                for (int r = 16 * s / NKS; r < 16 * (s + 1) / NKS; ++r) {
                    const int g4 = r >> 2;
                    if ((r & 3) == 0 && g4 + 1 < 4)     // the next group's -LSE log2 e, one group ahead
                        l4[(g4 + 1) & 1] = *reinterpret_cast<const f32x4*>(sL + 32 * qh + 8 * (g4 + 1) + 4 * h);
                    sacc[r] = fast_exp2(fmaf(sacc[r], c2, l4[g4 & 1][r & 3]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // (a wave whose keys all follow its queries gets P = 0 from the mask; skipping
        // it instead would split the accumulators' live ranges)
        if (CAUSAL && (q0 + 32 * qh < k0w + 31)) {      // key > query -> 0
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (mykey > q0 + 32 * qh + 8 * (r >> 2) + 4 * h + (r & 3)) sacc[r] = 0.f;
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = to_bf16(sacc[r]);
        __builtin_amdgcn_s_setprio(1);
        // dV^T += dO^T P (products m = s2 * NDT + dt) while dS = P (dP - D) is computed
        {
            constexpr int NM = 2 * NDT;
            auto frag = [&](int m) __attribute__((always_inline)) {
                return tlq.tr(sG, 16 * (m / NDT), m % NDT);
            };
            bf16x8 ring[PF];
#pragma unroll
            for (int m = 0; m < PF && m < NM; ++m) ring[m] = frag(m);
            f32x4 d4[2];
            d4[0] = *reinterpret_cast<const f32x4*>(sD + 32 * qh + 4 * h);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const bf16x8 a = ring[m % PF];
                if (m + PF < NM) ring[m % PF] = frag(m + PF);
                const int s2 = m / NDT, dt = m % NDT;
                dvacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s2], dvacc[dt], 0, 0, 0);
#pragma unroll
                for (int r = 16 * m / NM; r < 16 * (m + 1) / NM; ++r) {
                    const int g4 = r >> 2;
                    if ((r & 3) == 0 && g4 + 1 < 4)
                        d4[(g4 + 1) & 1] = *reinterpret_cast<const f32x4*>(sD + 32 * qh + 8 * (g4 + 1) + 4 * h);
                    sb[r >> 3][r & 7] = to_bf16(sacc[r] * (pacc[r] - d4[g4 & 1][r & 3]));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // dK^T += Q^T dS
        {
            constexpr int NM = 2 * NDT;
            auto frag = [&](int m) __attribute__((always_inline)) {
                return tlq.tr(sQ, 16 * (m / NDT), m % NDT);
            };
            bf16x8 ring[PF];
#pragma unroll
            for (int m = 0; m < PF && m < NM; ++m) ring[m] = frag(m);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const bf16x8 a = ring[m % PF];
                if (m + PF < NM) ring[m % PF] = frag(m + PF);
                dkacc[m % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[m / NDT], dkacc[m % NDT], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if constexpr (!SPARSE) {
        auto step = [&](int i, char* qc, char* gc, float* lc, float* dc, char* qn, char* gn) {
            wait_vmem_all();                            // this wave's loads of block i landed
            if (wave == 0) lc[lane] = -kLog2e * lreg;
            if (wave == 1) dc[lane] = lreg;
            __syncthreads();                            // everyone's loads landed; block i-1 fully read
            block_body(i, qc, gc, lc, dc, [&]() __attribute__((always_inline)) {
                if (i + 1 < nq) issue_block(i + 1, qn, gn);
            });
        };
        issue_block(i0, sQ0, sG0);
        int i = i0;
        for (; i + 1 < nq; i += 2) {
            step(i, sQ0, sG0, sL0, sD0, sQ1, sG1);
            step(i + 1, sQ1, sG1, sL1, sD1, sQ0, sG0);
        }
        if (i < nq) step(i, sQ0, sG0, sL0, sD0, sQ1, sG1);
    } else {
        // in: the next query block to visit (nq if none)
        auto step = [&](int i, int in, char* qc, char* gc, float* lc, float* dc, char* qn, char* gn) {
            wait_vmem_all();
            if (wave == 0) lc[lane] = -kLog2e * lreg;
            if (wave == 1) dc[lane] = lreg;
            __syncthreads();
            block_body(i, qc, gc, lc, dc, [&]() __attribute__((always_inline)) {
                if (in < nq) issue_block(in, qn, gn);
            });
        };
        // only the query blocks of kept mask rows (two 64-query blocks per mask block);
        // this workgroup's keys are mask column kb
        const int nmb = (N + kMaskBlock - 1) / kMaskBlock;
        MaskWalk mw;
        mw.init(bmask + head * mhead + kb, nmb, nmb, lane);
        int i = mw.next_unit(i0, nq, 2, lane);
        if (i < nq) issue_block(i, sQ0, sG0);
        while (i < nq) {
            int in = mw.next_unit(i + 1, nq, 2, lane);
            step(i, in, sQ0, sG0, sL0, sD0, sQ1, sG1);
            i = in;
            if (i >= nq) break;
            in = mw.next_unit(i + 1, nq, 2, lane);
            step(i, in, sQ1, sG1, sL1, sD1, sQ0, sG0);
            i = in;
        }
    }

    // Epilogue.  The two query halves' partials are summed in LDS, row-major (one key per
    // row, DP floats, 16-byte chunks XOR-swizzled by the row so that the MFMA-layout writes
    // and the row reads are free of bank conflicts), key group g's rows in the g-th Q/dO
    // buffer: dV first, then dK.  The first query half puts its partials there, the second
    // adds its own, then waves 2g and 2g + 1 store group g's rows, so each store instruction
    // writes contiguous memory.  The K/V tiles are free from the start of the epilogue, so
    // the next item's K and V rows are issued first and load during the sums.  The sums'
    // barriers order LDS only (lds_barrier), and every staging access names its Q/dO buffer
    // directly, so that the compiler sees it apart from the K/V tiles being loaded (through a
    // pointer chosen per wave it cannot, and would wait for those loads).
    wait_vmem_all();
    __syncthreads();                                    // every tile fully read
    {
        const int nitem = walk.item(t + 1);
        if (nitem >= 0) {
            int nhead, nkb;
            block_coords<CAUSAL, false>(nitem, nitems, nkblk, slots, nhead, nkb);
            issue_kv((size_t)nhead * (size_t)N * D, nkb * C::BN);
        }
    }
    {
        constexpr int NCHP = C::DP / 4 <= 16 ? 16 : 32;  // 16-byte chunks per LDS row (power of two)
        constexpr int GROUP_BYTES = 32 * NCHP * 16;      // one key group's rows
        static_assert(GROUP_BYTES <= C::Q_BYTES, "epilogue staging fits");
        auto soff = [](int row, int ch) { return (row * NCHP + (ch ^ (row & 15))) * 16; };
        // lane index made opaque here, so that the offsets below are computed per item and
        // not hoisted out of the item loop (where they would sit in registers the main loop needs)
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int l32e = lane_e & 31, he = lane_e >> 5, tid_e = 64 * wave + lane_e;
        auto sum_store = [&](const f32x16 (&acc)[C::NDT], G* __restrict__ dst, float mult) {
            // lane: key row l32 of the group; accumulator rows d = 32 dt + 8 g4 + 4 h + e -> chunk 8 dt + 2 g4 + h
            // (rows d >= D are padding, d = 80)
            auto put = [&](char* buf) __attribute__((always_inline)) {
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        if (32 * dt + 8 * g4 < D)
                            *reinterpret_cast<f32x4*>(buf + soff(l32e, 8 * dt + 2 * g4 + he)) =
                                f32x4{acc[dt][4 * g4], acc[dt][4 * g4 + 1], acc[dt][4 * g4 + 2], acc[dt][4 * g4 + 3]};
            };
            // every partial read before the first write, so that the reads are in flight together
            auto add = [&](char* buf) __attribute__((always_inline)) {
                f32x4 pk[C::NDT * 4];
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        if (32 * dt + 8 * g4 < D)
                            pk[4 * dt + g4] = *reinterpret_cast<const f32x4*>(buf + soff(l32e, 8 * dt + 2 * g4 + he));
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        if (32 * dt + 8 * g4 < D) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) pk[4 * dt + g4][e] += acc[dt][4 * g4 + e];
                            *reinterpret_cast<f32x4*>(buf + soff(l32e, 8 * dt + 2 * g4 + he)) = pk[4 * dt + g4];
                        }
            };
            // one branch per key group, each naming its buffer; the distinct empty asm
            // statements keep the compiler from merging the four into one access through
            // a selected pointer
            if (qh == 0) {
                if (kg == 0) { asm volatile("; put 0"); put(sQ0); asm volatile("; put 0 end"); }
                if (kg == 1) { asm volatile("; put 1"); put(sQ1); asm volatile("; put 1 end"); }
                if (kg == 2) { asm volatile("; put 2"); put(sG0); asm volatile("; put 2 end"); }
                if (kg == 3) { asm volatile("; put 3"); put(sG1); asm volatile("; put 3 end"); }
            }
            lds_barrier();
            if (qh == 1) {
                if (kg == 0) { asm volatile("; add 0"); add(sQ0); asm volatile("; add 0 end"); }
                if (kg == 1) { asm volatile("; add 1"); add(sQ1); asm volatile("; add 1 end"); }
                if (kg == 2) { asm volatile("; add 2"); add(sG0); asm volatile("; add 2 end"); }
                if (kg == 3) { asm volatile("; add 3"); add(sG1); asm volatile("; add 3 end"); }
            }
            lds_barrier();
            // waves 2g and 2g + 1 store group g's rows: D/4 chunks per key row, consecutive threads
            // take consecutive chunks of a row.  The stores are range-checked (rows past N fall
            // outside the buffer and are dropped), so no pass branches and the group's LDS reads
            // all issue before its first store.
            constexpr int CPR = D / 4, GTOTAL = 32 * CPR, GTHREADS = 128, NPASS = GTOTAL / GTHREADS;
            static_assert(GTOTAL % GTHREADS == 0, "whole passes");
            const int gt = tid_e & (GTHREADS - 1);
            const auto ro = make_rsrc(dst + hoff + (size_t)k0 * D, (uint32_t)(N - k0) * (uint32_t)(D * sizeof(G)));
            auto rows = [&](const char* buf, int g) __attribute__((always_inline)) {
                f32x4 a[NPASS];
#pragma unroll
                for (int pass = 0; pass < NPASS; ++pass) {
                    const int c = pass * GTHREADS + gt;
                    const int row = c / CPR, ch = c - row * CPR;
                    a[pass] = *reinterpret_cast<const f32x4*>(buf + soff(row, ch));
                }
#pragma unroll
                for (int pass = 0; pass < NPASS; ++pass) {
                    const int c = pass * GTHREADS + gt;
                    const int row = c / CPR, ch = c - row * CPR;
                    const int off = ((32 * g + row) * D + 4 * ch) * (int)sizeof(G);
                    if constexpr (sizeof(G) == 4) {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, a[pass] * mult), ro, off, 0, 0);
                    } else {
                        bf16x4 x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = to_bf16(a[pass][e] * mult);
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), ro, off, 0, 0);
                    }
                }
            };
            const int wg2 = wave >> 1;
            if (wg2 == 0) { asm volatile("; rows 0"); rows(sQ0, 0); asm volatile("; rows 0 end"); }
            if (wg2 == 1) { asm volatile("; rows 1"); rows(sQ1, 1); asm volatile("; rows 1 end"); }
            if (wg2 == 2) { asm volatile("; rows 2"); rows(sG0, 2); asm volatile("; rows 2 end"); }
            if (wg2 == 3) { asm volatile("; rows 3"); rows(sG1, 3); asm volatile("; rows 3 end"); }
            lds_barrier();                               // the staging rows are read
        };
        sum_store(dvacc, dV, 1.0f);                     // dV = (dV^T acc)^T
        sum_store(dkacc, dK, scale);                    // dK = scale * (dK^T acc)^T
    }
    }
}

// ----------------------------------------------------------------------------
// bf16 backward, part 2: dQ.  One workgroup per BM = 128 query rows (32 per
// wave, two workgroups per CU), iterating over key tiles of BN = 64 -- the same
// shape as the forward, and the same trick: work on transposes so that every
// accumulator lane holds ONE query.
//   S^T = K Q^T, dP^T = V dO^T        (A = K, V row reads; B = Q, dO registers)
//   P^T = exp2(S^T c2 - LSE log2 e), dS^T = P^T o (dP^T - D)   (per-lane LSE, D)
//   dQ^T += K^T dS^T                   (A = K^T by transpose reads; B = dS^T from
//                                       the accumulator registers, bf16)
// dQ is written once (no atomics, deterministic).
// ----------------------------------------------------------------------------
template <int D>
struct BwdQCfg {
    static constexpr int BM = 128, BN = 64, NKT = BN / 32;
    static constexpr int RB = D == 64 ? 128 : 256;
    static constexpr int DP = (D + 31) / 32 * 32, NDT = DP / 32;
    static constexpr int NKS = D / 16;
    static constexpr int T_BYTES = BN * RB;
    static_assert(4 * T_BYTES <= 80 * 1024, "two workgroups per CU");
};

template <int D, bool CAUSAL, typename G, bool SPARSE>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                      const bf16* __restrict__ V, const bf16* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ Dg,
                                                      const bf16* __restrict__ Og, G* __restrict__ dQ, int N,
                                                      int nqblk, float scale, const uint8_t* __restrict__ bmask,
                                                      long mhead, int slots)
{
    using C = BwdQCfg<D>;
    static_assert(kMaskBlock == C::BM && kMaskBlock == 2 * C::BN, "mask block = query block");
    constexpr int RB = C::RB;
    constexpr uint32_t ROWB = D * 2;
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
    const bf16* __restrict__ Kh = K + hoff;
    const bf16* __restrict__ Vh = V + hoff;
    const float c2 = scale * kLog2e;
    TileLane<RB, C::NKS, C::NDT, true> tl;
    tl.init(lane);

    // Q and dO fragments (B operands), this lane's -LSE*log2e and D
    bf16x8 qf[C::NKS], gf[C::NKS];
    float nlse, dq_d;
    {
        const uint32_t hb = (uint32_t)N * ROWB;
        const auto rq = make_rsrc(Q + hoff, hb), rg = make_rsrc(dO + hoff, hb);
        const uint32_t ro = (uint32_t)myq * ROWB + 16 * h;
#pragma unroll
        for (int s = 0; s < C::NKS; ++s) {
            qf[s] = __builtin_bit_cast(bf16x8, buf_ld16(rq, ro + 32 * s));
            gf[s] = __builtin_bit_cast(bf16x8, buf_ld16(rg, ro + 32 * s));
        }
        nlse = -kLog2e * buf_ld4f(make_rsrc(LSE + (size_t)head * N, (uint32_t)N * 4), myq * 4);
        if (Og != nullptr) {
            // D = rowsum(dO o O) from this lane's half row of O and the dO fragments, written for
            // the key-side kernel (rows past N read as zeros and are not written)
            const auto ro_o = make_rsrc(Og + hoff, hb);
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < C::NKS; ++s) {
                const bf16x8 o = __builtin_bit_cast(bf16x8, buf_ld16(ro_o, ro + 32 * s));
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)gf[s][e], acc);
            }
            dq_d = acc + xor32(acc);
            if (h == 0 && myq < N) Dg[(size_t)head * N + myq] = dq_d;
        } else {
            dq_d = buf_ld4f(make_rsrc(Dg + (size_t)head * N, (uint32_t)N * 4), myq * 4);
        }
    }

    f32x16 dqacc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[dt][r] = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + C::BN - 1) / C::BN;

    auto issue_tile = [&](int j, char* sK, char* sV) {
        const int kv0 = j * C::BN;
        const uint32_t bytes = (uint32_t)(N - kv0) * ROWB;        // rows past N read as zeros
        dma_rows<D, RB, true>(make_rsrc(Kh + (size_t)kv0 * D, bytes), sK, wave * (C::BN / 4), C::BN / 4, lane);
        dma_rows<D, RB, true>(make_rsrc(Vh + (size_t)kv0 * D, bytes), sV, wave * (C::BN / 4), C::BN / 4, lane);
    };

    // One key tile, ordered so that each wave's VALU work overlaps its own MFMAs:
    //   S^T = K Q^T;  dP^T = V dO^T while P^T = exp2(S^T c2 - LSE log2 e) is computed (in place);
    //   dS^T of keys 0-31;  dQ^T += K^T dS^T for keys 0-31 while dS^T of keys 32-63 is computed;
    //   dQ^T += K^T dS^T for keys 32-63.  Fragments go PF products ahead through small rings.
    auto tile_body = [&](int j, const char* sK, const char* sV) {
        static_assert(C::NKT == 2, "two 32-key halves per tile");
        const int kv0 = j * C::BN;
        // key kv0 + 4 h + cr is masked (follows the query, or lies past N) when cr > bound; only
        // tiles that cross the wave's diagonal or N need it.  A key past N reads as a zero row,
        // whose P = exp(-LSE) can overflow when every score of the row is very negative, so the
        // ragged tile is masked under both mask settings.
        const bool diag = (CAUSAL && kv0 + C::BN - 1 > q0w) || (kv0 + C::BN > N);
        const int bound = (CAUSAL ? min(myq, N - 1) : N - 1) - kv0 - 4 * h;
        f32x16 sacc[C::NKT], pacc[C::NKT];
        constexpr int NF = 2 * C::NKS, PF = 4;          // f = 2 s + kt
        {
            auto frag = [&](int f) __attribute__((always_inline)) { return tl.row(sK, 32 * (f & 1), f >> 1); };
            bf16x8 ring[PF];
#pragma unroll
            for (int f = 0; f < PF; ++f) ring[f] = frag(f);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const bf16x8 a = ring[f % PF];
                if (f + PF < NF) ring[f % PF] = frag(f + PF);
                sacc[f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[f >> 1], f < 2 ? f32x16{} : sacc[f & 1],
                                                                      0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        {
            auto frag = [&](int f) __attribute__((always_inline)) { return tl.row(sV, 32 * (f & 1), f >> 1); };
            bf16x8 ring[PF];
#pragma unroll
            for (int f = 0; f < PF; ++f) ring[f] = frag(f);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const bf16x8 a = ring[f % PF];
                if (f + PF < NF) ring[f % PF] = frag(f + PF);
                pacc[f & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[f >> 1], f < 2 ? f32x16{} : pacc[f & 1],
                                                                      0, 0, 0);
                // P of score elements [32 f / NF, 32 (f + 1) / NF), element e = 16 kt + r
#pragma unroll
                for (int e = 32 * f / NF; e < 32 * (f + 1) / NF; ++e)
                    sacc[e >> 4][e & 15] = fast_exp2(fmaf(sacc[e >> 4][e & 15], c2, nlse));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // dS^T = P^T o (dP^T - D) in bf16; on masked tiles, 0 where the key follows the query or
        // lies past N (this also replaces whatever a masked key's exponential gave, inf included)
        bf16x8 sb[C::NKT][2];
        auto ds_elem = [&](int kt, int r) __attribute__((always_inline)) {
            sb[kt][r >> 3][r & 7] = to_bf16(sacc[kt][r] * (pacc[kt][r] - dq_d));
        };
        auto ds_mask = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
            for (int w = 0; w < 8; ++w) {               // packed pair: elements r = 2w, 2w + 1
                const int r = 2 * w;
                u32x4 v = __builtin_bit_cast(u32x4, sb[kt][r >> 3]);
                uint32_t x = v[(r & 7) >> 1];
                if (32 * kt + 8 * (r >> 2) + (r & 3) > bound) x &= 0xFFFF0000u;
                if (32 * kt + 8 * (r >> 2) + (r & 3) + 1 > bound) x &= 0x0000FFFFu;
                v[(r & 7) >> 1] = x;
                sb[kt][r >> 3] = __builtin_bit_cast(bf16x8, v);
            }
        };
#pragma unroll
        for (int r = 0; r < 16; ++r) ds_elem(0, r);
        if (diag) ds_mask(0);
        {
            // dQ^T += K^T dS^T, m = (2 kt + s2) NDT + dt; the K^T fragments (transpose reads) go PF2
            // products ahead through a ring; dS^T of keys 32-63 between the products of keys 0-31
            constexpr int NM = 2 * C::NKT * C::NDT, NM0 = 2 * C::NDT, PF2 = 2;
            auto tfrag = [&](int m) __attribute__((always_inline)) {
                return tl.tr(sK, 16 * (m / C::NDT), m % C::NDT);
            };
            bf16x8 ring[PF2];
#pragma unroll
            for (int m = 0; m < PF2; ++m) ring[m] = tfrag(m);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m == NM0 && diag) ds_mask(1);
                const bf16x8 a = ring[m % PF2];
                if (m + PF2 < NM) ring[m % PF2] = tfrag(m + PF2);
                const int ks = m / C::NDT;             // 2 kt + s2
                dqacc[m % C::NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb[ks >> 1][ks & 1], dqacc[m % C::NDT],
                                                                            0, 0, 0);
                if (m < NM0) {
#pragma unroll
                    for (int r = 16 * m / NM0; r < 16 * (m + 1) / NM0; ++r) ds_elem(1, r);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    if constexpr (!SPARSE) {
        auto step = [&](int j, const char* kc, const char* vc, char* kn, char* vn) {
            wait_vmem_all();
            __syncthreads();
            if (j + 1 < ntiles) issue_tile(j + 1, kn, vn);
            if (!(CAUSAL && j * C::BN > q0w + 31))      // else every key of the tile follows this wave's rows
                tile_body(j, kc, vc);
        };
        issue_tile(0, sK0, sV0);
        int j = 0;
        for (; j + 1 < ntiles; j += 2) {
            step(j, sK0, sV0, sK1, sV1);
            step(j + 1, sK1, sV1, sK0, sV0);
        }
        if (j < ntiles) step(j, sK0, sV0, sK1, sV1);
    } else {
        // jn: the next tile to visit (ntiles if none)
        auto step = [&](int j, int jn, const char* kc, const char* vc, char* kn, char* vn) {
            wait_vmem_all();
            __syncthreads();
            if (jn < ntiles) issue_tile(jn, kn, vn);
            if (!(CAUSAL && j * C::BN > q0w + 31)) tile_body(j, kc, vc);
        };
        // only the tiles of kept key blocks (two 64-key tiles per mask block)
        const int nmb = (N + kMaskBlock - 1) / kMaskBlock;
        MaskWalk mw;
        mw.init(bmask + head * mhead + (size_t)qb * nmb, 1, nmb, lane);
        int j = mw.next_unit(0, ntiles, 2, lane);
        if (j < ntiles) issue_tile(j, sK0, sV0);
        while (j < ntiles) {
            int jn = mw.next_unit(j + 1, ntiles, 2, lane);
            step(j, jn, sK0, sV0, sK1, sV1);
            j = jn;
            if (j >= ntiles) break;
            jn = mw.next_unit(j + 1, ntiles, 2, lane);
            step(j, jn, sK1, sV1, sK0, sV0);
            j = jn;
        }
    }

    // dQ = scale * dQ^T acc (lane = query; 4 consecutive head-dim values per store)
    if (myq < N) {
        G* dst = dQ + hoff + (size_t)myq * D;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * dt + 8 * g4 + 4 * h;
                if (d0 < D) {
                    if constexpr (sizeof(G) == 4) {
                        f32x4 a;
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[e] = dqacc[dt][4 * g4 + e] * scale;
                        *reinterpret_cast<f32x4*>(dst + d0) = a;
                    } else {
                        bf16x4 a;
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[e] = to_bf16(dqacc[dt][4 * g4 + e] * scale);
                        *reinterpret_cast<bf16x4*>(dst + d0) = a;
                    }
                }
            }
    }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename T, int D>
static hipError_t pre_t(const void* O, const void* dO, int BH, int N, float* Dd, hipStream_t st)
{
    const long rows = (long)BH * N;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(stride_grid((rows + 31) / 32)), dim3(256), 0, st, (const T*)O,
                       (const T*)dO, Dd, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const void* O, const void* dO, bool bf16_in, int BH, int N, int d, float* Dd,
                          hipStream_t st)
{
    if (bf16_in) {
        switch (d) {
            case 64: return pre_t<bf16, 64>(O, dO, BH, N, Dd, st);
            case 80: return pre_t<bf16, 80>(O, dO, BH, N, Dd, st);
            case 128: return pre_t<bf16, 128>(O, dO, BH, N, Dd, st);
        }
    } else {
        switch (d) {
            case 64: return pre_t<float, 64>(O, dO, BH, N, Dd, st);
            case 80: return pre_t<float, 80>(O, dO, BH, N, Dd, st);
            case 128: return pre_t<float, 128>(O, dO, BH, N, Dd, st);
        }
    }
    return hipErrorInvalidValue;
}

template <int D, bool CAUSAL, typename G>
static hipError_t dkdv_t(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                         const float* Dd, int BH, int N, float scale, void* dK, void* dV, const uint8_t* bmask,
                         long mhead, hipStream_t st)
{
    const int nkblk = (N + BwdKVCfg<D>::BN - 1) / BwdKVCfg<D>::BN;
    const int nitems = nkblk * BH;
    // Dense: a persistent grid.  Block-sparse: one workgroup per item, since a mask makes the
    // items' costs unrelated to the static heavy-first order and the hardware's dynamic dispatch
    // balances them better (with nwg = nitems every workgroup walks exactly its own item).
    int nwg = nitems;
    if (!bmask)
        if (hipError_t e = persistent_grid(nitems, 1, items_split<CAUSAL>(nitems, nkblk), &nwg); e != hipSuccess)
            return e;
    const dim3 grid(nwg), block(64 * BwdKVCfg<D>::WAVES);
    const int slots = tune_lookup(kTuneDkdv, D, CAUSAL, N).slots;
    if (bmask)
        hipLaunchKernelGGL((bwd_dkdv_bf16<D, CAUSAL, G, true>), grid, block, 0, st, (const bf16*)Q, (const bf16*)K,
                           (const bf16*)V, (const bf16*)dO, LSE, Dd, (G*)dK, (G*)dV, N, nkblk, scale, bmask, mhead,
                           slots, nitems);
    else
        hipLaunchKernelGGL((bwd_dkdv_bf16<D, CAUSAL, G, false>), grid, block, 0, st, (const bf16*)Q, (const bf16*)K,
                           (const bf16*)V, (const bf16*)dO, LSE, Dd, (G*)dK, (G*)dV, N, nkblk, scale, nullptr, 0L,
                           slots, nitems);
    return hipGetLastError();
}

template <int D, bool CAUSAL, typename G>
static hipError_t dq_t(const void* Q, const void* K, const void* V, const void* dO, const float* LSE, float* Dd,
                       const void* O, int BH, int N, float scale, void* dQ, const uint8_t* bmask, long mhead,
                       hipStream_t st)
{
    const int nqblk = (N + BwdQCfg<D>::BM - 1) / BwdQCfg<D>::BM;
    const int slots = tune_lookup(kTuneDq, D, CAUSAL, N).slots;
    if (bmask)
        hipLaunchKernelGGL((bwd_dq_bf16<D, CAUSAL, G, true>), dim3(nqblk * BH), dim3(256), 0, st, (const bf16*)Q,
                           (const bf16*)K, (const bf16*)V, (const bf16*)dO, LSE, Dd, (const bf16*)O, (G*)dQ, N,
                           nqblk, scale, bmask, mhead, slots);
    else
        hipLaunchKernelGGL((bwd_dq_bf16<D, CAUSAL, G, false>), dim3(nqblk * BH), dim3(256), 0, st, (const bf16*)Q,
                           (const bf16*)K, (const bf16*)V, (const bf16*)dO, LSE, Dd, (const bf16*)O, (G*)dQ, N,
                           nqblk, scale, nullptr, 0L, slots);
    return hipGetLastError();
}

#define ATTN_DISPATCH_D_CAUSAL_G(FN, ...)                                                        \
    switch (d) {                                                                                 \
        case 64:                                                                                 \
            if (causal) return bf16_grad ? FN<64, true, bf16>(__VA_ARGS__) : FN<64, true, float>(__VA_ARGS__);    \
            return bf16_grad ? FN<64, false, bf16>(__VA_ARGS__) : FN<64, false, float>(__VA_ARGS__);             \
        case 80:                                                                                 \
            if (causal) return bf16_grad ? FN<80, true, bf16>(__VA_ARGS__) : FN<80, true, float>(__VA_ARGS__);    \
            return bf16_grad ? FN<80, false, bf16>(__VA_ARGS__) : FN<80, false, float>(__VA_ARGS__);             \
        case 128:                                                                                \
            if (causal) return bf16_grad ? FN<128, true, bf16>(__VA_ARGS__) : FN<128, true, float>(__VA_ARGS__);  \
            return bf16_grad ? FN<128, false, bf16>(__VA_ARGS__) : FN<128, false, float>(__VA_ARGS__);           \
    }                                                                                            \
    return hipErrorInvalidValue;

hipError_t launch_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                           const float* Dd, int BH, int N, int d, float scale, int causal, void* dK, void* dV,
                           bool bf16_grad, const uint8_t* bmask, long mhead, hipStream_t st)
{
    ATTN_DISPATCH_D_CAUSAL_G(dkdv_t, Q, K, V, dO, LSE, Dd, BH, N, scale, dK, dV, bmask, mhead, st)
}

hipError_t launch_bwd_dq(const void* Q, const void* K, const void* V, const void* dO, const float* LSE, float* Dd,
                         const void* O, int BH, int N, int d, float scale, int causal, void* dQ, bool bf16_grad,
                         const uint8_t* bmask, long mhead, hipStream_t st)
{
    ATTN_DISPATCH_D_CAUSAL_G(dq_t, Q, K, V, dO, LSE, Dd, O, BH, N, scale, dQ, bmask, mhead, st)
}

template <int D, bool CAUSAL>
static hipError_t f32_t(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                        const float* Dd, int BH, int N, float scale, float* dQacc, float* dK, float* dV,
                        const uint8_t* bmask, long mhead, hipStream_t st)
{
    using C = BwdCfg<float, D>;
    const long n4 = (long)BH * N * D / 4;
    hipLaunchKernelGGL(zero_f32_kernel, dim3(stride_grid((n4 + 255) / 256)), dim3(256), 0, st, dQacc, n4);
    const int nkblk = (N + C::BN - 1) / C::BN;
    const int slots = tune_lookup(kTuneBwdF32, D, CAUSAL, N).slots;
    if (bmask)
        hipLaunchKernelGGL((bwd_kernel_f32<D, CAUSAL, true>), dim3(nkblk * BH), dim3(C::THREADS), 0, st,
                           (const float*)Q, (const float*)K, (const float*)V, (const float*)dO, LSE, Dd, dQacc, dK,
                           dV, N, nkblk, scale, bmask, mhead, slots);
    else
        hipLaunchKernelGGL((bwd_kernel_f32<D, CAUSAL, false>), dim3(nkblk * BH), dim3(C::THREADS), 0, st,
                           (const float*)Q, (const float*)K, (const float*)V, (const float*)dO, LSE, Dd, dQacc, dK,
                           dV, N, nkblk, scale, nullptr, 0L, slots);
    return hipGetLastError();
}

hipError_t launch_bwd_f32(const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                          const float* Dd, int BH, int N, int d, float scale, int causal, float* dQacc, float* dK,
                          float* dV, const uint8_t* bmask, long mhead, hipStream_t st)
{
#define ATTN_F32_ARGS Q, K, V, dO, LSE, Dd, BH, N, scale, dQacc, dK, dV, bmask, mhead, st
    switch (d) {
        case 64: return causal ? f32_t<64, true>(ATTN_F32_ARGS) : f32_t<64, false>(ATTN_F32_ARGS);
        case 80: return causal ? f32_t<80, true>(ATTN_F32_ARGS) : f32_t<80, false>(ATTN_F32_ARGS);
        case 128: return causal ? f32_t<128, true>(ATTN_F32_ARGS) : f32_t<128, false>(ATTN_F32_ARGS);
    }
#undef ATTN_F32_ARGS
    return hipErrorInvalidValue;
}

}  // namespace attn
