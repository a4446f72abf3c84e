// Forward kernels: O = softmax(scale Q K^T) V and LSE, one fused pass.
//
// What they follow: FlashAttention-2 review, 'core algorithm' answer, section 2
// (1) tiling into T_r row blocks and T_c column blocks, (2) per-block S, P and
// P V with the running max m and running sum l, (3) one final adjustment;
// "IO-4 FlashAttention", sections 3-4 (block algorithm, online softmax).
// Split-Q work partitioning (each wave owns its own query rows and never
// exchanges partial results with other waves): FlashAttention-2 review, the
// Split-K vs Split-Q answer, section 2.
//
// gfx950 mapping shared by the kernels (each wave owns 32 query rows; a workgroup
// holds 4 waves, or 8 for the dense bf16 walks):
//   * The wave computes S^T = K Q^T with MFMA 32x32 tiles, so every lane of the
//     accumulator holds ONE query and 16 keys.  The running max, running sum and
//     rescale factor are then per-lane scalars; the only cross-lane step per
//     tile is one exchange with lane l^32, which holds the other 16 keys of the
//     same query.
//   * O^T = V^T P^T: the S^T accumulator registers (rounded to the MFMA operand
//     type) ARE the B operand of the next MFMA (the contraction over keys is
//     permuted to the accumulator's row order, and V^T is read with the same
//     permutation).
//   * Causal: column tiles entirely above the block's diagonal are never
//     loaded; tiles entirely above a wave's own rows are skipped by that wave;
//     the element mask runs only on tiles that cross the diagonal or N.
//
// fwd_kernel_f32 (fp32 inputs, MFMA 32x32x2 f32) stages K and V through
// registers into padded LDS (V transposed, key fastest).  bf16 (the hot path):
// fwd_kernel_bf16_pipe for dense walks, fwd_kernel_bf16_sparse for block-sparse
// ones, with the same arithmetic.
#include <float.h>

#include <type_traits>

#include "../../include/attn.h"
#include "attn_common.h"
#include "attn_launch.h"
#include "attn_tuning.h"

static_assert(ATTN_MASK_BLOCK == attn::kMaskBlock, "the ABI's mask block is the kernels'");

namespace attn {

template <typename T, int D>
struct FwdCfg {
    static_assert(sizeof(T) == 4, "the staged kernel serves fp32 inputs");
    static constexpr int QT = 1;
    static constexpr int THREADS = 256;
    static constexpr int BM = 4 * 32 * QT;          // query rows per workgroup
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int NKT = BN / 32;             // 32-key sub-tiles
    static constexpr int DP = (D + 31) / 32 * 32;   // head dim padded to the 32-row O^T tiles
    static constexpr int NDT = DP / 32;
    static constexpr int E = Mma<T>::E, KS = Mma<T>::KS, CH = Mma<T>::CH;
    static constexpr int NKS = D / KS;              // MFMA steps of the Q K^T contraction
    static constexpr int KPITCH = D + 4;                          // elements; conflict-free b128 reads
    static constexpr int VPITCH = BN + 4;                         // elements
    static constexpr int KBUF = BN * KPITCH;
    static constexpr int VBUF = DP * VPITCH;
    static constexpr int CPR = D / CH;              // 16-byte chunks per row
    static constexpr int KCHUNKS = BN * CPR;
    static constexpr int KLD = (KCHUNKS + THREADS - 1) / THREADS;
    static constexpr int VGROUPS = (BN / 4) * CPR;  // 4 keys x 1 chunk each
    static constexpr int VLD = (VGROUPS + THREADS - 1) / THREADS;
    static constexpr int SMEM_ELEMS = 2 * (KBUF + VBUF);
    static_assert(D % KS == 0, "head dim must be a multiple of the MFMA contraction");
    static_assert(D % CH == 0, "head dim must be a multiple of the chunk size");
    static_assert(SMEM_ELEMS * sizeof(T) <= 160 * 1024, "LDS budget");
};

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256) void fwd_kernel_f32(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int N, int nqblk, float c,
                                                      int negate_q, const uint8_t* __restrict__ bmask, long mhead,
                                                      int slots)
{
    typedef float T;
    using C = FwdCfg<T, D>;
    static_assert(kMaskBlock == 2 * C::BN && kMaskBlock == C::BM, "mask block = query block");
    constexpr int QT = C::QT;
    using M = Mma<T>;
    typedef typename M::frag frag;
    constexpr float NEG_INF = -__builtin_inff();

    __shared__ __attribute__((aligned(16))) T smem[C::SMEM_ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;

    int head, qb;
    block_coords<CAUSAL, true>(blockIdx.x, gridDim.x, nqblk, slots, head, qb);
    const int q0 = qb * C::BM;
    const int q0w = q0 + wave * 32 * QT;             // this wave's first query row
    const size_t hoff = (size_t)head * (size_t)N * D;
    const T* __restrict__ Kh = K + hoff;
    const T* __restrict__ Vh = V + hoff;
    constexpr uint32_t ROWB = D * sizeof(T);         // bytes per row

    // ---- Q fragments (B operand of S^T = K Q^T), held for the whole pass ----
    frag qf[QT][C::NKS];
    {
        const auto rq = make_rsrc(Q + hoff, (uint32_t)N * ROWB);
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            const uint32_t rowoff = (uint32_t)(q0w + 32 * t + l32) * ROWB;
#pragma unroll
            for (int s = 0; s < C::NKS; ++s) {
                const uint32_t off = rowoff + (s * C::KS + C::E * h) * sizeof(T);
                const float x = buf_ld4f(rq, off);
                qf[t][s] = negate_q ? -x : x;
            }
        }
    }

    // Rows D..DP-1 of the V^T buffers feed only discarded output rows; zero them once.
    if constexpr (C::DP > D) {
        for (int b = 0; b < 2; ++b) {
            T* Vl = smem + b * (C::KBUF + C::VBUF) + C::KBUF;
            for (int x = tid; x < (C::DP - D) * C::VPITCH; x += C::THREADS)
                Vl[D * C::VPITCH + x] = from_f32<T>(0.f);
        }
    }

    f32x16 oacc[C::NDT][QT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int t = 0; t < QT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][t][r] = 0.f;
    float mc[QT], l[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) { mc[t] = NEG_INF; l[t] = 0.f; }

    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + C::BN - 1) / C::BN;

    // ---- staging: global -> registers -> LDS (per-thread offsets are loop invariant) ----
    uint32_t koff[C::KLD], voff[C::VLD];
    int kst_row[C::KLD], kst_col[C::KLD], vst_g[C::VLD], vst_col[C::VLD];
#pragma unroll
    for (int i = 0; i < C::KLD; ++i) {
        const int f = tid + C::THREADS * i;
        kst_row[i] = f / C::CPR;
        kst_col[i] = f - kst_row[i] * C::CPR;
        koff[i] = kst_row[i] * ROWB + kst_col[i] * 16;
    }
#pragma unroll
    for (int i = 0; i < C::VLD; ++i) {
        const int f = tid + C::THREADS * i;
        vst_g[i] = f / C::CPR;
        vst_col[i] = f - vst_g[i] * C::CPR;
        voff[i] = 4 * vst_g[i] * ROWB + vst_col[i] * 16;
    }
    u32x4 kst[C::KLD];
    u32x4 vst[C::VLD][4];
    auto load_tile = [&](int j) {
        const int kv0 = j * C::BN;
        const uint32_t bytes = (uint32_t)(N - kv0) * ROWB;        // rows past N read as zeros
        const auto rk = make_rsrc(Kh + (size_t)kv0 * D, bytes);
        const auto rv = make_rsrc(Vh + (size_t)kv0 * D, bytes);
#pragma unroll
        for (int i = 0; i < C::KLD; ++i)
            if (C::KCHUNKS % C::THREADS == 0 || tid + C::THREADS * i < C::KCHUNKS) kst[i] = buf_ld16(rk, koff[i]);
#pragma unroll
        for (int i = 0; i < C::VLD; ++i)
            if (C::VGROUPS % C::THREADS == 0 || tid + C::THREADS * i < C::VGROUPS) {
#pragma unroll
                for (int e = 0; e < 4; ++e) vst[i][e] = buf_ld16(rv, voff[i] + e * ROWB);
            }
    };
    auto store_tile = [&](T* Kl) {
        T* Vl = Kl + C::KBUF;
#pragma unroll
        for (int i = 0; i < C::KLD; ++i)
            if (C::KCHUNKS % C::THREADS == 0 || tid + C::THREADS * i < C::KCHUNKS)
                st16(Kl + kst_row[i] * C::KPITCH + kst_col[i] * C::CH, kst[i]);
#pragma unroll
        for (int i = 0; i < C::VLD; ++i)
            if (C::VGROUPS % C::THREADS == 0 || tid + C::THREADS * i < C::VGROUPS) {
                const int g = vst_g[i], col = vst_col[i];
                // 4 keys x 4 head-dim values -> for each of the 4 dims, the 4 keys (16 bytes)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const int dd = col * C::CH + x;
                    st16(Vl + dd * C::VPITCH + 4 * g, u32x4{vst[i][0][x], vst[i][1][x], vst[i][2][x], vst[i][3][x]});
                }
            }
    };

    // ---- one key tile: S^T, online softmax, O^T += V^T P^T ----
    auto compute_tile = [&](const T* Kl, int kv0) {
        const T* Vl = Kl + C::KBUF;
        f32x16 sacc[C::NKT][QT];
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
            for (int t = 0; t < QT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kt][t][r] = 0.f;
#pragma unroll
        for (int s = 0; s < C::NKS; ++s) {
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt) {
                const T* src = Kl + (32 * kt + l32) * C::KPITCH + s * C::KS + C::E * h;
                const frag a = *src;
#pragma unroll
                for (int t = 0; t < QT; ++t) sacc[kt][t] = M::mma(a, qf[t][s], sacc[kt][t]);
            }
        }

        // mc[t] is the reference max in log2 units (max * scale * log2 e).  It only
        // moves when the tile's max exceeds it by more than kLazyLog2 (so every p
        // stays <= 2^kLazyLog2): most tiles then need no rescale of O and l at all.
        const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > q0w) || (kv0 + C::BN > N);
        frag pf[C::NKT][32 / C::KS][QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            if (need_mask) {
                const int q = q0w + 32 * t + l32;
#pragma unroll
                for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
                        if ((CAUSAL && key > q) || key >= N) sacc[kt][t][r] = NEG_INF;
                    }
            }
            float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; r += 2)
                    mx4[r >> 2] = max3f(mx4[r >> 2], sacc[kt][t][r], sacc[kt][t][r + 1]);
            float mx = max3f(mx4[0], mx4[1], fmaxf(mx4[2], mx4[3]));
            mx = fmaxf(mx, xor32(mx));
            const float mxc = (mx == NEG_INF) ? NEG_INF : mx * c;
            if (__builtin_amdgcn_ballot_w64(mxc > mc[t] + kLazyLog2) != 0) {
                const float mnew = fmaxf(mc[t], mxc);
                const float alpha = fast_exp2(mc[t] - mnew);       // 0 on the first tile
                l[t] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][t][r] *= alpha;
                mc[t] = mnew;
            }
            const float ms = mc[t];
            if (need_mask) {
#pragma unroll
                for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float sv = sacc[kt][t][r];
                        sacc[kt][t][r] = (sv == NEG_INF) ? 0.f : fast_exp2(fmaf(sv, c, -ms));
                    }
            } else {
#pragma unroll
                for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[kt][t][r] = fast_exp2(fmaf(sacc[kt][t][r], c, -ms));
            }
            // P in the MFMA operand type; the row sum is taken over exactly these values.
            {
                float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pf[kt][r][t] = sacc[kt][t][r];
                        ls[r & 3] += sacc[kt][t][r];
                    }
                l[t] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
            }
        }

        // O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt) {
#pragma unroll
            for (int s2 = 0; s2 < 32 / C::KS; ++s2) {
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) {
                    const T* vrow = Vl + (32 * dt + l32) * C::VPITCH + 32 * kt;
                    const frag a = vrow[8 * (s2 >> 2) + 4 * h + (s2 & 3)];
#pragma unroll
                    for (int t = 0; t < QT; ++t) oacc[dt][t] = M::mma(a, pf[kt][s2][t], oacc[dt][t]);
                }
            }
        }
    };

    // ---- main loop, unrolled by two so the LDS buffer offsets are constants ----
    if constexpr (!SPARSE) {
        auto step = [&](int j, T* Kl) {
            store_tile(Kl);
            __syncthreads();
            if (j + 1 < ntiles) load_tile(j + 1);
            const int kv0 = j * C::BN;
            if (!(CAUSAL && kv0 > q0w + 32 * QT - 1))    // else: every key is above this wave's rows
                compute_tile(Kl, kv0);
        };
        load_tile(0);
        for (int j = 0; j < ntiles; j += 2) {
            step(j, smem);
            if (j + 1 < ntiles) step(j + 1, smem + C::KBUF + C::VBUF);
        }
    } else {
        // jn: the next tile to visit (ntiles if none)
        auto step = [&](int j, int jn, T* Kl) {
            store_tile(Kl);
            __syncthreads();
            if (jn < ntiles) load_tile(jn);
            const int kv0 = j * C::BN;
            if (!(CAUSAL && kv0 > q0w + 32 * QT - 1)) compute_tile(Kl, kv0);
        };
        // only the tiles of kept key blocks (two 64-key tiles per mask block)
        const int nmb = (N + kMaskBlock - 1) / kMaskBlock;
        MaskWalk mw;
        mw.init(bmask + head * mhead + (size_t)qb * nmb, 1, nmb, lane);
        int j = mw.next_unit(0, ntiles, 2, lane);
        if (j < ntiles) load_tile(j);
        while (j < ntiles) {
            int jn = mw.next_unit(j + 1, ntiles, 2, lane);
            step(j, jn, smem);
            j = jn;
            if (j >= ntiles) break;
            jn = mw.next_unit(j + 1, ntiles, 2, lane);
            step(j, jn, smem + C::KBUF + C::VBUF);
            j = jn;
        }
    }

    // ---- epilogue: one division by l, O and LSE written once ----
    T* Oh = O + hoff;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const float lt = l[t] + xor32(l[t]);
        const float inv = (SPARSE && !(lt > 0.f)) ? 0.f : 1.0f / lt;     // no kept key: O = 0, LSE = -inf
        const int q = q0w + 32 * t + l32;
        if (q < N) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = 32 * dt + 8 * g + 4 * h;
                    if (d0 < D) {
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = oacc[dt][t][4 * g + e] * inv;
                        *reinterpret_cast<f32x4*>(Oh + (size_t)q * D + d0) = v;
                    }
                }
            if (h == 0) LSE[(size_t)head * N + q] = (mc[t] + __log2f(lt)) * kLn2;
        }
    }
}

// ----------------------------------------------------------------------------
// bf16 forward, block-sparse walks.  Same per-lane softmax as above; K and V tiles go
// straight from HBM/L2 into swizzled LDS rows (direct-to-LDS loads, no staging
// registers, no transposing stores) and V^T reaches the MFMA through transpose
// reads.  sK0/sK1/sV0/sV1 are separate __shared__ objects and the loop is unrolled by
// two, so the compiler can tell the next tile's in-flight loads from the current
// tile's reads.  4 waves (128 rows, one mask block) per workgroup, two workgroups per
// CU, <= 256 registers per wave.  Dense walks take fwd_kernel_bf16_pipe below, which
// does the same arithmetic in the same order (an all-kept mask gives identical bits).
// ----------------------------------------------------------------------------
template <int D, int WAVES>
struct FwdBf16Cfg {
    static constexpr int BM = 32 * WAVES, BN = 64, NKT = BN / 32;
    static constexpr int RB = D == 64 ? 128 : 256;
    static constexpr int DP = (D + 31) / 32 * 32, NDT = DP / 32;
    static constexpr int NKS = D / 16;
    static constexpr int T_BYTES = BN * RB;
    static_assert(4 * T_BYTES <= 80 * 1024, "two workgroups per CU");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2)
void fwd_kernel_bf16_sparse(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                          const bf16* __restrict__ V, bf16* __restrict__ O,
                                                          float* __restrict__ LSE, int N, int nqblk, float c,
                                                          int negate_q, const uint8_t* __restrict__ bmask,
                                                          long mhead, int slots)
{
    constexpr bool SPARSE = true;
    constexpr int WAVES = 4;
    using C = FwdBf16Cfg<D, WAVES>;
    static_assert(kMaskBlock == 2 * C::BN && kMaskBlock == C::BM, "mask block = query block");
    constexpr int RB = C::RB;
    constexpr uint32_t ROWB = D * 2;
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
    const bf16* __restrict__ Kh = K + hoff;
    const bf16* __restrict__ Vh = V + hoff;
    TileLane<RB, C::NKS, C::NDT, true> tl;
    tl.init(lane);

    // Q fragments (B operand of S^T = K Q^T), sign-flipped for a negative scale
    bf16x8 qf[C::NKS];
    {
        const auto rq = make_rsrc(Q + hoff, (uint32_t)N * ROWB);
        const uint32_t ro = (uint32_t)myq * ROWB + 16 * h;
#pragma unroll
        for (int s = 0; s < C::NKS; ++s) {
            u32x4 raw = buf_ld16(rq, ro + 32 * s);
            if (negate_q) raw ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }

    f32x16 oacc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float mc = NEG_INF, l = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + C::BN - 1) / C::BN;

    auto issue_tile = [&](int j, char* sK, char* sV) {
        const int kv0 = j * C::BN;
        const uint32_t bytes = (uint32_t)(N - kv0) * ROWB;        // rows past N read as zeros
        dma_rows<D, RB, true>(make_rsrc(Kh + (size_t)kv0 * D, bytes), sK, wave * (C::BN / WAVES), C::BN / WAVES, lane);
        dma_rows<D, RB, true>(make_rsrc(Vh + (size_t)kv0 * D, bytes), sV, wave * (C::BN / WAVES), C::BN / WAVES, lane);
    };

    auto tile_body = [&](int j, const char* sK, const char* sV) {
        const int kv0 = j * C::BN;
        f32x16 sacc[C::NKT];
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
        // K fragments are read PF products ahead through a small ring (sched_barrier keeps the order)
        {
            constexpr int NM = C::NKS * C::NKT, PF = 4;
            bf16x8 ring[PF];
#pragma unroll
            for (int i = 0; i < PF; ++i) ring[i] = tl.row(sK, 32 * (i % C::NKT), i / C::NKT);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                const int s = i / C::NKT, kt = i % C::NKT;
                const bf16x8 a = ring[i % PF];
                if (i + PF < NM) ring[i % PF] = tl.row(sK, 32 * ((i + PF) % C::NKT), (i + PF) / C::NKT);
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // lane: query myq, keys kv0 + 4 h + cr with cr = 32 kt + 8 (r/4) + r%4; a key is masked
        // when it follows the query or lies past N, i.e. when cr exceeds one per-lane bound
        const bool need_mask = (CAUSAL && kv0 + C::BN - 1 > q0w) || (kv0 + C::BN > N);
        if (need_mask) {
            const int bound = CAUSAL ? min(myq, N - 1) - kv0 - 4 * h : N - 1 - kv0 - 4 * h;
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kt + 8 * (r >> 2) + (r & 3) > bound) sacc[kt][r] = NEG_INF;
        }
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx4[r >> 2] = max3f(mx4[r >> 2], sacc[kt][r], sacc[kt][r + 1]);
        float mx = max3f(mx4[0], mx4[1], fmaxf(mx4[2], mx4[3]));
        mx = fmaxf(mx, xor32(mx));
        const float mxc = (mx == NEG_INF) ? NEG_INF : mx * c;
        // the reference max moves only when the tile's max exceeds it by 2^kLazyLog2
        if (__builtin_amdgcn_ballot_w64(mxc > mc + kLazyLog2) != 0) {
            const float mnew = fmaxf(mc, mxc);
            const float alpha = fast_exp2(mc - mnew);           // 0 on the first tile
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            mc = mnew;
        }
        // a masked score is -inf and c >= FLT_MIN, so exp2 gives 0 once mc is finite: a dense
        // walk's first tile gives every row a key (key 0, or keys below N), so only
        // block-sparse walks, whose rows may have seen no key yet, need the select
        if (SPARSE && need_mask) {
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float sv = sacc[kt][r];
                    sacc[kt][r] = (sv == NEG_INF) ? 0.f : fast_exp2(fmaf(sv, c, -mc));
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kt][r] = fast_exp2(fmaf(sacc[kt][r], c, -mc));
        }
        // P in bf16; the row sum is taken over exactly these values
        bf16x8 pf[C::NKT][2];
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[kt][s2][e] = to_bf16(sacc[kt][8 * s2 + e]);
                const u32x4 w = __builtin_bit_cast(u32x4, pf[kt][s2]);
#pragma unroll
                for (int x = 0; x < 4; ++x) ls[s2] = sum2_bf16(w[x], ls[s2]);
            }
        l += ls[0] + ls[1];
        // O^T += V^T P^T; the V^T fragments (transpose reads) go PF products ahead through a ring
        {
            constexpr int NT = 2 * C::NKT * C::NDT, PF = 4;
            auto tfrag = [&](int t) __attribute__((always_inline)) {
                return tl.tr(sV, 32 * (t / (2 * C::NDT)) + 16 * ((t / C::NDT) & 1), t % C::NDT);
            };
            bf16x8 ring[PF];
#pragma unroll
            for (int t = 0; t < PF; ++t) ring[t] = tfrag(t);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bf16x8 a = ring[t % PF];
                if (t + PF < NT) ring[t % PF] = tfrag(t + PF);
                const int kt = t / (2 * C::NDT), s2 = (t / C::NDT) & 1, dt = t % C::NDT;
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kt][s2], oacc[dt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    {
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

    // epilogue: one division by l, O and LSE written once (a row with no kept key:
    // O = 0 and LSE = -inf)
    const float lt = l + xor32(l);
    const float inv = (SPARSE && !(lt > 0.f)) ? 0.f : 1.0f / lt;
    if (myq < N) {
        bf16* dst = O + hoff + (size_t)myq * D;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * dt + 8 * g + 4 * h;
                if (d0 < D) {
                    bf16x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = to_bf16(oacc[dt][4 * g + e] * inv);
                    *reinterpret_cast<bf16x4*>(dst + d0) = v;
                }
            }
        if (h == 0) LSE[(size_t)head * N + myq] = (mc + __log2f(lt)) * kLn2;
    }
}

// ----------------------------------------------------------------------------
// bf16 forward, dense walks: the same arithmetic as fwd_kernel_bf16_sparse (same products
// in the same order, same roundings, same rescale decisions: bit-identical results),
// software-pipelined across key tiles so that each wave's softmax runs under its own
// MFMAs instead of between them.  Iteration j of a wave:
//   [A]  S_{j+1} = K_{j+1} Q^T   (16 MFMAs at d = 128)  with  exp2 of S_j, keys 0-31
//   [B1] O^T += V_j^T P_j^T, keys 0-31                   with  exp2 of S_j, keys 32-63
//   [B2] O^T += V_j^T P_j^T, keys 32-63                  with  the row max of S_{j+1}
// and the rare rescale of O and l (lazy, threshold 2^8) at the top, before the
// exponentials of S_j need the reference max.  K runs one tile ahead of V: at the top
// of iteration j (one barrier) K_{j+2} is issued, and V_{j+1} after the second score
// product (so that the step's direct-to-LDS loads do not all queue at the address unit
// at once), into the buffers that iteration j-1 finished reading; iteration j reads
// K_{j+1} and V_j.  A causal block's last three iterations, where some waves have no
// tile, run in a loop of their own with both loads at the top.  Wave priority steps
// 3, 2, 1, 0 through each iteration so that the two waves of a SIMD finish together.
// Q comes in and O goes out through each wave's own rows of an LDS stage, so that every
// global load and store instruction moves whole rows.
// 8 waves (256 query rows) per workgroup, 32 rows per wave, two waves per SIMD.
// ----------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1)
void fwd_kernel_bf16_pipe(const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
                          bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqblk, float c, int negate_q,
                          int slots)
{
    constexpr int WAVES = 8;
    using C = FwdBf16Cfg<D, WAVES>;
    static_assert(C::NKT == 2, "two 32-key halves per tile");
    constexpr int RB = C::RB, NKS = C::NKS, NDT = C::NDT;
    constexpr uint32_t ROWB = D * 2;
    constexpr float NEG_INF = -__builtin_inff();
    __shared__ __attribute__((aligned(1024))) char sK0[C::T_BYTES], sK1[C::T_BYTES];
    __shared__ __attribute__((aligned(1024))) char sV0[C::T_BYTES], sV1[C::T_BYTES];
    __shared__ __attribute__((aligned(256))) char sO[WAVES * 32 * RB];

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
    TileLane<RB, NKS, NDT, true> tl;
    tl.init(lane);

    // this wave's 32 query rows go to its own rows of sO (direct-to-LDS, whole rows per
    // instruction); sO holds nothing else until the epilogue stages O there
    dma_rows<D, RB, true>(make_rsrc(Q + hoff + (size_t)q0 * D, (uint32_t)(N - q0) * ROWB), sO, 32 * wave, 32, lane);
    bf16x8 qf[NKS];                             // read from sO once the prologue's loads landed

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float mc = NEG_INF, l = 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + C::BM) : N;
    const int ntiles = (kv_end + C::BN - 1) / C::BN;
    // this wave's last tile (causal: the last one holding a key at or before its last row)
    const int jlast = CAUSAL ? min(ntiles - 1, (q0w + 31) / C::BN) : ntiles - 1;

    auto issue = [&](const bf16* __restrict__ base, int j, char* tile) {
        const int kv0 = j * C::BN;
        const uint32_t bytes = (uint32_t)(N - kv0) * ROWB;        // rows past N read as zeros
        dma_rows<D, RB, true>(make_rsrc(base + (size_t)kv0 * D, bytes), tile, wave * (C::BN / WAVES),
                              C::BN / WAVES, lane);
    };
    auto need_mask = [&](int j) { return (CAUSAL && j * C::BN + C::BN - 1 > q0w) || (j * C::BN + C::BN > N); };
    // lane: query myq, keys kv0 + 4 h + cr with cr = 32 kt + 8 (r/4) + r%4; masked when cr > bound
    auto apply_mask = [&](f32x16 (&sacc)[2], int j) {
        const int kv0 = j * C::BN;
        const int bound = CAUSAL ? min(myq, N - 1) - kv0 - 4 * h : N - 1 - kv0 - 4 * h;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * kt + 8 * (r >> 2) + (r & 3) > bound) sacc[kt][r] = NEG_INF;
    };
    // the row max of a score tile, scaled to log2 units (both lanes of a query agree)
    auto row_max = [&](const float (&mx4)[4]) {
        float mx = max3f(mx4[0], mx4[1], fmaxf(mx4[2], mx4[3]));
        mx = fmaxf(mx, xor32(mx));
        return (mx == NEG_INF) ? NEG_INF : mx * c;
    };
    // the score product of tile j+1 as NKS * 2 MFMAs, with `work(i)` issued after MFMA i;
    // K fragments are read PF MFMAs ahead through a ring
    auto scores = [&](f32x16 (&sacc)[2], const char* sK, auto&& work) __attribute__((always_inline)) {
        constexpr int NM = NKS * 2, PF = 4;
        bf16x8 ring[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) ring[i] = tl.row(sK, 32 * (i % 2), i / 2);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            const int s = i / 2, kt = i % 2;
            const bf16x8 a = ring[i % PF];
            if (i + PF < NM) ring[i % PF] = tl.row(sK, 32 * ((i + PF) % 2), (i + PF) / 2);
            sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? f32x16{} : sacc[kt], 0, 0, 0);
            work(i);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // 16 max3 of a score tile into four partial maxima, `x` = slices of eight
    auto max_slice = [&](float (&mx4)[4], const f32x16 (&sacc)[2], int x) __attribute__((always_inline)) {
        const int kt = x >> 3, r = 2 * (x & 7);
        mx4[r >> 2] = max3f(mx4[r >> 2], sacc[kt][r], sacc[kt][r + 1]);
    };

    // prologue: K_0, V_0, K_1 in flight; S_0 and its (unmasked) row max
    f32x16 sA[2], sB[2];
    float mxc_next;
    issue(Kh, 0, sK0);
    issue(Vh, 0, sV0);
    if (ntiles > 1) issue(Kh, 1, sK1);
    wait_vmem_all();
    __syncthreads();
    // Q fragments (B operand of S^T = K Q^T), sign-flipped for a negative scale
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        u32x4 raw = __builtin_bit_cast(u32x4, tl.row(sO, 32 * wave, s));
        if (negate_q) raw ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qf[s] = __builtin_bit_cast(bf16x8, raw);
    }
    scores(sA, sK0, [&](int) {});
    {
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int x = 0; x < 16; ++x) max_slice(mx4, sA, x);
        mxc_next = row_max(mx4);
    }

    // One iteration: scur = S_j, snext <- S_{j+1}; sKn holds K_{j+1}, sVc V_j.  On a wave's last
    // tile, [A] still runs on whatever the K buffer holds (in bounds) and its result is never
    // used: a branch around it would make the compiler copy the live score tile at the join.
    // `sVl`: where V_{j+1} goes when this body issues it (after the second score product, so
    // that the step's loads do not all queue at the address unit at once), else null
    auto body = [&](int j, f32x16 (&scur)[2], f32x16 (&snext)[2], const char* sKn, const char* sVc, char* sVl)
        __attribute__((always_inline)) {
        // tiles crossing the diagonal or N (rare): mask S_j in place and take its max again
        float mxc = mxc_next;
        if (need_mask(j)) {
            apply_mask(scur, j);
            float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
            for (int x = 0; x < 16; ++x) max_slice(mx4, scur, x);
            mxc = row_max(mx4);
        }
        // the reference max moves only when the tile's max exceeds it by 2^kLazyLog2
        if (__builtin_amdgcn_ballot_w64(mxc > mc + kLazyLog2) != 0) {
            const float mnew = fmaxf(mc, mxc);
            const float alpha = fast_exp2(mc - mnew);               // 0 on the first tile
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            mc = mnew;
        }
        const float ms = mc;
        bf16x8 pf[2][2];
        float ls[2] = {0.f, 0.f};
        // exp2 of element r of key half kt (a masked -inf gives 0: mc is finite, c >= FLT_MIN);
        // P in bf16 and the row sum over exactly those values, eight elements at a time
        auto expo = [&](int kt, int r) __attribute__((always_inline)) {
            scur[kt][r] = fast_exp2(fmaf(scur[kt][r], c, -ms));
        };
        auto pack = [&](int kt, int s2) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[kt][s2][e] = to_bf16(scur[kt][8 * s2 + e]);
            const u32x4 w = __builtin_bit_cast(u32x4, pf[kt][s2]);
#pragma unroll
            for (int x = 0; x < 4; ++x) ls[s2] = sum2_bf16(w[x], ls[s2]);
        };
        // [A] the next tile's score MFMAs with the exponentials of keys 0-31
        scores(snext, sKn, [&](int i) __attribute__((always_inline)) {
            constexpr int NM = NKS * 2;
            if (i == 2 && sVl != nullptr && j + 1 < ntiles) issue(Vh, j + 1, sVl);
            if (i == NM / 2) __builtin_amdgcn_s_setprio(2);
#pragma unroll
            for (int r = 16 * i / NM; r < 16 * (i + 1) / NM; ++r) {
                expo(0, r);
                if (r == 7) pack(0, 0);
                if (r == 15) pack(0, 1);
            }
        });
        // O^T += V^T P^T: product t = (2 kt + s2) NDT + dt; V^T fragments PF products ahead
        constexpr int NT = 4 * NDT, PF = 4;
        auto tfrag = [&](int t) __attribute__((always_inline)) {
            return tl.tr(sVc, 32 * (t / (2 * NDT)) + 16 * ((t / NDT) & 1), t % NDT);
        };
        bf16x8 ring[PF];
#pragma unroll
        for (int t = 0; t < PF; ++t) ring[t] = tfrag(t);
        float mx4[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16x8 a = ring[t % PF];
            if (t + PF < NT) ring[t % PF] = tfrag(t + PF);
            const int kt = t / (2 * NDT), s2 = (t / NDT) & 1, dt = t % NDT;
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kt][s2], oacc[dt], 0, 0, 0);
            if (t == 0) __builtin_amdgcn_s_setprio(1);
            if (t == 2 * NDT) __builtin_amdgcn_s_setprio(0);
            if (t < 2 * NDT) {
                // [B1] keys 0-31 of P V, with the exponentials of keys 32-63
#pragma unroll
                for (int r = 16 * t / (2 * NDT); r < 16 * (t + 1) / (2 * NDT); ++r) {
                    expo(1, r);
                    if (r == 7) pack(1, 0);
                    if (r == 15) pack(1, 1);
                }
            } else {
                // [B2] keys 32-63 of P V, with the next tile's (unmasked) row max
                const int u = t - 2 * NDT;
#pragma unroll
                for (int x = 16 * u / (2 * NDT); x < 16 * (u + 1) / (2 * NDT); ++x) max_slice(mx4, snext, x);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mxc_next = row_max(mx4);
        l += ls[0] + ls[1];
    };

    // ALL: a step in which every wave of the workgroup has a tile (all but a causal block's last
    // three), so no wave skips the body and the body issues V; else V is issued here
    auto step = [&](auto all, int j, f32x16 (&scur)[2], f32x16 (&snext)[2], const char* sKn, const char* sVc,
                    char* sKl, char* sVl) __attribute__((always_inline)) {
        wait_vmem_all();                            // this wave's loads of K_{j+1} and V_j landed
        __syncthreads();                            // everyone's; iteration j-1 fully read
        // the two waves of a SIMD (w and w + 4) run the same step; by default the older one wins
        // every issue contest, finishes first and idles at the next barrier while the other runs
        // alone.  Priority 3, 2, 1, 0 at the quarters of the step gives the wave that is behind
        // the issue slots instead.
        __builtin_amdgcn_s_setprio(3);
        if (j + 2 < ntiles) issue(Kh, j + 2, sKl);
        if constexpr (decltype(all)::value) {
            body(j, scur, snext, sKn, sVc, sVl);
        } else {
            if (j + 1 < ntiles) issue(Vh, j + 1, sVl);
            if (j <= jlast) body(j, scur, snext, sKn, sVc, nullptr);
        }
    };
    // even j: K_{j+1} in sK1, V_j in sV0; loads K_{j+2} -> sK0, V_{j+1} -> sV1 (odd j mirrored)
    const int jbusy = CAUSAL ? min(ntiles, (q0 + 31) / C::BN + 1) : ntiles;    // wave 0's last tile + 1
    const std::integral_constant<bool, true> all_busy;
    const std::integral_constant<bool, false> some_idle;
    int j = 0;
    for (; j + 1 < jbusy; j += 2) {
        step(all_busy, j, sA, sB, sK1, sV0, sK0, sV1);
        step(all_busy, j + 1, sB, sA, sK0, sV1, sK1, sV0);
    }
    for (; j + 1 < ntiles; j += 2) {
        step(some_idle, j, sA, sB, sK1, sV0, sK0, sV1);
        step(some_idle, j + 1, sB, sA, sK0, sV1, sK1, sV0);
    }
    if (j < ntiles) step(some_idle, j, sA, sB, sK1, sV0, sK0, sV1);

    // epilogue: one division by l; O goes through this wave's own LDS rows (swizzled like a
    // K/V tile) so that every store instruction writes whole rows; LSE written once
    const float lt = l + xor32(l);
    const float inv = 1.0f / lt;
    {
        char* st = sO + wave * 32 * RB;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (32 * dt + 8 * g < D) {
                    bf16x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = to_bf16(oacc[dt][4 * g + e] * inv);
                    *reinterpret_cast<bf16x4*>(st + l32 * RB + swz<RB, true>(l32, 4 * dt + g) * 16 + 8 * h) = v;
                }
            }
        constexpr int CPR = D / 8, NCH = 32 * CPR;
        static_assert(NCH % 64 == 0, "whole store instructions");
        const auto ro = make_rsrc(O + hoff + (size_t)q0w * D, (uint32_t)(N > q0w ? N - q0w : 0) * ROWB);
#pragma unroll
        for (int i = 0; i < NCH / 64; ++i) {
            const int idx = 64 * i + lane, row = idx / CPR, ch = idx - row * CPR;
            const u32x4 v = ld16(st + row * RB + swz<RB, true>(row, ch) * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, row * (int)ROWB + ch * 16, 0, 0);
        }
    }
    if (myq < N && h == 0) LSE[(size_t)head * N + myq] = (mc + __log2f(lt)) * kLn2;
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_f32(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH, int N,
                                 float scale, const uint8_t* bmask, long mhead, hipStream_t st)
{
    using C = FwdCfg<float, D>;
    const int nqblk = (N + C::BM - 1) / C::BM;
    const float c = fabsf(scale) * kLog2e;
    const int negq = scale < 0.f;
    const int slots = tune_lookup(kTuneFwdF32, D, CAUSAL, N).slots;
    hipLaunchKernelGGL((fwd_kernel_f32<D, CAUSAL, SPARSE>), dim3(nqblk * BH), dim3(C::THREADS), 0, st,
                       (const float*)Q, (const float*)K, (const float*)V, (float*)O, LSE, N, nqblk, c, negq, bmask,
                       mhead, slots);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_fwd_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH, int N,
                                  float scale, const uint8_t* bmask, long mhead, hipStream_t st)
{
    const float c = fmaxf(fabsf(scale) * kLog2e, FLT_MIN);        // scale 0: -inf * c stays -inf
    const int negq = scale < 0.f;
    const int slots = tune_lookup(kTuneFwdBf16, D, CAUSAL, N).slots;
    if constexpr (SPARSE) {
        const int nqblk = (N + FwdBf16Cfg<D, 4>::BM - 1) / FwdBf16Cfg<D, 4>::BM;
        hipLaunchKernelGGL((fwd_kernel_bf16_sparse<D, CAUSAL>), dim3(nqblk * BH), dim3(256), 0, st, (const bf16*)Q,
                           (const bf16*)K, (const bf16*)V, (bf16*)O, LSE, N, nqblk, c, negq, bmask, mhead, slots);
    } else {
        const int nqblk = (N + FwdBf16Cfg<D, 8>::BM - 1) / FwdBf16Cfg<D, 8>::BM;
        hipLaunchKernelGGL((fwd_kernel_bf16_pipe<D, CAUSAL>), dim3(nqblk * BH), dim3(512), 0, st, (const bf16*)Q,
                           (const bf16*)K, (const bf16*)V, (bf16*)O, LSE, N, nqblk, c, negq, slots);
    }
    return hipGetLastError();
}

template <bool BF, int D, bool CAUSAL>
static hipError_t launch_fwd_dc(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH, int N,
                                float scale, const uint8_t* bmask, long mhead, hipStream_t st)
{
    if constexpr (BF) {
        if (bmask) return launch_fwd_bf16<D, CAUSAL, true>(Q, K, V, O, LSE, BH, N, scale, bmask, mhead, st);
        return launch_fwd_bf16<D, CAUSAL, false>(Q, K, V, O, LSE, BH, N, scale, nullptr, 0, st);
    } else {
        if (bmask) return launch_fwd_f32<D, CAUSAL, true>(Q, K, V, O, LSE, BH, N, scale, bmask, mhead, st);
        return launch_fwd_f32<D, CAUSAL, false>(Q, K, V, O, LSE, BH, N, scale, nullptr, 0, st);
    }
}

template <bool BF, int D>
static hipError_t launch_fwd_d(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH, int N,
                               float scale, int causal, const uint8_t* bmask, long mhead, hipStream_t st)
{
    if (causal) return launch_fwd_dc<BF, D, true>(Q, K, V, O, LSE, BH, N, scale, bmask, mhead, st);
    return launch_fwd_dc<BF, D, false>(Q, K, V, O, LSE, BH, N, scale, bmask, mhead, st);
}

hipError_t launch_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, bool bf16_in,
                      int BH, int N, int d, float scale, int causal, const uint8_t* bmask, long mhead,
                      hipStream_t st)
{
    if (bf16_in) {
        switch (d) {
            case 64: return launch_fwd_d<true, 64>(Q, K, V, O, LSE, BH, N, scale, causal, bmask, mhead, st);
            case 80: return launch_fwd_d<true, 80>(Q, K, V, O, LSE, BH, N, scale, causal, bmask, mhead, st);
            case 128: return launch_fwd_d<true, 128>(Q, K, V, O, LSE, BH, N, scale, causal, bmask, mhead, st);
        }
    } else {
        switch (d) {
            case 64: return launch_fwd_d<false, 64>(Q, K, V, O, LSE, BH, N, scale, causal, bmask, mhead, st);
            case 80: return launch_fwd_d<false, 80>(Q, K, V, O, LSE, BH, N, scale, causal, bmask, mhead, st);
            case 128: return launch_fwd_d<false, 128>(Q, K, V, O, LSE, BH, N, scale, causal, bmask, mhead, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
