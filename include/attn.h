/*
 * attn.h -- C ABI of the exact tiled attention library (libattn.so, gfx950).
 *
 * The operation (per head, Q, K, V in R^{N x d}):
 *     S = scale * Q K^T,  P = softmax(S) row-wise,  O = P V,
 *     LSE_i = log(sum_j exp(S_ij))             (natural log of the scaled scores)
 * "IO-4 FlashAttention", problem setup (softmax(QK^T/sqrt(d_k))V) and section 1;
 * FlashAttention-2 review, 'core algorithm' answer, section 1.  With causal = 1,
 * key j is masked for query i when j > i (the plainest reading; the pages do not
 * define a mask).
 *
 * The gradients of L = sum(dO o O), FlashAttention-2 review, 'core algorithm'
 * answer, section 2 (3) Backward Pass, read as the softmax Jacobian:
 *     dP = dO V^T,  D_i = sum_k dO_ik O_ik,  dS = P o (dP - D),
 *     dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Conventions shared by every entry point
 *   - Q, K, V, O, dO, dQ, dK, dV are device pointers to contiguous row-major
 *     [B, H, N, d] arrays (d fastest).  LSE and D are device fp32 [B, H, N].
 *   - d must be 64, 80 or 128 (else ATTN_EUNSUPPORTED).  B, H, N >= 1,
 *     N*d < 2^29 (one head below 2 GiB of fp32) and B*H*ceil(N/128) < 2^23 (the
 *     launch grids' limit) (else ATTN_EINVAL).  The total B*H*N*d is not limited
 *     otherwise: heads are addressed with 64-bit offsets.  Q, K, V have the same N.
 *   - scale must be finite (else ATTN_EINVAL); its sign is arbitrary.
 *   - Every pointer must be non-NULL and 16-byte aligned (else ATTN_EINVAL).
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it and the call returns without synchronising.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises, and keeps no state between calls apart from a
 *     thread-local copy of the last HIP error.
 *   - On ATTN_EINVAL / ATTN_EUNSUPPORTED nothing has been enqueued and no
 *     output has been written.  On ATTN_EHIP (a launch failed) the outputs are
 *     undefined and attn_last_hip_error() returns the hipError_t.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,        /* bad pointer, size, alignment, scale or flag   */
    ATTN_EUNSUPPORTED = 2,  /* valid request the library does not implement */
    ATTN_EHIP = 3,          /* a HIP runtime call failed                     */
    ATTN_ENOSPACE = 4       /* more than attn_bwd_noalloc's static scratch   */
} attn_status;

typedef enum {
    ATTN_F32 = 0,           /* IEEE binary32                                 */
    ATTN_BF16 = 1           /* bfloat16 (8-bit exponent, 7-bit mantissa)     */
} attn_dtype;

/* Forward.  Q, K, V: inputs of dtype `dt`.  O: output of dtype `dt` (written
 * once, rounded to nearest even when dt = ATTN_BF16).  LSE: fp32 output, the
 * saved row statistic the backward recomputes P from (FlashAttention-2 review,
 * 'core algorithm' answer, section 2 (3), item 1: the stored m and l, folded
 * into LSE = m + ln l).  Scores and probabilities stay on chip; nothing of
 * size N x N is written (FlashAttention-2 review, strengths answer: O(N)
 * extra memory).  Arithmetic: products of dt values accumulated in fp32; the
 * probabilities P are rounded to dt before the P V product. */
attn_status attn_fwd(const void* Q, const void* K, const void* V, attn_dtype dt,
                     int B, int H, int N, int d, float scale, int causal,
                     void* O, float* LSE, void* stream);

/* Backward preprocess: D_i = sum_k dO_ik O_ik in fp32, the row-wise inner
 * product the corrected dS formula needs (D_i = sum_j P_ij dP_ij).  O, dO:
 * dtype `dt`.  D: fp32 [B,H,N] output. */
attn_status attn_bwd_preprocess(const void* O, const void* dO, attn_dtype dt,
                                int B, int H, int N, int d, float* D, void* stream);

/* Backward, key side: dK and dV (fp32 outputs, written once).  One workgroup per
 * block of keys recomputes S and P from Q, K and the saved LSE
 * ("Recomputation", '[LLM] Flash Attention' blog; FlashAttention-2 review,
 * 'core algorithm' answer, section 2 (3)) and reduces dV = P^T dO and
 * dK = scale dS^T Q on chip.  D from attn_bwd_preprocess; LSE from attn_fwd with
 * the same scale and causal flag.  dt must be ATTN_BF16 (else ATTN_EUNSUPPORTED;
 * attn_bwd_main covers fp32 inputs). */
attn_status attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                          const float* LSE, const float* D, attn_dtype dt,
                          int B, int H, int N, int d, float scale, int causal,
                          float* dK, float* dV, void* stream);

/* Backward, query side: dQ = scale dS K (fp32 output, written once, no
 * atomics).  One workgroup per block of queries recomputes S^T, P^T and dS^T.
 * Same arguments and restrictions as attn_bwd_dkdv. */
attn_status attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                        const float* LSE, const float* D, attn_dtype dt,
                        int B, int H, int N, int d, float scale, int causal,
                        float* dQ, void* stream);

/* Backward, query side with the preprocess folded in: like attn_bwd_dq, but D
 * is an output.  Each workgroup computes D_i = sum_k dO_ik O_ik (fp32) for its
 * own query rows from O and the dO rows it loads anyway, uses it for dS, and
 * writes it to D for an attn_bwd_dkdv call that follows (same stream, or
 * ordered after this call).  O: device, dtype dt, [B,H,N,d] like Q, 16-byte
 * aligned.  D: device fp32 [B,H,N], 16-byte aligned, fully overwritten.  dQ as
 * in attn_bwd_dq.  dt must be ATTN_BF16 (else ATTN_EUNSUPPORTED); a null or
 * misaligned pointer gives ATTN_EINVAL and nothing is launched.  This is the
 * order attn_bwd takes for bf16 inputs: one pass over O and dO fewer than
 * attn_bwd_preprocess + attn_bwd_dq. */
attn_status attn_bwd_dq_d(const void* Q, const void* K, const void* V, const void* O,
                          const void* dO, const float* LSE, attn_dtype dt,
                          int B, int H, int N, int d, float scale, int causal,
                          float* D, float* dQ, void* stream);

/* Backward after the preprocess: dQ, dK, dV (fp32, written once).  bf16 inputs:
 * attn_bwd_dkdv then attn_bwd_dq.  fp32 inputs: one kernel for all three, with
 * dQ accumulated by fp32 atomics into dQ after zero-filling it. */
attn_status attn_bwd_main(const void* Q, const void* K, const void* V, const void* dO,
                          const float* LSE, const float* D, attn_dtype dt,
                          int B, int H, int N, int d, float scale, int causal,
                          float* dQ, float* dK, float* dV, void* stream);

/* Bytes of device workspace attn_bwd (and attn_bwd_blocksparse) needs for
 * gradients of dtype grad_dt: D (B*H*N fp32) rounded up to 256 bytes, the same
 * for both gradient dtypes (every gradient is written once in its own dtype, so
 * no fp32 staging buffer exists).  Returns 0 for invalid sizes or dtypes. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d, attn_dtype grad_dt);

/* Full backward.  bf16 inputs: attn_bwd_dq_d (dQ, and D into the workspace),
 * then attn_bwd_dkdv.  fp32 inputs: attn_bwd_preprocess + attn_bwd_main.  The
 * results do not depend on the order.  Q, K, V, O, dO: dtype
 * `dt`; LSE from attn_fwd with the same scale and causal flag.  dQ, dK, dV:
 * outputs of dtype grad_dt (ATTN_BF16 gradients need bf16 inputs, else
 * ATTN_EUNSUPPORTED).  workspace: device, 16-byte aligned, at least
 * attn_bwd_workspace_bytes(B, H, N, d, grad_dt) bytes (else ATTN_EINVAL). */
attn_status attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                     const void* dO, const float* LSE, attn_dtype dt,
                     int B, int H, int N, int d, float scale, int causal,
                     void* dQ, void* dK, void* dV, attn_dtype grad_dt,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same operation, arguments, kernels and results as attn_bwd, but
 * without the workspace argument: the one scratch buffer the backward needs (the
 * fp32 D rows, B*H*N floats) is a static device array of ATTN_NOALLOC_MAX_ROWS
 * floats (16 MiB) inside the library, one copy per GPU, held until the process
 * ends.  Its address is looked up once per device, on the first call made with
 * that device current.  B*H*N > ATTN_NOALLOC_MAX_ROWS gives ATTN_ENOSPACE and
 * nothing is launched; other errors as attn_bwd.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  Nothing in the scratch
 * needs to start at zero: each call overwrites the D rows it reads.  Every call
 * on one GPU shares that GPU's scratch, so calls that overlap on one GPU (on
 * streams not ordered with each other, or from several host threads) race and
 * must be serialised by the caller. */
#define ATTN_NOALLOC_MAX_ROWS (4 * 1024 * 1024)

attn_status attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* LSE, attn_dtype dt,
                             int B, int H, int N, int d, float scale, int causal,
                             void* dQ, void* dK, void* dV, attn_dtype grad_dt, void* stream);

/* Block-sparse attention.  FlashAttention-2 review, 'sparse/hybrid' answer,
 * section 3 (1) (Sparse FlashAttention): the score matrix is cut into blocks,
 * only the important blocks are computed, and the skipped ones are never moved
 * on chip.  Here a block mask decides which blocks count:
 *   block_mask: device uint8 [mask_heads][T][T], T = ceil(N / ATTN_MASK_BLOCK),
 *     row-major, no alignment needed.  Entry (a, b) nonzero keeps the scores of
 *     queries a*128 .. a*128+127 against keys b*128 .. b*128+127; zero drops
 *     them (S = -inf there: P = 0 and the K, V, Q, dO rows of the block are not
 *     loaded for it).  Applied on top of the causal mask when causal = 1.
 *   mask_heads: 1 (one mask for every head) or B*H (one per head, [B, H] order);
 *     anything else, or block_mask = NULL, gives ATTN_EINVAL.
 * A query row that keeps no key at all gets O = 0 and LSE = -inf, and adds
 * nothing to any gradient (its own dQ row is 0).  Every other argument, output
 * and error follows attn_fwd / attn_bwd; the backward must get the forward's
 * mask, scale and causal flag. */
#define ATTN_MASK_BLOCK 128

attn_status attn_fwd_blocksparse(const void* Q, const void* K, const void* V, attn_dtype dt,
                                 int B, int H, int N, int d, float scale, int causal,
                                 const unsigned char* block_mask, int mask_heads,
                                 void* O, float* LSE, void* stream);

attn_status attn_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O,
                                 const void* dO, const float* LSE, attn_dtype dt,
                                 int B, int H, int N, int d, float scale, int causal,
                                 const unsigned char* block_mask, int mask_heads,
                                 void* dQ, void* dK, void* dV, attn_dtype grad_dt,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* fp8 forward.  FlashAttention-2 review, research-directions answer: FP8
 * support is the gap it names for newer hardware.  Q, K, V: device OCP fp8
 * e4m3 ("e4m3fn": no infinities, max 448) [B,H,N,d] arrays whose real values
 * are q_descale * Q, k_descale * K, v_descale * V (one factor per tensor, any
 * finite value).  Computes the same O and LSE as attn_fwd on those real values,
 * with O in bf16 (RNE) and LSE in fp32.  d must be 64 or 128 (else
 * ATTN_EUNSUPPORTED).  Arithmetic: Q K^T from fp8 products, exact, summed in
 * fp32; the probabilities P are rounded to fp8 e4m3 (RNE, relative error at most
 * 2^-4, or 2^-10 absolute below 2^-6) before the P V product, and the row sum
 * is taken over exactly those rounded values; the largest P of each row is at
 * least 2^7.  Other arguments, errors and ownership as for attn_fwd. */
attn_status attn_fwd_fp8(const void* Q, const void* K, const void* V,
                         float q_descale, float k_descale, float v_descale,
                         int B, int H, int N, int d, float scale, int causal,
                         void* O, float* LSE, void* stream);

/* Static description of a status code (never NULL). */
const char* attn_status_str(attn_status s);

/* hipError_t behind the calling thread's last ATTN_EHIP (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
