/*
 * mfma_rate.h -- C ABI of the matrix-core rate probe (libmfma_rate.so, gfx950).
 *
 * A measurement aid, not part of the attention path: it gives the bf16 MFMA rate that
 * the chip sustains at the clock it actually holds under matrix-core load, so that the
 * attention kernels' rates can be read against that ceiling as well as against the
 * published 2.4 GHz figure.
 */
#ifndef MFMA_RATE_H
#define MFMA_RATE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `workgroups` workgroups of 256 threads (four waves, at most two workgroups
 * per CU, so two waves per SIMD).  Every wave issues `iters` rounds of four independent
 * v_mfma_f32_32x32x16_bf16 products (32768 FLOP each) back to back, with, per `mix`:
 *   0  nothing else (register operands);
 *   1  each product's A operand read from LDS (one ds_read_b128 per product, the next
 *      round's four read after this round's products), as the attention kernels feed
 *      their products;
 *   2  register operands, plus per product one v_exp_f32 of an FMA, one max and one add
 *      on independent chains (about an online softmax's VALU work per product);
 *   3  both.
 *   out:    device fp32 [workgroups * 256], written (a reduction of the accumulators, so
 *           that the products are not optimised away; the values carry no meaning).
 *   stamps: device uint64 [workgroups * 4]: per workgroup, its first wave's s_memtime
 *           (shader clock counter) before and after the products, then s_memrealtime
 *           (a constant 100 MHz counter) before and after.
 *   stream: hipStream_t as void* (NULL = default stream); the call enqueues and returns.
 * Returns 0, 1 for a bad argument (workgroups or iters < 1, mix outside 0-3, a NULL
 * pointer; nothing is launched), 3 if the launch failed.  The caller owns both buffers. */
int mfma_rate_probe(int workgroups, int iters, int mix, float* out, unsigned long long* stamps, void* stream);

#ifdef __cplusplus
}
#endif

#endif
