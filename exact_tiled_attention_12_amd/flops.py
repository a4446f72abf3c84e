"""FLOP accounting for attention throughput.

FlashAttention-2 review, answer on implementation cost, section 2 (1)
(operation count): the forward costs 4 N^2 d per head and the backward 2.5
times the forward.  With a causal mask only about half of the score matrix is
computed, so both are halved (the workload statement's convention).
"""


def attn_flops(B, H, N, d, causal=False, which="fwd"):
    fwd = 4.0 * N * N * d * B * H
    if causal:
        fwd *= 0.5
    if which == "fwd":
        return fwd
    if which == "bwd":
        return 2.5 * fwd
    if which == "fwd+bwd":
        return 3.5 * fwd
    raise ValueError(which)


def blocksparse_flops(mask, N, d, causal=False, which="fwd", block=128):
    """Algorithmic FLOPs of block-sparse attention: the forward's 4 d per kept
    (query, key) pair, the backward 2.5 times that.  mask: [T, T] (one mask for
    every head; pass heads via a leading dimension or multiply) or [..., T, T],
    nonzero = kept; with causal only the pairs with key <= query count, so an
    all-kept causal mask gives 4 d N (N + 1) / 2 per head."""
    import numpy as np
    m = np.asarray(mask.cpu() if hasattr(mask, "cpu") else mask) != 0
    T = m.shape[-1]
    sizes = np.minimum(block, N - block * np.arange(T))            # rows (keys) per block
    pairs = np.outer(sizes, sizes).astype(np.float64)
    if causal:
        tri = np.tril(np.ones((T, T), bool), -1)
        pairs = np.where(tri, pairs, 0.0)
        pairs[np.arange(T), np.arange(T)] = sizes * (sizes + 1) / 2.0
    fwd = 4.0 * d * float((m * pairs).sum())
    if which == "fwd":
        return fwd
    if which == "bwd":
        return 2.5 * fwd
    if which == "fwd+bwd":
        return 3.5 * fwd
    raise ValueError(which)
