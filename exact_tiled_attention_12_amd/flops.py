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
