"""The five attention workloads (shapes only; no arithmetic of the method).

Shapes follow the problem statement of the FlashAttention-2 review
(Q, K, V in R^{N x d}, batched over heads) and the (Batch, Head, SeqLen, Dim)
layout of the 'Flash Attention-3' blog's code example.  Workload 5 takes the
attention-layer shape of GPT-3 2.7B (d_model 2560 = 32 heads x 80), the model
the FlashAttention-2 review quotes its end-to-end training figure on.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class AttnConfig:
    index: int
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str          # "fp32" or "bf16"
    backward: bool
    qk_mult: float = 1.0  # Q and K are multiplied by this after drawing

    @property
    def seed(self):
        return 1000 + self.index


CONFIGS = {
    1: AttnConfig(1, "fp32 B1 H1 N256 d64 non-causal, forward", 1, 1, 256, 64, False, "fp32", False),
    2: AttnConfig(2, "bf16 B8 H16 N1024 d64 non-causal, forward", 8, 16, 1024, 64, False, "bf16", False),
    3: AttnConfig(3, "bf16 B4 H16 N4096 d128 causal, fwd+bwd", 4, 16, 4096, 128, True, "bf16", True),
    4: AttnConfig(4, "bf16 B1 H16 N16384 d128 causal (Q,K x0.5), fwd+bwd", 1, 16, 16384, 128, True,
                  "bf16", True, 0.5),
    5: AttnConfig(5, "bf16 B8 H32 N2048 d80 causal (GPT-3 2.7B layer shape), fwd+bwd", 8, 32, 2048,
                  80, True, "bf16", True),
}
