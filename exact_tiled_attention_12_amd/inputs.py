"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no arithmetic of the attention method: it only draws i.i.d. N(0, 1)
values with a seeded CPU generator (order Q, K, V, dO), applies the workload's
Q/K multiplier (an exact power of two) and rounds to the compute dtype (RNE).
"""
import torch

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _DT[name]


def make_inputs(B, H, N, d, dtype="bf16", seed=0, qk_mult=1.0, with_grad=True):
    """Returns CPU tensors (q, k, v, do) of shape [B, H, N, d] in `dtype`."""
    g = torch.Generator().manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32) if with_grad else None
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    dt = _DT[dtype]
    out = [q.to(dt), k.to(dt), v.to(dt)]
    out.append(None if do is None else do.to(dt))
    return tuple(out)


def config_inputs(cfg, with_grad=None):
    if with_grad is None:
        with_grad = cfg.backward
    return make_inputs(cfg.B, cfg.H, cfg.N, cfg.d, cfg.dtype, cfg.seed, cfg.qk_mult, with_grad)


def random_block_mask(T, density, seed, empty_rows=(), lead=()):
    """uint8 block mask of shape lead + (T, T): each entry kept with probability `density`
    (seeded), then the listed block rows cleared (queries that keep no key)."""
    g = torch.Generator().manual_seed(int(seed))
    m = (torch.rand(tuple(lead) + (T, T), generator=g) < density).to(torch.uint8)
    for a in empty_rows:
        m[..., a, :] = 0
    return m


def local_global_mask(T, window, n_global):
    """uint8 [T, T] block mask of a local + global pattern: query block a keeps key blocks
    b with |a - b| < window (local context) and the first n_global key blocks (global)."""
    a = torch.arange(T).view(T, 1)
    b = torch.arange(T).view(1, T)
    return (((a - b).abs() < window) | (b < n_global)).to(torch.uint8)


FP8_MAX = 448.0        # largest finite OCP e4m3 ("e4m3fn") value


def make_fp8_inputs(B, H, N, d, seed=0):
    """fp8 e4m3 inputs with per-tensor dequantisation factors: i.i.d. N(0, 1) draws
    (order Q, K, V, seeded), each tensor divided by max|x| / 448 and rounded to
    e4m3 (torch's conversion).  Returns ((q8, k8, v8), (sq, sk, sv)) on the CPU;
    the real inputs are sq * q8.float(), and so on."""
    g = torch.Generator().manual_seed(int(seed))
    shape = (B, H, N, d)
    xs = [torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3)]
    out, scales = [], []
    for x in xs:
        s = float(x.abs().max()) / FP8_MAX
        out.append((x / s).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn))
        scales.append(s)
    return tuple(out), tuple(scales)
