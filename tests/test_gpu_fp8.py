"""GPU checks of the fp8 forward (attn_fwd_fp8) against the fp64 oracle.

The oracle computes exact attention on the real inputs (the fp8 values times
their dequantisation factors, exact in fp64).  The kernel differs from it by its
documented roundings, which fix a per-element bound:
  * P is rounded to e4m3: |P~ - P| <= 2^-4 P (normal range) or <= 2^-10 (below
    2^-6), with the row's largest P >= 2^7, so relative to the row's sum the
    absolute part is at most 2^-17 per key;
  * O = sum_j P~_j v_j / sum_j P~_j, hence, with P the exact softmax,
      |O~_id - O_id| <= (2^-4 sum_j P_ij |v_jd - O_id| + 2^-17 sum_j |v_jd - O_id|) / (1 - 2^-4 - 2^-17 n_i)
    (n_i = keys the row sees), plus the bf16 rounding of O (2^-8 |O|) and 1e-5
    for the fp32 sums;
  * LSE from the same rounded sum: |LSE~ - LSE| <= -ln(1 - 2^-4 - 2^-17 n_i) + 1e-5.
The tests assert that bound element by element.  Typical errors are far below it
(the roundings of many keys average out) and are printed.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_12_amd import attn_fwd, attn_fwd_fp8
from exact_tiled_attention_12_amd.inputs import make_fp8_inputs

pytestmark = pytest.mark.gpu

EPS_P, EPS_ABS = 2.0 ** -4, 2.0 ** -17


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _real(t8, s):
    return t8.float().double() * s


def _check_head(o, lse, q, k, v, causal, scale=None):
    """o, lse: one head's GPU outputs (CPU tensors); q, k, v: real inputs [N, d] (fp64)."""
    O, L, P = oracle.fwd_probs(q, k, v, scale=scale, causal=causal)
    vv = v.numpy() if hasattr(v, "numpy") else v
    N = O.shape[0]
    n = (np.arange(N) + 1) if causal else np.full(N, N)
    den = 1.0 - EPS_P - EPS_ABS * n
    A, B = np.empty_like(O), np.empty_like(O)
    for i0 in range(0, N, 32):                                        # rows in chunks: [rows, N, d] at a time
        i1 = min(N, i0 + 32)
        dev_abs = np.abs(vv[None, :, :] - O[i0:i1, None, :])          # |v_jd - O_id|
        seen = np.ones((i1 - i0, N))
        if causal:
            seen = (np.arange(N)[None, :] <= np.arange(i0, i1)[:, None]).astype(np.float64)
        A[i0:i1] = np.einsum("ij,ijd->id", P[i0:i1], dev_abs)
        B[i0:i1] = np.einsum("ij,ijd->id", seen, dev_abs)
    bound_o = (EPS_P * A + EPS_ABS * B) / den[:, None] + 2.0 ** -8 * np.abs(O) + 1e-5
    bound_l = -np.log(den) + 1e-5
    eo = np.abs(o.double().numpy() - O)
    el = np.abs(lse.double().numpy() - L)
    assert (eo <= bound_o).all(), f"O: worst excess {float((eo - bound_o).max())}"
    assert (el <= bound_l).all(), f"LSE: worst excess {float((el - bound_l).max())}"
    return float(eo.max()), float(eo.mean()), float(el.max()), float(bound_o.max())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 130, 300, 1000])
def test_small_shapes(d, causal, N):
    _say(f"case fp8 d={d} causal={causal} N={N}")
    dev = _dev()
    (q8, k8, v8), (sq, sk, sv) = make_fp8_inputs(1, 2, N, d, seed=N + d + causal)
    o, lse = attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), sq, sk, sv, causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    for hh in range(2):
        r = _check_head(o[0, hh].cpu(), lse[0, hh].cpu(), _real(q8[0, hh], sq), _real(k8[0, hh], sk),
                        _real(v8[0, hh], sv), causal)
        _say(f"  head {hh}: O max {r[0]:.2e} mean {r[1]:.2e} (bound up to {r[3]:.2e}), LSE max {r[2]:.2e}")


@pytest.mark.parametrize("scale", [0.0, -0.07, 0.25])
def test_scale_and_sign(scale):
    """A zero scale (uniform P), a negative one (sign folded into Q) and a sharp one."""
    _say(f"case fp8 scale={scale}")
    dev = _dev()
    (q8, k8, v8), (sq, sk, sv) = make_fp8_inputs(1, 1, 200, 128, seed=3)
    o, lse = attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), sq, -sk, sv, scale=scale, causal=True)
    torch.cuda.synchronize()
    r = _check_head(o[0, 0].cpu(), lse[0, 0].cpu(), _real(q8[0, 0], sq), _real(k8[0, 0], -sk),
                    _real(v8[0, 0], sv), True, scale=scale)
    _say(f"  O max {r[0]:.2e} mean {r[1]:.2e}, LSE max {r[2]:.2e}")


def test_workload_size_sampled_heads():
    """B4 H16 N4096 d128 causal (the bf16 bench shape), two heads checked in full."""
    _say("case fp8 B4 H16 N4096 d128 causal")
    dev = _dev()
    B, H, N, d = 4, 16, 4096, 128
    (q8, k8, v8), (sq, sk, sv) = make_fp8_inputs(B, H, N, d, seed=44)
    o, lse = attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), sq, sk, sv, causal=True)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (3, 15)):
        r = _check_head(o[b, h].cpu(), lse[b, h].cpu(), _real(q8[b, h], sq), _real(k8[b, h], sk),
                        _real(v8[b, h], sv), True)
        _say(f"  head ({b},{h}): O max {r[0]:.2e} mean {r[1]:.2e}, LSE max {r[2]:.2e}")


def test_matches_bf16_kernel_on_same_values_statistically():
    """On inputs that bf16 holds exactly (fp8 values times powers of two), the fp8 and bf16
    kernels differ only by the rounding of P: mean |difference| stays near 2^-4 / sqrt(keys)."""
    _say("case fp8 vs bf16 kernel")
    dev = _dev()
    (q8, k8, v8), _ = make_fp8_inputs(1, 4, 2048, 128, seed=9)
    s = 2.0 ** -7                                    # power of two: exact in bf16
    o8, l8 = attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), s, s, s, causal=False)
    qb, kb, vb = ((t.float() * s).to(torch.bfloat16).to(dev) for t in (q8, k8, v8))
    ob, lb = attn_fwd(qb, kb, vb, causal=False)
    torch.cuda.synchronize()
    diff = (o8.float() - ob.float()).abs()
    _say(f"  mean |O8 - O16| {diff.mean().item():.2e}, max {diff.max().item():.2e}, "
         f"LSE max {(l8 - lb).abs().max().item():.2e}")
    assert diff.mean().item() < 2.0 ** -4 / math.sqrt(64) * float(vb.float().abs().mean())


def test_beyond_4096_causal():
    """B1 H2 N4500 d128 causal: past N = 4096 the launch table gives the causal d = 128 fp8
    forward its 128-key tile; both heads checked in full against the bound."""
    _say("case fp8 B1 H2 N4500 d128 causal (128-key tiles)")
    dev = _dev()
    (q8, k8, v8), (sq, sk, sv) = make_fp8_inputs(1, 2, 4500, 128, seed=45)
    o, lse = attn_fwd_fp8(q8.to(dev), k8.to(dev), v8.to(dev), sq, sk, sv, causal=True)
    torch.cuda.synchronize()
    for hh in range(2):
        r = _check_head(o[0, hh].cpu(), lse[0, hh].cpu(), _real(q8[0, hh], sq), _real(k8[0, hh], sk),
                        _real(v8[0, hh], sv), True)
        _say(f"  head {hh}: O max {r[0]:.2e} mean {r[1]:.2e}, LSE max {r[2]:.2e}")
