"""GPU parity of the split backward entry points, and of a problem past 2^31 elements.

attn_bwd itself runs attn_bwd_dq_d + attn_bwd_dkdv (bf16) or attn_bwd_preprocess +
the fused fp32 kernel; these tests also cover the entry points a caller can chain
by hand (FlashAttention-2 review, 'core algorithm' answer, section 2 (3) Backward
Pass: D, then the recomputing backward):
  * attn_bwd_preprocess, then attn_bwd_main (bf16: key side + query side reading D;
    fp32: the fused kernel with dQ atomics);
  * attn_bwd_preprocess, then attn_bwd_dq (the query-side kernel's branch that reads
    D instead of computing it) and attn_bwd_dkdv.
Every output is NaN-poisoned first and compared with the fp64 oracle element by
element: bf16 against the per-element bound derived from the kernels' roundings
(tests/bf16_bound.py), fp32 against 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_12_amd import (attn_bwd, attn_bwd_dkdv, attn_bwd_dq, attn_bwd_dq_d, attn_bwd_main,
                                          attn_bwd_preprocess, attn_fwd, prepare)
from exact_tiled_attention_12_amd.inputs import make_inputs

from bf16_bound import bounds as bf16_bounds

pytestmark = pytest.mark.gpu
NAN = float("nan")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _nan_like(t, dtype=torch.float32):
    return torch.full(t.shape, NAN, dtype=dtype, device=t.device)


def _check_D(D, o, do):
    """D against the fp64 row sums of the same (GPU) O and dO: fp32 accumulation of d products."""
    od = o.double().cpu() * do.double().cpu()
    ref = od.sum(-1).numpy()
    bound = 2 * od.shape[-1] * 2.0 ** -24 * od.abs().sum(-1).numpy() + 1e-30
    err = np.abs(D.double().cpu().numpy() - ref)
    assert not np.isnan(err).any()
    assert np.all(err <= bound), f"D: {err.max():.3e}"


def _check_grads(q, k, v, do, grads, causal, dtype):
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            ref = oracle.bwd(q[b, h], k[b, h], v[b, h], do[b, h], causal=causal)
            bd = bf16_bounds(q[b, h], k[b, h], v[b, h], do[b, h], causal=causal) if dtype == "bf16" else None
            for n, g, r in zip(("dQ", "dK", "dV"), grads, ref):
                err = np.abs(g[b, h].double().cpu().numpy() - r)
                assert not np.isnan(err).any(), f"head ({b},{h}) {n}: NaN"
                if dtype == "bf16":
                    ratio = float((err / bd[n]).max())
                    _say(f"  head ({b},{h}) {n}: max err {err.max():.2e}, err/bound {ratio:.3f}")
                    assert ratio <= 1.0, f"head ({b},{h}) {n}: outside the derived bound"
                else:
                    _say(f"  head ({b},{h}) {n}: max err {err.max():.2e}")
                    assert err.max() <= 1e-5, f"head ({b},{h}) {n}: {err.max()}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_preprocess_then_main(dtype, d, causal):
    N = 333
    _say(f"case preprocess + main dtype={dtype} d={d} causal={causal} N={N}")
    dev = _dev()
    q, k, v, do = make_inputs(1, 3, N, d, dtype, seed=900 + d + causal)
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn_fwd(qg, kg, vg, causal=causal)
    D = attn_bwd_preprocess(o, dog, D=_nan_like(lse))
    dq, dk, dv = (_nan_like(qg) for _ in range(3))
    attn_bwd_main(qg, kg, vg, dog, lse, D, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    _check_D(D, o, dog)
    _check_grads(q, k, v, do, (dq, dk, dv), causal, dtype)


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_query_side_reading_D(d, causal):
    """attn_bwd_preprocess, then attn_bwd_dq (D read, not computed) and attn_bwd_dkdv."""
    N = 333
    _say(f"case preprocess + dq (D read) + dkdv d={d} causal={causal} N={N}")
    dev = _dev()
    q, k, v, do = make_inputs(1, 3, N, d, "bf16", seed=950 + d + causal)
    qg, kg, vg, dog = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn_fwd(qg, kg, vg, causal=causal)
    D = attn_bwd_preprocess(o, dog, D=_nan_like(lse))
    dq = attn_bwd_dq(qg, kg, vg, dog, lse, D, causal=causal, dq=_nan_like(qg))
    dk, dv = attn_bwd_dkdv(qg, kg, vg, dog, lse, D, causal=causal, dk=_nan_like(qg), dv=_nan_like(qg))
    torch.cuda.synchronize()
    _check_D(D, o, dog)
    _check_grads(q, k, v, do, (dq, dk, dv), causal, "bf16")


def test_more_than_2_31_elements():
    """B1 H4097 N4096 d128 causal: 2^31 + 2^19 elements per tensor, so the last head starts at
    element 2^31.  Heads 0..4095 repeat eight seeded heads; the last head is drawn from a seed
    of its own.  Heads 0, 4095 and 4096 are compared with the oracle in full (forward and
    backward), every output NaN-poisoned first."""
    B, H, N, d = 1, 4097, 4096, 128
    assert B * H * N * d > 2 ** 31
    _say(f"case more than 2^31 elements: B{B} H{H} N{N} d{d} causal")
    dev = _dev()
    base = make_inputs(1, 8, N, d, "bf16", seed=2031)
    last = make_inputs(1, 1, N, d, "bf16", seed=2032)
    big = []
    for t, t_last in zip(base, last):
        g = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
        tg = t.to(dev)
        for h0 in range(0, H - 1, 8):
            g[:, h0:h0 + 8] = tg
        g[:, H - 1:] = t_last.to(dev)
        big.append(g)
    qg, kg, vg, dog = big
    o = torch.full_like(qg, NAN)
    lse = torch.full((B, H, N), NAN, device=dev)
    attn_fwd(qg, kg, vg, causal=True, out=o, lse=lse)
    dq, dk, dv = (torch.full((B, H, N, d), NAN, device=dev) for _ in range(3))
    attn_bwd(qg, kg, vg, o, dog, lse, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for hh in (0, H - 2, H - 1):
        src = last if hh == H - 1 else tuple(t[:, hh % 8:hh % 8 + 1] for t in base)
        qh, kh, vh, doh = (t[0, 0] for t in src)
        O_ref, L_ref = oracle.fwd(qh, kh, vh, causal=True)
        dQ, dK, dV = oracle.bwd(qh, kh, vh, doh, causal=True)
        errs = {}
        for n, g, r in (("O", o, O_ref), ("LSE", lse, L_ref), ("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
            errs[n] = float(np.abs(g[0, hh].float().cpu().numpy() - r).max())
        _say(f"  head {hh}:", {n: f"{e:.2e}" for n, e in errs.items()})
        for n, e in errs.items():
            assert e <= 2e-2, f"head {hh} {n}: {e}"
    # every head written: no NaN left anywhere (checked on the device)
    for t in (o, lse, dq, dk, dv):
        assert not torch.isnan(t).any()


def test_prepared_launches_match_direct_calls():
    """prepare() marshals a call once and launches nothing; each launch() then gives the same bits as
    the direct call (the bf16 kernels are deterministic), also into outputs prepare() allocated and
    with a workspace the binding allocated inside the call."""
    dev = _dev()
    _say("case prepared launches: B=2 H=3 N=300 d=128 causal bf16")
    q, k, v, do = (t.to(dev) for t in make_inputs(2, 3, 300, 128, "bf16", seed=31))
    o_ref, l_ref = attn_fwd(q, k, v, causal=True)
    D_ref = torch.empty_like(l_ref)
    dq_ref, _ = attn_bwd_dq_d(q, k, v, o_ref, do, l_ref, D=D_ref, causal=True)
    dk_ref, dv_ref = attn_bwd_dkdv(q, k, v, do, l_ref, D_ref, causal=True)
    o, lse, D, dq, dk, dv = (_nan_like(t, t.dtype) for t in (o_ref, l_ref, D_ref, dq_ref, dk_ref, dv_ref))
    fwd, _ = prepare(attn_fwd, q, k, v, causal=True, out=o, lse=lse)
    qside, _ = prepare(attn_bwd_dq_d, q, k, v, o, do, lse, D=D, causal=True, dq=dq)
    kside, _ = prepare(attn_bwd_dkdv, q, k, v, do, lse, D, causal=True, dk=dk, dv=dv)
    fwd2, (o2, l2) = prepare(attn_fwd, q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(dq).all() and torch.isnan(dk).all()
    # attn_bwd with no workspace: the binding allocates one inside the call, kept alive by the launch
    full, grads = prepare(attn_bwd, q, k, v, o_ref, do, l_ref, causal=True)
    grads_ref = attn_bwd(q, k, v, o_ref, do, l_ref, causal=True)
    for g in grads:
        g.fill_(float("nan"))
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    for rep in range(3):
        fwd()
        qside()
        kside()
        fwd2()
        full()
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ (attn_bwd)", "dK (attn_bwd)", "dV (attn_bwd)"), grads, grads_ref):
            assert torch.equal(a, b), f"launch {rep}: {name} differs from the direct call"
        for name, a, b in (("O", o, o_ref), ("LSE", lse, l_ref), ("D", D, D_ref), ("dQ", dq, dq_ref),
                           ("dK", dk, dk_ref), ("dV", dv, dv_ref), ("O (allocated)", o2, o_ref),
                           ("LSE (allocated)", l2, l_ref)):
            assert torch.equal(a, b), f"launch {rep}: {name} differs from the direct call"
