"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: max-abs error <= 1e-5 for fp32 inputs and <= 2e-2 for bf16 inputs on
O, LSE, dQ, dK and dV; the oracle receives the exact (bf16-rounded) inputs.
Small shapes are compared element by element everywhere; the five workloads
run at full size in the launch configuration the benchmark times, with every
output NaN-poisoned first and every element of every head compared with the
oracle.  Off the workloads (sharp softmaxes, extreme scales), where gradients
grow past the workloads' magnitude, bf16 outputs are held to the per-element
bound derived from the kernels' roundings (tests/bf16_bound.py) instead.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_12_amd import attn_bwd, attn_bwd_dkdv, attn_bwd_dq_d, attn_fwd
from exact_tiled_attention_12_amd.configs import CONFIGS
from exact_tiled_attention_12_amd.inputs import config_inputs, make_inputs

from bf16_bound import bounds as bf16_bounds

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}
NAN = float("nan")


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _err(gpu, ref):
    """Largest |gpu - ref| (NaN if any element is NaN, so an unwritten output fails)."""
    return float(np.abs(gpu.detach().float().cpu().numpy() - ref).max())


def _run(q, k, v, do, causal, scale=None, grad_dtype=torch.float32):
    """Forward (and backward) with every output NaN-poisoned first."""
    dev = _dev()
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    o = torch.full_like(qg, NAN)
    lse = torch.full(qg.shape[:-1], NAN, device=dev)
    attn_fwd(qg, kg, vg, scale=scale, causal=causal, out=o, lse=lse)
    grads = None
    if do is not None:
        grads = tuple(torch.full(q.shape, NAN, dtype=grad_dtype, device=dev) for _ in range(3))
        attn_bwd(qg, kg, vg, o, do.to(dev), lse, scale=scale, causal=causal, grad_dtype=grad_dtype,
                 dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return o, lse, grads


def _assert_within_bound(name, gpu, ref, bound):
    """Element-wise |gpu - ref| <= bound; prints the largest error and its share of the bound."""
    err = np.abs(gpu.detach().float().cpu().double().numpy() - ref)
    assert not np.isnan(err).any(), f"{name}: NaN (an element left unwritten or a non-finite result)"
    ratio = float(np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0)).max())
    _say(f"    {name}: max err {err.max():.2e}, max err/bound {ratio:.3f}, max |ref| {np.abs(ref).max():.2e}")
    assert ratio <= 1.0, f"{name}: error outside the derived bound (ratio {ratio:.3f})"


def _check_full(q, k, v, do, causal, dtype, scale=None, tol=None, grad_dtype=torch.float32, derived=False):
    """Element-wise comparison of every output.  derived=True (bf16 only, used off the five
    workloads, where a sharper softmax makes the gradients larger than the workloads'
    magnitude of about 4) holds each head to the per-element bound derived from the
    kernels' roundings (tests/bf16_bound.py) instead of the fixed bar."""
    tol = TOL[dtype] if tol is None else tol
    o, lse, grads = _run(q, k, v, do, causal, scale, grad_dtype)
    O_ref, L_ref = oracle.fwd(q, k, v, scale=scale, causal=causal)
    refs = {"O": (o, O_ref), "LSE": (lse, L_ref)}
    if do is not None:
        dQ, dK, dV = oracle.bwd(q, k, v, do, scale=scale, causal=causal)
        refs.update(dQ=(grads[0], dQ), dK=(grads[1], dK), dV=(grads[2], dV))
    if derived:
        assert dtype == "bf16"
        B, H = q.shape[:2]
        for b in range(B):
            for h in range(H):
                bd = bf16_bounds(q[b, h], k[b, h], v[b, h], None if do is None else do[b, h], scale=scale,
                                 causal=causal, grad_bf16=grad_dtype == torch.bfloat16)
                _say(f"  head ({b}, {h}):")
                for n, (g, r) in refs.items():
                    _assert_within_bound(n, g[b, h], r[b, h], bd[n])
        return o, lse, grads
    errs = {n: _err(g, r) for n, (g, r) in refs.items()}
    _say("  max-abs errors:", {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= tol, f"{n}: {e} > {tol}"
    return o, lse, grads


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 3, 17, 64, 130, 257])
def test_small_shapes(dtype, d, causal, N):
    _say(f"case small dtype={dtype} d={d} causal={causal} N={N}")
    q, k, v, do = make_inputs(1, 2, N, d, dtype, seed=N * 1000 + d + causal)
    _check_full(q, k, v, do, causal, dtype)


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_multi_tile(d, causal):
    """Several 256-row blocks and 128-key blocks with a ragged tail, grid >= 256 workgroups."""
    N = 1000
    _say(f"case ragged d={d} causal={causal} N={N}")
    q, k, v, do = make_inputs(2, 33, N, d, "bf16", seed=77 + d)
    dev = _dev()
    o, lse, (dq, dk, dv) = _run(q, k, v, do, causal)
    for hh in range(66):      # every head (outputs NaN-poisoned by _run)
        b, h = divmod(hh, 33)
        O_ref, L_ref = oracle.fwd(q[b, h], k[b, h], v[b, h], causal=causal)
        dQ, dK, dV = oracle.bwd(q[b, h], k[b, h], v[b, h], do[b, h], causal=causal)
        errs = [_err(o[b, h], O_ref), _err(lse[b, h], L_ref), _err(dq[b, h], dQ), _err(dk[b, h], dK),
                _err(dv[b, h], dV)]
        _say("  head", hh, [f"{e:.2e}" for e in errs])
        assert max(errs) <= TOL["bf16"]
    assert dev.type == "cuda"


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.3])
def test_scale_edge_values(scale):
    """scale = 0 (uniform weights), a negative scale and a large one, against the derived bound."""
    _say(f"case scale={scale}")
    q, k, v, do = make_inputs(1, 3, 150, 64, "bf16", seed=5)
    _check_full(q, k, v, do, True, "bf16", scale=scale, derived=True)
    _check_full(q, k, v, do, False, "bf16", scale=scale, derived=True)


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores(d, causal):
    """Scores that keep growing along the keys, so the running row max moves far past its
    reference on later tiles, in the first and in the second 32-key half of a tile: key
    rows are scaled by a ramp (1 + j/48), with extra factors on keys 96-127 and 320-351.
    Held to the derived bound."""
    N = 700
    _say(f"case rising scores d={d} causal={causal} N={N}")
    q, k, v, do = make_inputs(1, 2, N, d, "bf16", seed=300 + d + causal)
    ramp = 1.0 + torch.arange(N, dtype=torch.float32) / 48.0
    ramp[96:128] *= 3.0
    ramp[320:352] *= 2.0
    k = (k.float() * ramp[:, None]).to(torch.bfloat16)
    _check_full(q, k, v, do, causal, "bf16", derived=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_very_negative_scores_ragged(d, causal):
    """Every key row equal (u) and Q = -16 u, so every score of a row is about -16 |u|^2 / sqrt(d)
    and LSE is about -120: a key past N (read as a zero row) would get P = exp(-LSE) = inf, which
    only masking keeps out of the gradients.  N % 64 != 0; gradients must be finite and inside
    the derived bound."""
    N = 1000
    _say(f"case very negative scores d={d} causal={causal} N={N}")
    q, k, v, do = make_inputs(1, 2, N, d, "bf16", seed=71 + d + causal)
    u = k[:, :, :1, :].float()
    k = u.expand(-1, -1, N, -1).to(torch.bfloat16).contiguous()
    q = (-16.0 * u).expand(-1, -1, N, -1).to(torch.bfloat16).contiguous()
    o, lse, grads = _check_full(q, k, v, do, causal, "bf16", derived=True)
    assert float(lse.min()) < -100.0
    for g in grads:
        assert torch.isfinite(g).all()


@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_query_side_with_folded_preprocess(d, causal):
    """attn_bwd_dq_d (dQ, and D = rowsum(dO o O) computed per query row) followed by
    attn_bwd_dkdv on that D: gradients against the oracle, D against the fp64 row sums of
    the same bf16 O and dO (fp32 accumulation bound)."""
    N = 700
    _say(f"case dq_d d={d} causal={causal} N={N}")
    dev = _dev()
    q, k, v, do = make_inputs(1, 3, N, d, "bf16", seed=500 + d + causal)
    qg, kg, vg, dog = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = attn_fwd(qg, kg, vg, causal=causal)
    D = torch.full(lse.shape, float("nan"), dtype=torch.float32, device=dev)
    dq, D = attn_bwd_dq_d(qg, kg, vg, o, dog, lse, D=D, causal=causal)
    dk, dv = attn_bwd_dkdv(qg, kg, vg, dog, lse, D, causal=causal)
    torch.cuda.synchronize()
    od = o.double().cpu() * do.double()
    D_ref = od.sum(-1).numpy()
    bound = 1e-5 * od.abs().sum(-1).numpy() + 1e-6
    assert np.all(np.abs(D.double().cpu().numpy() - D_ref) <= bound)
    for hh in range(3):
        dQ, dK, dV = oracle.bwd(q[0, hh], k[0, hh], v[0, hh], do[0, hh], causal=causal)
        errs = [_err(dq[0, hh], dQ), _err(dk[0, hh], dK), _err(dv[0, hh], dV)]
        _say("  head", hh, [f"{e:.2e}" for e in errs])
        assert max(errs) <= TOL["bf16"]


def test_bf16_gradients_option():
    _say("case bf16 grads")
    q, k, v, do = make_inputs(1, 2, 300, 128, "bf16", seed=9)
    _check_full(q, k, v, do, True, "bf16", grad_dtype=torch.bfloat16)


def test_forward_deterministic_and_overwrites_nan_poison():
    _say("case determinism / NaN poison")
    dev = _dev()
    q, k, v, _ = make_inputs(2, 4, 777, 128, "bf16", seed=3, with_grad=False)
    qg, kg, vg = q.to(dev), k.to(dev), v.to(dev)
    o1 = torch.full_like(qg, float("nan"))
    l1 = torch.full(qg.shape[:-1], float("nan"), device=dev)
    attn_fwd(qg, kg, vg, causal=True, out=o1, lse=l1)
    o2, l2 = attn_fwd(qg, kg, vg, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_backward_overwrites_nan_poison():
    _say("case bwd NaN poison")
    dev = _dev()
    q, k, v, do = make_inputs(1, 3, 333, 80, "bf16", seed=4)
    qg, kg, vg, dg = (t.to(dev) for t in (q, k, v, do))
    o, lse = attn_fwd(qg, kg, vg, causal=True)
    dq, dk, dv = (torch.full(q.shape, float("nan"), device=dev) for _ in range(3))
    attn_bwd(qg, kg, vg, o, dg, lse, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


# ---------------------------------------------------------------------------
# The five workloads at full size, every element of every head.
# ---------------------------------------------------------------------------
_FULL = {}


def _full_run(idx):
    """Workload idx at full size, in the launch configuration the benchmark times (attn_fwd, then
    attn_bwd: the query-side kernel with D, then the key side), every output NaN-poisoned first.
    Returns CPU copies.  One workload is kept at a time; its parts reuse it."""
    if idx not in _FULL:
        _FULL.clear()
        cfg = CONFIGS[idx]
        q, k, v, do = config_inputs(cfg)
        o, lse, grads = _run(q, k, v, do, cfg.causal)
        cpu = lambda t: t.detach().cpu()
        _FULL[idx] = (q, k, v, do, cpu(o), cpu(lse), None if grads is None else tuple(cpu(g) for g in grads))
    return _FULL[idx]


# (workload, part, parts): the heads of a workload are split into parts so that each test's
# oracle work stays near half a minute on the host
FULL_PARTS = [(1, 0, 1), (2, 0, 1), (5, 0, 2), (5, 1, 2), (3, 0, 2), (3, 1, 2), (4, 0, 4), (4, 1, 4), (4, 2, 4),
              (4, 3, 4)]


@pytest.mark.parametrize("idx,part,parts", FULL_PARTS)
def test_workload_every_element(idx, part, parts):
    cfg = CONFIGS[idx]
    _say(f"case workload {idx} every element, part {part + 1} of {parts}: {cfg.name}")
    q, k, v, do, o, lse, grads = _full_run(idx)
    BH = cfg.B * cfg.H
    tol = TOL[cfg.dtype]
    flat = lambda t: t.reshape(BH, cfg.N, *t.shape[3:])
    h0, h1 = part * BH // parts, (part + 1) * BH // parts
    worst = {}
    for hh in range(h0, h1):
        qh, kh, vh = flat(q)[hh], flat(k)[hh], flat(v)[hh]
        O_ref, L_ref = oracle.fwd(qh, kh, vh, causal=cfg.causal)
        errs = {"O": _err(flat(o)[hh], O_ref), "LSE": _err(flat(lse)[hh], L_ref)}
        if grads is not None:
            dQ, dK, dV = oracle.bwd(qh, kh, vh, flat(do)[hh], causal=cfg.causal)
            for n, g, r in zip(("dQ", "dK", "dV"), grads, (dQ, dK, dV)):
                errs[n] = _err(flat(g)[hh], r)
        for n, e in errs.items():
            assert e <= tol, f"head {hh} {n}: {e} > {tol}"      # NaN (an unwritten element) fails too
            worst[n] = max(worst.get(n, 0.0), e)
    _say(f"  heads {h0}..{h1 - 1}, largest errors:", {n: f"{e:.2e}" for n, e in worst.items()})


def test_long_sequence_sampled():
    """N = 65536 (four times the longest workload): sampled query rows (O, LSE, dQ) of both
    heads and key rows (dK, dV) of one, each evaluated by the oracle from its definition."""
    N = 65536
    _say(f"case long sequence N={N}")
    q, k, v, do = make_inputs(1, 2, N, 128, "bf16", seed=65)
    o, lse, (dq, dk, dv) = _run(q, k, v, do, True)
    rng = np.random.default_rng(65)
    rows = np.unique(np.concatenate([[0, 1, 4095, 4096, 32767, N - 1], rng.integers(0, N, 10)]))
    for hh in (0, 1):
        Or, Lr, dQr = oracle.rows(q[0, hh], k[0, hh], v[0, hh], do[0, hh], rows, causal=True)
        ridx = torch.as_tensor(rows)
        errs = {"O": _err(o[0, hh][ridx], Or), "LSE": _err(lse[0, hh][ridx], Lr), "dQ": _err(dq[0, hh][ridx], dQr)}
        if hh == 1:          # key rows need every query's statistics: O(N^2 d) on the CPU, one head
            dKc, dVc = oracle.cols(q[0, hh], k[0, hh], v[0, hh], do[0, hh], rows, causal=True)
            errs.update(dK=_err(dk[0, hh][ridx], dKc), dV=_err(dv[0, hh][ridx], dVc))
        _say(f"  head {hh}:", {n: f"{e:.2e}" for n, e in errs.items()})
        for n, e in errs.items():
            assert e <= TOL["bf16"], f"head {hh} {n}: {e}"


@pytest.mark.parametrize("causal", [True, False])
def test_key_side_walk_uneven_heads(causal):
    """B1 H3 N = 11000 d = 64: 86 key blocks x 3 heads = 258 (head, key block) items, more than
    the GPU has CUs and with B*H not a multiple of 8, so the key side's persistent grid walks
    one GPU-wide sequence and some workgroups take two items (the lightest blocks of the last
    heads).  Sampled key rows (dK, dV) of every head, the last 300 keys among them."""
    N = 11000
    _say(f"case key-side walk, uneven heads, causal={causal}")
    q, k, v, do = make_inputs(1, 3, N, 64, "bf16", seed=110 + causal)
    o, lse, (dq, dk, dv) = _run(q, k, v, do, causal)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 127, 128, 5000, N - 300, N - 129, N - 1], rng.integers(N - 300, N, 6),
                                     rng.integers(0, N, 4)]))
    ridx = torch.as_tensor(rows)
    for hh in range(3):
        dKc, dVc = oracle.cols(q[0, hh], k[0, hh], v[0, hh], do[0, hh], rows, causal=causal)
        errs = {"dK": _err(dk[0, hh][ridx], dKc), "dV": _err(dv[0, hh][ridx], dVc)}
        _say(f"  head {hh}:", {n: f"{e:.2e}" for n, e in errs.items()})
        for n, e in errs.items():
            assert e <= TOL["bf16"], f"head {hh} {n}: {e}"
