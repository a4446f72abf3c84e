"""GPU parity of the block-sparse entry points (attn_fwd_blocksparse /
attn_bwd_blocksparse) against the fp64 oracle with the same block mask.

Bar: the dense path's (max-abs <= 1e-5 fp32, <= 2e-2 bf16, set at output
magnitudes of about 1-4), scaled with the output's magnitude where it is larger:
a query block that keeps only a ragged key block of a few keys gets gradients
of 5-20, and the bf16 roundings of P and dS are relative to the values.  So the
bar is max(tol, r * max|ref|) with r = 1e-2 (bf16, as the dense scale edge
cases use) and r = 2.5e-6 (fp32: 1e-5 at magnitude 4).  Rows that keep no key
must give exactly O = 0, LSE = -inf and dQ = 0.  Masks:
seeded random ones with an empty block row, one shared mask and one per head,
the all-kept and the lower-triangular masks (which must reproduce the dense
kernels bit for bit), the all-dropped mask, and a local + global pattern at the
size of the N = 4096 workload.  N = 9000 (71 mask blocks) crosses the kernels'
64-block mask window.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_12_amd import attn_bwd, attn_bwd_blocksparse, attn_fwd, attn_fwd_blocksparse
from exact_tiled_attention_12_amd.inputs import local_global_mask, make_inputs, random_block_mask

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}
REL = {"fp32": 2.5e-6, "bf16": 1e-2}
BLK = 128


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _cmp(name, gpu, ref, dtype):
    """max-abs error; entries that are -inf in the reference must be -inf on the GPU."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), ninf), f"{name}: -inf pattern differs"
    if not (~ninf).any():
        return 0.0
    e = float(np.abs(g[~ninf] - ref[~ninf]).max())
    bar = max(TOL[dtype], REL[dtype] * float(np.abs(ref[~ninf]).max()))
    assert e <= bar, f"{name}: {e} > {bar}"
    return e


def _run(q, k, v, do, mask, causal, grad_dtype=torch.float32):
    dev = _dev()
    qg, kg, vg, dg, mg = q.to(dev), k.to(dev), v.to(dev), do.to(dev), mask.to(dev)
    o, lse = attn_fwd_blocksparse(qg, kg, vg, mg, causal=causal)
    grads = attn_bwd_blocksparse(qg, kg, vg, o, dg, lse, mg, causal=causal, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return o, lse, grads


def _check_full(q, k, v, do, mask, causal, dtype):
    o, lse, (dq, dk, dv) = _run(q, k, v, do, mask, causal)
    O, L = oracle.fwd(q, k, v, causal=causal, block_mask=mask)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=causal, block_mask=mask)
    errs = {n: _cmp(n, g, r, dtype) for n, g, r in
            (("O", o, O), ("LSE", lse, L), ("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV))}
    _say("  max-abs errors:", {n: f"{e:.2e}" for n, e in errs.items()})
    empty = np.isneginf(L)
    if empty.any():
        assert (o.float().cpu().numpy()[empty] == 0).all() and (dq.cpu().numpy()[empty] == 0).all()
    return o, lse, (dq, dk, dv)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 80, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [130, 300, 1000])
def test_random_masks(dtype, d, causal, N):
    """Shared mask (one for every head) with an empty block row, element by element."""
    _say(f"case blocksparse dtype={dtype} d={d} causal={causal} N={N}")
    T = (N + BLK - 1) // BLK
    q, k, v, do = make_inputs(1, 2, N, d, dtype, seed=N + d + causal)
    mask = random_block_mask(T, 0.55, seed=N * 7 + d, empty_rows=(T // 2,))
    _check_full(q, k, v, do, mask, causal, dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_per_head_masks(causal):
    _say(f"case blocksparse per-head masks causal={causal}")
    B, H, N, d = 2, 3, 700, 128
    T = (N + BLK - 1) // BLK
    q, k, v, do = make_inputs(B, H, N, d, "bf16", seed=21 + causal)
    mask = random_block_mask(T, 0.5, seed=99, lead=(B, H))
    mask[0, 1, 2] = 0                                     # an empty block row in one head only
    _check_full(q, k, v, do, mask, causal, "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 80), ("fp32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_all_kept_and_lower_triangle_match_dense_bitwise(dtype, d, causal):
    """Same tiles in the same order as the dense kernels: identical bits (fp32 dQ aside, see below).
    d = 80 takes the row sum on the matrix core (padding rows of O^T) in both forward kernels."""
    _say(f"case blocksparse all-kept dtype={dtype} d={d} causal={causal}")
    dev = _dev()
    N = 777
    T = (N + BLK - 1) // BLK
    q, k, v, do = (t.to(dev) for t in make_inputs(2, 2, N, d, dtype, seed=8))
    o, lse = attn_fwd(q, k, v, causal=causal)
    grads = attn_bwd(q, k, v, o, do, lse, causal=causal)
    masks = [torch.ones(T, T, dtype=torch.uint8)]
    if causal:
        masks.append(torch.tril(torch.ones(T, T, dtype=torch.uint8)))
    for m in masks:
        m = m.to(dev)
        o2, lse2 = attn_fwd_blocksparse(q, k, v, m, causal=causal)
        grads2 = attn_bwd_blocksparse(q, k, v, o2, do, lse2, m, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        # fp32 inputs sum dQ with float atomics, whose order varies from run to run
        if dtype == "fp32":
            assert (grads[0] - grads2[0]).abs().max().item() <= 1e-6
        else:
            assert torch.equal(grads[0], grads2[0])
        assert torch.equal(grads[1], grads2[1]) and torch.equal(grads[2], grads2[2])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_all_dropped(dtype):
    _say(f"case blocksparse all-dropped dtype={dtype}")
    dev = _dev()
    N = 260
    T = (N + BLK - 1) // BLK
    q, k, v, do = (t.to(dev) for t in make_inputs(1, 2, N, 64, dtype, seed=2))
    m = torch.zeros(T, T, dtype=torch.uint8, device=dev)
    o, lse = attn_fwd_blocksparse(q, k, v, m, causal=False)
    dq, dk, dv = attn_bwd_blocksparse(q, k, v, o, do, lse, m, causal=False)
    torch.cuda.synchronize()
    assert (o == 0).all() and torch.isneginf(lse).all()
    assert (dq == 0).all() and (dk == 0).all() and (dv == 0).all()


def test_bf16_gradients_option():
    _say("case blocksparse bf16 grads")
    N, d = 520, 128
    T = (N + BLK - 1) // BLK
    q, k, v, do = make_inputs(1, 2, N, d, "bf16", seed=31)
    mask = random_block_mask(T, 0.6, seed=5, empty_rows=(1,))
    o, lse, grads = _run(q, k, v, do, mask, True, grad_dtype=torch.bfloat16)
    dQ, dK, dV = oracle.bwd(q, k, v, do, causal=True, block_mask=mask)
    for n, g, r in (("dQ", grads[0], dQ), ("dK", grads[1], dK), ("dV", grads[2], dV)):
        assert g.dtype == torch.bfloat16
        _cmp(n, g, r, "bf16")


def _sampled(q, k, v, do, mask, causal, o, lse, dq, dk, dv, heads, rows):
    for (b, h) in heads:
        m = mask if mask.dim() == 2 else mask[b, h]
        Or, Lr, dQr = oracle.rows(q[b, h], k[b, h], v[b, h], do[b, h], rows, causal=causal, block_mask=m)
        dKc, dVc = oracle.cols(q[b, h], k[b, h], v[b, h], do[b, h], rows, causal=causal, block_mask=m)
        ridx = torch.as_tensor(rows)
        errs = {n: _cmp(n, g[b, h][ridx], r, "bf16") for n, g, r in
                (("O", o, Or), ("LSE", lse, Lr), ("dQ", dq, dQr), ("dK", dk, dKc), ("dV", dv, dVc))}
        _say(f"  head ({b},{h}):", {n: f"{e:.2e}" for n, e in errs.items()})


def test_local_global_at_workload_size():
    """B4 H16 N4096 d128 causal with a local (4 blocks) + global (1 block) mask, sampled rows/keys."""
    _say("case blocksparse local+global N=4096")
    B, H, N, d = 4, 16, 4096, 128
    q, k, v, do = make_inputs(B, H, N, d, "bf16", seed=3)
    mask = local_global_mask(N // BLK, 4, 1)
    o, lse, (dq, dk, dv) = _run(q, k, v, do, mask, True)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 127, 128, 1000, 2047, N - 1], rng.integers(0, N, 20)]))
    _sampled(q, k, v, do, mask, True, o, lse, dq, dk, dv, [(0, 0), (3, 15)], rows)


@pytest.mark.parametrize("causal", [False, True])
def test_beyond_one_mask_window(causal):
    """N = 9000: 71 mask blocks, so the kernels' 64-block window of the mask is reloaded."""
    _say(f"case blocksparse N=9000 causal={causal}")
    N, d = 9000, 64
    T = (N + BLK - 1) // BLK
    q, k, v, do = make_inputs(1, 2, N, d, "bf16", seed=40 + causal)
    mask = random_block_mask(T, 0.15, seed=13, lead=(1, 2))
    mask[..., 70, :] = 0
    mask[..., 70, 69] = 1                 # the last block row keeps one block beyond the first window
    mask[..., 66, :64] = 0                # and block row 66 keeps only blocks of the second window
    o, lse, (dq, dk, dv) = _run(q, k, v, do, mask, causal)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 64 * 128, 66 * 128 + 5, 8300, N - 1], rng.integers(0, N, 12)]))
    _sampled(q, k, v, do, mask, causal, o, lse, dq, dk, dv, [(0, 0), (0, 1)], rows)
