"""The autograd wrapper (flash_attention / FlashAttentionFn) in a training step.

A small multi-head self-attention layer (fp64 projections, attention in the
kernels' dtype) takes one SGD step twice: once on the GPU with the kernels, once
on the CPU with the oracle's forward and backward in place of the kernels.  The
two graphs are identical apart from the attention itself: both round Q, K, V,
O and dO to the attention dtype at the same points, so the only difference is
the kernels' arithmetic against the fp64 oracle.

Bar: the kernels' outputs meet 1e-5 (fp32) / 2e-2 (bf16) absolute at magnitudes
of about 1-4 (the parity tests); a weight gradient sums B*N such rows times
activations of magnitude ~1, so its error is compared relative to its largest
entry: 1e-4 for fp32 and 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_12_amd import attn
from exact_tiled_attention_12_amd.autograd import FlashAttentionFn, flash_attention


class OracleAttention(torch.autograd.Function):
    """The oracle's forward/backward as an autograd function (CPU, test-side only).

    Outputs and gradients are returned in the inputs' dtype, as the kernels do."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        ctx.save_for_backward(q, k, v)
        ctx.scale, ctx.causal = scale, causal
        O, _ = oracle.fwd(q, k, v, scale=scale, causal=causal)
        return torch.from_numpy(O).to(q.dtype)

    @staticmethod
    def backward(ctx, do):
        q, k, v = ctx.saved_tensors
        dQ, dK, dV = oracle.bwd(q, k, v, do.to(q.dtype), scale=ctx.scale, causal=ctx.causal)
        return (torch.from_numpy(dQ).to(q.dtype), torch.from_numpy(dK).to(q.dtype),
                torch.from_numpy(dV).to(q.dtype), None, None)


def _layer(params, x, H, dt, causal, attention):
    """y = MHA(x): per-head [B, H, N, d] views of the projections (non-contiguous)."""
    Wq, Wk, Wv, Wo = params
    B, N, dm = x.shape
    d = dm // H
    heads = lambda t: t.view(B, N, H, d).transpose(1, 2)
    q, k, v = heads(x @ Wq), heads(x @ Wk), heads(x @ Wv)
    o = attention(q.to(dt), k.to(dt), v.to(dt), d ** -0.5, causal).to(torch.float64)
    return o.transpose(1, 2).reshape(B, N, dm) @ Wo


def _sgd_step(params, x, target, H, dt, causal, attention, lr=0.5):
    ps = [p.detach().clone().requires_grad_(True) for p in params]
    loss = ((_layer(ps, x, H, dt, causal, attention) - target) ** 2).mean()
    loss.backward()
    grads = [p.grad.detach().clone() for p in ps]
    with torch.no_grad():
        new = [p - lr * g for p, g in zip(ps, grads)]
        loss2 = ((_layer(new, x, H, dt, causal, attention) - target) ** 2).mean()
    return float(loss.detach()), grads, new, float(loss2)


def _setup(B, N, H, d, seed):
    g = torch.Generator().manual_seed(seed)
    dm = H * d
    x = torch.randn(B, N, dm, generator=g, dtype=torch.float64)
    target = torch.randn(B, N, dm, generator=g, dtype=torch.float64)
    params = [torch.randn(dm, dm, generator=g, dtype=torch.float64) * dm ** -0.5 for _ in range(4)]
    return x, target, params


# ---------------------------------------------------------------- CPU checks

def test_oracle_attention_gradient_matches_finite_differences():
    """The test-side oracle autograd function against central differences (fp64, tiny)."""
    g = torch.Generator().manual_seed(4)
    q, k, v = (torch.randn(1, 2, 5, 3, generator=g, dtype=torch.float64, requires_grad=True) for _ in range(3))
    for causal in (False, True):
        assert torch.autograd.gradcheck(lambda a, b, c: OracleAttention.apply(a, b, c, 0.7, causal), (q, k, v),
                                        eps=1e-6, atol=1e-8, rtol=1e-6)


def test_wrapper_refuses_cpu_tensors():
    """No CPU fallback: tensors that are not on a GPU are rejected."""
    q = torch.randn(1, 1, 8, 64)
    with pytest.raises(ValueError, match="GPU"):
        flash_attention(q, q, q)


# ---------------------------------------------------------------- GPU checks

def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _relerr(a, b):
    a, b = a.detach().cpu().double(), b.detach().cpu().double()
    return float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))


@pytest.mark.gpu
@pytest.mark.parametrize("dt,tol", [(torch.float32, 1e-4), (torch.bfloat16, 2e-2)])
@pytest.mark.parametrize("H,d", [(2, 128), (3, 80), (4, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_training_step_matches_oracle(dt, tol, H, d, causal):
    dev = _dev()
    print(f"case training step dt={dt} H={H} d={d} causal={causal}", flush=True)
    x, target, params = _setup(2, 150, H, d, seed=H * 100 + d + causal)
    ref = _sgd_step(params, x, target, H, dt, causal, OracleAttention.apply)
    gpu = _sgd_step([p.to(dev) for p in params], x.to(dev), target.to(dev), H, dt, causal,
                    lambda q, k, v, s, c: flash_attention(q, k, v, scale=s, causal=c))
    torch.cuda.synchronize()
    errs = [_relerr(g, r) for g, r in zip(gpu[1], ref[1])] + [_relerr(p, r) for p, r in zip(gpu[2], ref[2])]
    print("  loss", gpu[0], ref[0], "after step", gpu[3], ref[3], "max rel err", f"{max(errs):.2e}", flush=True)
    assert abs(gpu[0] - ref[0]) <= tol * abs(ref[0])
    assert abs(gpu[3] - ref[3]) <= tol * abs(ref[3])
    assert max(errs) <= tol
    assert gpu[3] < gpu[0]                      # the step lowered the loss


@pytest.mark.gpu
def test_wrapper_returns_input_dtype_and_saves_no_quadratic_state():
    dev = _dev()
    print("case wrapper dtypes", flush=True)
    q, k, v = (torch.randn(1, 2, 300, 128, device=dev, dtype=torch.bfloat16, requires_grad=True) for _ in range(3))
    o = flash_attention(q, k, v, causal=True)
    assert o.dtype == torch.bfloat16 and o.shape == q.shape
    saved = o.grad_fn.saved_tensors
    assert max(t.numel() for t in saved) == q.numel()           # inputs and O; LSE is B*H*N
    o.float().sum().backward()
    assert q.grad.dtype == torch.bfloat16 and k.grad.dtype == torch.bfloat16 and v.grad.dtype == torch.bfloat16
    # the same gradients as the explicit calls through the C ABI
    o2, lse = attn.attn_fwd(q.detach(), k.detach(), v.detach(), causal=True)
    dq, dk, dv = attn.attn_bwd(q.detach(), k.detach(), v.detach(), o2, torch.ones_like(o2), lse, causal=True,
                               grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)
    assert isinstance(o.grad_fn, FlashAttentionFn._backward_cls)
    assert np.isfinite(q.grad.float().cpu().numpy()).all()
