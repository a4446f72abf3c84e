"""attn_bwd_noalloc (the allocation-free backward) against attn_bwd, through the C ABI.

The two entry points run the same kernels; only where the D rows live differs (the
library's static device scratch instead of a caller workspace), so their outputs
must agree bit for bit, except fp32-input dQ, which the fp32 kernel accumulates with
float atomics in no fixed order (held to 1e-6 instead, a tenth of the fp32 bar).
Two calls in a row, the second with a smaller input, show that the shared scratch
carries nothing from one call into the next.  Also checked:
a request past the scratch's limit is rejected before anything is launched.
"""
import pytest
import torch

from exact_tiled_attention_12_amd import attn_bwd, attn_bwd_noalloc, attn_fwd
from exact_tiled_attention_12_amd.attn import ATTN_ENOSPACE, NOALLOC_MAX_ROWS, AttnError
from exact_tiled_attention_12_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _pair(B, H, N, d, dtype, causal, grad_dtype, seed):
    dev = _dev()
    q, k, v, do = (t.to(dev) for t in make_inputs(B, H, N, d, dtype, seed=seed))
    o, lse = attn_fwd(q, k, v, causal=causal)
    ref = attn_bwd(q, k, v, o, do, lse, causal=causal, grad_dtype=grad_dtype)
    got = tuple(torch.full(q.shape, float("nan"), dtype=grad_dtype, device=dev) for _ in range(3))
    attn_bwd_noalloc(q, k, v, o, do, lse, *got, causal=causal)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype,grad_dtype", [("bf16", torch.float32), ("bf16", torch.bfloat16),
                                              ("fp32", torch.float32)])
@pytest.mark.parametrize("causal", [True, False])
def test_noalloc_matches_attn_bwd_twice(dtype, grad_dtype, causal):
    print(f"case no-alloc dtype={dtype} grads={grad_dtype} causal={causal}", flush=True)
    # a larger call, then a smaller one (shorter rows, fewer heads, another head dim)
    for (B, H, N, d, seed) in ((2, 8, 1500, 128, 11), (1, 3, 333, 80, 12)):
        ref, got = _pair(B, H, N, d, dtype, causal, grad_dtype, seed)
        for n, r, g in zip(("dQ", "dK", "dV"), ref, got):
            if dtype == "fp32" and n == "dQ":
                err = float((r - g).abs().max())
                assert err <= 1e-6, f"B{B} H{H} N{N} d{d} dQ: {err} from attn_bwd"
            else:
                assert torch.equal(r, g), f"B{B} H{H} N{N} d{d} {n}: differs from attn_bwd"


def test_noalloc_rejects_more_rows_than_its_scratch():
    dev = _dev()
    N = NOALLOC_MAX_ROWS // 4 + 1                  # B * H * N = NOALLOC_MAX_ROWS + 4
    shape = (1, 4, N, 64)
    t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(shape[:-1], dtype=torch.float32, device=dev)
    g = torch.empty(shape, dtype=torch.float32, device=dev)
    with pytest.raises(AttnError) as e:
        attn_bwd_noalloc(t, t, t, t, t, lse, g, g, g)
    assert e.value.status == ATTN_ENOSPACE
