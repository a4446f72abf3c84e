"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

Every request below fails validation, which the library performs before its
first HIP call; the pointers are never dereferenced.
"""
import ctypes
import math
import os
import re

import pytest

from exact_tiled_attention_12_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p(0x10000)          # non-null, 16-byte aligned, never touched
MIS = ctypes.c_void_p(0x10008)        # misaligned
NUL = ctypes.c_void_p(0)


def _declared_functions():
    with open(os.path.join(ROOT, "include", "attn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:attn_status|size_t|const char\*|int)\s+(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert set(_declared_functions()) == set(attn.EXPORTED)


@pytest.mark.parametrize("name", _declared_functions())
def test_library_exports_symbol(name):
    assert hasattr(attn.lib(), name)


def fwd(*, dt=1, B=1, H=1, N=16, d=64, scale=0.125, causal=0, q=P, o=P, lse=P):
    return attn.lib().attn_fwd(q, P, P, dt, B, H, N, d, scale, causal, o, lse, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(d=96), attn.ATTN_EUNSUPPORTED),
    (dict(d=32), attn.ATTN_EUNSUPPORTED),
    (dict(d=0), attn.ATTN_EINVAL),
    (dict(N=0), attn.ATTN_EINVAL),
    (dict(B=0), attn.ATTN_EINVAL),
    (dict(H=-1), attn.ATTN_EINVAL),
    (dict(dt=2), attn.ATTN_EINVAL),
    (dict(scale=math.nan), attn.ATTN_EINVAL),
    (dict(scale=math.inf), attn.ATTN_EINVAL),
    (dict(causal=2), attn.ATTN_EINVAL),
    (dict(q=NUL), attn.ATTN_EINVAL),
    (dict(q=MIS), attn.ATTN_EINVAL),
    (dict(o=NUL), attn.ATTN_EINVAL),
    (dict(lse=MIS), attn.ATTN_EINVAL),
    (dict(B=1024, H=1024, N=1024, d=64), attn.ATTN_EINVAL),    # B*H*ceil(N/128) >= 2^23 (grid limit)
    (dict(B=1, H=1, N=1 << 22, d=128), attn.ATTN_EINVAL),      # one head's fp32 rows >= 2 GiB
])
def test_fwd_rejects_before_launch(kw, expect):
    assert fwd(**kw) == expect


def test_bwd_rejects_before_launch():
    L = attn.lib()
    ws = L.attn_bwd_workspace_bytes(1, 1, 16, 64, attn.ATTN_F32)
    assert ws == 256
    args = lambda d=64, wsb=ws, g=attn.ATTN_F32, w=P, dt=attn.ATTN_BF16: (
        P, P, P, P, P, P, dt, 1, 1, 16, d, 0.125, 1, P, P, P, g, w, ctypes.c_size_t(wsb), None)
    assert L.attn_bwd(*args(wsb=ws - 1)) == attn.ATTN_EINVAL
    assert L.attn_bwd(*args(d=100)) == attn.ATTN_EUNSUPPORTED
    assert L.attn_bwd(*args(g=5)) == attn.ATTN_EINVAL
    assert L.attn_bwd(*args(w=NUL)) == attn.ATTN_EINVAL
    assert L.attn_bwd(*args(dt=attn.ATTN_F32, g=attn.ATTN_BF16)) == attn.ATTN_EUNSUPPORTED
    assert L.attn_bwd_main(P, P, P, P, P, P, 1, 1, 1, 16, 64, math.nan, 0, P, P, P, None) == attn.ATTN_EINVAL
    assert L.attn_bwd_preprocess(P, MIS, 1, 1, 1, 16, 64, P, None) == attn.ATTN_EINVAL
    # the split key-side / query-side passes exist for bf16 inputs only
    assert L.attn_bwd_dkdv(P, P, P, P, P, P, attn.ATTN_F32, 1, 1, 16, 64, 0.1, 0, P, P, None) == attn.ATTN_EUNSUPPORTED
    assert L.attn_bwd_dq(P, P, P, P, P, P, attn.ATTN_F32, 1, 1, 16, 64, 0.1, 0, P, None) == attn.ATTN_EUNSUPPORTED
    assert L.attn_bwd_dq(P, P, P, P, P, NUL, attn.ATTN_BF16, 1, 1, 16, 64, 0.1, 0, P, None) == attn.ATTN_EINVAL
    # dQ with the preprocess folded in: O (4th) and D (an output here) are checked like the rest
    dq_d = lambda o=P, D=P, dt=attn.ATTN_BF16, d=64: L.attn_bwd_dq_d(P, P, P, o, P, P, dt, 1, 1, 16, d, 0.1, 0, D, P,
                                                                     None)
    assert dq_d(dt=attn.ATTN_F32) == attn.ATTN_EUNSUPPORTED
    assert dq_d(o=MIS) == attn.ATTN_EINVAL
    assert dq_d(o=NUL) == attn.ATTN_EINVAL
    assert dq_d(D=NUL) == attn.ATTN_EINVAL
    assert dq_d(d=96) == attn.ATTN_EUNSUPPORTED


def test_blocksparse_rejects_bad_masks_before_launch():
    L = attn.lib()
    M = ctypes.c_void_p(0x20001)           # byte mask: no alignment needed, never read here
    fwd = lambda mask=M, heads=1, B=2, H=3, d=64, **kw: L.attn_fwd_blocksparse(
        P, P, P, attn.ATTN_BF16, B, H, 300, d, 0.125, kw.get("causal", 1), mask, heads, P, P, None)
    assert fwd(mask=NUL) == attn.ATTN_EINVAL
    assert fwd(heads=0) == attn.ATTN_EINVAL
    assert fwd(heads=5) == attn.ATTN_EINVAL                  # neither 1 nor B*H = 6
    assert fwd(heads=6, d=96) == attn.ATTN_EUNSUPPORTED
    assert fwd(heads=6, causal=2) == attn.ATTN_EINVAL
    ws = L.attn_bwd_workspace_bytes(2, 3, 300, 64, attn.ATTN_F32)
    bwd = lambda mask=M, heads=1, wsb=ws: L.attn_bwd_blocksparse(
        P, P, P, P, P, P, attn.ATTN_BF16, 2, 3, 300, 64, 0.125, 0, mask, heads, P, P, P, attn.ATTN_F32, P,
        ctypes.c_size_t(wsb), None)
    assert bwd(mask=NUL) == attn.ATTN_EINVAL
    assert bwd(heads=7) == attn.ATTN_EINVAL
    assert bwd(heads=6, wsb=ws - 1) == attn.ATTN_EINVAL


def test_fp8_rejects_before_launch():
    L = attn.lib()
    f = lambda q=P, d=128, sq=1.0, scale=0.1, causal=0: L.attn_fwd_fp8(q, P, P, sq, 1.0, 1.0, 1, 2, 64, d, scale,
                                                                       causal, P, P, None)
    assert f(d=80) == attn.ATTN_EUNSUPPORTED          # 64-byte contraction steps: d = 64 or 128
    assert f(d=96) == attn.ATTN_EUNSUPPORTED
    assert f(sq=math.nan) == attn.ATTN_EINVAL
    assert f(sq=math.inf) == attn.ATTN_EINVAL
    assert f(scale=math.nan) == attn.ATTN_EINVAL
    assert f(causal=3) == attn.ATTN_EINVAL
    assert f(q=MIS) == attn.ATTN_EINVAL
    assert f(q=NUL) == attn.ATTN_EINVAL


def test_noalloc_rejects_before_launch():
    L = attn.lib()
    f = lambda B=1, H=2, N=64, d=128, q=P, dt=attn.ATTN_BF16: L.attn_bwd_noalloc(
        q, P, P, P, P, P, dt, B, H, N, d, 0.1, 1, P, P, P, attn.ATTN_F32, None)
    # more rows than the static scratch holds: rejected before any HIP call
    assert f(B=1, H=4, N=attn.NOALLOC_MAX_ROWS // 4 + 1, d=64) == attn.ATTN_ENOSPACE
    assert f(d=96) == attn.ATTN_EUNSUPPORTED
    assert f(N=0) == attn.ATTN_EINVAL


def test_workspace_sizes():
    L = attn.lib()
    rows = 4 * 16 * 4096
    for g in (attn.ATTN_F32, attn.ATTN_BF16):       # D only, whatever the gradients' dtype
        assert L.attn_bwd_workspace_bytes(4, 16, 4096, 128, g) == rows * 4
        assert L.attn_bwd_workspace_bytes(1, 1, 3, 64, g) == 256
        assert L.attn_bwd_workspace_bytes(0, 16, 4096, 128, g) == 0
    assert L.attn_bwd_workspace_bytes(1, 1, 3, 64, 7) == 0       # not a dtype
    # more than 2^31 elements in all: valid (heads are addressed with 64-bit offsets)
    assert L.attn_bwd_workspace_bytes(1, 4097, 4096, 128, attn.ATTN_F32) == 4097 * 4096 * 4
    assert fwd(B=1, H=4097, N=4096, d=128, q=MIS) == attn.ATTN_EINVAL      # reaches the pointer checks


# ---- the Python binding checks every tensor's shape and dtype before it touches a device ----
def _t(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case", ["k_shape", "v_dtype", "out_shape", "lse_dtype", "lse_shape"])
def test_binding_rejects_mismatched_forward_buffers(case):
    import torch
    q = _t((1, 2, 40, 64))
    kw = dict(k=_t((1, 2, 40, 64)), v=_t((1, 2, 40, 64)))
    extra = {}
    if case == "k_shape":
        kw["k"] = _t((1, 2, 41, 64))
    elif case == "v_dtype":
        kw["v"] = _t((1, 2, 40, 64), torch.float32)
    elif case == "out_shape":
        extra["out"] = _t((1, 2, 40, 80))
    elif case == "lse_dtype":
        extra["lse"] = _t((1, 2, 40), torch.bfloat16)
    else:
        extra["lse"] = _t((1, 2, 41), torch.float32)
    with pytest.raises(ValueError, match="must"):
        attn.attn_fwd(q, kw["k"], kw["v"], **extra)


@pytest.mark.parametrize("case", ["dq_dtype", "dk_shape", "do_dtype", "lse_shape", "workspace_small", "grad_dtype"])
def test_binding_rejects_mismatched_backward_buffers(case):
    import torch
    shp = (1, 2, 40, 64)
    q, k, v, o, do = (_t(shp) for _ in range(5))
    lse = _t(shp[:-1], torch.float32)
    kw = {}
    if case == "dq_dtype":
        kw["dq"] = _t(shp, torch.bfloat16)           # default gradients are fp32
    elif case == "dk_shape":
        kw["dk"] = _t((1, 2, 40, 32), torch.float32)
    elif case == "do_dtype":
        do = _t(shp, torch.float32)
    elif case == "lse_shape":
        lse = _t((1, 2, 39), torch.float32)
    elif case == "workspace_small":
        kw["workspace"] = _t((16,), torch.uint8)
    else:
        kw["grad_dtype"] = torch.float16
    with pytest.raises((ValueError, TypeError), match="must"):
        attn.attn_bwd(q, k, v, o, do, lse, **kw)


def test_binding_rejects_mismatched_split_backward_buffers():
    import torch
    shp = (1, 2, 40, 64)
    q, k, v, o, do = (_t(shp) for _ in range(5))
    lse, D = _t(shp[:-1], torch.float32), _t(shp[:-1], torch.float32)
    with pytest.raises(ValueError, match="must"):
        attn.attn_bwd_dkdv(q, k, v, do, lse, _t(shp[:-1], torch.bfloat16))
    with pytest.raises(ValueError, match="must"):
        attn.attn_bwd_dq(q, k, v, do, lse, D, dq=_t(shp, torch.bfloat16))
    with pytest.raises(ValueError, match="must"):
        attn.attn_bwd_dq_d(q, k, v, _t((1, 2, 40, 128)), do, lse)
    with pytest.raises(ValueError, match="must"):
        attn.attn_bwd_main(q, k, v, do, lse, D, dv=_t((1, 1, 40, 64), torch.float32))
    with pytest.raises(ValueError, match="must"):
        attn.attn_bwd_preprocess(o, _t((1, 2, 40, 80)))


def test_status_strings():
    L = attn.lib()
    for s in range(5):
        assert L.attn_status_str(s)
    assert L.attn_status_str(99) == b"unknown status"
    assert L.attn_last_hip_error() == 0


def _probe_lib():
    from exact_tiled_attention_12_amd.build_probe import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        pytest.fail(f"{PROBE_PATH} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(PROBE_PATH)
    L.mfma_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.mfma_rate_probe.restype = ctypes.c_int
    return L


def test_probe_header_matches_library():
    with open(os.path.join(ROOT, "include", "mfma_rate.h")) as f:
        declared = re.findall(r"^\s*int\s+(\w+)\s*\(", f.read(), re.M)
    assert declared == ["mfma_rate_probe"]
    assert hasattr(_probe_lib(), "mfma_rate_probe")


@pytest.mark.parametrize("wg,iters,mix,out,stamps", [(0, 1, 0, P, P), (1, 0, 0, P, P), (1, 1, -1, P, P), (1, 1, 4, P, P),
                                                   (1, 1, 0, NUL, P), (1, 1, 0, P, NUL)])
def test_probe_rejects_before_launch(wg, iters, mix, out, stamps):
    assert _probe_lib().mfma_rate_probe(wg, iters, mix, out, stamps, None) == 1


def test_prepare_checks_like_the_call_and_leaves_no_recording():
    import torch
    q = _t((1, 2, 40, 64))
    with pytest.raises(ValueError, match="must"):
        attn.prepare(attn.attn_fwd, q, _t((1, 2, 41, 64)), q)
    assert attn._recording is None
    with pytest.raises(ValueError, match="GPU"):
        attn.prepare(attn.attn_fwd, q, q, q, out=torch.zeros_like(q))
    assert attn._recording is None
