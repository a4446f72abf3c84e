"""Python binding of libattn.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h.  PyTorch supplies device
memory (tensors) and the stream (the current HIP stream of the tensors'
device).  There is no fallback: if the library is missing or the tensors are
not on a GPU, the calls raise.
"""
import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP, ATTN_ENOSPACE = 0, 1, 2, 3, 4
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = ("attn_fwd", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_d", "attn_bwd_main",
            "attn_bwd_workspace_bytes", "attn_bwd", "attn_fwd_blocksparse", "attn_bwd_blocksparse",
            "attn_fwd_fp8", "attn_bwd_noalloc", "attn_status_str", "attn_last_hip_error")
MASK_BLOCK = 128        # ATTN_MASK_BLOCK: rows and keys per block-mask entry
NOALLOC_MAX_ROWS = 4 * 1024 * 1024      # ATTN_NOALLOC_MAX_ROWS: B*H*N limit of attn_bwd_noalloc

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().attn_status_str(status).decode()
        if status == ATTN_EHIP:
            msg += f" (hipError {lib().attn_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def use_library(path):
    """Loads the library from `path` instead of the in-tree libattn.so (before the first call;
    the launch-parameter sweep times candidate builds this way)."""
    global LIB_PATH
    if _lib is not None and os.path.abspath(path) != os.path.abspath(LIB_PATH):
        raise RuntimeError("the library is already loaded")
    LIB_PATH = path


def lib():
    """Loads libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.attn_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp]
        L.attn_bwd_preprocess.argtypes = [vp, vp, i, i, i, i, i, vp, vp]
        L.attn_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp]
        L.attn_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp]
        L.attn_bwd_dq_d.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp]
        L.attn_bwd_main.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, vp]
        L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
        L.attn_bwd_workspace_bytes.restype = sz
        L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, i, vp, sz, vp]
        L.attn_fwd_blocksparse.argtypes = [vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, vp, vp]
        L.attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, vp, vp, i, vp,
                                           sz, vp]
        L.attn_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, i, i, i, i, f, i, vp, vp, vp]
        L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, i, vp]
        for name in ("attn_fwd", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dq_d", "attn_bwd_main",
                     "attn_bwd", "attn_fwd_blocksparse", "attn_bwd_blocksparse", "attn_fwd_fp8",
                     "attn_bwd_noalloc"):
            getattr(L, name).restype = i
        L.attn_status_str.argtypes = [i]
        L.attn_status_str.restype = ctypes.c_char_p
        L.attn_last_hip_error.argtypes = []
        L.attn_last_hip_error.restype = i
        _lib = L
    return _lib


def _dt(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# While prepare() runs a binding function, its C calls are recorded here instead of made, with
# every tensor whose pointer they carry (so that those buffers outlive the prepared launch).
_recording = None


def _ptr(t):
    if t is not None and _recording is not None:
        _recording[1].append(t)
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def _check_inputs(*ts):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda":
            raise ValueError("tensors must be on a GPU")
        if t.device != dev:
            raise ValueError("tensors on different devices")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, name, shape, dtype):
    """Raises unless tensor t (an argument called `name`) has exactly this shape and dtype: the
    C ABI takes raw pointers and cannot tell a wrong-sized buffer from a right one."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _expect_like_q(q, **ts):
    for name, t in ts.items():
        _expect(t, name, q.shape, q.dtype)


def _expect_rows(q, **ts):
    """fp32 [B, H, N] row statistics (LSE, D)."""
    for name, t in ts.items():
        _expect(t, name, q.shape[:-1], torch.float32)


def _workspace(workspace, need, dev):
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold at least {need} bytes")
    return workspace


def _call(name, *args):
    if _recording is not None:
        _recording[0].append((getattr(lib(), name), name, args))
        return
    st = getattr(lib(), name)(*args)
    if st != ATTN_OK:
        raise AttnError(st, name)


def prepare(fn, *args, **kwargs):
    """Checks and marshals one call of a binding function (attn_fwd, attn_bwd, attn_bwd_dq_d, ...)
    once, without launching anything, and returns (launch, result).  launch() re-issues exactly
    the C calls that fn would have made: same buffers, same scalars, same stream, status checked.
    It skips the per-call Python checks, which cost more than a short kernel runs (a loop that
    enqueues one fixed launch many times otherwise keeps the GPU waiting on the host).  result is
    what fn returned (its output tensors); launch keeps every buffer the calls use alive."""
    global _recording
    if _recording is not None:
        raise RuntimeError("prepare() does not nest")
    _recording = ([], [])
    try:
        result = fn(*args, **kwargs)
        calls, keep = _recording
    finally:
        _recording = None

    def launch():
        for f, name, cargs in calls:
            st = f(*cargs)
            if st != ATTN_OK:
                raise AttnError(st, name)
    launch.buffers = keep
    return launch, result


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O = softmax(scale Q K^T) V and LSE.  Returns (O, LSE)."""
    B, H, N, d = _shape(q)
    _dt(q)
    _expect_like_q(q, k=k, v=v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect_like_q(q, out=o)
    _expect_rows(q, lse=l)
    _check_inputs(q, k, v, o, l)
    _call("attn_fwd", _ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, N, d, float(scale), int(bool(causal)),
          _ptr(o), _ptr(l), _stream(q, stream))
    return o, l


def attn_bwd_workspace_bytes(B, H, N, d, grad_dtype=torch.float32):
    return int(lib().attn_bwd_workspace_bytes(B, H, N, d, _gdt(grad_dtype)))


def _gdt(grad_dtype):
    if grad_dtype == torch.bfloat16:
        return ATTN_BF16
    if grad_dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"gradients must be float32 or bfloat16, not {grad_dtype}")


def attn_bwd_preprocess(o, do, D=None, stream=None):
    """D = rowsum(dO o O), fp32 [B, H, N]."""
    B, H, N, d = _shape(o)
    _dt(o)
    _expect_like_q(o, do=do)
    D = torch.empty((B, H, N), dtype=torch.float32, device=o.device) if D is None else D
    _expect_rows(o, D=D)
    _check_inputs(o, do, D)
    _call("attn_bwd_preprocess", _ptr(o), _ptr(do), _dt(o), B, H, N, d, _ptr(D), _stream(o, stream))
    return D


def _grad(t, q, dtype=torch.float32, name="gradient"):
    """A caller's gradient buffer (checked: [B, H, N, d] of `dtype`), or a new one."""
    if t is None:
        return torch.empty(q.shape, dtype=dtype, device=q.device)
    _expect(t, name, q.shape, dtype)
    return t


def attn_bwd_dkdv(q, k, v, do, lse, D, scale=None, causal=False, dk=None, dv=None, stream=None):
    """dK, dV (fp32, written once).  bf16 inputs only."""
    B, H, N, d = _shape(q)
    _expect_like_q(q, k=k, v=v, do=do)
    _expect_rows(q, lse=lse, D=D)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dk, dv = _grad(dk, q), _grad(dv, q)
    _check_inputs(q, k, v, do, lse, D, dk, dv)
    _call("attn_bwd_dkdv", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(dk), _ptr(dv), _stream(q, stream))
    return dk, dv


def attn_bwd_dq(q, k, v, do, lse, D, scale=None, causal=False, dq=None, stream=None):
    """dQ (fp32, written once).  bf16 inputs only."""
    B, H, N, d = _shape(q)
    _expect_like_q(q, k=k, v=v, do=do)
    _expect_rows(q, lse=lse, D=D)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = _grad(dq, q)
    _check_inputs(q, k, v, do, lse, D, dq)
    _call("attn_bwd_dq", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(dq), _stream(q, stream))
    return dq


def attn_bwd_dq_d(q, k, v, o, do, lse, D=None, scale=None, causal=False, dq=None, stream=None):
    """(dQ, D): dQ (fp32, written once) with the preprocess folded in: D = rowsum(dO o O) is
    computed per query row, used, and returned for an attn_bwd_dkdv call.  bf16 inputs only."""
    B, H, N, d = _shape(q)
    _expect_like_q(q, k=k, v=v, o=o, do=do)
    if D is None:
        D = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _expect_rows(q, lse=lse, D=D)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = _grad(dq, q)
    _check_inputs(q, k, v, o, do, lse, D, dq)
    _call("attn_bwd_dq_d", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(D), _ptr(dq), _stream(q, stream))
    return dq, D


def attn_bwd_main(q, k, v, do, lse, D, scale=None, causal=False, dq=None, dk=None, dv=None, stream=None):
    """dQ, dK, dV (fp32, written once) given D from attn_bwd_preprocess."""
    B, H, N, d = _shape(q)
    _dt(q)
    _expect_like_q(q, k=k, v=v, do=do)
    _expect_rows(q, lse=lse, D=D)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq, dk, dv = _grad(dq, q), _grad(dk, q), _grad(dv, q)
    _check_inputs(q, k, v, do, lse, D, dq, dk, dv)
    _call("attn_bwd_main", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(D), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _stream(q, stream))
    return dq, dk, dv


def attn_bwd(q, k, v, o, do, lse, scale=None, causal=False, grad_dtype=torch.float32, workspace=None,
             dq=None, dk=None, dv=None, stream=None):
    """Full backward.  Returns (dQ, dK, dV) in grad_dtype."""
    B, H, N, d = _shape(q)
    _dt(q)
    _expect_like_q(q, k=k, v=v, o=o, do=do)
    _expect_rows(q, lse=lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gdt = _gdt(grad_dtype)
    workspace = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d, grad_dtype), q.device)
    dq, dk, dv = (_grad(t, q, grad_dtype, n) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    _check_inputs(q, k, v, o, do, lse, dq, dk, dv, workspace)
    _call("attn_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), gdt, _ptr(workspace),
          ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(q, stream))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None, causal=False, stream=None):
    """attn_bwd without a workspace: the library's static device scratch holds D, so the C call
    allocates nothing (the caller passes the gradient buffers, of one dtype: float32 or bfloat16).
    B*H*N must not exceed NOALLOC_MAX_ROWS.  Calls that overlap on one GPU race on the scratch."""
    B, H, N, d = _shape(q)
    _dt(q)
    _expect_like_q(q, k=k, v=v, o=o, do=do)
    _expect_rows(q, lse=lse)
    gdt = _gdt(dq.dtype)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, n, q.shape, dq.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_inputs(q, k, v, o, do, lse, dq, dk, dv)
    _call("attn_bwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), gdt, _stream(q, stream))
    return dq, dk, dv


def _block_mask(mask, q):
    """(uint8 device mask, mask_heads) from a [T, T] mask or a [B, H, T, T] one (nonzero = kept)."""
    B, H, N, _ = _shape(q)
    T = (N + MASK_BLOCK - 1) // MASK_BLOCK
    if mask.dtype != torch.uint8:
        raise TypeError("block mask must be uint8")
    if tuple(mask.shape) == (T, T):
        heads = 1
    elif tuple(mask.shape) == (B, H, T, T):
        heads = B * H
    else:
        raise ValueError(f"block mask must be [{T}, {T}] or [{B}, {H}, {T}, {T}]")
    return mask, heads


def attn_fwd_blocksparse(q, k, v, block_mask, scale=None, causal=False, out=None, lse=None, stream=None):
    """Forward restricted to the kept blocks of block_mask (uint8 [T, T] or [B, H, T, T],
    T = ceil(N / 128)).  Rows that keep no key get O = 0 and LSE = -inf.  Returns (O, LSE)."""
    B, H, N, d = _shape(q)
    _dt(q)
    _expect_like_q(q, k=k, v=v)
    m, heads = _block_mask(block_mask, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _expect_like_q(q, out=o)
    _expect_rows(q, lse=l)
    _check_inputs(q, k, v, o, l, m)
    _call("attn_fwd_blocksparse", _ptr(q), _ptr(k), _ptr(v), _dt(q), B, H, N, d, float(scale),
          int(bool(causal)), _ptr(m), heads, _ptr(o), _ptr(l), _stream(q, stream))
    return o, l


def attn_bwd_blocksparse(q, k, v, o, do, lse, block_mask, scale=None, causal=False, grad_dtype=torch.float32,
                         workspace=None, dq=None, dk=None, dv=None, stream=None):
    """Backward of attn_fwd_blocksparse (same mask, scale and causal flag).  Returns (dQ, dK, dV)."""
    B, H, N, d = _shape(q)
    _dt(q)
    _expect_like_q(q, k=k, v=v, o=o, do=do)
    _expect_rows(q, lse=lse)
    m, heads = _block_mask(block_mask, q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    gdt = _gdt(grad_dtype)
    workspace = _workspace(workspace, attn_bwd_workspace_bytes(B, H, N, d, grad_dtype), q.device)
    dq, dk, dv = (_grad(t, q, grad_dtype, n) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    _check_inputs(q, k, v, o, do, lse, dq, dk, dv, workspace, m)
    _call("attn_bwd_blocksparse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _dt(q), B, H, N, d,
          float(scale), int(bool(causal)), _ptr(m), heads, _ptr(dq), _ptr(dk), _ptr(dv), gdt, _ptr(workspace),
          ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(q, stream))
    return dq, dk, dv


def attn_fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale=None, causal=False, out=None, lse=None,
                 stream=None):
    """Forward on fp8 e4m3 inputs (torch.float8_e4m3fn, [B, H, N, d], d = 64 or 128) whose real values are
    descale * tensor.  Returns (O in bf16, LSE in fp32)."""
    B, H, N, d = _shape(q8)
    for t in (q8, k8, v8):
        if t.dtype != torch.float8_e4m3fn or t.shape != q8.shape:
            raise ValueError("q8, k8, v8 must be float8_e4m3fn tensors of one shape")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None else lse
    _expect(o, "out", q8.shape, torch.bfloat16)
    _expect_rows(q8, lse=l)
    _check_inputs(q8, k8, v8, o, l)
    _call("attn_fwd_fp8", _ptr(q8), _ptr(k8), _ptr(v8), float(q_descale), float(k_descale), float(v_descale),
          B, H, N, d, float(scale), int(bool(causal)), _ptr(o), _ptr(l), _stream(q8, stream))
    return o, l
