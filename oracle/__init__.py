"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports, calls or loads it, and the two share no code.

This module is argument marshalling around ``attn_oracle.c``: it converts
inputs to contiguous float64 numpy arrays, loops over leading (batch, head)
dimensions and calls the C functions one head at a time.  All arithmetic is in
the C file, which cites the passages it follows.
"""
import ctypes
import os

import numpy as np

from .build import LIB_PATH, build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        # ATTN_ORACLE_LIB: another build of attn_oracle.c (the mutation test of the pins
        # loads deliberately broken copies this way, in subprocesses of its own)
        path = os.environ.get("ATTN_ORACLE_LIB", LIB_PATH)
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            _build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        L, D, I, M = ctypes.c_long, ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        lib.oracle_fwd.argtypes = [dp, dp, dp, L, L, D, I, M, L, dp, dp, dp]
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, L, L, D, I, M, L, dp, dp, dp, dp, dp]
        lib.oracle_fwd_online.argtypes = [dp, dp, dp, L, L, D, I, M, L, L, L, dp, dp]
        lib.oracle_rows.argtypes = [dp, dp, dp, dp, L, L, D, I, M, L, lp, L, dp, dp, dp]
        lib.oracle_cols.argtypes = [dp, dp, dp, dp, L, L, D, I, M, L, lp, L, dp, dp]
        for f in (lib.oracle_fwd, lib.oracle_bwd, lib.oracle_fwd_online, lib.oracle_rows,
                  lib.oracle_cols):
            f.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _f64(x):
    if hasattr(x, "detach"):                       # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with code {rc}")


def _heads(shape):
    if len(shape) < 2:
        raise ValueError("expected [..., N, d]")
    return int(np.prod(shape[:-2], dtype=np.int64)), shape[-2], shape[-1]


MASK_BLOCK = 128     # the block edge the kernels' masks use; the oracle takes any


def _masks(block_mask, lead, N, block):
    """Per-head uint8 [T, T] masks (T = ceil(N / block)) from None, one [T, T] mask for
    every head, or masks with the inputs' leading dimensions: a list of nh arrays or None."""
    nh = int(np.prod(lead, dtype=np.int64))
    if block_mask is None:
        return [None] * nh
    m = block_mask.detach().cpu().numpy() if hasattr(block_mask, "detach") else np.asarray(block_mask)
    m = (m != 0).astype(np.uint8)
    T = (N + block - 1) // block
    if m.shape == (T, T):
        m = np.broadcast_to(m, (nh, T, T))
    elif m.shape == tuple(lead) + (T, T):
        m = m.reshape(nh, T, T)
    else:
        raise ValueError(f"block mask of shape {m.shape}, expected ({T}, {T}) or {tuple(lead) + (T, T)}")
    return [np.ascontiguousarray(m[h]) for h in range(nh)]


def _mp(m):
    return None if m is None else m.ctypes.data_as(ctypes.c_void_p)


def default_scale(d):
    """1/sqrt(d): 'IO-4 FlashAttention' problem setup; 'Flash Attention-3' code example."""
    return 1.0 / float(np.sqrt(d))


def num_threads():
    return _load().oracle_num_threads()


def fwd(q, k, v, scale=None, causal=False, block_mask=None, block=MASK_BLOCK):
    """Naive forward with explicit S and P.  Returns (O, LSE) as float64."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nh, N, d = _heads(q.shape)
    if scale is None:
        scale = default_scale(d)
    ms = _masks(block_mask, q.shape[:-2], N, block)
    qh, kh, vh = q.reshape(nh, N, d), k.reshape(nh, N, d), v.reshape(nh, N, d)
    O = np.empty((nh, N, d))
    LSE = np.empty((nh, N))
    for h in range(nh):
        _check(lib.oracle_fwd(_ptr(qh[h]), _ptr(kh[h]), _ptr(vh[h]), N, d, float(scale),
                              int(bool(causal)), _mp(ms[h]), int(block), _ptr(O[h]), _ptr(LSE[h]), None),
               "oracle_fwd")
    return O.reshape(q.shape), LSE.reshape(q.shape[:-1])


def fwd_probs(q, k, v, scale=None, causal=False, block_mask=None, block=MASK_BLOCK):
    """Single head [N, d]: returns (O, LSE, P) with the explicit N x N P."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    m = _masks(block_mask, (), N, block)[0]
    O, LSE, P = np.empty((N, d)), np.empty(N), np.empty((N, N))
    _check(lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), N, d, float(scale), int(bool(causal)), _mp(m), int(block),
                          _ptr(O), _ptr(LSE), _ptr(P)), "oracle_fwd")
    return O, LSE, P


def bwd(q, k, v, do, scale=None, causal=False, return_D=False, block_mask=None, block=MASK_BLOCK):
    """Naive backward.  Returns (dQ, dK, dV) [+ (D, D2) if return_D]."""
    lib = _load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    nh, N, d = _heads(q.shape)
    if scale is None:
        scale = default_scale(d)
    ms = _masks(block_mask, q.shape[:-2], N, block)
    r = lambda a: a.reshape(nh, N, d)
    qh, kh, vh, gh = r(q), r(k), r(v), r(do)
    dQ, dK, dV = np.empty((nh, N, d)), np.empty((nh, N, d)), np.empty((nh, N, d))
    D, D2 = np.empty((nh, N)), np.empty((nh, N))
    for h in range(nh):
        _check(lib.oracle_bwd(_ptr(qh[h]), _ptr(kh[h]), _ptr(vh[h]), _ptr(gh[h]), N, d,
                              float(scale), int(bool(causal)), _mp(ms[h]), int(block), _ptr(dQ[h]), _ptr(dK[h]),
                              _ptr(dV[h]), _ptr(D[h]), _ptr(D2[h])), "oracle_bwd")
    out = (dQ.reshape(q.shape), dK.reshape(q.shape), dV.reshape(q.shape))
    if return_D:
        out = out + (D.reshape(q.shape[:-1]), D2.reshape(q.shape[:-1]))
    return out


def fwd_online(q, k, v, scale=None, causal=False, Br=2, Bc=2, block_mask=None, block=MASK_BLOCK):
    """Forward by the tiled online recurrence.  Returns (O, LSE)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    nh, N, d = _heads(q.shape)
    if scale is None:
        scale = default_scale(d)
    ms = _masks(block_mask, q.shape[:-2], N, block)
    qh, kh, vh = q.reshape(nh, N, d), k.reshape(nh, N, d), v.reshape(nh, N, d)
    O = np.empty((nh, N, d))
    LSE = np.empty((nh, N))
    for h in range(nh):
        _check(lib.oracle_fwd_online(_ptr(qh[h]), _ptr(kh[h]), _ptr(vh[h]), N, d, float(scale),
                                     int(bool(causal)), _mp(ms[h]), int(block), int(Br), int(Bc), _ptr(O[h]),
                                     _ptr(LSE[h])), "oracle_fwd_online")
    return O.reshape(q.shape), LSE.reshape(q.shape[:-1])


def rows(q, k, v, do, row_idx, scale=None, causal=False, block_mask=None, block=MASK_BLOCK):
    """Single head [N, d]: (O, LSE, dQ) of the given query rows (dQ None if do is None)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    do = None if do is None else _f64(do)
    N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    idx = np.ascontiguousarray(np.asarray(row_idx, dtype=np.int64))
    n = idx.shape[0]
    O, LSE = np.empty((n, d)), np.empty(n)
    dQ = None if do is None else np.empty((n, d))
    m = _masks(block_mask, (), N, block)[0]
    _check(lib.oracle_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(do), N, d, float(scale),
                           int(bool(causal)), _mp(m), int(block), idx.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                           n, _ptr(O), _ptr(LSE), _ptr(dQ)), "oracle_rows")
    return O, LSE, dQ


def cols(q, k, v, do, col_idx, scale=None, causal=False, block_mask=None, block=MASK_BLOCK):
    """Single head [N, d]: (dK, dV) of the given key rows."""
    lib = _load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    idx = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int64))
    n = idx.shape[0]
    dK, dV = np.empty((n, d)), np.empty((n, d))
    m = _masks(block_mask, (), N, block)[0]
    _check(lib.oracle_cols(_ptr(q), _ptr(k), _ptr(v), _ptr(do), N, d, float(scale),
                           int(bool(causal)), _mp(m), int(block), idx.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                           n, _ptr(dK), _ptr(dV)), "oracle_cols")
    return dK, dV
