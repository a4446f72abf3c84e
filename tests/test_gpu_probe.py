"""The matrix-core rate probe (libmfma_rate.so) that bench.py reads its measured ceilings from:
its products and side work give the values they must, in every mix, and its clock stamps advance.

The probe's operands are fixed per lane (A row m, contraction k = 8 h + e: bf16(0.001 (m + 32 h + e));
B: bf16(1 - 0.01 e)), so each of its four accumulator chains ends at iters * (A B) in the 32x32
MFMA output layout, and each thread writes the sum of its chains and of its VALU chains."""
import ctypes

import numpy as np
import pytest
import torch

from exact_tiled_attention_12_amd.build_probe import PROBE_PATH

pytestmark = pytest.mark.gpu


def _lib():
    L = ctypes.CDLL(PROBE_PATH)
    L.mfma_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.mfma_rate_probe.restype = ctypes.c_int
    return L


def _bf16(x):
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def _expected(iters, mix):
    """Per thread of a 256-thread workgroup: the value the probe writes (fp64)."""
    m = np.arange(32)[:, None]
    A = np.concatenate([_bf16(0.001 * (m + 32 * h + np.arange(8)[None, :])) for h in (0, 1)], axis=1)  # 32 x 16
    B = np.tile(_bf16(1.0 - 0.01 * np.arange(8))[:, None], (2, 32))                                       # 16 x 32
    D = A @ B
    out = np.empty(256)
    for t in range(256):
        lane = t & 63
        n, h = lane % 32, lane // 32
        rows = [8 * (r // 4) + 4 * h + (r % 4) for r in range(16)]
        c = 4 * iters * D[rows, n].sum()
        x = np.float32(0.1) * np.float32(lane) + np.array([0.0, 0.25, 0.5, 0.75])
        y, z = np.zeros(4), np.zeros(4)
        if mix & 2:
            x = x.astype(np.float64)
            for _ in range(iters):
                x = np.exp2(0.5 * x - 0.75)
                y = np.maximum(y, x)
                z = z + x
        out[t] = x.sum() + y.sum() + z.sum() + c
    return out


@pytest.mark.parametrize("mix", [0, 1, 2, 3])
def test_probe_values_and_stamps(mix):
    print(f"case probe mix={mix}", flush=True)
    wg, iters = 6, 64
    dev = torch.device("cuda:0")
    out = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device=dev)
    stamps = torch.zeros(wg * 4, dtype=torch.int64, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    assert _lib().mfma_rate_probe(wg, iters, mix, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stamps.data_ptr()),
                                  ctypes.c_void_p(st)) == 0
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(wg, 256)
    exp = _expected(iters, mix)
    err = np.abs(got - exp[None, :]).max() / np.abs(exp).max()
    print(f"  max relative error {err:.2e}", flush=True)
    assert err < 1e-4
    s = stamps.cpu().numpy().reshape(wg, 4)
    assert (s[:, 1] > s[:, 0]).all() and (s[:, 3] > s[:, 2]).all()
    mhz = (s[:, 1] - s[:, 0]) / ((s[:, 3] - s[:, 2]) / 100e6) / 1e6
    print(f"  shader clock {np.median(mhz):.0f} MHz", flush=True)
    assert 100 < np.median(mhz) < 5000
