"""Builds libmfma_rate.so, the matrix-core rate probe that bench.py reads the roofline against
(same hipcc flags as libattn.so)."""
import os
import subprocess

from .build import CSRC, FLAGS, HERE, HIPCC

PROBE_PATH = os.path.join(HERE, "libmfma_rate.so")


def build(verbose=False):
    tmp = PROBE_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, os.path.join(CSRC, "mfma_rate.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError("hipcc failed:\n" + errs)
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    print(build(verbose=True))
