"""bench.py's host-side readers of rocprofv3 output (no GPU): the post-warm-up kernel statistics
and the per-kernel GFX clock, on small CSV files with known answers, and the multi-GPU refusal."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(f'"{h}"' for h in header) + "\n")
        for r in rows:
            f.write(",".join(f'"{v}"' if isinstance(v, str) else str(v) for v in r) + "\n")


def test_trace_summary_skips_warmup_launches(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    # kernel A: 3 launches of 10, 20, 30 us; kernel B: 2 launches of 5, 7 us (start order scrambled)
    rows = [("void a<1>(int)", 0, 10_000), ("void b(int)", 500_000, 505_000), ("void a<1>(int)", 100_000, 120_000),
            ("void a<1>(int)", 200_000, 230_000), ("void b(int)", 600_000, 607_000)]
    _write(p, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.trace_summary(str(p), skip=1)
    out = capsys.readouterr().out.splitlines()
    a = next(l for l in out if "void a<1>" in l)
    b = next(l for l in out if "void b(int)" in l)
    assert "| 3 | 2 | 25.0 | 25.0 | 20.0 | 30.0 |" in a           # the 10 us warm-up launch left out
    assert "| 2 | 1 | 7.0 | 7.0 | 7.0 | 7.0 |" in b


def test_clock_summary_divides_by_xcds_and_duration(tmp_path, capsys):
    pre = tmp_path / "run"
    _write(str(pre) + "_agent_info.csv", ["Agent_Type", "Num_Xcc"], [("CPU", 0), ("GPU", 8)])
    # two dispatches of one kernel, 100 us each; GRBM_COUNT summed over 8 XCDs at 2.0 and 1.5 GHz
    name = "void (anonymous namespace)::k<3>(int, float*)"
    _write(str(pre) + "_kernel_trace.csv", ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [(1, name, 0, 100_000), (2, name, 200_000, 300_000)])
    _write(str(pre) + "_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"],
           [(1, name, "GRBM_COUNT", 8 * 2.0e9 * 100e-6), (2, name, "GRBM_COUNT", 8 * 1.5e9 * 100e-6),
            (2, name, "GRBM_GUI_ACTIVE", 1.0)])
    bench.clock_summary(str(pre), skip=0)
    out = capsys.readouterr().out
    assert "XCDs per dispatch: 8" in out
    line = next(l for l in out.splitlines() if "k<3>" in l)
    assert line.startswith("| `void (anonymous namespace)::k<3>` | 2 | 100.0 | 1750 |")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU only" in r.stderr
