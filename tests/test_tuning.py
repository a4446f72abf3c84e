"""The launch-parameter table (csrc/attn_tuning.h) and its generator (CPU only)."""
import os
import shutil
import subprocess

from exact_tiled_attention_12_amd import tune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RESULTS = os.path.join(ROOT, "profiles", "tuning_sweep_results.json")


def test_table_is_what_the_committed_sweep_gives(tmp_path):
    """Re-running the selection on the committed timings reproduces the committed table."""
    h = tmp_path / "attn_tuning.h"
    shutil.copy(tune.TABLE_H, h)
    tune.apply(RESULTS, table_path=str(h), report_path=str(tmp_path / "report.md"))
    with open(tune.TABLE_H) as f:
        assert h.read_text() == f.read()


def test_lookup_rules(tmp_path):
    """First matching entry wins, d = 0 matches any head dim, the force macros override."""
    src = tmp_path / "t.cpp"
    src.write_text('''
#include <cstdio>
#include "attn_tuning.h"
int main() {
    using namespace attn;
    const TuneEntry a = tune_lookup(kTuneDq, 128, 1, 4096), b = tune_lookup(kTuneDq, 128, 1, 4097);
    const TuneEntry c = tune_lookup(kTuneDq, 64, 1, 100), e = tune_lookup(kTuneFwdFp8, 128, 1, 16384);
    printf("%d %d %d %d %d\\n", a.slots, b.slots, c.slots, e.slots, e.key_tile);
    return 0;
}
''')
    inc = os.path.join(ROOT, "exact_tiled_attention_12_amd", "csrc")
    out = []
    for extra in ([], ["-DATTN_TUNE_FORCE_SLOTS=16", "-DATTN_TUNE_FORCE_KEY_TILE=128"]):
        exe = tmp_path / ("t" + str(len(extra)))
        subprocess.run(["g++", "-std=c++17", "-I", inc, *extra, "-o", str(exe), str(src)], check=True)
        out.append(subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split())
    # committed sweep: dQ d=128 causal takes 128 up to N = 4096 and 64 beyond; d = 64 falls to the d = 0 default
    assert out[0] == ["128", "64", "64", "32", "64"]
    assert out[1] == ["16", "16", "16", "16", "128"]
