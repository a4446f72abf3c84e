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


def _table_rows():
    """The committed table's entries as (kernel, d, causal, n_max, slots, key_tile)."""
    import re
    text = open(tune.TABLE_H).read()
    body = text[text.index("kTuneTable[] = {"):text.index("// ---- generated table: end")]
    rows = []
    for m in re.finditer(r"\{(kTune\w+), (\d+), (\d), ([^,]+), (\d+), (\d+)\}", body):
        n_max = (1 << 30) if m.group(4).strip() == "1 << 30" else int(m.group(4))
        rows.append((m.group(1), int(m.group(2)), int(m.group(3)), n_max, int(m.group(5)), int(m.group(6))))
    return rows


def _expected(rows, kernel, d, causal, n):
    """The lookup rule: first entry of the kernel with d equal (or 0), the same causal flag and N <= n_max;
    otherwise slots 64, key tile 64."""
    for k, dd, c, n_max, s, kt in rows:
        if k == kernel and (dd == 0 or dd == d) and c == causal and n <= n_max:
            return s, kt
    return 64, 64


def test_lookup_rules(tmp_path):
    """First matching entry wins, d = 0 matches any head dim, the force macros override: the C++ lookup
    agrees with the rule applied to the committed table's rows."""
    rows = _table_rows()
    assert rows, "no table rows parsed"
    queries = [("kTuneDq", 128, 1, 4096), ("kTuneDq", 128, 1, 4097), ("kTuneDq", 64, 1, 100),
               ("kTuneFwdFp8", 128, 1, 16384), ("kTuneDkdv", 80, 1, 2048), ("kTuneFwdBf16", 128, 0, 4096),
               ("kTuneDkdv", 128, 1, 4096), ("kTuneDkdv", 128, 1, 4097), ("kTuneFwdBf16", 128, 1, 4097)]
    calls = "\n".join(f'    {{ const TuneEntry t = tune_lookup({k}, {d}, {c}, {n}); printf("%d %d\\n", t.slots, t.key_tile); }}'
                      for k, d, c, n in queries)
    src = tmp_path / "t.cpp"
    src.write_text(f"""
#include <cstdio>
#include "attn_tuning.h"
int main() {{
    using namespace attn;
{calls}
    return 0;
}}
""")
    inc = os.path.join(ROOT, "exact_tiled_attention_12_amd", "csrc")
    out = []
    for extra in ([], ["-DATTN_TUNE_FORCE_SLOTS=16", "-DATTN_TUNE_FORCE_KEY_TILE=128"]):
        exe = tmp_path / ("t" + str(len(extra)))
        subprocess.run(["g++", "-std=c++17", "-I", inc, *extra, "-o", str(exe), str(src)], check=True)
        got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
        out.append([tuple(int(x) for x in l.split()) for l in got if l.strip()])
    assert out[0] == [_expected(rows, *q) for q in queries]
    assert out[1] == [(16, 128)] * len(queries)
