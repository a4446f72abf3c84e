"""The kernels' workgroup -> work-item mappings are bijections (CPU, no GPU needed).

block_coords (XCD grouping, causal heavy-first order) and ItemWalk (the key-side
kernel's persistent walk) are compiled from the kernels' own header as host code
(tests/host_walk.cpp) and evaluated for every workload shape, for every `slots`
value the launch table can give, for head counts that are not multiples of 8 and
for other compute-unit counts.  A slip in either mapping would leave some (head,
block) pair uncomputed, or computed twice, which sampled parity checks can miss.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SLOTS = (16, 32, 64, 128)           # every value in the launch table (and the sweep's candidates)

# (B*H, N) of the five workloads, ragged and uneven shapes, and a long sequence
SHAPES = [(1, 256), (128, 1024), (64, 4096), (16, 16384), (256, 2048),
          (66, 1000), (3, 11000), (6, 300), (13, 777), (2, 65536), (4097, 4096)]


@pytest.fixture(scope="module")
def walk(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("walk") / "libwalk.so")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    subprocess.run([hipcc, "--offload-host-only", "-x", "hip", "-O1", "-fPIC", "-shared", "-std=c++17", "-o", out,
                    os.path.join(HERE, "host_walk.cpp")], check=True, capture_output=True)
    L = ctypes.CDLL(out)
    ip = ctypes.POINTER(ctypes.c_int)
    L.walk_block_coords.argtypes = [ctypes.c_int] * 5 + [ip, ip]
    L.walk_items.argtypes = [ctypes.c_int] * 5 + [ip]
    L.persistent_workgroups.argtypes = [ctypes.c_int] * 4
    return L


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _coords(L, causal, heavy_last, nb, nblk, slots):
    head = np.full(nb, -1, dtype=np.int32)
    blk = np.full(nb, -1, dtype=np.int32)
    assert L.walk_block_coords(int(causal), int(heavy_last), nb, nblk, slots, _ip(head), _ip(blk)) == 0
    return head, blk


def _assert_bijection(head, blk, BH, nblk, what):
    assert head.min() >= 0 and head.max() < BH, what
    assert blk.min() >= 0 and blk.max() < nblk, what
    code = head.astype(np.int64) * nblk + blk
    assert np.array_equal(np.sort(code), np.arange(BH * nblk)), f"{what}: not a bijection"


# (kernel, rows per block, heavy_last): forward bf16 dense (256 rows), block-sparse and fp32
# forward, fp8 forward and the query-side backward (128 rows), fp32 backward (128 keys)
GRIDS = [("fwd_dense", 256, True), ("fwd_128", 128, True), ("dq", 128, True), ("bwd_f32", 128, False)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("BH,N", SHAPES)
def test_block_coords_bijective(walk, BH, N, causal):
    for name, rows, heavy_last in GRIDS:
        nblk = (N + rows - 1) // rows
        for slots in SLOTS:
            head, blk = _coords(walk, causal, heavy_last, BH * nblk, nblk, slots)
            _assert_bijection(head, blk, BH, nblk, f"{name} BH={BH} N={N} causal={causal} slots={slots}")


@pytest.mark.parametrize("ncu", [256, 304, 80, 8])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("BH,N", SHAPES)
def test_key_side_walk_bijective(walk, BH, N, causal, ncu):
    """Persistent key side: one workgroup per CU walks its share of the (head, 128-key block)
    items; every item is visited once, and block_coords maps the items onto the pairs."""
    nkblk = (N + 127) // 128
    nitems = nkblk * BH
    split = (BH % 8 == 0) if causal else (nitems % 8 == 0)
    nwg = walk.persistent_workgroups(nitems, 1, int(split), ncu)
    steps = nitems // nwg + 2
    items = np.full((nwg, steps), -2, dtype=np.int32)
    assert walk.walk_items(nwg, nitems, nkblk, int(causal), steps, _ip(items)) == 0
    seen = []
    for row in items:
        stop = np.where(row < 0)[0]
        assert stop.size and row[stop[0]] == -1         # every workgroup's walk ends
        seen.extend(row[: stop[0]].tolist())
    assert sorted(seen) == list(range(nitems)), f"BH={BH} N={N} causal={causal} ncu={ncu}"
    for slots in SLOTS:
        head, blk = _coords(walk, causal, False, nitems, nkblk, slots)
        _assert_bijection(head, blk, BH, nkblk, f"dkdv BH={BH} N={N} causal={causal} slots={slots}")


@pytest.mark.parametrize("BH,N", [(64, 4096), (16, 16384), (256, 2048), (128, 1024), (32, 8192), (8, 4096),
                                  (64, 2816), (128, 2600), (48, 3000), (96, 1500)])
def test_query_side_groups_fill_shader_engine_rounds(walk, BH, N):
    """An XCD dispatches its workgroups in order, consecutive ones to its four shader engines in
    turn, so block_coords gives the causal query-side grids a multiple of four heads per group:
    every four consecutive workgroups of an XCD then hold blocks of one index (equal cost), or,
    with fewer heads left in a group, each of them before the next index."""
    for name, rows, heavy_last in GRIDS:
        if not heavy_last:
            continue
        nblk = (N + rows - 1) // rows
        hx = BH // 8
        for slots in SLOTS:
            head, blk = _coords(walk, True, True, BH * nblk, nblk, slots)
            for x in range(8):
                h, b = head[x::8], blk[x::8]            # XCD x's sequence
                assert np.all(h // hx == x), f"{name} BH={BH} N={N} slots={slots}: heads leave XCD {x}"
                # groups of G heads (a multiple of 4, or all of the XCD's), the last one possibly smaller;
                # each group's positions run rank by rank over its heads
                p = 0
                while p < len(b):
                    # the group's heads: the positions before the block index changes
                    q = p
                    while q < len(b) and b[q] == b[p]:
                        q += 1
                    gh = q - p
                    assert gh == hx or gh % 4 == 0 or p + gh * nblk == len(b), \
                        f"{name} BH={BH} N={N} slots={slots} XCD {x}: group of {gh} heads at {p}"
                    for r in range(nblk):                                  # rank r: one index, gh heads
                        seg = slice(p + r * gh, p + (r + 1) * gh)
                        assert len(set(b[seg].tolist())) == 1 and len(set(h[seg].tolist())) == gh, \
                            f"{name} BH={BH} N={N} slots={slots} XCD {x} rank {r} at {p}"
                    p += gh * nblk
