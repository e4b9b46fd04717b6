"""Host-only tests of the tile schedule (no GPU).

A small C++ harness links the library's planner source and walks every
workgroup through the kernels' own item decoder: every non-padded output tile
must be visited exactly once, no padded tile may appear, and the counts must
match the closed forms  items = sum_b H*ceil(n_b/T_out),
pairs = sum_b H*ceil(n_b/T_out)*ceil(n_b/T_in).
The harness is built with the host address and undefined-behaviour sanitizers.
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sigmoid_attention_amd", "csrc")
TILES = {"fwd": (128, 64), "bwd_dq": (128, 64), "bwd_dkdv": (128, 64)}


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_harness")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{CSRC}", os.path.join(ROOT, "tests", "plan_harness.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


def run(harness, B, H, L, d, lens, outer=128, inner=64):
    out = subprocess.run([harness, str(B), str(H), str(L), str(d), str(outer), str(inner), *map(str, lens)],
                         check=True, capture_output=True, text=True)
    return json.loads(out.stdout)


def closed_forms(H, lens, outer, inner):
    lens = np.asarray(lens, dtype=np.int64)
    items = int((H * -(-lens // outer)).sum())
    pairs = int((H * -(-lens // outer) * -(-lens // inner)).sum())
    return items, pairs


CASES = [
    ("tiny", 2, 2, 128, [128, 77]),
    ("all_zero", 3, 4, 256, [0, 0, 0]),
    ("one_token", 1, 1, 64, [1]),
    ("tile_edges", 5, 3, 300, [127, 128, 129, 64, 65]),
    ("single_head_long", 1, 1, 8192, [8192]),
    ("few_heads_long", 1, 4, 8192, [8192]),
    ("many_sequences", 300, 8, 512, list(np.random.default_rng(1).integers(0, 513, 300))),
    ("many_full_sequences", 600, 2, 256, [256] * 599 + [255]),
    ("short_cells_1024", 1024, 16, 256, [256] * 1024),
    ("short_cells_4096", 4096, 4, 128, [128] * 4096),
    ("ragged_cells_3000", 3000, 2, 512, list(np.random.default_rng(2).integers(0, 513, 3000))),
    ("beyond_one_table", 4500, 1, 64, list(np.random.default_rng(3).integers(0, 65, 4500))),
    ("wide_lengths", 2100, 1, 70000, [1] * 2099 + [70000]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("pass_", sorted(TILES))
def test_schedule_covers_every_tile_once(harness, case, pass_):
    _, B, H, L, lens = case
    outer, inner = TILES[pass_]
    r = run(harness, B, H, L, 64, lens, outer, inner)
    items, pairs = closed_forms(H, lens, outer, inner)
    assert r["missing"] == 0 and r["dup"] == 0 and r["extra"] == 0 and r["bad"] == 0, r
    assert r["zero_bad"] == 0, r
    assert r["items"] == items == r["stats_items"], r
    assert r["pairs"] == pairs == r["stats_pairs"], r
    if items == 0 and all(n == L for n in lens):
        assert r["launches"] == 0
    if B <= (2048 if L > 65535 else 4096) and items > 0:
        assert r["launches"] == 1, r  # one launch per pass up to a length table's capacity
    assert r["max_piece_seqs"] <= 64, r


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_schedule_on_workloads(harness, name):
    w = workloads.WORKLOADS[name]
    lens = workloads.lengths(name)
    for pass_, (outer, inner) in TILES.items():
        r = run(harness, w.B, w.H, w.Lmax, w.d, lens, outer, inner)
        items, pairs = closed_forms(w.H, lens, outer, inner)
        assert r["missing"] == 0 and r["dup"] == 0 and r["extra"] == 0 and r["bad"] == 0, r
        assert r["zero_bad"] == 0, r
        assert (r["items"], r["pairs"]) == (items, pairs)
        # Longest-first over 8 XCD lists keeps the per-XCD tile-pair load even
        # (a batch with fewer items than XCD lists cannot be even).
        if items >= 64:
            assert r["xcd_imbalance"] < 0.05, (pass_, r)


def test_padding_skip_counts():
    """Tile pairs grow with the covered tiles, not with Lmax: a batch padded to
    4096 with lengths 2048 visits a quarter of the dense pairs."""
    items_full, pairs_full = closed_forms(16, [4096] * 16, 128, 64)
    items_half, pairs_half = closed_forms(16, [2048] * 16, 128, 64)
    assert pairs_half * 4 == pairs_full and items_half * 2 == items_full
