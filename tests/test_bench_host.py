"""Host-side logic of bench.py (no GPU): the FLOP convention, the covered-tile
count, the kernel-source hash that guards stored traffic counters, and the
one-GPU rule."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_pair_flops_closed_forms():
    # H d n^2 per sequence; causal: H d n (n + 1) / 2
    assert bench.pair_flops([3, 5], 2, 64) == 2 * 64 * (9 + 25)
    assert bench.pair_flops([3, 5], 2, 64, causal=True) == 2 * 64 * (6 + 15)
    assert bench.pair_flops([0, 0], 4, 128) == 0.0


def test_flop_units_sum_to_the_convention():
    u = bench.KERNEL_FLOP_UNITS
    assert u["fwd"] + u["bwd"] == 14            # 4 n^2 d forward + 10 n^2 d backward
    assert u["bwd_dq"] + u["bwd_dkdv"] == u["bwd"]
    for k, (fast, split) in bench.EXECUTED_UNITS.items():
        assert fast >= u[k] and split >= fast


def test_algorithmic_bytes_and_bound():
    import workloads
    w = workloads.WORKLOADS["many_b4096h16d64_l128"]
    lens = [128] * w.B
    tensor = 4096 * 16 * 128 * 64 * 2  # one full [B, H, Lmax, d] 16-bit tensor
    assert bench.kernel_bytes("bwd", lens, w) == 7 * tensor
    assert bench.kernel_bytes("fwd", lens, w) == 4 * tensor
    # padded rows are written but not read
    assert bench.kernel_bytes("fwd", [64] * w.B, w) == 3 * tensor / 2 + tensor
    # 10 n^2 d FLOP over 7 n d 2 bytes per (sequence, head): 91 FLOP/byte at
    # n = 128, below the 312.5 of 2.5 PFLOP/s over 8 TB/s; about 1460 at 2048
    flops = 10 * bench.pair_flops(lens, w.H, w.d)
    r = bench.roofline_bound(flops, bench.kernel_bytes("bwd", lens, w), 1.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["frac"] == r["hbm_frac"]
    assert abs(r["achieved"] - 7 * tensor / 1e-3 / 1e9) < 0.01
    h = workloads.WORKLOADS[workloads.HEADLINE]
    hl = [h.Lmax] * h.B
    r = bench.roofline_bound(10 * bench.pair_flops(hl, h.H, h.d), bench.kernel_bytes("bwd", hl, h), 1.0)
    assert r["bound"] == "mfma" and r["frac"] == r["mfma_frac"]
    assert bench.one_tile_bwd(w, "fast") and not bench.one_tile_bwd(w, "split") and not bench.one_tile_bwd(h, "fast")
    assert bench.executed_units("bwd", w, "fast") == 10 and bench.executed_units("bwd", h, "fast") == 14


def test_covered_pairs():
    # 300 rows -> 3 tiles of 128 x 5 tiles of 64; 1 row -> 1 x 1; 0 rows -> none
    assert bench.covered_pairs([300, 1, 0], 2, 128, 64) == 2 * (15 + 1)


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // one\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    h1 = bench.kernel_source_hash()
    src.write_text("// a new comment\nint f() {\n  return 1;  // two\n}\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
