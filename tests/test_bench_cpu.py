"""Host-side checks of bench.py: the algorithmic work its rooflines divide by,
the choice of the binding peak, its statistics, and its refusal of more than
one GPU. No GPU is used."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def full_selection(cfg):
    ns = np.zeros((cfg["n_q"] // 64, cfg["hkv"], 2), dtype=np.int64)
    ns[..., 0] = cfg["top_chunks"]
    ns[..., 1] = cfg["top_groups"]
    return ns


# (GFLOP, MiB) of one attention launch with every block keeping its full
# budget, as derived from the workload shapes: flops 4 d per attended
# (query, key) pair over all query heads, the diagonal tile's masked half
# excluded; bytes Q read + O written + the K/V rows of each (block, KV head)
# working set, loaded per block as the pages do (LCFT, section 2.1,
# "Exact-token attention"). Every block of these three workloads has more
# candidates than its budget, so the full selection is the one routing makes.
EXPECTED = {2: (24.7128, 128.0), 3: (152.5049, 352.0), 4: (144.9719, 576.0)}


@pytest.mark.parametrize("cid", sorted(EXPECTED))
def test_algorithmic_counts_of_the_workloads(cid):
    cfg = bench.synth_config(cid)
    flops, byts, pairs = bench.algorithmic(cfg, full_selection(cfg))
    gflop, mib = EXPECTED[cid]
    assert flops / 1e9 == pytest.approx(gflop, rel=1e-5)
    assert byts / 2**20 == mib
    assert flops == 4 * cfg["d"] * pairs


def test_16k_counts_by_hand():
    """The 16K segment by hand: 32 blocks x 8 KV heads, each attending 3 fixed
    chunks (one sink, two local) and 64 groups of 8 tokens of history plus its
    own causal 64-token block, for 4 query heads of 64 rows."""
    cfg = bench.synth_config(2)
    hist = 3 * 64 + 64 * 8
    pairs = 32 * 8 * 4 * (64 * hist + 64 * 65 // 2)
    kv_rows = 32 * 8 * (hist + 64)
    flops, byts, _ = bench.algorithmic(cfg, full_selection(cfg))
    assert flops == 4.0 * 128 * pairs
    assert byts == 2.0 * 32 * 2048 * 128 * 2 + 2.0 * kv_rows * 128 * 2


def test_roofline_takes_the_binding_peak():
    c2, c3 = bench.synth_config(2), bench.synth_config(3)
    r2 = bench.roofline(c2, full_selection(c2), 50.0, "route_attend_bf16", with_traffic=False)
    r3 = bench.roofline(c3, full_selection(c3), 170.0, "attend_bf16", with_traffic=False)
    assert r2["bound"] == "hbm" and r2["unit"] == "GB/s" and r2["peak"] == 8000.0
    assert r2["frac"] == pytest.approx(128 * 2**20 / 50e-6 / 8e12)
    assert r3["bound"] == "mfma" and r3["unit"] == "TFLOP/s" and r3["peak"] == 2500.0
    assert r3["frac"] == pytest.approx(152.50489344e9 / 170e-6 / 2.5e15)
    for r in (r2, r3):
        assert r["achieved"] / r["peak"] == pytest.approx(r["frac"])


def test_stats():
    s = bench.stats(list(range(1, 12)))
    assert s == {"mean": 6.0, "median": 6.0, "p10": 2.0, "p90": 10.0, "n": 11}
    with pytest.raises(AssertionError):
        bench.stats([1.0, float("nan")])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
