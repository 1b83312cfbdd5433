"""GPU parity of the HIP path with the CPU oracle, through the C ABI.

Bars: routing index sets bit-exact wherever the oracle certifies the boundary
(every boundary of the planted workloads is certified); summaries bit-exact
for bfloat16 keys (their float64 sums are exact, then rounded once) and
within one float32 ulp for float32 keys; outputs within the tolerances of
tests/harness.py. Workloads are the five seeded synthetic configurations at
full size; attention is compared element by element on sampled items.
"""
import numpy as np
import pytest

import oracle
import synth
from harness import bf16_round, check_outputs, check_routing, gpu_run, inputs, oracle_route

pytestmark = pytest.mark.gpu

# items compared element by element per workload (first, last and spread blocks)
SAMPLE_BLOCKS = {0: None, 1: [0, 1, 2, 31, 62, 63], 2: [0, 13, 31], 3: [0, 40, 63], 4: [0, 31]}


def sampled_items(cfg, cfg_id):
    nb = cfg["n_q"] // 64
    blocks = SAMPLE_BLOCKS[cfg_id] or list(range(nb))
    return [(b, h) for b in blocks for h in range(cfg["hkv"])]


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_summaries(cfg_id):
    cfg, x, f = inputs(cfg_id)
    print(f"[summaries] {cfg['name']}", flush=True)
    gpu = gpu_run(cfg, x)
    gs, cs = oracle.summaries(cfg, f["k"])
    gs32, cs32 = gs.astype(np.float32), cs.astype(np.float32)
    if cfg["dtype"] == "bf16":
        np.testing.assert_array_equal(gpu["gs"], gs32)
        np.testing.assert_array_equal(gpu["cs"], cs32)
    else:
        for a, b in ((gpu["gs"], gs32), (gpu["cs"], cs32)):
            ulp = np.abs(np.spacing(b))
            assert (np.abs(a - b) <= ulp).all()


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_routing_and_attention_end_to_end(cfg_id):
    """GPU route + GPU attend against the oracle's own routing and attention."""
    cfg, x, f = inputs(cfg_id)
    print(f"[end-to-end] {cfg['name']}", flush=True)
    gpu = gpu_run(cfg, x)
    ref = oracle_route(cfg, f)
    n, uncert, mism = check_routing(cfg, gpu, ref, f)
    print(f"  items={n} uncertified boundaries={uncert} differing sets={mism}", flush=True)
    assert uncert == 0, f"{uncert} uncertified boundaries in a planted workload"
    assert mism == 0
    items = sampled_items(cfg, cfg_id)
    idx = [b * cfg["hkv"] + h for b, h in items]
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1][idx], ref[2][idx, 1])
    mx, mean, lerr = check_outputs(cfg, gpu, items, ro, rl)
    print(f"  items={n} max_abs={mx:.3g} mean_abs={mean:.3g} lse={lerr:.3g}", flush=True)
    if cfg["dtype"] == "bf16":
        # the float32 output mode: the same bars on the output before its
        # rounding to bfloat16, which must give the bfloat16 output exactly
        g32 = gpu_run(cfg, x, out_f32=True)
        for name in ("chunk_idx", "group_idx", "n_sel", "lse"):
            np.testing.assert_array_equal(g32[name], gpu[name])
        mx, mean, lerr = check_outputs(cfg, g32, items, ro, rl)
        print(f"  float32 output: max_abs={mx:.3g} mean_abs={mean:.3g}", flush=True)
        np.testing.assert_array_equal(bf16_round(g32["out"]), gpu["out"])


@pytest.mark.parametrize("cfg_id", [3, 4])
def test_host_tier_matches_device_resident(cfg_id):
    """History K/V and group summaries in pinned host memory (split at the first
    query): indices and outputs are bit-identical to the all-HBM run."""
    cfg, x, f = inputs(cfg_id)
    print(f"[host tier] {cfg['name']} split={cfg['tier_split']}", flush=True)
    a = gpu_run(cfg, x)
    b = gpu_run(cfg, x, split=cfg["tier_split"])
    for key in ("chunk_idx", "group_idx", "n_sel"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["lse"], b["lse"])


def test_host_tier_group_stage_reads_host_summaries():
    """A tiered run whose group stage must choose (top_groups < groups of the kept
    chunks), so group summaries are read from pinned host memory."""
    cfg, x, f = inputs(2)
    split = 8192
    print(f"[host tier, choosing group stage] split={split}", flush=True)
    a = gpu_run(cfg, x)
    b = gpu_run(cfg, x, split=split)
    for key in ("chunk_idx", "group_idx", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(a[key], b[key])


def test_deterministic_reruns():
    cfg, x, f = inputs(2)
    a = gpu_run(cfg, x)
    b = gpu_run(cfg, x)
    for key in ("gs", "cs", "chunk_idx", "group_idx", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(a[key], b[key])


@pytest.mark.parametrize("cfg_id", [1, 2])
def test_attention_with_oracle_selection(cfg_id):
    """hga_attend fed the oracle's own selection, compared on sampled items."""
    cfg, x, f = inputs(cfg_id)
    ref = oracle_route(cfg, f)
    nb, hkv = cfg["n_q"] // 64, cfg["hkv"]
    gpu = gpu_run(cfg, x, group_idx=ref[1].reshape(nb, hkv, -1), n_sel=ref[2].reshape(nb, hkv, 2))
    items = sampled_items(cfg, cfg_id)
    idx = [b * hkv + h for b, h in items]
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1][idx], ref[2][idx, 1])
    check_outputs(cfg, gpu, items, ro, rl)


@pytest.mark.parametrize("case", ["f32", "bf16_d64_g4", "split_below_q_start", "wide_windows"])
def test_host_tier_cache_small_shapes(case):
    """The host-tier path (history chunks marked, given cache slots and copied
    once each) is bit-identical to the all-HBM run on small shapes: fp32,
    d = 64 with 4-token groups, a split well below the first query (the local
    windows and some kept groups then come from HBM), wide sink/local windows."""
    from test_gpu_edges import small
    over = {"f32": dict(dtype="f32", d=64, rope_theta=None),
            "bf16_d64_g4": dict(d=64, group=4, top_groups=20),
            "split_below_q_start": dict(L=2048, n_q=512),
            "wide_windows": dict(L=2048, n_q=512, sink=192, local=256)}[case]
    cfg = small(**over)
    x = synth.make_inputs(cfg)
    split = {"split_below_q_start": 768, "wide_windows": 1024}.get(case, cfg["L"] - cfg["n_q"])
    print(f"[host tier cache] {case} split={split}", flush=True)
    a = gpu_run(cfg, x)
    b = gpu_run(cfg, x, split=split)
    for key in ("chunk_idx", "group_idx", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(a[key], b[key])


def test_host_tier_cache_keys_past_the_last_query():
    from test_gpu_edges import small
    cfg = small(L=1024, n_q=256)
    x = synth.make_inputs(cfg)
    a = gpu_run(cfg, x, q_start=512, seq_len=1024)
    b = gpu_run(cfg, x, q_start=512, seq_len=1024, split=384)
    for key in ("chunk_idx", "group_idx", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(a[key], b[key])
