"""hga_route_attend (routing and attention in one call) against hga_route
followed by hga_attend: both run the same router and attention code, so every
output is bit-identical; on a small workload also against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from harness import check_outputs, check_routing, gpu_run, inputs, oracle_route
from test_gpu_edges import CASES, small

pytestmark = pytest.mark.gpu

KEYS = ("chunk_idx", "group_idx", "n_sel", "out", "lse")


def assert_identical(a, b, what):
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"


@pytest.mark.parametrize("name", list(CASES))
def test_fused_matches_separate_calls_edge_cases(name):
    cfg = small(**CASES[name])
    print(f"[fused edge] {name}", flush=True)
    x = synth.make_inputs(cfg)
    assert_identical(gpu_run(cfg, x), gpu_run(cfg, x, fused=True), name)


@pytest.mark.parametrize("cfg_id", [0, 1, 2, 3, 4])
def test_fused_matches_separate_calls_workloads(cfg_id):
    cfg, x, _ = inputs(cfg_id)
    print(f"[fused workload] {cfg['name']}", flush=True)
    assert_identical(gpu_run(cfg, x), gpu_run(cfg, x, fused=True), cfg["name"])


def test_fused_against_oracle():
    cfg, x, f = inputs(1)
    gpu = gpu_run(cfg, x, fused=True)
    ref = oracle_route(cfg, f)
    n, uncert, mism = check_routing(cfg, gpu, ref, f)
    print(f"  items={n} uncertified boundaries={uncert} differing sets={mism}", flush=True)
    assert uncert == 0 and mism == 0
    items = oracle.all_items(cfg)
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1], ref[2][:, 1])
    check_outputs(cfg, gpu, items, ro, rl)


def test_fused_host_tier_runs_the_two_steps():
    """K/V partly in pinned host memory: the call gathers after routing."""
    cfg, x, _ = inputs(3)
    split = cfg["tier_split"]
    assert_identical(gpu_run(cfg, x, split=split), gpu_run(cfg, x, split=split, fused=True), "host tier")


def test_fused_with_keys_past_the_last_query():
    cfg = small(L=1024, n_q=256)
    x = synth.make_inputs(cfg)
    a = gpu_run(cfg, x, q_start=512, seq_len=1024)
    b = gpu_run(cfg, x, q_start=512, seq_len=1024, fused=True)
    assert_identical(a, b, "q_start + n_q < seq_len")
