"""GPU edge cases against the oracle on small shapes (several tiles, ragged
routed tiles, degenerate budgets and windows, other GQA ratios, head sizes
and group sizes, float32, invalid selection entries, empty query range)."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hga_amd as hga
import oracle
import synth
from harness import DEV, check_outputs, check_routing, gpu_run, hga_cfg, oracle_route, to_dev

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="edge", L=1024, n_q=512, hq=8, hkv=2, d=128, dtype="bf16", rope_theta=1e4,
                chunk=64, group=8, q_block=64, top_chunks=4, top_groups=12, sink=64, local=128,
                shared_rank=0, shared_scale=0.0, n_plant_chunks=2, groups_per_plant_chunk=1,
                plant_chunks=(1, 6), alpha=1.0, beta=16.0, tier_split=0, cfg_id=60)
    base.update(kw)
    return synth.config(base)


CASES = {
    "base": dict(),
    "gqa1": dict(hq=2, hkv=2),
    "gqa2": dict(hq=4, hkv=2),
    "gqa6": dict(hq=12, hkv=2),
    "gqa8": dict(hq=16, hkv=2),
    "d64": dict(d=64),
    "group4": dict(group=4, top_groups=20),
    "group16": dict(group=16, top_groups=6),
    "group64": dict(group=64, top_groups=3),
    "group1": dict(group=1, top_groups=70),
    "no_routing": dict(top_chunks=0, top_groups=0),
    "no_groups": dict(top_groups=0),
    "no_windows": dict(sink=0, local=0),
    "ragged13": dict(top_groups=13),
    "budget_covers_all": dict(top_chunks=16, top_groups=128),
    "wide_windows": dict(sink=192, local=256),
    "single_block": dict(n_q=64),
    "from_zero": dict(L=512, n_q=512),
    "one_chunk": dict(L=64, n_q=64),
    "f32_d64": dict(dtype="f32", d=64, rope_theta=None),
    "f32_d128_g3": dict(dtype="f32", d=128, hq=6, hkv=2, rope_theta=None),
    "f32_d32_group4": dict(dtype="f32", d=32, group=4, top_groups=9, rope_theta=None),
    "f32_d4": dict(dtype="f32", d=4, rope_theta=None, n_plant_chunks=0),
    # more than one scoring round (256 summary rows each): about 700 chunk
    # candidates in three rounds (the router kernel, two in flight), and
    # 384 groups of 48 kept chunks in two rounds (also inside the fused kernel)
    "chunk_rounds3": dict(L=64 * 700, n_q=128, top_chunks=8, top_groups=24),
    "group_rounds2": dict(L=64 * 80, n_q=128, top_chunks=48, top_groups=100),
    # the largest selections: the longest sequence the library takes (4,096
    # chunks; 4,092 chunk candidates, 64 keys per lane in the selecting
    # wave), 1,500 chunks (32 per lane), and the group stage over 4,096 and
    # 1,600 groups with the bfloat16 attention's largest group budget
    "max_seq_len": dict(L=64 * 4096, n_q=64, hq=2, hkv=1, d=64, top_chunks=8, top_groups=24,
                        n_plant_chunks=8, plant_chunks=(1, 4090)),
    "candidates_1500": dict(L=64 * 1500, n_q=64, hq=2, hkv=1, d=64, top_chunks=8, top_groups=24,
                            n_plant_chunks=8, plant_chunks=(1, 1495)),
    "max_group_candidates": dict(L=64 * 600, n_q=64, hq=2, hkv=1, d=64, top_chunks=512, top_groups=2048,
                                 n_plant_chunks=8, plant_chunks=(1, 595)),
    "group_candidates_1600": dict(L=64 * 600, n_q=64, hq=2, hkv=1, d=64, top_chunks=200, top_groups=700,
                                  n_plant_chunks=8, plant_chunks=(1, 595)),
    # at the fused kernel's selection bound: 512 chunk and 512 group
    # candidates (the fused kernel), then one chunk candidate more (the
    # router kernel, then the attention kernel)
    "select_bound_512": dict(L=64 * 516, n_q=64, top_chunks=64, top_groups=200, n_plant_chunks=8,
                             plant_chunks=(1, 510)),
    "select_bound_513": dict(L=64 * 517, n_q=64, top_chunks=64, top_groups=200, n_plant_chunks=8,
                             plant_chunks=(1, 510)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_edge_case_end_to_end(name):
    cfg = small(**CASES[name])
    print(f"[edge] {name}", flush=True)
    x = synth.make_inputs(cfg)
    f = {n: synth.to_f64(x[n], cfg["dtype"]) for n in ("q", "k", "v")}
    gpu = gpu_run(cfg, x)
    ref = oracle_route(cfg, f)
    n, uncert, mism = check_routing(cfg, gpu, ref, f)
    print(f"  items={n} uncertified boundaries={uncert} differing sets={mism}", flush=True)
    assert mism == 0
    items = oracle.all_items(cfg)
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1], ref[2][:, 1])
    check_outputs(cfg, gpu, items, ro, rl)


def test_queries_before_the_end_of_the_keys():
    """q_start + n_q < seq_len: keys past the last query are never read."""
    cfg = small(L=1024, n_q=256)
    x = synth.make_inputs(cfg)
    gpu = gpu_run(cfg, x, q_start=512, seq_len=1024)
    sub = dict(cfg, L=768)
    f = {"q": synth.to_f64(x["q"], "bf16"), "k": synth.to_f64(x["k"], "bf16")[:, :768],
         "v": synth.to_f64(x["v"], "bf16")[:, :768]}
    ref = oracle_route(sub, f)
    n, uncert, mism = check_routing(sub, gpu, ref, f)
    print(f"  items={n} uncertified boundaries={uncert} differing sets={mism}", flush=True)
    assert mism == 0
    items = oracle.all_items(sub)
    ro, rl = oracle.attend(sub, f["q"], f["k"], f["v"], items, ref[1], ref[2][:, 1])
    check_outputs(sub, gpu, items, ro, rl)


def test_invalid_selection_entries_are_skipped():
    """Negative, duplicate, fixed-chunk and not-yet-closed entries mixed into an
    ascending selection change nothing."""
    cfg = small(top_groups=8)
    x = synth.make_inputs(cfg)
    f = {n: synth.to_f64(x[n], "bf16") for n in ("q", "k", "v")}
    ref = oracle_route(cfg, f)
    nb, hkv = cfg["n_q"] // 64, cfg["hkv"]
    wide = dict(cfg, top_groups=24)
    gi = np.full((nb * hkv, 24), -1, np.int32)
    ns = np.zeros((nb * hkv, 2), np.int32)
    for n, (b, h) in enumerate(oracle.all_items(cfg)):
        s = cfg["L"] - cfg["n_q"] + 64 * b
        row = [-5, 0]                                   # negative; a group of the sink chunk
        for j in ref[1][n][: ref[2][n, 1]]:
            row += [int(j), int(j)]                     # duplicates
        row += [s // 8, s // 8 + 3, 10**6]              # groups not closed before the block
        gi[n, :len(row)] = row
        ns[n] = (ref[2][n, 0], len(row))
    gpu = gpu_run(wide, x, group_idx=gi.reshape(nb, hkv, 24), n_sel=ns.reshape(nb, hkv, 2))
    items = oracle.all_items(cfg)
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1], ref[2][:, 1])
    check_outputs(cfg, gpu, items, ro, rl)


def test_empty_query_range_writes_nothing():
    cfg = small()
    x = synth.make_inputs(cfg)
    c = hga_cfg(cfg)
    q, k = to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16")
    out = torch.full_like(q, 3.0)
    ns = torch.full((1, 2, 2), -7, dtype=torch.int32, device=DEV)
    hga.hga_route(c, q, 1024, 0, 1024, k, k, ns, ns, ns)
    hga.hga_attend(c, q, 1024, 0, 1024, k, k, ns, ns, out)
    torch.cuda.synchronize()
    assert (ns == -7).all() and (out == 3.0).all()


# Exact ties: integer queries and keys whose chunks repeat with a short period,
# so many scores are exactly equal on both sides (exact in float64 in any
# order). The boundary then falls inside a class of equal scores, and the
# lower-index rule alone decides which members are kept (fixed by the task's
# statement of the method; "Long-Context Fine-Tuning with Limited VRAM",
# section 2.1, "Chunk selection" and "Group selection").
TIE_CASES = {
    "g2_d64": dict(d=64, hq=4, hkv=2, L=2048, n_q=512, top_chunks=4, top_groups=12, chunk_period=5),
    "g4_d128": dict(d=128, hq=8, hkv=2, L=2048, n_q=512, top_chunks=6, top_groups=20, chunk_period=7),
    "g2_block16": dict(d=64, hq=4, hkv=2, L=1024, n_q=256, q_block=16, top_chunks=3, top_groups=10,
                       chunk_period=4),
    "group4": dict(d=64, hq=4, hkv=2, L=2048, n_q=256, group=4, top_chunks=4, top_groups=23, chunk_period=6),
}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", list(TIE_CASES))
def test_exact_ties_take_the_lower_index(name, fused):
    cfg = small(rope_theta=None, n_plant_chunks=0, integer_values=(-2, 2), **TIE_CASES[name])
    print(f"[ties] {name} fused={fused}", flush=True)
    x = synth.make_inputs(cfg)
    f = {n: synth.to_f64(x[n], cfg["dtype"]) for n in ("q", "k", "v")}
    gpu = gpu_run(cfg, x, fused=fused)
    ref = oracle_route(cfg, f)
    dg = ref[3]
    ties = int((dg[:, oracle.DG_GAP_C] == 0).sum() + (dg[:, oracle.DG_GAP_G] == 0).sum())
    n, uncert, mism = check_routing(cfg, gpu, ref, f)
    print(f"  items={n} boundaries at an exact tie={ties} uncertified={uncert} differing sets={mism}", flush=True)
    assert ties >= n // 2, "the periodic integer keys should put most boundaries on an exact tie"
    assert mism == 0, "the lower-index rule decides every tie: the sets must equal the oracle's"
    nitems = len(oracle.all_items(cfg))
    np.testing.assert_array_equal(gpu["chunk_idx"].reshape(nitems, -1), ref[0])
    np.testing.assert_array_equal(gpu["group_idx"].reshape(nitems, -1), ref[1])
    np.testing.assert_array_equal(gpu["n_sel"].reshape(nitems, 2), ref[2])
    items = oracle.all_items(cfg)
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1], ref[2][:, 1])
    check_outputs(cfg, gpu, items, ro, rl)
