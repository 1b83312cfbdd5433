"""The segment-streaming driver (hga_stream_forward) and the chunk-range
summary build against the one-shot calls: summaries, indices, outputs and LSE
are bit-identical (every chunk's summaries and every block's routing and
attention depend only on the chunks before it, which the driver has committed
when it reaches the block)."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hga_amd as hga
import synth
from harness import DEV, hga_cfg, to_dev
from test_gpu_edges import small

pytestmark = pytest.mark.gpu


def run(cfg, x, segment=None):
    """One-shot (segment None: summaries, then one hga_route_attend over every
    position) or streamed in segments. Every position queries (n_q == L)."""
    c = hga_cfg(cfg)
    dt, L, d, g, hkv = cfg["dtype"], cfg["L"], cfg["d"], cfg["group"], cfg["hkv"]
    assert cfg["n_q"] == L
    nb = L // cfg["q_block"]
    q, k, v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
    gs = torch.full((hkv, L // g, d), float("nan"), device=DEV)
    cs = torch.full((hkv, L // 64, d), float("nan"), device=DEV)
    ci = torch.full((nb, hkv, cfg["top_chunks"]), -7, dtype=torch.int32, device=DEV)
    gi = torch.full((nb, hkv, cfg["top_groups"]), -7, dtype=torch.int32, device=DEV)
    ns = torch.full((nb, hkv, 2), -7, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(cfg["hq"], L, device=DEV)
    if segment is None:
        hga.hga_build_summaries(c, k, L, gs, cs)
        hga.hga_route_attend(c, q, 0, L, L, cs, gs, k, v, ci, gi, ns, out, lse)
    else:
        hga.hga_stream_forward(c, q, k, v, L, segment, cs, gs, ci, gi, ns, out, lse)
    torch.cuda.synchronize()
    return dict(gs=gs.cpu().numpy(), cs=cs.cpu().numpy(), chunk_idx=ci.cpu().numpy(),
                group_idx=gi.cpu().numpy(), n_sel=ns.cpu().numpy(),
                out=out.float().cpu().numpy(), lse=lse.cpu().numpy())


def assert_identical(a, b, what):
    for key in a:
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"


CASES = {
    "bf16_seg256": (dict(L=1024, n_q=1024), 256),
    "bf16_ragged_seg384": (dict(L=1024, n_q=1024), 384),
    "bf16_one_segment": (dict(L=1024, n_q=1024), 1024),
    "bf16_seg64": (dict(L=512, n_q=512), 64),
    "bf16_gqa8": (dict(L=1024, n_q=1024, hq=16, hkv=2), 256),
    "f32": (dict(L=1024, n_q=1024, dtype="f32", d=64, rope_theta=None), 256),
    "bf16_block16_seg192": (dict(L=1024, n_q=1024, q_block=16), 192),
    "bf16_block1_seg64": (dict(L=256, n_q=256, q_block=1), 64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_stream_matches_one_shot_small(name):
    over, segment = CASES[name]
    cfg = small(**over)
    print(f"[stream] {name}", flush=True)
    x = synth.make_inputs(cfg)
    assert_identical(run(cfg, x), run(cfg, x, segment), name)


@pytest.mark.parametrize("cfg_id,segment", [(0, 256), (1, 1024)])
def test_stream_matches_one_shot_workloads(cfg_id, segment):
    cfg = synth.config(cfg_id)
    print(f"[stream] {cfg['name']} segment={segment}", flush=True)
    x = synth.make_inputs(cfg)
    assert_identical(run(cfg, x), run(cfg, x, segment), cfg["name"])


def test_stream_16k_in_training_segments():
    """The 16K training-segment workload with every position querying, streamed
    in its 2,048-token segments."""
    cfg = synth.config(2, n_q=16384)
    x = synth.make_inputs(cfg)
    assert_identical(run(cfg, x), run(cfg, x, 2048), "16K in 2048-token segments")


def test_summary_range_matches_full_build():
    cfg = small(L=2048, n_q=512)
    x = synth.make_inputs(cfg)
    c = hga_cfg(cfg)
    L, d, g, hkv = cfg["L"], cfg["d"], cfg["group"], cfg["hkv"]
    k = to_dev(x["k"], "bf16")
    full = [torch.empty(hkv, L // g, d, device=DEV), torch.empty(hkv, L // 64, d, device=DEV)]
    part = [torch.full_like(full[0], float("nan")), torch.full_like(full[1], float("nan"))]
    hga.hga_build_summaries(c, k, L, *full)
    for c0, c1 in ((0, 5), (5, 5), (5, 17), (17, L // 64)):
        hga.hga_build_summaries_range(c, k, L, c0, c1, *part)
    torch.cuda.synchronize()
    for a, b in zip(full, part):
        assert torch.equal(a, b)
