"""hga_route_attend_noalloc (no workspace; the spread attention's partial
states in the library's static device scratch array) against hga_route_attend
given the workspace hga_workspace_size asks for: the same kernels run, so
every output is bit-identical. Two decoding calls in a row, the second with a
smaller input (fewer sequences, a shorter history), leave the first call's
partial states in the array; then a prefill shape, which needs no scratch."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hga_amd as hga
from harness import DEV, inputs, to_dev

pytestmark = pytest.mark.gpu


def decode_call(cfg_id, batch, pos, noalloc):
    """One decoded token at position pos of workload cfg_id for `batch`
    sequences (folded into the heads), through one of the two entry points."""
    base, x, _ = inputs(cfg_id)
    L, d, g = base["L"], base["d"], base["group"]
    hq, hkv = batch * base["hq"], batch * base["hkv"]
    c = hga.make_config(hq, hkv, d, base["top_chunks"], base["top_groups"], base["sink"], base["local"],
                        dtype=base["dtype"], group_size=g, q_block=1)
    k = to_dev(x["k"], base["dtype"]).repeat(batch, 1, 1).contiguous()
    v = to_dev(x["v"], base["dtype"]).repeat(batch, 1, 1).contiguous()
    q = to_dev(x["q"][:, -1:], base["dtype"]).repeat(batch, 1, 1).contiguous()
    gs = torch.empty(hkv, L // g, d, device=DEV)
    cs = torch.empty(hkv, L // 64, d, device=DEV)
    hga.hga_build_summaries_range(c, k, L, 0, pos // 64, gs, cs)
    ci = torch.full((1, hkv, base["top_chunks"]), -7, dtype=torch.int32, device=DEV)
    gi = torch.full((1, hkv, base["top_groups"]), -7, dtype=torch.int32, device=DEV)
    ns = torch.full((1, hkv, 2), -7, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((hq, 1), float("nan"), device=DEV)
    wsb = hga.hga_workspace_size(c, L, 1, hga.HGA_WS_ATTEND)
    assert wsb > 0, "few items: the spread attention (which takes the scratch) must run"
    if noalloc:
        hga.hga_route_attend_noalloc(c, q, pos, 1, L, cs, gs, k, v, ci, gi, ns, out, lse)
    else:
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        hga.hga_route_attend(c, q, pos, 1, L, cs, gs, k, v, ci, gi, ns, out, lse, ws, wsb)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in (("ci", ci), ("gi", gi), ("ns", ns), ("out", out.view(torch.int16)),
                                              ("lse", lse))}


def assert_identical(a, b, what):
    for key in a:
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"
    assert np.isfinite(a["lse"]).all()


def test_noalloc_matches_route_attend_on_two_calls():
    # 16K history, 2 sequences (16 items in 3 ranges each), then the 4K
    # workload at position 2047, one sequence (8 items, fewer ranges)
    for cfg_id, batch, pos in ((2, 2, 16383), (1, 1, 2047)):
        print(f"[noalloc] workload {cfg_id} batch {batch} position {pos}", flush=True)
        b = decode_call(cfg_id, batch, pos, noalloc=True)
        a = decode_call(cfg_id, batch, pos, noalloc=False)
        assert_identical(a, b, f"workload {cfg_id}")


def test_noalloc_prefill_needs_no_scratch():
    cfg, x, _ = inputs(1)
    L, nq, hkv, d, g = cfg["L"], cfg["n_q"], cfg["hkv"], cfg["d"], cfg["group"]
    c = hga.make_config(cfg["hq"], hkv, d, cfg["top_chunks"], cfg["top_groups"], cfg["sink"], cfg["local"],
                        dtype=cfg["dtype"], group_size=g)
    assert hga.hga_workspace_size(c, L, nq, hga.HGA_WS_ATTEND) == 0
    q, k, v = (to_dev(x[n], cfg["dtype"]) for n in ("q", "k", "v"))
    gs = torch.empty(hkv, L // g, d, device=DEV)
    cs = torch.empty(hkv, L // 64, d, device=DEV)
    hga.hga_build_summaries(c, k, L, gs, cs)
    res = []
    for noalloc in (True, False):
        nb = nq // 64
        ci = torch.empty(nb, hkv, cfg["top_chunks"], dtype=torch.int32, device=DEV)
        gi = torch.empty(nb, hkv, cfg["top_groups"], dtype=torch.int32, device=DEV)
        ns = torch.empty(nb, hkv, 2, dtype=torch.int32, device=DEV)
        out = torch.empty_like(q)
        lse = torch.empty(cfg["hq"], nq, device=DEV)
        if noalloc:
            hga.hga_route_attend_noalloc(c, q, 0, nq, L, cs, gs, k, v, ci, gi, ns, out, lse)
        else:
            hga.hga_route_attend(c, q, 0, nq, L, cs, gs, k, v, ci, gi, ns, out, lse)
        torch.cuda.synchronize()
        res.append({"ci": ci.cpu().numpy(), "gi": gi.cpu().numpy(), "ns": ns.cpu().numpy(),
                    "out": out.view(torch.int16).cpu().numpy(), "lse": lse.cpu().numpy()})
    assert_identical(res[1], res[0], "prefill")


def test_noalloc_refuses_a_host_tier():
    cfg, x, _ = inputs(1)
    c = hga.make_config(cfg["hq"], cfg["hkv"], cfg["d"], cfg["top_chunks"], cfg["top_groups"], cfg["sink"],
                        cfg["local"], dtype=cfg["dtype"])
    fake = 0x10000
    with pytest.raises(hga.HgaError) as ei:
        hga.hga_route_attend_noalloc(c, fake, 1024, 64, 4096, fake, fake, (fake, fake, 1024), (fake, fake, 1024),
                                     fake, fake, fake, fake)
    assert ei.value.status == hga.HGA_ERR_UNSUPPORTED
