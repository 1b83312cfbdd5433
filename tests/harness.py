"""Shared helpers of the GPU tests: device upload, pinned host tiers, one call
of the whole path through the C ABI, and the comparison rules."""
from __future__ import annotations

import functools

import numpy as np
import torch

import hierarchical_sparse_attention_hga_amd as hga
from hierarchical_sparse_attention_hga_amd.memory import split_to_host
import oracle
import synth

DEV = torch.device("cuda:0")

# Output tolerances against the float64 oracle. bfloat16: the workload's
# stated bar (max-abs 2e-2, mean-abs 1e-3). float32: scores and softmax in
# float32 over at most a few thousand tokens keep the relative error near
# 1e-6; the bar leaves two orders of magnitude of room.
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=1e-3, lse_abs=1e-3),
       "f32": dict(max_abs=1e-4, mean_abs=1e-5, lse_abs=1e-4)}


def to_dev(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def hga_cfg(cfg, out_f32=False):
    """The library config of a workload; ``out_f32`` (bfloat16 workloads) asks
    for the float32 output mode (HGA_BF16_F32OUT)."""
    assert not out_f32 or cfg["dtype"] == "bf16"
    return hga.make_config(cfg["hq"], cfg["hkv"], cfg["d"], cfg["top_chunks"], cfg["top_groups"],
                           cfg["sink"], cfg["local"], dtype="bf16_f32out" if out_f32 else cfg["dtype"],
                           group_size=cfg["group"],
                           q_block=cfg["q_block"], softmax_scale=cfg.get("softmax_scale") or 0.0)


def gpu_run(cfg, x, split=0, group_idx=None, n_sel=None, q_start=None, seq_len=None, fused=False,
            capacity=None, spread=False, out_f32=False):
    """Run summaries, routing and attention through the C ABI.

    ``group_idx``/``n_sel`` (numpy, [nb][hkv][kg] / [nb][hkv][2]) replace the
    GPU routing as the attention's input when given. With ``fused`` routing
    and attention run through hga_route_attend. With ``capacity`` (a multiple
    of 64 above the sequence, as a decoding cache is), K/V and the summary
    buffers hold that many tokens, every row past the sequence is NaN, and only
    the summaries of the sequence's whole chunks are built. With ``spread`` the
    call gets the workspace hga_workspace_size(HGA_WS_ATTEND) asks for (asserted
    nonzero), with which calls of few items spread each item's tiles over
    several workgroups. With ``out_f32`` the output is written in float32
    (HGA_BF16_F32OUT). Returns numpy arrays.
    """
    assert not (fused and group_idx is not None)
    c = hga_cfg(cfg, out_f32)
    dt = cfg["dtype"]
    L = cfg["L"] if seq_len is None else seq_len
    nq = cfg["n_q"]
    q0 = L - nq if q_start is None else q_start
    nb, hkv, d, g = nq // cfg["q_block"], cfg["hkv"], cfg["d"], cfg["group"]
    q, k, v = to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt)
    L_seq = L
    if capacity is not None:
        assert capacity % 64 == 0 and capacity >= L and seq_len is None and q_start is None
        pad = lambda t: torch.cat([t, torch.full((hkv, capacity - L, d), float("nan"), dtype=t.dtype,
                                                 device=DEV)], dim=1).contiguous()
        k, v, L = pad(k), pad(v), capacity
    gs = torch.full((hkv, L // g, d), float("nan"), device=DEV)
    cs = torch.full((hkv, L // 64, d), float("nan"), device=DEV)
    ci = torch.full((nb, hkv, cfg["top_chunks"]), -7, dtype=torch.int32, device=DEV)
    gi = torch.full((nb, hkv, cfg["top_groups"]), -7, dtype=torch.int32, device=DEV)
    ns = torch.full((nb, hkv, 2), -7, dtype=torch.int32, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=DEV)
    lse = torch.empty(cfg["hq"], nq, device=DEV)
    if capacity is not None:
        hga.hga_build_summaries_range(c, k, L, 0, L_seq // 64, gs, cs)
    else:
        hga.hga_build_summaries(c, k, L, gs, cs)
    pins = []
    if split > 0:
        gpin, _, gs_t = split_to_host(gs, split // g)
        gs_t = (gs_t[0], gs_t[1], split)          # the group-summary split is counted in tokens
        kpin, _, k_t = split_to_host(k, split)
        vpin, _, v_t = split_to_host(v, split)
        pins = [gpin, kpin, vpin]
    else:
        gs_t, k_t, v_t = gs, k, v
    ws = None
    wsb = 0
    if split > 0:
        wsb = hga.hga_workspace_size(c, L, nq, hga.HGA_WS_ATTEND_TIERED)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    elif spread:
        wsb = hga.hga_workspace_size(c, L, nq, hga.HGA_WS_ATTEND)
        assert wsb > 0
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    if fused:
        hga.hga_route_attend(c, q, q0, nq, L, cs, gs_t, k_t, v_t, ci, gi, ns, out, lse, ws, wsb)
    else:
        hga.hga_route(c, q, q0, nq, L, cs, gs_t, ci, gi, ns)
        gi_in, ns_in = gi, ns
        if group_idx is not None:
            gi_in = torch.from_numpy(np.ascontiguousarray(group_idx, dtype=np.int32)).to(DEV)
            ns_in = torch.from_numpy(np.ascontiguousarray(n_sel, dtype=np.int32)).to(DEV)
        hga.hga_attend(c, q, q0, nq, L, k_t, v_t, gi_in, ns_in, out, lse, ws, wsb)
    torch.cuda.synchronize()
    res = dict(gs=gs.cpu().numpy(), cs=cs.cpu().numpy(), chunk_idx=ci.cpu().numpy(),
               group_idx=gi.cpu().numpy(), n_sel=ns.cpu().numpy(),
               out=out.float().cpu().numpy().astype(np.float64), lse=lse.cpu().numpy().astype(np.float64))
    for p in pins:
        p.free()
    return res


@functools.lru_cache(maxsize=4)
def inputs(cfg_id, **over):
    cfg = synth.config(cfg_id, **over)
    x = synth.make_inputs(cfg)
    f = {n: synth.to_f64(x[n], cfg["dtype"]) for n in ("q", "k", "v")}
    return cfg, x, f


def oracle_route(cfg, f):
    sums = (oracle.summaries(cfg, f["k"]), oracle.abs_summaries(cfg, f["k"]))
    return oracle.route(cfg, f["q"], f["k"], sums=sums)


def check_routing(cfg, gpu, ref, f):
    """The GPU's routing of every item against the oracle's ``ref`` (from
    oracle_route on the float64 inputs ``f``).

    A certified boundary (gap above twice the bound eps) has one correct
    answer: the GPU's kept set must equal the oracle's. Where a boundary is
    not certified several selections are correct, and the GPU's must be one of
    them: oracle.valid_selection over the oracle's scores of every candidate
    (for the group stage, the groups of the chunks the GPU kept). Exact ties
    are uncertified boundaries too (gap 0); the callers assert that the GPU's
    sets equal the oracle's there as well, which is the lower-index rule.
    Returns (items, uncertified boundaries, items whose kept sets differ from
    the oracle's)."""
    ci_r, gi_r, ns_r, dg = ref
    kc, kg = cfg["top_chunks"], cfg["top_groups"]
    n_items = ci_r.shape[0]
    ci_g = gpu["chunk_idx"].reshape(n_items, kc)
    gi_g = gpu["group_idx"].reshape(n_items, kg)
    ns_g = gpu["n_sel"].reshape(n_items, 2)
    cert = [(oracle.certified(dg[n], "chunk"), oracle.certified(dg[n], "group")) for n in range(n_items)]
    loose = [n for n in range(n_items) if not (cert[n][0] and cert[n][1])]
    uncert = sum((not cc) + (not cg) for cc, cg in cert)
    tables = {}
    if loose:
        items = oracle.all_items(cfg)
        csc, gsc, eps = oracle.route_scores(cfg, f["q"], f["k"], [items[n] for n in loose])
        tables = {n: (csc[i], gsc[i], eps[i]) for i, n in enumerate(loose)}
    gpc = cfg["chunk"] // cfg["group"]
    mism = 0
    for n in range(n_items):
        cc, cg = cert[n]
        nsc, nsg = int(ns_g[n, 0]), int(ns_g[n, 1])
        same_c = np.array_equal(ci_g[n], ci_r[n]) and nsc == ns_r[n, 0]
        same_g = np.array_equal(gi_g[n], gi_r[n]) and nsg == ns_r[n, 1]
        mism += int(not (same_c and same_g))
        if cc:
            assert same_c, f"item {n}: certified chunk set differs: {ci_g[n]} vs {ci_r[n]}"
        if cc and cg:
            assert same_g, f"item {n}: certified group set differs: {gi_g[n]} vs {gi_r[n]}"
        if n in tables:
            csc, gsc, eps = tables[n]
            kept_c = ci_g[n][:nsc]
            assert np.all(ci_g[n][nsc:] == -1) and np.all(gi_g[n][nsg:] == -1), f"item {n}: padding"
            assert np.all(np.diff(kept_c) > 0) and np.all(np.diff(gi_g[n][:nsg]) > 0), f"item {n}: not ascending"
            assert oracle.valid_selection(csc, kept_c, kc, eps[0]), \
                f"item {n}: chunk set {kept_c} is not a correct selection at its uncertified boundary"
            mask = np.full(gsc.shape, np.nan)
            for m in kept_c:
                mask[m * gpc:(m + 1) * gpc] = gsc[m * gpc:(m + 1) * gpc]
            assert oracle.valid_selection(mask, gi_g[n][:nsg], kg, eps[1]), \
                f"item {n}: group set {gi_g[n][:nsg]} is not a correct selection at its uncertified boundary"
    return n_items, uncert, mism


def item_rows(cfg, out, items):
    """Gather [n][G][B][d] rows of a [Hq][n_q][d] array for (b, h) items."""
    G, B = cfg["hq"] // cfg["hkv"], cfg["q_block"]
    return np.stack([np.stack([out[h * G + r, b * B:(b + 1) * B] for r in range(G)]) for b, h in items])


def bf16_round(a):
    """float32 values rounded to bfloat16 (to nearest, ties to even), as
    float64."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_half_spacing(o):
    """Half the gap from each bfloat16 value to the next one away from zero:
    the most its own round-to-nearest can have moved it."""
    _, e = np.frexp(np.abs(o))
    return np.ldexp(1.0, e - 9)


def check_outputs(cfg, gpu, items, ref_out, ref_lse, beyond_output_rounding=False):
    """Bars of TOL on the outputs and the LSE of the given items.

    With ``beyond_output_rounding`` (bfloat16 only) each output's error is
    first reduced by its own final rounding to bfloat16 (bf16_half_spacing):
    over a token set of a few tokens the output is not averaged down, and the
    storage rounding of a value near 1 alone is ~1e-3 on average, the whole
    mean-abs bar; what remains bounds the arithmetic error before it."""
    tol = TOL[cfg["dtype"]]
    o = item_rows(cfg, gpu["out"], items)
    l = item_rows(cfg, gpu["lse"][..., None], items)[..., 0]
    err = np.abs(o - ref_out)
    if beyond_output_rounding:
        assert cfg["dtype"] == "bf16"
        err = np.maximum(err - bf16_half_spacing(o), 0.0)
    assert np.isfinite(o).all()
    max_abs, mean_abs = float(err.max()), float(err.mean())
    lerr = float(np.abs(l - ref_lse).max())
    assert max_abs <= tol["max_abs"], f"max abs error {max_abs}"
    assert mean_abs <= tol["mean_abs"], f"mean abs error {mean_abs}"
    assert lerr <= tol["lse_abs"], f"lse error {lerr}"
    return max_abs, mean_abs, lerr
