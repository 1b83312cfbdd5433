"""Benchmark of the HGA routed-attention forward on one MI355X.

A step is one pass of the whole path over one layer of one synthetic input:
hga_build_summaries_range (group and chunk summaries of the chunks the step's
own positions close; the history's summaries are resident, built when their
chunks closed, as the pages keep them), then hga_route_attend (block queries,
chunk stage, group stage and exact routed attention), all on one stream with
every input already in HBM. The rate with every chunk's summaries rebuilt
each step is reported alongside. With at most
4 query heads per KV head hga_route_attend is one kernel; with more (the 64K
layer's 8) the step runs the router and the attention kernels, timed apart.
The 16K step through the separate hga_route and hga_attend calls is reported
alongside.

The workload is the 16,384-token training-segment shape (Qwen3-8B heads:
32 query / 8 KV heads, head_dim 128, bf16, 2,048 active queries over a
14,336-token history, top-16 chunks, top-64 groups, sink 64, local 128).
The same line also reports the 65,536-token Qwen3-30B-A3B-shaped layer with
its history in HBM and, separately, with its history in pinned host memory
(that rate includes the PCIe transfer of the routed set), and the
131,072-token long-evaluation layer with its history in pinned host memory.

It also reports the backward of the attention over the 16K workload's
2,048-query active segment (hga_attend_backward: dQ, and dK, dV of the
segment's keys; the history is detached) against bf16 MFMA peak, and one-token decoding (query block of one token, routing over
the resident summaries of the closed chunks, then attention) at the end of the
16K and 64K sequences for batches of sequences, as generated tokens per
second with the fused kernel's HBM roofline.

Output: one JSON line (see the keys below). ``roofline`` covers the kernel
that does the attention (the route-and-attend kernel, or the attention kernel
where routing runs apart): the attention's algorithmic flops or bytes over
that kernel's mean duration, measured with HIP events on the launch stream
over the timed steps; ``cpu_baseline`` is the CPU oracle on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # flop/s, MI355X dense bf16 MFMA
PEAK_F32_MFMA = 157.3e12

METRIC = "routed-attn query-tokens/sec per layer at 16K/64K; % of HBM or MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=160)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload index (default: the 16K segment)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 64K lines")
    ap.add_argument("--backward", action="store_true", help="only the backward line of --config")
    ap.add_argument("--decode-batch", type=int, default=0, metavar="B",
                    help="only the one-token decoding line of --config for a batch of B sequences")
    ap.add_argument("--host-tier", action="store_true",
                    help="main line with the history (tokens before the first query) in pinned host memory")
    ap.add_argument("--traffic-kib", type=float, nargs=2, default=None, metavar=("FETCH", "WRITE"),
                    help="attention kernel FETCH_SIZE and WRITE_SIZE per dispatch (KiB, as rocprofv3 "
                         "reports them) for the roofline traffic field")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size, to scale the HBM byte counters."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4}), flush=True)


def algorithmic(cfg, n_sel):
    """Attention flops and bytes of one launch from the kept selection.

    flops = 4 d x (attended query-key pairs) over all query heads;
    bytes = Q read + O write + per-(block, KV head) K/V rows of its token set.
    """
    d, G, hkv = cfg["d"], cfg["hq"] // cfg["hkv"], cfg["hkv"]
    nb = cfg["n_q"] // 64
    q0 = cfg["L"] - cfg["n_q"]
    esz = 2 if cfg["dtype"] == "bf16" else 4
    ns = n_sel.reshape(nb, hkv, 2)
    pairs = 0
    kv_rows = 0
    for b in range(nb):
        s = q0 + 64 * b
        ms = s // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        fixed = 64 * (a + ms - bb)
        for h in range(hkv):
            hist = fixed + cfg["group"] * int(ns[b, h, 1])
            pairs += G * (64 * hist + 64 * 65 // 2)
            kv_rows += hist + 64
    flops = 4.0 * d * pairs
    qo = 2.0 * cfg["hq"] * cfg["n_q"] * d * esz
    byts = qo + 2.0 * kv_rows * d * esz
    return flops, byts, pairs


def to_dev(a, dtype, dev):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


class Workload:
    """Device buffers and one step of the path for one configuration."""

    def __init__(self, cfg_id, split=0, fused=None):
        import torch

        import hierarchical_sparse_attention_hga_amd as hga
        import synth
        from hierarchical_sparse_attention_hga_amd.memory import split_to_host

        self.torch, self.hga = torch, hga
        self.cfg = cfg = synth.config(cfg_id)
        self.x = x = synth.make_inputs(cfg)
        self.c = hga.make_config(cfg["hq"], cfg["hkv"], cfg["d"], cfg["top_chunks"], cfg["top_groups"],
                                 cfg["sink"], cfg["local"], dtype=cfg["dtype"], group_size=cfg["group"])
        DEV = torch.device("cuda:0")
        L, nq, hkv, d = cfg["L"], cfg["n_q"], cfg["hkv"], cfg["d"]
        self.L, self.nq, self.q0 = L, nq, L - nq
        nb = nq // 64
        self.q, k, v = (to_dev(x[n], cfg["dtype"], DEV) for n in ("q", "k", "v"))
        self.gs = torch.empty(hkv, L // cfg["group"], d, device=DEV)
        self.cs = torch.empty(hkv, L // 64, d, device=DEV)
        self.ci = torch.empty(nb, hkv, cfg["top_chunks"], dtype=torch.int32, device=DEV)
        self.gi = torch.empty(nb, hkv, cfg["top_groups"], dtype=torch.int32, device=DEV)
        self.ns = torch.empty(nb, hkv, 2, dtype=torch.int32, device=DEV)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(cfg["hq"], nq, device=DEV)
        self.k_full = k
        self.split = split
        # one kernel exactly where hga_route_attend fuses (bf16, K/V on the
        # device, at most 256 query rows per item: G <= 4 for blocks of 64);
        # otherwise the two calls are timed apart
        if fused is None:
            fused = cfg["dtype"] == "bf16" and split == 0 and cfg["hq"] // hkv <= 4
        self.fused = fused
        self.n_stages = 2 if fused else 3
        self.pins = []
        self.ws, self.wsb = None, 0
        # the history's summaries are resident before the step (built when
        # their chunks closed); each step builds those of the chunks its own
        # positions close
        hga.hga_build_summaries(self.c, k, L, self.gs, self.cs)
        torch.cuda.synchronize()
        self.seg_chunks = (self.q0 // 64, L // 64)
        if split > 0:
            gpin, _, gs_t = split_to_host(self.gs, split // cfg["group"])
            self.gs_t = (gs_t[0], gs_t[1], split)
            kpin, _, self.k_t = split_to_host(k, split)
            vpin, _, self.v_t = split_to_host(v, split)
            self.pins = [gpin, kpin, vpin]
            self.wsb = hga.hga_workspace_size(self.c, L, nq, hga.HGA_WS_ATTEND_TIERED)
            self.ws = torch.empty(self.wsb, dtype=torch.uint8, device=DEV)
        else:
            self.gs_t, self.k_t, self.v_t = self.gs, k, v

    def step(self, ev=None, timed=-1):
        """One step; with ev, HIP events on the launch stream bracket stage
        `timed` (0 summaries, 1 routing or routing + attention, 2 attention)."""
        hga, c = self.hga, self.c

        def mark(stage, k):
            if ev is not None and stage == timed:
                ev[k].record()
        mark(0, 0)
        if self.split == 0:
            hga.hga_build_summaries_range(c, self.k_full, self.L, *self.seg_chunks, self.gs, self.cs)
        mark(0, 1)
        mark(1, 0)
        if self.fused:
            hga.hga_route_attend(c, self.q, self.q0, self.nq, self.L, self.cs, self.gs_t, self.k_t, self.v_t,
                                 self.ci, self.gi, self.ns, self.out, self.lse, self.ws, self.wsb)
            mark(1, 1)
        else:
            hga.hga_route(c, self.q, self.q0, self.nq, self.L, self.cs, self.gs_t, self.ci, self.gi, self.ns)
            mark(1, 1)
            mark(2, 0)
            hga.hga_attend(c, self.q, self.q0, self.nq, self.L, self.k_t, self.v_t, self.gi, self.ns,
                           self.out, self.lse, self.ws, self.wsb)
            mark(2, 1)

    # one step in SAMPLE_PERIOD carries a pair of timing events (measured: a
    # pair on every second step costs about 5% of the step, on every eighth
    # nothing measurable)
    SAMPLE_PERIOD = 8

    def run(self, steps, warmup):
        """Time `steps` steps. Every SAMPLE_PERIOD-th step brackets one stage
        with HIP events on the launch stream, the stages in turn; stage times
        are means over their own samples."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        per = self.SAMPLE_PERIOD
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        which = [(i // per) % self.n_stages if i % per == 0 else -1 for i in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i], which[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stage = [[evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(steps) if which[i] == j]
                 for j in range(self.n_stages)]   # us
        return wall, stage

    def free(self):
        for p in self.pins:
            p.free()


def source_sha256():
    """Digest of every kernel source (csrc/*.hip and *.h, in name order): a
    counter run is valid only for the sources it was taken on."""
    import glob
    import hashlib
    files = sorted(glob.glob(os.path.join(ROOT, "hierarchical_sparse_attention_hga_amd", "csrc", "*.hip")) +
                   glob.glob(os.path.join(ROOT, "hierarchical_sparse_attention_hga_amd", "csrc", "*.h")))
    return hashlib.sha256(b"".join(open(f, "rb").read() for f in files)).hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` ("route_attend_bf16", "attend_bf16" or
    "attend_backward", the latter summed over its kernels) from the committed
    rocprofv3 counter runs
    (profiles/<kernel>_<workload>.traffic.json), or None when they are missing
    or were taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if source_sha256() != rec["source_sha256"]:
        return None
    return 1024.0 * (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"])


def roofline(cfg, n_sel, attend_us, kernel, with_traffic=True):
    flops, byts, _ = algorithmic(cfg, n_sel)
    traffic = measured_traffic(cfg["name"], kernel) if with_traffic else None
    t_mfma = flops / PEAK_BF16
    t_hbm = byts / PEAK_HBM
    t = attend_us * 1e-6
    if t_mfma >= t_hbm:
        return {"kernel": kernel, "bound": "mfma", "achieved": flops / t / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": flops / t / PEAK_BF16, "traffic": traffic, "traffic_unit": "HBM bytes per launch",
                "algorithmic_flops": flops, "algorithmic_bytes": byts}
    return {"kernel": kernel, "bound": "hbm", "achieved": byts / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": byts / t / PEAK_HBM, "traffic": traffic, "traffic_unit": "HBM bytes per launch",
            "algorithmic_flops": flops, "algorithmic_bytes": byts}


def host_link_bytes(cfg, n_sel, group_idx, split):
    """Bytes one step moves across the host link on the host-tier path: K and V
    of every history chunk (below split) that some (block, KV head) needs (its
    sink and local chunks, the chunks of its kept groups), each once."""
    nb, hkv, g = cfg["n_q"] // 64, cfg["hkv"], cfg["group"]
    q0 = cfg["L"] - cfg["n_q"]
    ns = n_sel.reshape(nb, hkv, 2)
    gi = group_idx.reshape(nb, hkv, -1)
    need = [set() for _ in range(hkv)]
    for b in range(nb):
        ms = (q0 + 64 * b) // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        for h in range(hkv):
            need[h].update(m for m in list(range(a)) + list(range(bb, ms)) if m * 64 < split)
            need[h].update(int(j) * g // 64 for j in gi[b, h, :int(ns[b, h, 1])] if j >= 0 and int(j) * g < split)
    esz = 2 if cfg["dtype"] == "bf16" else 4
    return sum(len(n) for n in need) * 64 * cfg["d"] * esz * 2


def cpu_baseline(cfg_id, min_seconds=10.0):
    """The oracle timed on the host cores: summaries, routing and attention of
    every (block, KV head) of the layer, repeated until at least min_seconds
    of CPU work have run."""
    import oracle
    import synth
    cfg = synth.config(cfg_id)
    x = synth.make_inputs(cfg)
    f = {n: synth.to_f64(x[n], cfg["dtype"]) for n in ("q", "k", "v")}
    reps, t0 = 0, time.perf_counter()
    while True:
        sums = (oracle.summaries(cfg, f["k"]), oracle.abs_summaries(cfg, f["k"]))
        ci, gi, ns, dg = oracle.route(cfg, f["q"], f["k"], sums=sums)
        oracle.attend(cfg, f["q"], f["k"], f["v"], oracle.all_items(cfg), gi, ns[:, 1])
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": reps * cfg["n_q"] / el, "unit": "query-tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"float64 C oracle, whole layer ({cfg['n_q']} queries, all {cfg['hkv']} KV heads: "
                      f"summaries, routing, attention) repeated {reps}x in {el:.1f} s"}


class Result:
    """Timing of one workload: wall time of the timed steps and per-stage
    means and medians (us)."""

    def __init__(self, w, wall, stage):
        self.cfg, self.fused, self.wall = w.cfg, w.fused, wall
        self.ns = w.ns.cpu().numpy()
        self.split = w.split
        self.host_bytes = host_link_bytes(w.cfg, self.ns, w.gi.cpu().numpy(), w.split) if w.split else 0
        self.mean = [float(np.mean(x)) if x else float("nan") for x in stage]
        self.med = [float(np.median(x)) if x else float("nan") for x in stage]

    def stages(self, which):
        v = self.mean if which == "mean" else self.med
        if self.fused:
            return {"summaries": v[0], "route_attend": v[1]}
        return {"summaries": v[0], "route": v[1], "attend": v[2]}

    def roofline(self, with_traffic=True):
        if self.fused:
            return roofline(self.cfg, self.ns, self.mean[1], "route_attend_bf16", with_traffic)
        return roofline(self.cfg, self.ns, self.mean[2], "attend_bf16", with_traffic)


def stream_line(passes, warmup):
    """The 16K training-segment sequence with every position querying, run by
    hga_stream_forward in its 2,048-token segments (each: summaries of the
    chunks it closes, then routing and attention of its queries); query-tokens
    per second over whole passes."""
    import torch

    import hierarchical_sparse_attention_hga_amd as hga
    import synth
    cfg = synth.config(2, n_q=16384)
    x = synth.make_inputs(cfg)
    DEV = torch.device("cuda:0")
    L, hkv, d, g = cfg["L"], cfg["hkv"], cfg["d"], cfg["group"]
    c = hga.make_config(cfg["hq"], hkv, d, cfg["top_chunks"], cfg["top_groups"], cfg["sink"], cfg["local"],
                        dtype=cfg["dtype"], group_size=g)
    q, k, v = (to_dev(x[n], cfg["dtype"], DEV) for n in ("q", "k", "v"))
    gs = torch.empty(hkv, L // g, d, device=DEV)
    cs = torch.empty(hkv, L // 64, d, device=DEV)
    ci = torch.empty(L // 64, hkv, cfg["top_chunks"], dtype=torch.int32, device=DEV)
    gi = torch.empty(L // 64, hkv, cfg["top_groups"], dtype=torch.int32, device=DEV)
    ns = torch.empty(L // 64, hkv, 2, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(cfg["hq"], L, device=DEV)

    def one():
        hga.hga_stream_forward(c, q, k, v, L, 2048, cs, gs, ci, gi, ns, out, lse)
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(passes):
        one()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    return {"value": passes * L / el, "unit": "query-tokens/s", "ms_per_pass": el / passes * 1e3,
            "note": "16,384 positions all querying, 8 segments of 2,048: per segment the summaries of its 32 "
                    "chunks, then routing and attention of its queries against the committed history"}


def decode_bytes(cfg, pos, n_sel):
    """HBM bytes one (sequence, KV head) item of a one-token decoding step
    must move: the chunk summaries it scores (all candidates when the chunk
    stage selects), the group summaries of its kept chunks (when the group
    stage selects), K and V of its token set (fixed chunks, kept groups, the
    open chunk up to the token), its G queries and outputs (with LSE) and its
    index rows."""
    d, G, g = cfg["d"], cfg["hq"] // cfg["hkv"], cfg["group"]
    esz = 2 if cfg["dtype"] == "bf16" else 4
    ms = pos // 64
    a = min(cfg["sink"] // 64, ms)
    bb = max(ms - cfg["local"] // 64, a)
    ncand = bb - a
    nsc = int(n_sel[0])
    nsg = int(n_sel[1])
    rows = (ncand if 0 < nsc < ncand else 0) + (64 // g * nsc if 0 < nsg < 64 // g * nsc else 0)
    tokens = 64 * (a + ms - bb) + g * nsg + (pos - 64 * ms + 1)
    return (4 * d * rows + 2 * esz * d * tokens + 2 * G * d * esz + 4 * G
            + 4 * (cfg["top_chunks"] + cfg["top_groups"] + 2))


def decode_line(cfg_id, batch, steps, warmup):
    """One-token decoding steps over a batch of sequences at the end of
    workload cfg_id's sequence (position L - 1, history L - 1 tokens): per
    step, hga_route_attend with q_block 1 over the resident summaries of the
    closed chunks, given the workspace hga_workspace_size asks for (nonzero
    for few items: the attention then spreads each item over several
    workgroups). The batch is folded into the heads (sequence-major
    [batch x heads]); every sequence repeats the workload's K/V and last query
    at its own addresses. Summaries are built before timing (each closes once
    per 64 generated tokens). Timed with HIP events around one launch in eight on the
    launch stream."""
    import torch

    import hierarchical_sparse_attention_hga_amd as hga
    import synth
    base = synth.config(cfg_id)
    x = synth.make_inputs(base)
    DEV = torch.device("cuda:0")
    L, d, g = base["L"], base["d"], base["group"]
    hq, hkv = batch * base["hq"], batch * base["hkv"]
    c = hga.make_config(hq, hkv, d, base["top_chunks"], base["top_groups"], base["sink"], base["local"],
                        dtype=base["dtype"], group_size=g, q_block=1)
    k = to_dev(x["k"], base["dtype"], DEV).repeat(batch, 1, 1).contiguous()
    v = to_dev(x["v"], base["dtype"], DEV).repeat(batch, 1, 1).contiguous()
    q = to_dev(x["q"][:, -1:], base["dtype"], DEV).repeat(batch, 1, 1).contiguous()
    del x
    gs = torch.empty(hkv, L // g, d, device=DEV)
    cs = torch.empty(hkv, L // 64, d, device=DEV)
    ci = torch.empty(1, hkv, base["top_chunks"], dtype=torch.int32, device=DEV)
    gi = torch.empty(1, hkv, base["top_groups"], dtype=torch.int32, device=DEV)
    ns = torch.empty(1, hkv, 2, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(hq, 1, device=DEV)
    pos = L - 1
    hga.hga_build_summaries_range(c, k, L, 0, pos // 64, gs, cs)
    wsb = hga.hga_workspace_size(c, L, 1, hga.HGA_WS_ATTEND)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=DEV)

    def one():
        hga.hga_route_attend(c, q, pos, 1, L, cs, gs, k, v, ci, gi, ns, out, lse, ws, wsb)
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    per = Workload.SAMPLE_PERIOD
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if i % per == 0:
            evs[i][0].record()
        one()
        if i % per == 0:
            evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(0, steps, per)]))
    nsel = ns.cpu().numpy().reshape(hkv, 2)
    byts = float(sum(decode_bytes(base, pos, nsel[h]) for h in range(hkv)))
    # one kernel unless the block has more than two scoring rounds of chunk
    # candidates (then the router kernel, then the attention kernel) or the
    # attention spreads the items (router, ranges, merge)
    fused = (pos // 64 - base["sink"] // 64 - base["local"] // 64 <= 512 and base["hq"] // base["hkv"] <= 256
             and wsb == 0)
    kname = ("route_attend_bf16" if fused else
             "route_kernel + attend_split_bf16 + attend_combine" if wsb else "route_kernel + attend_bf16")
    traffic = measured_traffic(f"{base['name']}-decode-b{batch}", "route_attend_bf16") if fused else None
    del k, v, gs, cs, ws
    torch.cuda.empty_cache()
    return {"value": steps * batch / wall, "unit": "generated tokens/s", "kernel_us_mean": us,
            "ms_per_step": wall / steps * 1e3,
            "config": {"workload": f"{base['name']}-decode", "batch": batch, "history": pos,
                       "q_heads": base["hq"], "kv_heads": base["hkv"], "q_block": 1},
            "roofline": {"kernel": kname, "bound": "hbm", "achieved": byts / (us * 1e-6) / 1e9,
                         "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": byts / (us * 1e-6) / PEAK_HBM,
                         "traffic": traffic, "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": byts}}


def backward_flops(cfg, n_sel, group_idx):
    """Algorithmic flops of one backward call: S and dP once over every
    attended (query, key) pair, dQ over every pair, and dK, dV over the pairs
    whose key lies in the call's own positions (history keys are detached):
    2 d flops per pair and product, so 6 d per pair plus 4 d per segment pair."""
    d, G, hkv, g = cfg["d"], cfg["hq"] // cfg["hkv"], cfg["hkv"], cfg["group"]
    nb = cfg["n_q"] // 64
    q0 = cfg["L"] - cfg["n_q"]
    ns = n_sel.reshape(nb, hkv, 2)
    gi = group_idx.reshape(nb, hkv, -1)
    pairs = pairs_seg = 0
    for b in range(nb):
        s = q0 + 64 * b
        ms = s // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        fixed = list(range(a)) + list(range(bb, ms))
        diag = 64 * 65 // 2
        for h in range(hkv):
            kept = gi[b, h, :int(ns[b, h, 1])]
            pairs += G * (64 * (64 * len(fixed) + g * len(kept)) + diag)
            seg_fixed = sum(1 for m in fixed if 64 * m >= q0)
            seg_kept = int((kept * g >= q0).sum())
            pairs_seg += G * (64 * (64 * seg_fixed + g * seg_kept) + diag)
    return 2.0 * d * (3 * pairs + 2 * pairs_seg)


def backward_line(cfg_id, steps, warmup):
    """hga_attend_backward over the active segment of workload cfg_id (its n_q
    queries; keys before q_start are detached history), after one forward
    that provides the kept groups, output and LSE; timed with HIP events on
    the launch stream around one call in Workload.SAMPLE_PERIOD."""
    import torch

    hga = __import__("hierarchical_sparse_attention_hga_amd")
    w = Workload(cfg_id)
    w.step()
    torch.cuda.synchronize()
    cfg = w.cfg
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1337)
    dout = torch.randn(w.q.shape, generator=gen, device="cuda:0").to(torch.bfloat16)
    dq = torch.empty_like(w.q)
    dk = torch.empty(cfg["hkv"], w.nq, cfg["d"], dtype=torch.bfloat16, device="cuda:0")
    dv = torch.empty_like(dk)
    wsb = hga.hga_workspace_size(w.c, w.L, w.nq, hga.HGA_WS_BACKWARD)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")

    def one():
        hga.hga_attend_backward(w.c, w.q, w.q0, w.nq, w.L, w.k_full, w.v_t, w.gi, w.ns, w.out, w.lse, dout,
                                dq, dk, dv, ws, wsb)
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    per = Workload.SAMPLE_PERIOD
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if i % per == 0:
            evs[i][0].record()
        one()
        if i % per == 0:
            evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = float(np.mean([evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(0, steps, per)]))
    flops = backward_flops(cfg, w.ns.cpu().numpy(), w.gi.cpu().numpy())
    w.free()
    return {"value": steps * cfg["n_q"] / wall, "unit": "query-tokens/s", "call_us_mean": us,
            "ms_per_step": wall / steps * 1e3,
            "config": {"workload": f"{cfg['name']}-backward", "n_q": cfg["n_q"], "history": w.q0},
            "roofline": {"kernel": "hga_attend_backward (bwd_dq_kernel, then bwd_dkv_kernel)", "bound": "mfma",
                         "achieved": flops / (us * 1e-6) / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                         "frac": flops / (us * 1e-6) / PEAK_BF16,
                         "traffic": measured_traffic(f"{cfg['name']}-backward", "attend_backward"),
                         "traffic_unit": "HBM bytes per call (both kernels)", "algorithmic_flops": flops}}


def route_bytes(cfg, n_sel):
    """HBM bytes of hga_route over every (block, KV head) of the workload: the
    block's G x 64 query rows, the chunk summaries it scores (all candidates,
    when the chunk stage selects), the group summaries of its kept chunks
    (when the group stage selects), and its index rows."""
    d, G, hkv, g = cfg["d"], cfg["hq"] // cfg["hkv"], cfg["hkv"], cfg["group"]
    esz = 2 if cfg["dtype"] == "bf16" else 4
    nb = cfg["n_q"] // 64
    q0 = cfg["L"] - cfg["n_q"]
    ns = n_sel.reshape(nb, hkv, 2)
    rows = 0
    for b in range(nb):
        ms = (q0 + 64 * b) // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        for h in range(hkv):
            nsc, nsg = int(ns[b, h, 0]), int(ns[b, h, 1])
            rows += (bb - a if 0 < nsc < bb - a else 0) + (64 // g * nsc if 0 < nsg < 64 // g * nsc else 0)
    return (nb * hkv * G * 64 * d * esz + 4.0 * d * rows
            + 4 * nb * hkv * (cfg["top_chunks"] + cfg["top_groups"] + 2))


def stage_hbm(cfg_id, reps=20):
    """Achieved HBM rates of the summary build (every chunk of the sequence)
    and of the router alone: algorithmic bytes over the mean of reps
    back-to-back calls (HIP events on the launch stream around all of them)."""
    import torch
    w = Workload(cfg_id)
    cfg, hga = w.cfg, w.hga

    def mean_us(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    sum_us = mean_us(lambda: hga.hga_build_summaries(w.c, w.k_full, w.L, w.gs, w.cs))
    route_us = mean_us(lambda: hga.hga_route(w.c, w.q, w.q0, w.nq, w.L, w.cs, w.gs_t, w.ci, w.gi, w.ns))
    esz = 2 if cfg["dtype"] == "bf16" else 4
    d, hkv, L = cfg["d"], cfg["hkv"], cfg["L"]
    sum_bytes = hkv * L * d * esz + 4.0 * hkv * (L // cfg["group"] + L // 64) * d
    r_bytes = route_bytes(cfg, w.ns.cpu().numpy())
    w.free()
    out = {}
    for name, byts, us in (("summaries_full_build", sum_bytes, sum_us), ("routing", r_bytes, route_us)):
        out[name] = {"us": us, "algorithmic_bytes": byts, "achieved_GBps": byts / (us * 1e-6) / 1e9,
                     "frac_of_hbm_peak": byts / (us * 1e-6) / PEAK_HBM}
    return out


def full_summary_us(cfg_id, reps=20):
    """Mean time of hga_build_summaries over every chunk of workload cfg_id's
    sequence (HIP events on the launch stream)."""
    import torch
    w = Workload(cfg_id)
    for _ in range(3):
        w.hga.hga_build_summaries(w.c, w.k_full, w.L, w.gs, w.cs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        w.hga.hga_build_summaries(w.c, w.k_full, w.L, w.gs, w.cs)
    e1.record()
    torch.cuda.synchronize()
    w.free()
    return e0.elapsed_time(e1) / reps * 1e3


def synth_config(cfg_id):
    import synth
    return synth.config(cfg_id)


def measure(cfg_id, steps, warmup, split=0, fused=None):
    w = Workload(cfg_id, split, fused)
    wall, stage = w.run(steps, warmup)
    r = Result(w, wall, stage)
    w.free()
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by KV head, each GPU running its heads' items with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.init()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.backward:
        print(json.dumps(backward_line(args.config, args.steps, args.warmup)), flush=True)
        return
    if args.decode_batch:
        print(json.dumps(decode_line(args.config, args.decode_batch, args.steps, args.warmup)), flush=True)
        return
    split = 0
    if args.host_tier:
        import synth
        split = synth.config(args.config)["tier_split"] or (synth.config(args.config)["L"] -
                                                            synth.config(args.config)["n_q"])
    main_r = measure(args.config, args.steps, args.warmup, split=split)
    cfg = main_r.cfg
    value = args.steps * cfg["n_q"] / main_r.wall
    line = {
        "metric": METRIC, "value": value, "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_r.wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded; Qwen3-shaped heads, rank-8 shared component, planted groups)",
        "config": {"workload": cfg["name"], "seq_len": cfg["L"], "n_q": cfg["n_q"], "q_heads": cfg["hq"],
                   "kv_heads": cfg["hkv"], "head_dim": cfg["d"], "top_chunks": cfg["top_chunks"],
                   "top_groups": cfg["top_groups"], "sink": cfg["sink"], "local": cfg["local"],
                   "kv_residency": "host-pinned history" if split else "hbm"},
        "stages_us_mean": main_r.stages("mean"),
        "stages_us_median": main_r.stages("median"),
        "roofline": main_r.roofline(),
    }
    if split:
        line["host_link_bytes_per_step"] = main_r.host_bytes
    if not args.no_extra:
        extra = {}
        # the rate with the summaries prebuilt (kept resident, as the pages do):
        # query tokens over the routing + gather + attention stage times
        rest = sum(main_r.mean[1:])
        extra["summaries_prebuilt"] = {
            "value": cfg["n_q"] / (rest * 1e-6), "unit": "query-tokens/s",
            "note": "n_q / (mean routing + gather + attention stage time); summary build excluded"}
        if not split:
            full_us = full_summary_us(args.config)
            extra["full_summary_rebuild"] = {
                "value": cfg["n_q"] / ((full_us + rest) * 1e-6), "unit": "query-tokens/s",
                "summaries_us": full_us,
                "note": "the step with the summaries of every chunk of the sequence rebuilt (history included) "
                        "instead of only the chunks the step's positions close"}
        half = max(args.steps // 2, 5)
        extra["stage_hbm"] = stage_hbm(args.config)
        if main_r.fused:
            sep = measure(args.config, half, args.warmup, fused=False)
            extra["separate_calls"] = {
                "value": half * sep.cfg["n_q"] / sep.wall, "unit": "query-tokens/s",
                "note": "same step through hga_route then hga_attend; roofline of the attention kernel alone",
                "stages_us_mean": sep.stages("mean"), "roofline": sep.roofline(with_traffic=False)}
        if args.config == 2:
            extra["16k_streamed_2048_segments"] = stream_line(max(args.steps // 6, 3), 2)
        if args.config != 3:
            r3 = measure(3, half, args.warmup)
            extra["64k_hbm"] = {"value": half * r3.cfg["n_q"] / r3.wall, "unit": "query-tokens/s",
                                "stages_us_mean": r3.stages("mean"), "roofline": r3.roofline()}
            rh = measure(3, 24, 2, split=r3.cfg["tier_split"])
            extra["64k_host_tier_pcie_inclusive"] = {
                "value": 24 * rh.cfg["n_q"] / rh.wall, "unit": "query-tokens/s",
                "note": "history K/V and group summaries in pinned host memory; each history chunk any block "
                        "needs crosses the host link once per step into an HBM cache, then attention",
                "host_link_bytes_per_step": rh.host_bytes,
                "stages_us_mean": rh.stages("mean")}
            r4 = measure(4, 24, 2, split=synth_config(4)["tier_split"])
            extra["128k_host_tier_pcie_inclusive"] = {
                "value": 24 * r4.cfg["n_q"] / r4.wall, "unit": "query-tokens/s",
                "note": "the 131,072-token long-evaluation layer (Qwen3-8B heads, top-64 chunks, top-512 groups, "
                        "64 planted needle groups per head): history K/V and group summaries in pinned host "
                        "memory, the final 2,048 queries in HBM; each history chunk any block needs crosses "
                        "the host link once per step",
                "host_link_bytes_per_step": r4.host_bytes,
                "stages_us_mean": r4.stages("mean")}
        extra["backward_16k_segment"] = backward_line(2, 80, 5)
        extra["decode_16k_batch64"] = decode_line(2, 64, 80, 5)
        extra["decode_16k_single_sequence"] = decode_line(2, 1, 80, 5)
        extra["decode_64k_batch32"] = decode_line(3, 32, 80, 5)
        line["also"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
