"""Benchmark of the HGA routed-attention forward on one MI355X.

A step is one pass of the whole path over one layer of one synthetic input:
hga_build_summaries_range (group and chunk summaries of the chunks the step's
own positions close; the history's summaries are resident, built when their
chunks closed, as the pages keep them), then hga_route_attend (block queries,
chunk stage, group stage and exact routed attention), all on one stream with
every input already in HBM. With at most 4 query heads per KV head
hga_route_attend is one kernel; with more (the 64K layer's 8) the step runs
the router and the attention kernels, timed apart.

`value` is the workload's query tokens over the mean duration of the timed
steps with the caches flushed: each of the timed steps runs after a 512 MiB
buffer is written (outside its pair of HIP events on the launch stream), so
the L2 caches and the 256 MB Infinity Cache hold none of the step's data, as
in a model where the other layers' weights and activations pass through the
caches between two calls of this layer. `value_warm` is the same steps run
back to back (wall clock between two device synchronizations), with the
layer's data left in the caches by the previous step. Then every stage is
timed call by call with HIP event pairs, warm and flushed; each reports mean,
median, p10 and p90.

The workload is the 16,384-token training-segment shape (Qwen3-8B heads:
32 query / 8 KV heads, head_dim 128, bf16, 2,048 active queries over a
14,336-token history, top-16 chunks, top-64 groups, sink 64, local 128).
`also` reports the same figures for the tiny float32 1K workload, the
Qwen3-8B 4K layer and the 65,536-token Qwen3-30B-A3B-shaped layer with its
history in HBM; the 64K and 131,072-token layers with their history in
pinned host memory (PCIe-inclusive, with the bytes they move over the host
link and the box's measured pinned host-to-device rate); the summary build
and the router against HBM; the 16K step through the separate calls; the 16K
sequence streamed in segments; the backward of the attention over the 16K
segment; and one-token decoding at the end of the 16K and 64K sequences.

``roofline`` covers the kernel that does the attention (the route-and-attend
kernel, or the attention kernel where routing runs apart): the attention's
algorithmic flops or bytes over that kernel's mean warm duration;
``cpu_baseline`` is the CPU oracle on the same workload, per stage, on all
host threads and on one.
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
PEAK_F32 = 157.3e12        # flop/s, MI355X float32 vector
PEAK_HOST_LINK = 64e9      # B/s, PCIe 5.0 x16 per direction (nominal)

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
    ap.add_argument("--cached-host-tier", action="store_true",
                    help="only the lines of --config through the persistent host-tier cache (planted groups shared "
                         "by all blocks, and a separate set per 4 blocks)")
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


_FLUSH = []


def cache_flusher(mib=512):
    """A call that writes `mib` MiB of device memory: more than the 256 MB
    Infinity Cache and every L2, so the next call finds none of its data
    cached (the buffer is allocated once)."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0"))
    buf = _FLUSH[0]
    return lambda: buf.fill_(1)


def event_us(call, n, flush=None, warm=2):
    """Durations (us) of n calls, each bracketed by a pair of HIP events on
    the current stream (the stream the library launches on), after `warm`
    untimed calls; with flush, it runs before each call, outside the pair."""
    import torch
    for _ in range(warm):
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]


def stats(us):
    """Mean, median, p10 and p90 of a list of durations (us)."""
    a = np.asarray(us, dtype=np.float64)
    assert a.size > 0 and np.isfinite(a).all()
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def timed_calls(call, steps, warmup, samples=None):
    """Wall-clock time of `steps` calls back to back, then event statistics
    of `samples` (default max(steps, 20)) warm calls and as many with the
    caches flushed before each."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = samples or max(steps, 20)
    return wall, stats(event_us(call, n)), stats(event_us(call, n, cache_flusher()))


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

    def stage_calls(self):
        """The step's stages in order, as (name, call) pairs: the summaries of
        the chunks the step's positions close, then routing and attention in
        one call (one kernel) or in two."""
        hga, c = self.hga, self.c
        calls = []
        if self.split == 0:
            calls.append(("summaries", lambda: hga.hga_build_summaries_range(c, self.k_full, self.L, *self.seg_chunks,
                                                                             self.gs, self.cs)))
        if self.fused:
            calls.append(("route_attend", lambda: hga.hga_route_attend(
                c, self.q, self.q0, self.nq, self.L, self.cs, self.gs_t, self.k_t, self.v_t, self.ci, self.gi,
                self.ns, self.out, self.lse, self.ws, self.wsb)))
        else:
            calls.append(("route", lambda: hga.hga_route(c, self.q, self.q0, self.nq, self.L, self.cs, self.gs_t,
                                                         self.ci, self.gi, self.ns)))
            calls.append(("attend", lambda: hga.hga_attend(c, self.q, self.q0, self.nq, self.L, self.k_t, self.v_t,
                                                           self.gi, self.ns, self.out, self.lse, self.ws, self.wsb)))
        return calls

    def step(self):
        for _, call in self.stage_calls():
            call()

    def run(self, steps, warmup, samples):
        """Time `steps` steps back to back (wall clock between two device
        synchronizations), then every stage and the whole step with HIP event
        pairs on the launch stream: `samples` calls back to back (warm), and
        as many with a 512 MiB buffer written before each (the L2 caches and
        the 256 MB Infinity Cache then hold none of the step's data)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        stages = {"warm": {}, "flushed": {}}
        flush = cache_flusher()
        for name, call in self.stage_calls() + [("step", self.step)]:
            stages["warm"][name] = event_us(call, samples)
            # the timed steps of the headline rate: exactly `steps` of them
            stages["flushed"][name] = event_us(call, steps if name == "step" else samples, flush)
        return wall, stages

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


def measured_traffic(workload, kernel, flushed=False):
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
    sfx = "_after_flush" if flushed else ""
    return 1024.0 * (rec["fetch_kib" + sfx] * rec["fetch_factor"] + rec["write_kib" + sfx] * rec["write_factor"])


def roofline(cfg, n_sel, attend_us, kernel, with_traffic=True, flushed=False):
    """The attention's algorithmic flops and bytes over the mean launch
    duration of the kernel that runs it, against whichever MI355X peak binds
    (bf16 MFMA or HBM; the float32 path against the float32 peak)."""
    flops, byts, _ = algorithmic(cfg, n_sel)
    traffic = measured_traffic(cfg["name"], kernel, flushed) if with_traffic else None
    peak_flops = PEAK_BF16 if cfg["dtype"] == "bf16" else PEAK_F32
    t_mfma = flops / peak_flops
    t_hbm = byts / PEAK_HBM
    t = attend_us * 1e-6
    base = {"kernel": kernel, "traffic": traffic, "traffic_unit": "HBM bytes per launch",
            "algorithmic_flops": flops, "algorithmic_bytes": byts, "kernel_us_mean": attend_us}
    if t_mfma >= t_hbm:
        return {"bound": "mfma" if cfg["dtype"] == "bf16" else "alu", "achieved": flops / t / 1e12,
                "peak": peak_flops / 1e12, "unit": "TFLOP/s", "frac": flops / t / peak_flops, **base}
    return {"bound": "hbm", "achieved": byts / t / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": byts / t / PEAK_HBM, **base}


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


def cpu_baseline(cfg_id, seconds=10.0, sample_blocks=4):
    """The oracle timed on the host cores, per stage: summaries of every chunk
    of the sequence, routing and attention of the (block, KV head) items.

    All threads: the whole layer, repeated for about `seconds`. One thread: the
    summaries once, routing and attention of the items of `sample_blocks`
    blocks spread over the layer (all KV heads), scaled to the layer by item
    count. query-tokens/s = n_q / (summaries + routing + attention)."""
    import oracle
    import synth
    cfg = synth.config(cfg_id)
    x = synth.make_inputs(cfg)
    f = {n: synth.to_f64(x[n], cfg["dtype"]) for n in ("q", "k", "v")}
    items = oracle.all_items(cfg)
    nthreads = oracle.threads()

    def stages(its, reps_for=None):
        t = {"summaries": 0.0, "routing": 0.0, "attention": 0.0}
        reps = 0
        t_end = time.perf_counter() + (reps_for or 0.0)
        while True:
            t0 = time.perf_counter()
            sums = (oracle.summaries(cfg, f["k"]), oracle.abs_summaries(cfg, f["k"]))
            t1 = time.perf_counter()
            ci, gi, ns, _ = oracle.route(cfg, f["q"], f["k"], items=its, sums=sums)
            t2 = time.perf_counter()
            oracle.attend(cfg, f["q"], f["k"], f["v"], its, gi, ns[:, 1])
            t3 = time.perf_counter()
            t["summaries"] += t1 - t0
            t["routing"] += t2 - t1
            t["attention"] += t3 - t2
            reps += 1
            if reps_for is None or time.perf_counter() >= t_end:
                break
        return {k: v / reps for k, v in t.items()}, reps

    full, reps = stages(items, seconds)
    nb = cfg["n_q"] // cfg["q_block"]
    blocks = sorted(set(int(round(i * (nb - 1) / max(sample_blocks - 1, 1))) for i in range(sample_blocks)))
    sample = [(b, h) for b in blocks for h in range(cfg["hkv"])]
    oracle.set_threads(1)
    try:
        one, _ = stages(sample)
    finally:
        oracle.set_threads(nthreads)
    scale = len(items) / len(sample)
    one = {"summaries": one["summaries"], "routing": one["routing"] * scale, "attention": one["attention"] * scale}
    rate = lambda t: cfg["n_q"] / sum(t.values())
    return {"value": rate(full), "unit": "query-tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"float64 C oracle on {cfg['name']}: the whole layer ({cfg['n_q']} queries, all "
                      f"{cfg['hkv']} KV heads; summaries of every chunk, routing, attention) repeated {reps}x on "
                      f"{nthreads} threads; one thread: summaries, then routing and attention of blocks {blocks} "
                      f"(all KV heads) scaled to the layer by item count",
            "stages_s": full,
            "one_thread": {"value": rate(one), "unit": "query-tokens/s", "cores": 1, "stages_s": one}}


class Result:
    """Timing of one workload: wall time of the timed steps and per-stage
    statistics (us), warm and with the caches flushed."""

    def __init__(self, w, wall, stages, steps):
        self.cfg, self.fused, self.wall, self.steps = w.cfg, w.fused, wall, steps
        self.ns = w.ns.cpu().numpy()
        self.gi = w.gi.cpu().numpy()
        self.split = w.split
        self.host_bytes = host_link_bytes(w.cfg, self.ns, self.gi, w.split) if w.split else 0
        self.warm = {k: stats(v) for k, v in stages["warm"].items()}
        self.flushed = {k: stats(v) for k, v in stages["flushed"].items()}

    @property
    def value(self):
        """n_q over the mean flushed step (the timed steps)."""
        return self.cfg["n_q"] / (self.flushed["step"]["mean"] * 1e-6)

    @property
    def value_warm(self):
        """n_q x steps over the wall clock of the warm steps, back to back."""
        return self.steps * self.cfg["n_q"] / self.wall

    def attention_stage(self):
        return "route_attend" if self.fused else "attend"

    def kernel_name(self):
        if self.cfg["dtype"] != "bf16":
            return "attend_f32"
        return "route_attend_bf16" if self.fused else "attend_bf16"

    def roofline(self, flushed=True, with_traffic=True):
        st = (self.flushed if flushed else self.warm)[self.attention_stage()]
        # the counters are of the all-HBM kernels; the host-tier path runs another instantiation
        return roofline(self.cfg, self.ns, st["mean"], self.kernel_name(), with_traffic and not self.split, flushed)

    def line(self, with_traffic=True):
        """The workload's measured figures as one JSON object."""
        out = {"value": self.value, "unit": "query-tokens/s", "value_warm": self.value_warm,
               "ms_per_step": self.flushed["step"]["mean"] * 1e-3,
               "ms_per_step_warm": self.wall / self.steps * 1e3,
               "stages_us_flushed": self.flushed, "stages_us": self.warm,
               "roofline": self.roofline(with_traffic=with_traffic),
               "roofline_warm": self.roofline(flushed=False, with_traffic=with_traffic)}
        if self.split:
            out["host_link_bytes_per_step"] = self.host_bytes
        return out


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
    per 64 generated tokens). Wall clock over the steps; each call's duration
    from HIP event pairs on the launch stream (warm, and with the caches
    flushed)."""
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
    wall, warm, flushed = timed_calls(one, steps, warmup)
    us = warm["mean"]
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
    return {"value": steps * batch / wall, "unit": "generated tokens/s", "call_us": warm, "call_us_flushed": flushed,
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
    that provides the kept groups, output and LSE; wall clock over the calls,
    and each call's duration from HIP event pairs on the launch stream."""
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
    wall, warm, flushed = timed_calls(one, steps, warmup)
    us = warm["mean"]
    flops = backward_flops(cfg, w.ns.cpu().numpy(), w.gi.cpu().numpy())
    w.free()
    return {"value": steps * cfg["n_q"] / wall, "unit": "query-tokens/s", "call_us": warm, "call_us_flushed": flushed,
            "ms_per_step": wall / steps * 1e3,
            "config": {"workload": f"{cfg['name']}-backward", "n_q": cfg["n_q"], "history": w.q0},
            "roofline": {"kernel": "hga_attend_backward (bwd_dq_kernel, then bwd_dkv_kernel)", "bound": "mfma",
                         "achieved": flops / (us * 1e-6) / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                         "frac": flops / (us * 1e-6) / PEAK_BF16,
                         "traffic": measured_traffic(f"{cfg['name']}-backward", "attend_backward"),
                         "traffic_unit": "HBM bytes per call (both kernels)", "algorithmic_flops": flops}}


def route_bytes(cfg, n_sel):
    """Algorithmic HBM bytes of hga_route over every (block, KV head) of the
    workload: each KV head's chunk summaries once (every chunk that some block
    scores, when the chunk stage selects), the group summaries of each item's
    kept chunks (when its group stage selects), the query rows once, and the
    index rows written."""
    d, G, hkv, g = cfg["d"], cfg["hq"] // cfg["hkv"], cfg["hkv"], cfg["group"]
    esz = 2 if cfg["dtype"] == "bf16" else 4
    nb = cfg["n_q"] // 64
    q0 = cfg["L"] - cfg["n_q"]
    ns = n_sel.reshape(nb, hkv, 2)
    scored = [set() for _ in range(hkv)]
    gs_rows = 0
    for b in range(nb):
        ms = (q0 + 64 * b) // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        for h in range(hkv):
            nsc, nsg = int(ns[b, h, 0]), int(ns[b, h, 1])
            if 0 < nsc < bb - a:
                scored[h].update(range(a, bb))
            if 0 < nsg < 64 // g * nsc:
                gs_rows += 64 // g * nsc
    cs_rows = sum(len(x) for x in scored)
    return (cfg["hq"] * cfg["n_q"] * d * esz + 4.0 * d * (cs_rows + gs_rows)
            + 4 * nb * hkv * (cfg["top_chunks"] + cfg["top_groups"] + 2))


def stage_hbm(cfg_id, samples=20):
    """Achieved HBM rates of the summary build (every chunk of the sequence)
    and of the router alone: algorithmic bytes over the mean duration of
    `samples` calls, each between HIP events on the launch stream."""
    w = Workload(cfg_id)
    cfg, hga = w.cfg, w.hga
    for _ in range(3):
        w.step()
    sum_us = stats(event_us(lambda: hga.hga_build_summaries(w.c, w.k_full, w.L, w.gs, w.cs), samples))
    route_us = stats(event_us(lambda: hga.hga_route(w.c, w.q, w.q0, w.nq, w.L, w.cs, w.gs_t, w.ci, w.gi, w.ns),
                              samples))
    esz = 2 if cfg["dtype"] == "bf16" else 4
    d, hkv, L = cfg["d"], cfg["hkv"], cfg["L"]
    sum_bytes = hkv * L * d * esz + 4.0 * hkv * (L // cfg["group"] + L // 64) * d
    r_bytes = route_bytes(cfg, w.ns.cpu().numpy())
    w.free()
    out = {}
    for name, byts, st in (("summaries_full_build", sum_bytes, sum_us), ("routing", r_bytes, route_us)):
        us = st["mean"]
        out[name] = {"us": st, "algorithmic_bytes": byts, "achieved_GBps": byts / (us * 1e-6) / 1e9,
                     "frac_of_hbm_peak": byts / (us * 1e-6) / PEAK_HBM}
    out["routing"]["note"] = ("latency-bound: a chain of dependent memory round trips per item (block query, "
                              "chunk scores, selection, group scores, selection)")
    return out


def full_summary_us(cfg_id, samples=20):
    """Duration statistics of hga_build_summaries over every chunk of
    workload cfg_id's sequence (HIP events on the launch stream)."""
    w = Workload(cfg_id)
    for _ in range(3):
        w.hga.hga_build_summaries(w.c, w.k_full, w.L, w.gs, w.cs)
    st = stats(event_us(lambda: w.hga.hga_build_summaries(w.c, w.k_full, w.L, w.gs, w.cs), samples))
    w.free()
    return st


def synth_config(cfg_id):
    import synth
    return synth.config(cfg_id)


def measure(cfg_id, steps, warmup, split=0, fused=None, samples=None):
    w = Workload(cfg_id, split, fused)
    wall, stages = w.run(steps, warmup, samples or max(steps, 20))
    r = Result(w, wall, stages, steps)
    w.free()
    return r


def host_link_rate(mib=256, samples=10):
    """Achievable pinned host-to-device copy rate of the box (B/s): the
    median of `samples` copies of `mib` MiB from pinned host memory."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(mib << 20, dtype=torch.uint8, device="cuda:0")
    us = stats(event_us(lambda: dst.copy_(src, non_blocking=True), samples))
    return (mib << 20) / (us["median"] * 1e-6)


def host_tier_line(cfg_id, steps, warmup, link_rate, note):
    r = measure(cfg_id, steps, warmup, split=synth_config(cfg_id)["tier_split"])
    line = r.line()
    t = r.flushed["attend"]["mean"] * 1e-6
    line["note"] = note
    line["host_link"] = {"bytes_per_step": r.host_bytes, "attend_stage_GBps": r.host_bytes / t / 1e9,
                         "frac_of_nominal_64GBps": r.host_bytes / t / PEAK_HOST_LINK,
                         "measured_pinned_h2d_GBps": link_rate / 1e9,
                         "note": "history bytes the step moves over the host link over the whole attention stage "
                                 "(the copy, then the attention): a lower bound of the link's achieved rate"}
    return line


def cached_host_tier_line(cfg_id, steps, warmup, link_rate, share=None, calls_of=None):
    """The layer with its history (tokens before the first query) in pinned
    host memory, through a persistent HBM cache (hga_route_attend_cached).

    cold: a call on an emptied cache of every history chunk (each distinct
    history group crosses the host link once); warm: the same call
    repeated (every group resident; the rate of `value`). With `calls_of`, a
    rolling pass: the queries in consecutive calls of `calls_of` queries each,
    on a cache with the fewest slots such calls allow (chunks are evicted),
    with the hit rate of its K/V requests. `share` plants a separate set of
    relevant groups for every `share` consecutive query blocks, so blocks of
    different sets route to different chunks. Every figure is taken with
    everything on one stream and, as "overlap", with the copies on a second
    stream while the blocks that need none of them are attended."""
    import torch

    import hierarchical_sparse_attention_hga_amd as hga
    import synth
    from hierarchical_sparse_attention_hga_amd.memory import split_to_host
    over = dict(plant_block_share=share) if share else {}
    cfg = synth.config(cfg_id, **over)
    x = synth.make_inputs(cfg)
    DEV = torch.device("cuda:0")
    L, nq, hkv, d, g = cfg["L"], cfg["n_q"], cfg["hkv"], cfg["d"], cfg["group"]
    q0, split = L - nq, cfg["tier_split"] or L - nq
    c = hga.make_config(cfg["hq"], hkv, d, cfg["top_chunks"], cfg["top_groups"], cfg["sink"], cfg["local"],
                        dtype=cfg["dtype"], group_size=g)
    q, k, v = (to_dev(x[n], cfg["dtype"], DEV) for n in ("q", "k", "v"))
    del x
    gs = torch.empty(hkv, L // g, d, device=DEV)
    cs = torch.empty(hkv, L // 64, d, device=DEV)
    hga.hga_build_summaries(c, k, L, gs, cs)
    torch.cuda.synchronize()
    gpin, _, gs_t = split_to_host(gs, split // g)
    kpin, _, k_t = split_to_host(k, split)
    vpin, _, v_t = split_to_host(v, split)
    gs_t = (gs_t[0], gs_t[1], split)
    del k, v
    esz = 2 if cfg["dtype"] == "bf16" else 4

    def make(n_q, kv_slots, gs_slots):
        size = hga.hga_tier_cache_size(c, split, kv_slots, gs_slots)
        mem = torch.empty(size + 256, dtype=torch.uint8, device=DEV)
        cache = hga.tier_cache((mem.data_ptr() + 255) // 256 * 256, size, split, kv_slots, gs_slots)
        hga.hga_tier_cache_init(c, cache)
        wsb = hga.hga_workspace_size(c, L, n_q, hga.HGA_WS_ATTEND_CACHED)
        return mem, cache, torch.empty(wsb, dtype=torch.uint8, device=DEV), wsb

    def counts(mem, cache):
        off = cache.mem - mem.data_ptr()
        raw = mem[off:off + 8 * len(hga.TC_COUNTERS)].cpu().numpy().view(np.int64)
        return dict(zip(hga.TC_COUNTERS, (int(r) for r in raw)))

    side = torch.cuda.Stream()   # default priority

    def caller(cache, ws, wsb, qs, n_q, overlap=True):
        nb = n_q // 64
        ci = torch.empty(nb, hkv, cfg["top_chunks"], dtype=torch.int32, device=DEV)
        gi = torch.empty(nb, hkv, cfg["top_groups"], dtype=torch.int32, device=DEV)
        ns = torch.empty(nb, hkv, 2, dtype=torch.int32, device=DEV)
        qv = q[:, qs - q0:qs - q0 + n_q].contiguous()
        out = torch.empty_like(qv)
        lse = torch.empty(cfg["hq"], n_q, device=DEV)
        return lambda: hga.hga_route_attend_cached(c, qv, qs, n_q, L, cs, gs_t, k_t, v_t, cache, ci, gi, ns, out, lse,
                                                   ws, wsb, copy_stream=side if overlap else None)

    nch = split // 64
    gs_all = hga.hga_tier_cache_min_slots(c, L, nq, hga.HGA_TC_GS)
    mem, cache, ws, wsb = make(nq, nch, gs_all)
    colds = {}
    for overlap in (False, True):
        call = caller(cache, ws, wsb, q0, nq, overlap)
        call()                       # the kernels' first launches (code loading) out of the cold figure
        hga.hga_tier_cache_init(c, cache)
        cold_us = event_us(call, 1, warm=0)[0]
        cold = counts(mem, cache)
        colds[overlap] = {"us": cold_us, "host_link_bytes": cold["kv_bytes"] + cold["gs_bytes"],
                          "host_link_GBps": (cold["kv_bytes"] + cold["gs_bytes"]) / (cold_us * 1e-6) / 1e9,
                          "kv_requests": cold["kv_requests"], "kv_misses": cold["kv_misses"]}
    _, warm_overlap, _ = timed_calls(call, steps, warmup)
    wall, warm, flushed = timed_calls(caller(cache, ws, wsb, q0, nq, False), steps, warmup)
    line = {"value": steps * nq / wall, "unit": "query-tokens/s", "ms_per_step": wall / steps * 1e3,
            "call_us": warm, "call_us_flushed": flushed, "call_us_overlap": warm_overlap,
            "cold_call": colds[False], "cold_call_overlap": colds[True],
            "warm_counters_after": counts(mem, cache),
            "measured_pinned_h2d_GBps": link_rate / 1e9,
            "config": {"workload": cfg["name"] + (f"-plant-share{share}" if share else ""), "split": split,
                       "kv_slots": nch, "gs_slots": gs_all}}
    del mem, cache, ws
    if calls_of:
        kv_min = hga.hga_tier_cache_min_slots(c, L, calls_of, hga.HGA_TC_KV)
        gs_min = hga.hga_tier_cache_min_slots(c, L, calls_of, hga.HGA_TC_GS)
        mem, cache, ws, wsb = make(calls_of, kv_min, gs_min)
        def rolling_pass(overlap):
            calls = [caller(cache, ws, wsb, qs, calls_of, overlap) for qs in range(q0, L, calls_of)]
            for fn in calls:      # one pass to settle (the cache then holds the last calls' chunks)
                fn()
            before = counts(mem, cache)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for fn in calls:
                fn()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            after = counts(mem, cache)
            return len(calls), el, {k2: after[k2] - before[k2] for k2 in after}

        _, el_overlap, _ = rolling_pass(True)
        ncalls, el, dlt = rolling_pass(False)
        line["rolling"] = {
            "value": nq / el, "value_overlap": nq / el_overlap, "unit": "query-tokens/s", "calls": ncalls,
            "queries_per_call": calls_of,
            "kv_slots": kv_min, "gs_slots": gs_min,
            "kv_hit_rate": 1.0 - dlt["kv_misses"] / max(dlt["kv_requests"], 1),
            "gs_hit_rate": 1.0 - dlt["gs_misses"] / max(dlt["gs_requests"], 1) if dlt["gs_requests"] else None,
            "host_link_bytes_per_pass": dlt["kv_bytes"] + dlt["gs_bytes"],
            "host_link_GBps": (dlt["kv_bytes"] + dlt["gs_bytes"]) / el / 1e9,
            "counters": dlt,
            "note": "the layer's queries in consecutive calls through one cache with the fewest slots such calls "
                    "allow; hit rate = 1 - K/V groups copied / history groups the calls' blocks attended"}
        del mem, cache, ws
    for p in (gpin, kpin, vpin):
        p.free()
    torch.cuda.empty_cache()
    return line


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
        print(json.dumps(backward_line(args.config, args.steps, args.warmup), allow_nan=False), flush=True)
        return
    if args.cached_host_tier:
        link = host_link_rate()
        for share in (None, 4):
            print(json.dumps(cached_host_tier_line(args.config, args.steps, args.warmup, link, share=share,
                                                   calls_of=256), allow_nan=False), flush=True)
        return
    if args.decode_batch:
        print(json.dumps(decode_line(args.config, args.decode_batch, args.steps, args.warmup), allow_nan=False),
              flush=True)
        return
    split = 0
    if args.host_tier:
        split = synth_config(args.config)["tier_split"] or (synth_config(args.config)["L"] -
                                                            synth_config(args.config)["n_q"])
    main_r = measure(args.config, args.steps, args.warmup, split=split)
    cfg = main_r.cfg
    ml = main_r.line()
    line = {
        "metric": METRIC, "value": ml["value"], "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ml["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded; Qwen3-shaped heads, rank-8 shared component, planted groups)",
        "config": {"workload": cfg["name"], "seq_len": cfg["L"], "n_q": cfg["n_q"], "q_heads": cfg["hq"],
                   "kv_heads": cfg["hkv"], "head_dim": cfg["d"], "top_chunks": cfg["top_chunks"],
                   "top_groups": cfg["top_groups"], "sink": cfg["sink"], "local": cfg["local"],
                   "kv_residency": "host-pinned history" if split else "hbm"},
        "value_warm": ml["value_warm"], "ms_per_step_warm": ml["ms_per_step_warm"],
        "stages_us_flushed": ml["stages_us_flushed"], "stages_us": ml["stages_us"],
        "roofline": ml["roofline"], "roofline_warm": ml["roofline_warm"],
    }
    if split:
        line["host_link_bytes_per_step"] = main_r.host_bytes
    if not args.no_extra:
        extra = {}
        half = max(args.steps // 2, 10)
        rest = sum(v["mean"] for k, v in main_r.flushed.items() if k not in ("summaries", "step"))
        extra["summaries_prebuilt"] = {
            "value": cfg["n_q"] / (rest * 1e-6), "unit": "query-tokens/s",
            "note": "n_q / (mean flushed routing + gather + attention stage time); summary build excluded"}
        if not split:
            full = full_summary_us(args.config)
            extra["full_summary_rebuild"] = {
                "value": cfg["n_q"] / ((full["mean"] + rest) * 1e-6), "unit": "query-tokens/s",
                "summaries_us": full,
                "note": "the step with the summaries of every chunk of the sequence rebuilt (history included) "
                        "instead of only the chunks the step's positions close"}
        extra["stage_hbm"] = stage_hbm(args.config)
        if main_r.fused:
            sep = measure(args.config, half, args.warmup, fused=False)
            sl = sep.line(with_traffic=False)
            extra["separate_calls"] = {
                "value": sl["value"], "unit": "query-tokens/s", "stages_us": sl["stages_us"],
                "note": "same step through hga_route then hga_attend; roofline of the attention kernel alone",
                "roofline": sl["roofline"]}
        names = {0: "tiny_fp32_1k", 1: "qwen3_8b_4k", 2: "qwen3_8b_segment_16k", 3: "qwen3_30b_a3b_64k_hbm"}
        for cid in (0, 1, 3):
            if cid != args.config:
                extra[names[cid]] = measure(cid, half, args.warmup).line()
        link = host_link_rate()
        extra["64k_host_tier_pcie_inclusive"] = host_tier_line(
            3, max(half, 20), 2, link,
            "history K/V and group summaries in pinned host memory; each history chunk any block needs crosses "
            "the host link once per step into an HBM cache, then attention")
        extra["128k_host_tier_pcie_inclusive"] = host_tier_line(
            4, max(half, 20), 2, link,
            "the 131,072-token long-evaluation layer (Qwen3-8B heads, top-64 chunks, top-512 groups, 64 planted "
            "needle groups per head): history K/V and group summaries in pinned host memory, the final 2,048 "
            "queries in HBM; each history chunk any block needs crosses the host link once per step")
        extra["64k_host_tier_cached"] = cached_host_tier_line(3, max(half, 20), 2, link, calls_of=256)
        extra["64k_host_tier_cached_block_varying"] = cached_host_tier_line(3, max(half, 20), 2, link, share=4,
                                                                            calls_of=256)
        if args.config == 2:
            extra["16k_streamed_2048_segments"] = stream_line(max(args.steps // 6, 3), 2)
        extra["backward_16k_segment"] = backward_line(2, half, 3)
        extra["decode_16k_batch64"] = decode_line(2, 64, half, 3)
        extra["decode_16k_single_sequence"] = decode_line(2, 1, half, 3)
        extra["decode_64k_batch32"] = decode_line(3, 32, half, 3)
        line["also"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(line, allow_nan=False), flush=True)


if __name__ == "__main__":
    main()
