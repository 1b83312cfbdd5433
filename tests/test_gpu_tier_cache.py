"""The persistent host-tier cache (hga_route_attend_cached) on the GPU.

The history (tokens below the split) of K, V and the group summaries lives in
pinned host memory; a cache in HBM keeps the K/V rows of history groups and
the group summaries of history chunks across calls ("Long-Context Fine-Tuning
with Limited VRAM", section 2.1, "Group selection" and "Exact-token
attention"; section 4.5, table 8). Whatever the cache holds, every call's
routing, outputs and LSE must be bit-identical to hga_route_attend with
everything in HBM (itself compared with the oracle in test_gpu_parity.py and
test_gpu_edges.py). The counters must account for every request: a call's
K/V requests are the history groups its (block, KV head) items attend, each
miss is a group copied because the cache lacked it, and a call that repeats
the previous call's queries on a cache large enough for both misses nothing.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hga_amd as hga
import synth
from harness import DEV, hga_cfg, to_dev
from hierarchical_sparse_attention_hga_amd.memory import split_to_host
from test_gpu_edges import small

pytestmark = pytest.mark.gpu

KEYS = ("chunk_idx", "group_idx", "n_sel", "out", "lse")


class Setup:
    """Device and host buffers of one workload: K, V and summaries of the
    whole sequence in HBM, and the same history split into pinned memory."""

    def __init__(self, cfg, x, split):
        self.cfg, self.split = cfg, split
        self.c = hga_cfg(cfg)
        dt, L, hkv, d, g = cfg["dtype"], cfg["L"], cfg["hkv"], cfg["d"], cfg["group"]
        self.q_all = to_dev(x["q"], dt)
        self.k, self.v = to_dev(x["k"], dt), to_dev(x["v"], dt)
        self.gs = torch.empty(hkv, L // g, d, device=DEV)
        self.cs = torch.empty(hkv, L // 64, d, device=DEV)
        hga.hga_build_summaries(self.c, self.k, L, self.gs, self.cs)
        torch.cuda.synchronize()
        gpin, _, gs_t = split_to_host(self.gs, split // g)
        self.gs_t = (gs_t[0], gs_t[1], split)
        kpin, _, self.k_t = split_to_host(self.k, split)
        vpin, _, self.v_t = split_to_host(self.v, split)
        self.pins = [gpin, kpin, vpin]
        self.side = torch.cuda.Stream()   # copy stream of the overlapped calls (default priority)

    def free(self):
        for p in self.pins:
            p.free()

    def outputs(self, q_start, n_q):
        cfg = self.cfg
        nb, hkv = n_q // cfg["q_block"], cfg["hkv"]
        return dict(chunk_idx=torch.full((nb, hkv, cfg["top_chunks"]), -7, dtype=torch.int32, device=DEV),
                    group_idx=torch.full((nb, hkv, cfg["top_groups"]), -7, dtype=torch.int32, device=DEV),
                    n_sel=torch.full((nb, hkv, 2), -7, dtype=torch.int32, device=DEV),
                    out=torch.full((cfg["hq"], n_q, cfg["d"]), float("nan"), dtype=self.q_all.dtype, device=DEV),
                    lse=torch.full((cfg["hq"], n_q), float("nan"), device=DEV))

    def q(self, q_start, n_q):
        q0 = self.cfg["L"] - self.cfg["n_q"]
        return self.q_all[:, q_start - q0:q_start - q0 + n_q].contiguous()

    def hbm(self, q_start, n_q):
        o = self.outputs(q_start, n_q)
        hga.hga_route_attend(self.c, self.q(q_start, n_q), q_start, n_q, self.cfg["L"], self.cs, self.gs, self.k,
                             self.v, o["chunk_idx"], o["group_idx"], o["n_sel"], o["out"], o["lse"])
        torch.cuda.synchronize()
        return fetch(o)

    def cached(self, cache, q_start, n_q, overlap=False):
        o = self.outputs(q_start, n_q)
        L = self.cfg["L"]
        wsb = hga.hga_workspace_size(self.c, L, n_q, hga.HGA_WS_ATTEND_CACHED)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        hga.hga_route_attend_cached(self.c, self.q(q_start, n_q), q_start, n_q, L, self.cs, self.gs_t, self.k_t,
                                    self.v_t, cache, o["chunk_idx"], o["group_idx"], o["n_sel"], o["out"], o["lse"],
                                    ws, wsb, copy_stream=self.side if overlap else None)
        torch.cuda.synchronize()
        return fetch(o)


def fetch(o):
    res = {k: t.cpu().numpy() for k, t in o.items() if k != "out"}
    res["out"] = o["out"].view(torch.int16 if o["out"].dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    return res


def make_cache(st, kv_slots, gs_slots):
    size = hga.hga_tier_cache_size(st.c, st.split, kv_slots, gs_slots)
    mem = torch.empty(size + 256, dtype=torch.uint8, device=DEV)
    base = (mem.data_ptr() + 255) // 256 * 256
    cache = hga.tier_cache(base, size, st.split, kv_slots, gs_slots)
    hga.hga_tier_cache_init(st.c, cache)
    return mem, cache


def counters(mem, cache):
    base = cache.mem - mem.data_ptr()
    raw = mem[base:base + 8 * len(hga.TC_COUNTERS)].cpu().numpy().view(np.int64)
    return dict(zip(hga.TC_COUNTERS, (int(v) for v in raw)))


def kv_requests(cfg, res, q_start, split):
    """History groups the call's (block, KV head) items attend: their usable
    kept groups below the split and every group of their fixed chunks below
    it (the token set of the method's exact-token attention)."""
    g, B, kg = cfg["group"], cfg["q_block"], cfg["top_groups"]
    gpc = 64 // g
    nb, hkv = res["n_sel"].shape[:2]
    total = 0
    for b in range(nb):
        s = q_start + b * B
        ms = s // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        fixed = [m for m in list(range(a)) + list(range(bb, ms)) if m * 64 < split]
        for h in range(hkv):
            n = int(min(max(res["n_sel"][b, h, 1], 0), kg))
            kept = [int(j) for j in res["group_idx"][b, h, :n]
                    if j >= 0 and (j + 1) * g <= s and (j * g) // 64 >= a and (j * g) // 64 < bb]
            total += sum(1 for j in kept if j * g < split) + gpc * len(fixed)
    return total


def unique_groups(cfg, res, q_start, split):
    """Distinct (KV head, history group) pairs the call's items attend."""
    g, B, kg = cfg["group"], cfg["q_block"], cfg["top_groups"]
    gpc = 64 // g
    nb, hkv = res["n_sel"].shape[:2]
    seen = set()
    for b in range(nb):
        s = q_start + b * B
        ms = s // 64
        a = min(cfg["sink"] // 64, ms)
        bb = max(ms - cfg["local"] // 64, a)
        for h in range(hkv):
            for m in list(range(a)) + list(range(bb, ms)):
                if m * 64 < split:
                    seen.update((h, m * gpc + u) for u in range(gpc))
            n = int(min(max(res["n_sel"][b, h, 1], 0), kg))
            for j in res["group_idx"][b, h, :n]:
                if j >= 0 and j * g < split and (j + 1) * g <= s and a <= (j * g) // 64 < bb:
                    seen.add((h, int(j)))
    return len(seen)


def assert_same(a, b, what):
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"


# queries of each call (start, count): neighbouring blocks, a repeat, distant
# blocks, the last blocks, the first again
CALLS = [(2048, 128), (2176, 128), (2048, 128), (3072, 128), (3968, 128), (2048, 128)]


@pytest.mark.parametrize("case,overlap", [("bf16", False), ("bf16", True), ("bf16_d64_g4", True), ("f32", True)])
def test_cache_across_calls_with_evictions(case, overlap):
    """A cache with the fewest slots the calls allow (so chunks are evicted
    between calls), the group stage choosing (its summaries go through the
    cache too): six calls over different query ranges, each bit-identical to
    the all-HBM call; the counters add up. With overlap the copies run on a
    second stream while the blocks that need none of them are attended (calls
    mixing such blocks with others: a repeat, a neighbour)."""
    over = {"bf16": dict(),
            "bf16_d64_g4": dict(d=64, group=4, top_groups=20),
            "f32": dict(dtype="f32", d=64, rope_theta=None)}[case]
    # every query block plants its own relevant groups, so calls at different
    # positions route to different chunks (more chunks than the cache holds)
    cfg = small(**dict(dict(L=4096, n_q=2048, top_chunks=4, top_groups=12, plant_block_share=1, n_plant_chunks=4,
                            plant_chunks=(1, 30)), **over))
    x = synth.make_inputs(cfg)
    split = 2048
    st = Setup(cfg, x, split)
    try:
        kv_min = hga.hga_tier_cache_min_slots(st.c, cfg["L"], 128, hga.HGA_TC_KV)
        gs_min = hga.hga_tier_cache_min_slots(st.c, cfg["L"], 128, hga.HGA_TC_GS)
        assert 0 < kv_min < split // 64 and 0 < gs_min < split // 64
        mem, cache = make_cache(st, kv_min, gs_min)
        prev = counters(mem, cache)
        assert all(v == 0 for v in prev.values())
        for i, (q0, n) in enumerate(CALLS):
            print(f"[tier cache] {case} overlap={overlap} call {i}: queries [{q0}, {q0 + n})", flush=True)
            ref = st.hbm(q0, n)
            got = st.cached(cache, q0, n, overlap)
            assert_same(ref, got, f"{case} call {i}")
            now = counters(mem, cache)
            req = kv_requests(cfg, ref, q0, split)
            assert now["calls"] == i + 1
            assert now["kv_requests"] - prev["kv_requests"] == req
            assert 0 <= now["kv_misses"] - prev["kv_misses"] <= unique_groups(cfg, ref, q0, split)
            esz = 2 if cfg["dtype"] == "bf16" else 4
            assert now["kv_bytes"] - prev["kv_bytes"] == (now["kv_misses"] - prev["kv_misses"]) * 2 * cfg["group"] * \
                cfg["d"] * esz
            assert now["gs_misses"] - prev["gs_misses"] <= now["gs_requests"] - prev["gs_requests"]
            print(f"  {dict((k, now[k] - prev[k]) for k in now)}", flush=True)
            prev = now
        assert prev["kv_evictions"] > 0 and prev["gs_evictions"] > 0, "the small cache should have evicted chunks"
    finally:
        st.free()


@pytest.mark.parametrize("share,overlap", [(None, False), (4, True)])
def test_cache_64k_layer(share, overlap):
    """The 64K Qwen3-30B-A3B-shaped layer with its history in pinned host
    memory and a cache of every history chunk: the first call copies each
    distinct history group once (across all query blocks), the second copies
    nothing; both bit-identical to the all-HBM call. With block-varying
    planting (each set of four consecutive query blocks routes to its own
    chunks) the first call copies more. With overlap, the first call's blocks
    all wait for the copies and the second call's need none."""
    over = dict(plant_block_share=share) if share else {}
    cfg = synth.config(3, **over)
    x = synth.make_inputs(cfg)
    split = cfg["tier_split"]
    st = Setup(cfg, x, split)
    try:
        q0, n = cfg["L"] - cfg["n_q"], cfg["n_q"]
        nch = split // 64
        assert hga.hga_tier_cache_min_slots(st.c, cfg["L"], n, hga.HGA_TC_KV) == nch
        assert hga.hga_tier_cache_min_slots(st.c, cfg["L"], n, hga.HGA_TC_GS) == 0   # the group stage keeps all
        mem, cache = make_cache(st, nch, 0)
        ref = st.hbm(q0, n)
        for call in range(2):
            print(f"[tier cache] 64K share={share} overlap={overlap} call {call}", flush=True)
            got = st.cached(cache, q0, n, overlap)
            assert_same(ref, got, f"64K call {call}")
            c = counters(mem, cache)
            print(f"  {c}", flush=True)
            assert c["kv_requests"] == (call + 1) * kv_requests(cfg, ref, q0, split)
            assert c["kv_misses"] == unique_groups(cfg, ref, q0, split)   # the second call misses nothing
            assert c["gs_requests"] == 0 and c["kv_evictions"] == 0
    finally:
        st.free()
