"""Seeded synthetic inputs for HGA routed attention.

This module is the only code shared by the CPU oracle and the HIP path. It holds
workload descriptions and random-number generation only: no step of the routing
or attention method is computed here. Inputs stand in for the pages' PG19 text
and RULER-style planted values (Long-Context Fine-Tuning with Limited VRAM,
section 3 and table 1; section 4.6), which are not available.

Recipe (every tensor is drawn from ``numpy.random.default_rng([seed, cfg, id])``
with seed 1337, the matched seed of that paper's table 1):

* Q [Hq][Nq][d], K [Hkv][L][d], V [Hkv][L][d] ~ N(0, 1).
* Optional rank-r shared component (r = 8, scale 0.5): one basis
  U_h in R^{r x d} ~ N(0, 1/r) per KV head, shared by that head's Q, K and V;
  each token of each tensor adds ``scale * c_t @ U_h`` with c_t ~ N(0, I_r).
* Optional RoPE (rotate-half convention, inv_freq_i = theta^(-2i/d), absolute
  positions; queries sit at positions L - Nq + i), applied in float64.
* Planted structure, added after RoPE: a unit direction u_h per KV head; every
  query of the KV head's query heads gets ``+alpha * u_h``; the keys of the
  planted 8-token groups get ``+beta * u_h``. Planted groups lie in distinct
  chunks drawn without replacement from ``plant_chunks`` (half-open range).
* Values are rounded to float32 (round to nearest even) and, for bf16 configs,
  then to bfloat16 (round to nearest even). bf16 data is carried as uint16 bit
  patterns.
"""
from __future__ import annotations

import copy
import numpy as np

SEED = 1337

# Tensor ids for the counter-free seeding scheme default_rng([SEED, cfg, id]).
_T_Q, _T_K, _T_V, _T_U, _T_CQ, _T_CK, _T_CV, _T_DIR, _T_PCH, _T_PGR = range(10)

# The five workloads. Head-major layouts: Q [Hq][n_q][d], K/V [Hkv][L][d].
CONFIGS = [
    dict(name="tiny-fp32-1k", L=1024, n_q=1024, hq=1, hkv=1, d=64, dtype="f32",
         rope_theta=None, chunk=64, group=8, q_block=64, top_chunks=4, top_groups=8,
         sink=64, local=64, shared_rank=0, shared_scale=0.0,
         n_plant_chunks=4, groups_per_plant_chunk=1, plant_chunks=(1, 14),
         alpha=1.0, beta=16.0, tier_split=0),
    dict(name="qwen3-8b-4k", L=4096, n_q=4096, hq=32, hkv=8, d=128, dtype="bf16",
         rope_theta=1e6, chunk=64, group=8, q_block=64, top_chunks=8, top_groups=16,
         sink=64, local=64, shared_rank=8, shared_scale=0.5,
         n_plant_chunks=8, groups_per_plant_chunk=2, plant_chunks=(1, 62),
         alpha=1.0, beta=8.0, tier_split=0),
    dict(name="qwen3-8b-segment-16k", L=16384, n_q=2048, hq=32, hkv=8, d=128, dtype="bf16",
         rope_theta=1e6, chunk=64, group=8, q_block=64, top_chunks=16, top_groups=64,
         sink=64, local=128, shared_rank=8, shared_scale=0.5,
         n_plant_chunks=16, groups_per_plant_chunk=1, plant_chunks=(1, 222),
         alpha=1.0, beta=16.0, tier_split=0),
    dict(name="qwen3-30b-a3b-64k", L=65536, n_q=4096, hq=32, hkv=4, d=128, dtype="bf16",
         rope_theta=1e7, chunk=64, group=8, q_block=64, top_chunks=32, top_groups=256,
         sink=64, local=128, shared_rank=8, shared_scale=0.5,
         n_plant_chunks=32, groups_per_plant_chunk=1, plant_chunks=(1, 958),
         alpha=1.0, beta=16.0, tier_split=65536 - 4096),
    dict(name="long-eval-128k", L=131072, n_q=2048, hq=32, hkv=8, d=128, dtype="bf16",
         rope_theta=1e6, chunk=64, group=8, q_block=64, top_chunks=64, top_groups=512,
         sink=64, local=128, shared_rank=0, shared_scale=0.0,
         n_plant_chunks=64, groups_per_plant_chunk=1, plant_chunks=(1, 2014),
         alpha=1.0, beta=16.0, tier_split=131072 - 2048),
]


def config(i_or_cfg, **overrides) -> dict:
    """Return a copy of workload ``i`` (or of a given dict) with overrides applied."""
    cfg = copy.deepcopy(CONFIGS[i_or_cfg] if isinstance(i_or_cfg, int) else i_or_cfg)
    cfg.update(overrides)
    cfg.setdefault("cfg_id", i_or_cfg if isinstance(i_or_cfg, int) else 99)
    return cfg


def q_start(cfg) -> int:
    return cfg["L"] - cfg["n_q"]


# ---------------------------------------------------------------- rounding helpers
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(x, dtype: str) -> np.ndarray:
    """Exact float64 view of stored input data (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------- generation
def _rng(cfg, tid):
    return np.random.default_rng([SEED, int(cfg.get("cfg_id", 99)), int(cfg.get("seed", 0)), tid])


def _rope(x, pos, theta):
    """Rotate-half RoPE of x [H][T][d] (float64) at integer positions pos [T]."""
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half].copy(), x[..., half:].copy()
    x[..., :half] = x1 * c - x2 * s
    x[..., half:] = x2 * c + x1 * s
    return x


def _integer_inputs(cfg: dict) -> dict:
    """Inputs with exact ties: Q and K entries are integers drawn uniformly from
    ``integer_values`` = (lo, hi) (inclusive), and the keys repeat with a period
    of ``chunk_period`` chunks (chunk m holds the keys of chunk m mod period),
    so summaries, and every score built from them, repeat exactly. Small
    integers are exact in bfloat16, and their means over power-of-two counts
    and the dot products of such means are exact in float64, so equal scores
    are equal on every evaluation order. V ~ N(0, 1). No RoPE, no planting."""
    L, nq, hq, hkv, d, c = cfg["L"], cfg["n_q"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["chunk"]
    lo, hi = cfg["integer_values"]
    per = int(cfg.get("chunk_period", 0)) or L // c
    q = _rng(cfg, _T_Q).integers(lo, hi + 1, size=(hq, nq, d)).astype(np.float64)
    base = _rng(cfg, _T_K).integers(lo, hi + 1, size=(hkv, per * c, d)).astype(np.float64)
    reps = -(-L // (per * c))
    k = np.tile(base, (1, reps, 1))[:, :L]
    v = _rng(cfg, _T_V).standard_normal((hkv, L, d))
    out = {"planted": [[] for _ in range(hkv)]}
    for name, x in (("q", q), ("k", k), ("v", v)):
        x32 = x.astype(np.float32)
        out[name] = f32_to_bf16_bits(x32) if cfg["dtype"] == "bf16" else x32
    return out


def make_inputs(cfg: dict) -> dict:
    """Generate Q, K, V for workload ``cfg``.

    Returns a dict with ``q`` [Hq][n_q][d], ``k`` and ``v`` [Hkv][L][d] in storage
    format (float32, or uint16 bf16 bits), and ``planted`` = list per KV head of
    the planted global group indices (sorted).
    """
    L, nq, hq, hkv, d = cfg["L"], cfg["n_q"], cfg["hq"], cfg["hkv"], cfg["d"]
    G = hq // hkv
    q0 = L - nq
    if cfg.get("integer_values"):
        return _integer_inputs(cfg)
    q = _rng(cfg, _T_Q).standard_normal((hq, nq, d))
    k = _rng(cfg, _T_K).standard_normal((hkv, L, d))
    v = _rng(cfg, _T_V).standard_normal((hkv, L, d))
    r = int(cfg.get("shared_rank", 0))
    if r > 0 and cfg.get("shared_scale", 0.0) != 0.0:
        sc = float(cfg["shared_scale"])
        U = _rng(cfg, _T_U).standard_normal((hkv, r, d)) * np.sqrt(1.0 / r)
        cq = _rng(cfg, _T_CQ).standard_normal((hq, nq, r))
        ck = _rng(cfg, _T_CK).standard_normal((hkv, L, r))
        cv = _rng(cfg, _T_CV).standard_normal((hkv, L, r))
        for h in range(hkv):
            k[h] += sc * (ck[h] @ U[h])
            v[h] += sc * (cv[h] @ U[h])
            for g in range(G):
                q[h * G + g] += sc * (cq[h * G + g] @ U[h])
    if cfg.get("rope_theta"):
        th = float(cfg["rope_theta"])
        _rope(q, np.arange(q0, L), th)
        _rope(k, np.arange(L), th)
    planted = []
    npc = int(cfg.get("n_plant_chunks", 0))
    gpc = int(cfg.get("groups_per_plant_chunk", 1))
    c, g = cfg["chunk"], cfg["group"]
    share = cfg.get("plant_block_share")
    if npc > 0 and share:
        return _finish(cfg, q, k, v, _plant_per_block_sets(cfg, q, k, int(share)))
    if npc > 0:
        dirs = _rng(cfg, _T_DIR).standard_normal((hkv, d))
        dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
        rch = _rng(cfg, _T_PCH)
        rgr = _rng(cfg, _T_PGR)
        lo, hi = cfg["plant_chunks"]
        hi = min(hi, L // c)
        for h in range(hkv):
            chunks = np.sort(rch.choice(np.arange(lo, hi), size=min(npc, hi - lo), replace=False))
            groups = []
            for m in chunks:
                within = np.sort(rgr.choice(c // g, size=gpc, replace=False))
                for u in within:
                    j = int(m) * (c // g) + int(u)
                    groups.append(j)
                    k[h, j * g:(j + 1) * g, :] += cfg["beta"] * dirs[h]
            planted.append(sorted(groups))
            q[h * G:(h + 1) * G] += cfg["alpha"] * dirs[h]
    else:
        planted = [[] for _ in range(hkv)]
    return _finish(cfg, q, k, v, planted)


def _finish(cfg, q, k, v, planted):
    """Round to the stored formats (float32, then bfloat16 bits)."""
    out = {"planted": planted}
    for name, x in (("q", q), ("k", k), ("v", v)):
        x32 = x.astype(np.float32)
        out[name] = f32_to_bf16_bits(x32) if cfg["dtype"] == "bf16" else x32
    return out


def _plant_per_block_sets(cfg, q, k, share):
    """Block-varying planting: the query blocks are taken `share` at a time
    (consecutive blocks of q_block queries); each set s of blocks gets its own
    unit direction u_{h,s} per KV head and its own n_plant_chunks planted
    groups (in distinct chunks of plant_chunks, drawn per set): the set's
    queries get +alpha u_{h,s}, the planted groups' keys +beta u_{h,s}. Blocks
    of different sets then route to different chunks. Returns the planted
    groups per KV head (all sets, sorted)."""
    L, nq, hq, hkv, d = cfg["L"], cfg["n_q"], cfg["hq"], cfg["hkv"], cfg["d"]
    G, c, g, B = hq // hkv, cfg["chunk"], cfg["group"], cfg["q_block"]
    npc, gpc = int(cfg["n_plant_chunks"]), int(cfg.get("groups_per_plant_chunk", 1))
    nsets = -(-(nq // B) // share)
    dirs = _rng(cfg, _T_DIR).standard_normal((hkv, nsets, d))
    dirs /= np.linalg.norm(dirs, axis=2, keepdims=True)
    rch, rgr = _rng(cfg, _T_PCH), _rng(cfg, _T_PGR)
    lo, hi = cfg["plant_chunks"]
    hi = min(hi, L // c)
    planted = []
    for h in range(hkv):
        groups = set()
        for st in range(nsets):
            chunks = rch.choice(np.arange(lo, hi), size=min(npc, hi - lo), replace=False)
            for m in np.sort(chunks):
                for u in np.sort(rgr.choice(c // g, size=gpc, replace=False)):
                    j = int(m) * (c // g) + int(u)
                    groups.add(j)
                    k[h, j * g:(j + 1) * g, :] += cfg["beta"] * dirs[h, st]
            rows = slice(st * share * B, min((st + 1) * share * B, nq))
            q[h * G:(h + 1) * G, rows] += cfg["alpha"] * dirs[h, st]
        planted.append(sorted(groups))
    return planted
