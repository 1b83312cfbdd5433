"""CPU oracle for the HGA routed-attention forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It wraps ``hga_oracle.c`` (plain C, float64, see that file's
header for the steps and the readings of the pages it follows) through ctypes
and shares no code with the HIP path. Inputs arrive as the exact float64
widening of the stored bf16/fp32 values.
"""
from __future__ import annotations

import ctypes as C
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hga_oracle.c")
LIB_PATH = os.path.join(_HERE, "liborc.so")

# diagnostics row layout (mirrors the enum in hga_oracle.c)
DG_NCAND_C, DG_GAP_C, DG_EPS_C, DG_UNROUNDED_EQ_C, DG_NCAND_G, DG_GAP_G, DG_EPS_G, DG_UNROUNDED_EQ_G = range(8)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no floating-point contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Cfg(C.Structure):
    _fields_ = [("hq", C.c_int32), ("hkv", C.c_int32), ("d", C.c_int32),
                ("chunk", C.c_int32), ("group", C.c_int32), ("q_block", C.c_int32),
                ("top_chunks", C.c_int32), ("top_groups", C.c_int32),
                ("sink", C.c_int32), ("local", C.c_int32),
                ("seq_len", C.c_int64), ("n_q", C.c_int64), ("scale", C.c_double)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = C.CDLL(LIB_PATH)
        P = C.c_void_p
        lib.orc_summaries.argtypes = [C.POINTER(_Cfg), P, P, P]
        lib.orc_abs_summaries.argtypes = [C.POINTER(_Cfg), P, P, P]
        lib.orc_route.argtypes = [C.POINTER(_Cfg), P, P, P, P, P, C.c_int, P, P, P, P, P]
        lib.orc_attend.argtypes = [C.POINTER(_Cfg), P, P, P, C.c_int, P, P, P, P, P]
        lib.orc_attend_backward.argtypes = [C.POINTER(_Cfg), P, P, P, P, P, P, P, P, P, P, P, P]
        lib.orc_token_set.argtypes = [C.POINTER(_Cfg), C.c_int, P, C.c_int, P, C.c_int64]
        lib.orc_token_set.restype = C.c_int64
        assert lib.orc_diag_width() == 8
        lib.orc_threads.restype = C.c_int
        lib.orc_set_threads.argtypes = [C.c_int]
        lib.orc_route_scores.argtypes = [C.POINTER(_Cfg), P, P, P, P, P, C.c_int, P, P, P, P]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def make_cfg(cfg: dict) -> _Cfg:
    scale = cfg.get("softmax_scale") or 1.0 / math.sqrt(cfg["d"])
    return _Cfg(cfg["hq"], cfg["hkv"], cfg["d"], cfg["chunk"], cfg["group"], cfg["q_block"],
                cfg["top_chunks"], cfg["top_groups"], cfg["sink"], cfg["local"],
                cfg["L"], cfg["n_q"], float(scale))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def summaries(cfg, k64):
    """Step 1: group and chunk means of the keys (float64)."""
    lib = _load()
    L, d, hkv = cfg["L"], cfg["d"], cfg["hkv"]
    k64 = _f64(k64)
    gs = np.empty((hkv, L // cfg["group"], d))
    cs = np.empty((hkv, L // cfg["chunk"], d))
    lib.orc_summaries(C.byref(make_cfg(cfg)), _ptr(k64), _ptr(gs), _ptr(cs))
    return gs, cs


def abs_summaries(cfg, k64):
    lib = _load()
    L, d, hkv = cfg["L"], cfg["d"], cfg["hkv"]
    k64 = _f64(k64)
    ga = np.empty((hkv, L // cfg["group"], d))
    ca = np.empty((hkv, L // cfg["chunk"], d))
    lib.orc_abs_summaries(C.byref(make_cfg(cfg)), _ptr(k64), _ptr(ga), _ptr(ca))
    return ga, ca


def all_items(cfg):
    nb = cfg["n_q"] // cfg["q_block"]
    return [(b, h) for b in range(nb) for h in range(cfg["hkv"])]


def route(cfg, q64, k64, items=None, sums=None):
    """Steps 2-5 for a list of (block, kv_head) items.

    Returns chunk_idx [n][kc], group_idx [n][kg] (ascending, -1 padded),
    n_sel [n][2] and diag [n][8] (see the DG_* column names).
    """
    lib = _load()
    items = all_items(cfg) if items is None else items
    it = np.ascontiguousarray(np.asarray(items, dtype=np.int32).reshape(-1, 2))
    n = it.shape[0]
    if sums is None:
        sums = (summaries(cfg, k64), abs_summaries(cfg, k64))
    (gs, cs), (ga, ca) = sums
    q64 = _f64(q64)
    kc, kg = cfg["top_chunks"], cfg["top_groups"]
    ci = np.empty((n, max(kc, 0)), np.int32)
    gi = np.empty((n, max(kg, 0)), np.int32)
    ns = np.empty((n, 2), np.int32)
    dg = np.empty((n, 8), np.float64)
    lib.orc_route(C.byref(make_cfg(cfg)), _ptr(q64), _ptr(ga), _ptr(ca), _ptr(gs), _ptr(cs),
                  n, _ptr(it), _ptr(ci), _ptr(gi), _ptr(ns), _ptr(dg))
    return ci, gi, ns, dg


def route_scores(cfg, q64, k64, items, sums=None):
    """Decision scores of every candidate of both stages, for each (block,
    KV head) item: chunk_sc [n][L/chunk] (NaN where a chunk is not a
    candidate of the item), group_sc [n][L/group] (every group of every
    candidate chunk; NaN elsewhere) and eps [n][2], the error bounds of the
    two stages over all of these scores. Used where a boundary is not
    certified and several selections are correct."""
    lib = _load()
    it = np.ascontiguousarray(np.asarray(items, dtype=np.int32).reshape(-1, 2))
    n = it.shape[0]
    if sums is None:
        sums = (summaries(cfg, k64), abs_summaries(cfg, k64))
    (gs, cs), (ga, ca) = sums
    csc = np.empty((n, cfg["L"] // cfg["chunk"]))
    gsc = np.empty((n, cfg["L"] // cfg["group"]))
    eps = np.empty((n, 2))
    lib.orc_route_scores(C.byref(make_cfg(cfg)), _ptr(_f64(q64)), _ptr(ga), _ptr(ca), _ptr(gs), _ptr(cs),
                         n, _ptr(it), _ptr(csc), _ptr(gsc), _ptr(eps))
    return csc, gsc, eps


def attend(cfg, q64, k64, v64, items, group_idx, n_groups):
    """Steps 6-7: exact causal attention over each item's token set.

    Returns out [n][G][B][d] and lse [n][G][B] (float64).
    """
    lib = _load()
    it = np.ascontiguousarray(np.asarray(items, dtype=np.int32).reshape(-1, 2))
    n = it.shape[0]
    G, B, d = cfg["hq"] // cfg["hkv"], cfg["q_block"], cfg["d"]
    kg = cfg["top_groups"]
    gi = np.ascontiguousarray(np.asarray(group_idx, dtype=np.int32).reshape(n, kg))
    ng = np.ascontiguousarray(np.asarray(n_groups, dtype=np.int32).reshape(n))
    out = np.empty((n, G, B, d))
    lse = np.empty((n, G, B))
    lib.orc_attend(C.byref(make_cfg(cfg)), _ptr(_f64(q64)), _ptr(_f64(k64)), _ptr(_f64(v64)), n,
                   _ptr(it), _ptr(gi), _ptr(ng), _ptr(out), _ptr(lse))
    return out, lse


def attend_backward(cfg, q64, k64, v64, dout64, group_idx, n_groups, with_abs=False):
    """Backward of step 7 with the routing fixed, over every (block, KV head).

    group_idx [nb][hkv][kg], n_groups [nb][hkv]; dout [Hq][n_q][d]. Returns dq
    [Hq][n_q][d] and dk, dv [Hkv][L][d] (float64; every key row, zero where no
    query attends it); with ``with_abs`` also their magnitude companions
    (dq_abs, dk_abs, dv_abs: the same sums over term magnitudes, see
    orc_attend_backward), for error bounds.
    """
    lib = _load()
    nb, hkv, kg = cfg["n_q"] // cfg["q_block"], cfg["hkv"], cfg["top_groups"]
    gi = np.ascontiguousarray(np.asarray(group_idx, dtype=np.int32).reshape(nb, hkv, kg))
    ng = np.ascontiguousarray(np.asarray(n_groups, dtype=np.int32).reshape(nb, hkv))
    q64, k64, v64, dout64 = _f64(q64), _f64(k64), _f64(v64), _f64(dout64)
    dq = np.empty_like(q64)
    dk = np.empty_like(k64)
    dv = np.empty_like(v64)
    ab = (np.empty_like(q64), np.empty_like(k64), np.empty_like(v64)) if with_abs else (None, None, None)
    lib.orc_attend_backward(C.byref(make_cfg(cfg)), _ptr(q64), _ptr(k64), _ptr(v64), _ptr(dout64),
                            _ptr(gi), _ptr(ng), _ptr(dq), _ptr(dk), _ptr(dv), *(_ptr(a) for a in ab))
    return (dq, dk, dv, *ab) if with_abs else (dq, dk, dv)


def token_set(cfg, b, group_idx, n_groups):
    """Step 6: ascending token positions attended by block ``b``."""
    lib = _load()
    gi = np.ascontiguousarray(np.asarray(group_idx, dtype=np.int32))
    cap = cfg["L"]
    buf = np.empty(cap, np.int32)
    n = lib.orc_token_set(C.byref(make_cfg(cfg)), int(b), _ptr(gi), int(n_groups), _ptr(buf), cap)
    return buf[:n].copy()


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().orc_threads())


def set_threads(n: int) -> None:
    """Run the oracle's loops on n OpenMP threads from now on."""
    _load().orc_set_threads(int(n))


def valid_selection(scores, kept, k, eps) -> bool:
    """Several selections are correct at a boundary that is not certified:
    with v the k-th largest of the candidates' scores (NaN entries are not
    candidates), a kept set is correct when it holds min(k, candidates)
    distinct candidates, every candidate scoring above v + 2 eps, and none
    scoring below v - 2 eps (any evaluation order within the bound eps could
    have produced it)."""
    cand = np.flatnonzero(~np.isnan(scores))
    kept = np.asarray(kept, dtype=np.int64)
    kk = min(k, cand.size)
    if kept.size != kk or np.unique(kept).size != kk or not np.isin(kept, cand).all():
        return False
    if kk == 0 or kk == cand.size:
        return True
    v = np.sort(scores[cand])[::-1][kk - 1]
    must = cand[scores[cand] > v + 2.0 * eps]
    never = cand[scores[cand] < v - 2.0 * eps]
    return bool(np.isin(must, kept).all() and not np.isin(never, kept).any())


def certified(diag_row, stage: str) -> bool:
    """A boundary is certified when the gap between the k-th and (k+1)-th
    scores exceeds twice the error bound: every evaluation order then keeps
    the same set."""
    gap, eps = (diag_row[DG_GAP_C], diag_row[DG_EPS_C]) if stage == "chunk" else \
               (diag_row[DG_GAP_G], diag_row[DG_EPS_G])
    return bool(gap > 2.0 * eps)


def run(cfg, q64, k64, v64, items=None):
    """Route then attend (the whole forward) for a list of items."""
    items = all_items(cfg) if items is None else items
    ci, gi, ns, dg = route(cfg, q64, k64, items)
    out, lse = attend(cfg, q64, k64, v64, items, gi, ns[:, 1])
    return dict(chunk_idx=ci, group_idx=gi, n_sel=ns, diag=dg, out=out, lse=lse)
