"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every test here runs on the CPU. Each one is chosen so that a plausible slip in
the oracle (a dropped window, a wrong tie rule, an off-by-one in the causal
mask, a transposed operand) fails at least one of them.

Source of the method: "Long-Context Fine-Tuning with Limited VRAM", section 2.1.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(**kw):
    base = dict(L=256, n_q=256, hq=2, hkv=1, d=8, chunk=16, group=4, q_block=16,
                top_chunks=3, top_groups=5, sink=16, local=16, dtype="f32", rope_theta=None,
                shared_rank=0, shared_scale=0.0, n_plant_chunks=0, groups_per_plant_chunk=1,
                plant_chunks=(1, 2), alpha=0.0, beta=0.0, tier_split=0, cfg_id=50)
    base.update(kw)
    return base


def rand_qkv(cfg, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((cfg["hq"], cfg["n_q"], cfg["d"]))
    k = rng.standard_normal((cfg["hkv"], cfg["L"], cfg["d"]))
    v = rng.standard_normal((cfg["hkv"], cfg["L"], cfg["d"]))
    return q, k, v


def dense_causal(cfg, q, k, v):
    """Textbook dense causal attention (full score matrix, masked softmax)."""
    G = cfg["hq"] // cfg["hkv"]
    q0 = cfg["L"] - cfg["n_q"]
    scale = cfg.get("softmax_scale") or 1.0 / math.sqrt(cfg["d"])
    out = np.empty_like(q)
    lse = np.empty(q.shape[:2])
    pos_q = np.arange(q0, cfg["L"])[:, None]
    pos_k = np.arange(cfg["L"])[None, :]
    for hq in range(cfg["hq"]):
        s = scale * (q[hq] @ k[hq // G].T)
        s = np.where(pos_k <= pos_q, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        den = p.sum(axis=1, keepdims=True)
        out[hq] = (p / den) @ v[hq // G]
        lse[hq] = (m + np.log(den))[:, 0]
    return out, lse


def oracle_full(cfg, q, k, v):
    """Run the oracle on every item; return out [Hq][n_q][d], lse, and the routing."""
    res = oracle.run(cfg, q, k, v)
    G, B = cfg["hq"] // cfg["hkv"], cfg["q_block"]
    out = np.empty((cfg["hq"], cfg["n_q"], cfg["d"]))
    lse = np.empty((cfg["hq"], cfg["n_q"]))
    for n, (b, h) in enumerate(oracle.all_items(cfg)):
        for r in range(G):
            out[h * G + r, b * B:(b + 1) * B] = res["out"][n, r]
            lse[h * G + r, b * B:(b + 1) * B] = res["lse"][n, r]
    return out, lse, res


# ------------------------------------------------------------------ step 1
def test_summaries_closed_form_ramp():
    """Keys K[h][t][e] = (h+1) t + e/2: group j's mean is (h+1)(g j + (g-1)/2) + e/2."""
    cfg = tiny_cfg(hkv=2, hq=2, L=128, n_q=64)
    L, d, g, c = cfg["L"], cfg["d"], cfg["group"], cfg["chunk"]
    t = np.arange(L)[None, :, None]
    h = np.arange(2)[:, None, None]
    e = np.arange(d)[None, None, :]
    k = (h + 1) * t + 0.5 * e + 0.0 * t
    gs, cs = oracle.summaries(cfg, k)
    j = np.arange(L // g)[None, :, None]
    m = np.arange(L // c)[None, :, None]
    np.testing.assert_array_equal(gs, (h + 1) * (g * j + (g - 1) / 2) + 0.5 * e)
    np.testing.assert_array_equal(cs, (h + 1) * (c * m + (c - 1) / 2) + 0.5 * e)


def test_summaries_constant_and_chunk_is_mean_of_groups():
    cfg = tiny_cfg()
    k = np.full((1, cfg["L"], cfg["d"]), 0.375)
    gs, cs = oracle.summaries(cfg, k)
    assert np.all(gs == 0.375) and np.all(cs == 0.375)
    _, k, _ = rand_qkv(cfg, 3)
    gs, cs = oracle.summaries(cfg, k)
    per = cfg["chunk"] // cfg["group"]
    np.testing.assert_allclose(cs, gs.reshape(1, -1, per, cfg["d"]).mean(axis=2), rtol=0, atol=1e-15)


# ------------------------------------------------------------------ hand-worked example
def test_hand_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_L20.json")))
    cfg = tiny_cfg(**fx["config"])
    k = np.array(fx["k"], float)[None]
    q = np.array(fx["q"], float)[None]
    v = np.stack([np.arange(cfg["L"], dtype=float), np.ones(cfg["L"])], axis=1)[None]
    ci, gi, ns, dg = oracle.route(cfg, q, k, [(0, 0)])
    exp = fx["expected"]
    assert ci[0].tolist() == exp["chunk_idx"]
    assert gi[0].tolist() == exp["group_idx"]
    assert ns[0].tolist() == exp["n_sel"]
    assert oracle.token_set(cfg, 0, gi[0], ns[0, 1]).tolist() == exp["token_set"]
    out, lse = oracle.attend(cfg, q, k, v, [(0, 0)], gi, ns[:, 1])
    env = {"exp": math.exp, "log": math.log}
    for pos, expr in exp["out_0_closed_form"].items():
        i = int(pos) - 16
        assert out[0, 0, i, 0] == pytest.approx(eval(expr, env), rel=1e-14)
        assert out[0, 0, i, 1] == pytest.approx(1.0, rel=1e-14)
    for pos, expr in exp["lse_closed_form"].items():
        assert lse[0, 0, int(pos) - 16] == pytest.approx(eval(expr, env), rel=1e-14)


# ------------------------------------------------------------------ steps 4, 5: selection
def _designed_chunk_scores(cfg, weights):
    """Queries all equal e_0, chunk m keys all equal weights[m] e_0: score_m = weights[m]."""
    L, d, c = cfg["L"], cfg["d"], cfg["chunk"]
    q = np.zeros((cfg["hq"], cfg["n_q"], d)); q[..., 0] = 1.0
    k = np.zeros((1, L, d))
    for m in range(L // c):
        k[0, m * c:(m + 1) * c, 0] = weights[m]
    return q, k


def test_chunk_stage_closed_form_scores():
    cfg = tiny_cfg(n_q=16, top_chunks=4, top_groups=0)
    nc = cfg["L"] // cfg["chunk"]            # 16 chunks; the block is chunk 15
    rng = np.random.default_rng(7)
    w = rng.permutation(nc).astype(float)
    q, k = _designed_chunk_scores(cfg, w)
    ci, gi, ns, dg = oracle.route(cfg, q, k, [(0, 0)])
    cand = [m for m in range(nc - 1) if m != 0 and m != nc - 2]   # sink 0, local 14
    expect = sorted(sorted(cand, key=lambda m: -w[m])[:4])
    assert ci[0].tolist() == expect
    assert ns[0, 0] == 4 and dg[0, oracle.DG_NCAND_C] == len(cand)


def test_exact_ties_go_to_lower_index():
    cfg = tiny_cfg(n_q=16, top_chunks=3, top_groups=4)
    q = np.ones((cfg["hq"], 16, cfg["d"]))
    k = np.ones((1, cfg["L"], cfg["d"]))
    ci, gi, ns, _ = oracle.route(cfg, q, k, [(0, 0)])
    assert ci[0].tolist() == [1, 2, 3]          # chunk 0 is the sink
    assert gi[0].tolist() == [4, 5, 6, 7]       # the first 4 groups of chunk 1


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_exhaustive_subset_search(seed):
    """For small candidate counts, enumerate every k-subset: the kept set is the
    unique subset where each kept item beats each dropped one (higher score, or
    an equal score and a lower index)."""
    cfg = tiny_cfg(L=176, n_q=16, top_chunks=3, top_groups=4, d=4)
    rng = np.random.default_rng(100 + seed)
    q = rng.standard_normal((cfg["hq"], 16, cfg["d"]))
    k = rng.integers(-2, 3, size=(1, cfg["L"], cfg["d"])).astype(float)   # frequent ties
    ci, gi, ns, dg = oracle.route(cfg, q, k, [(0, 0)])
    # decision score: float64 block-mean query against the float32-rounded summary
    qbar = q[:, :16].reshape(-1, cfg["d"]).mean(axis=0)
    gs, cs = oracle.summaries(cfg, k)

    def score(vec):
        return float(np.dot(qbar, vec.astype(np.float32).astype(np.float64)))

    def beats(x, y, sc):
        return sc[x] > sc[y] or (sc[x] == sc[y] and x < y)

    def brute(cands, sc, kk):
        kk = min(kk, len(cands))
        good = [S for S in itertools.combinations(cands, kk)
                if all(beats(x, y, sc) for x in S for y in cands if y not in S)]
        assert len(good) == 1
        return sorted(good[0])

    nc = cfg["L"] // cfg["chunk"]
    cands = [m for m in range(1, nc - 2)]
    scc = {m: score(cs[0, m]) for m in cands}
    selc = brute(cands, scc, 3)
    assert ci[0].tolist() == selc
    gcands = [m * 4 + u for m in selc for u in range(4)]
    scg = {j: score(gs[0, j]) for j in gcands}
    assert gi[0].tolist() == brute(gcands, scg, 4)


def test_selection_is_permutation_equivariant():
    """Swapping the contents of two candidate chunks swaps them in the selection."""
    cfg = tiny_cfg(n_q=16, top_chunks=4, top_groups=6)
    q, k, _ = rand_qkv(cfg, 11)
    q += 0.5
    k[0, 16 * 9:16 * 10] += 1.0
    ci, gi, ns, _ = oracle.route(cfg, q, k, [(0, 0)])
    a, b = 3, 9
    k2 = k.copy()
    k2[0, 16 * a:16 * (a + 1)], k2[0, 16 * b:16 * (b + 1)] = k[0, 16 * b:16 * (b + 1)], k[0, 16 * a:16 * (a + 1)]
    ci2, gi2, _, _ = oracle.route(cfg, q, k2, [(0, 0)])
    sw = {a: b, b: a}
    assert sorted(sw.get(m, m) for m in ci[0]) == ci2[0].tolist()
    gmap = lambda j: sw.get(j // 4, j // 4) * 4 + j % 4
    assert sorted(gmap(j) for j in gi[0]) == gi2[0].tolist()


# ------------------------------------------------------------------ step 7: attention
@pytest.mark.parametrize("hq,hkv,ragged", [(1, 1, False), (4, 2, False), (6, 3, True)])
def test_dense_equivalence_when_budget_covers_everything(hq, hkv, ragged):
    """With kc >= every candidate and kg >= all their groups, routed attention is
    dense causal attention (the token set is every earlier token)."""
    L = 176 if ragged else 256
    cfg = tiny_cfg(L=L, n_q=L - 32, hq=hq, hkv=hkv, top_chunks=L // 16, top_groups=L // 4)
    q, k, v = rand_qkv(cfg, 5)
    out, lse, res = oracle_full(cfg, q, k, v)
    ref, rlse = dense_causal(cfg, q, k, v)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("q_block,L,n_q", [(1, 183, 1), (1, 256, 40), (4, 180, 72), (8, 256, 104)])
def test_dense_equivalence_small_query_blocks(q_block, L, n_q):
    """Blocks smaller than a chunk (q_block = 1 is per-token decoding), with a
    sequence that may end inside an open chunk: under a budget that covers
    every candidate the token set is every earlier token, so the result is
    dense causal attention. Dropping the open chunk's earlier tokens, or taking
    the windows from the block instead of its chunk, fails this."""
    cfg = tiny_cfg(L=L, n_q=n_q, q_block=q_block, hq=4, hkv=2, top_chunks=L // 16, top_groups=L // 4)
    q, k, v = rand_qkv(cfg, 15)
    out, lse, _ = oracle_full(cfg, q, k, v)
    ref, rlse = dense_causal(cfg, q, k, v)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("q_block", [1, 4])
def test_no_routing_budget_small_blocks_is_chunk_diagonal_attention(q_block):
    """With no windows and no budget a block sees only its own open chunk up to
    itself: dense causal attention restricted to each chunk."""
    cfg = tiny_cfg(sink=0, local=0, top_chunks=0, top_groups=0, hq=2, hkv=1, q_block=q_block, n_q=128)
    q, k, v = rand_qkv(cfg, 16)
    out, lse, _ = oracle_full(cfg, q, k, v)
    c, q0 = cfg["chunk"], cfg["L"] - cfg["n_q"]
    for m in range(q0 // c, cfg["L"] // c):
        sub = tiny_cfg(L=c, n_q=c, hq=2, hkv=1)
        sl = slice(m * c, (m + 1) * c)
        ref, rlse = dense_causal(sub, q[:, m * c - q0:(m + 1) * c - q0], k[:, sl], v[:, sl])
        np.testing.assert_allclose(out[:, m * c - q0:(m + 1) * c - q0], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, m * c - q0:(m + 1) * c - q0], rlse, rtol=0, atol=1e-12)


def test_single_token_block_query_is_the_head_mean():
    """q_block = 1, G = 1: the block query is the query itself, so the kept
    chunks are the top kc of q . CS[m] over the non-fixed closed chunks (brute
    force over the float32-rounded summaries, ties to the lower index)."""
    cfg = tiny_cfg(L=250, n_q=1, q_block=1, hq=1, hkv=1, sink=16, local=32, top_chunks=4, top_groups=6)
    q, k, v = rand_qkv(cfg, 17)
    ci, gi, ns, _ = oracle.route(cfg, q, k, [(0, 0)])
    gs, cs = oracle.summaries(cfg, k)
    s = 249
    ms = s // 16
    cand = [m for m in range(ms) if not (m < 1 or m >= ms - 2)]
    sc = {m: float(np.dot(q[0, 0], cs[0, m].astype(np.float32).astype(np.float64))) for m in cand}
    keep = sorted(sorted(cand, key=lambda m: (-sc[m], m))[:4])
    assert ci[0].tolist() == keep
    groups = [4 * m + u for m in keep for u in range(4)]
    gsc = {j: float(np.dot(q[0, 0], gs[0, j].astype(np.float32).astype(np.float64))) for j in groups}
    assert gi[0].tolist() == sorted(sorted(groups, key=lambda j: (-gsc[j], j))[:6])
    assert ns[0].tolist() == [4, 6]


def test_no_routing_budget_is_block_diagonal_attention():
    cfg = tiny_cfg(sink=0, local=0, top_chunks=0, top_groups=0, hq=2, hkv=1)
    q, k, v = rand_qkv(cfg, 6)
    out, lse, _ = oracle_full(cfg, q, k, v)
    B = cfg["q_block"]
    for b in range(cfg["n_q"] // B):
        sub = tiny_cfg(L=B, n_q=B, hq=2, hkv=1)
        ref, rlse = dense_causal(sub, q[:, b * B:(b + 1) * B], k[:, b * B:(b + 1) * B], v[:, b * B:(b + 1) * B])
        np.testing.assert_allclose(out[:, b * B:(b + 1) * B], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, b * B:(b + 1) * B], rlse, rtol=0, atol=1e-12)


def test_constant_values_and_uniform_weights():
    """Constant V gives O = V; Q = 0 gives uniform weights, so O is the mean of V
    over the visible kept tokens and LSE = log(count)."""
    cfg = tiny_cfg()
    q, k, v = rand_qkv(cfg, 8)
    vc = np.full_like(v, -1.25)
    out, _, _ = oracle_full(cfg, q, k, vc)
    np.testing.assert_allclose(out, -1.25, rtol=0, atol=1e-13)
    q0 = np.zeros_like(q)
    out, lse, res = oracle_full(cfg, q0, k, v)
    B = cfg["q_block"]
    for n, (b, h) in enumerate(oracle.all_items(cfg)):
        T = oracle.token_set(cfg, b, res["group_idx"][n], res["n_sel"][n, 1])
        for i in (0, 5, B - 1):
            pos = b * B + i
            vis = T[T <= pos]
            np.testing.assert_allclose(out[0, pos], v[0, vis].mean(axis=0), atol=1e-13)
            assert lse[0, pos] == pytest.approx(math.log(len(vis)), abs=1e-13)


def test_causality_future_keys_do_not_change_past_outputs():
    cfg = tiny_cfg(top_chunks=2, top_groups=3)
    q, k, v = rand_qkv(cfg, 9)
    out, lse, _ = oracle_full(cfg, q, k, v)
    rng = np.random.default_rng(1)
    for p in (37, 100, 170, 250):
        k2, v2 = k.copy(), v.copy()
        k2[:, p + 1:] += rng.standard_normal(k2[:, p + 1:].shape) * 3
        v2[:, p + 1:] -= 2.0
        o2, l2, _ = oracle_full(cfg, q, k2, v2)
        np.testing.assert_array_equal(o2[:, :p + 1], out[:, :p + 1])
        np.testing.assert_array_equal(l2[:, :p + 1], lse[:, :p + 1])
        assert not np.array_equal(o2[:, p + 1:], out[:, p + 1:])


# ------------------------------------------------------------------ step 6 invariants
@pytest.mark.parametrize("cfg_over", [dict(), dict(sink=32, local=48, top_chunks=4, top_groups=7),
                                      dict(sink=0, local=16, top_chunks=1, top_groups=4, n_q=128),
                                      dict(q_block=1, n_q=40, top_chunks=2, top_groups=5),
                                      dict(q_block=4, L=252, n_q=100, sink=32, top_chunks=3, top_groups=6)])
def test_routing_and_token_set_invariants(cfg_over):
    cfg = tiny_cfg(**cfg_over)
    q, k, v = rand_qkv(cfg, 12)
    items = oracle.all_items(cfg)
    ci, gi, ns, dg = oracle.route(cfg, q, k, items)
    c, g, B = cfg["chunk"], cfg["group"], cfg["q_block"]
    q0 = cfg["L"] - cfg["n_q"]
    for n, (b, h) in enumerate(items):
        s = q0 + b * B
        ms = s // c
        fixed = {m for m in range(ms) if m < cfg["sink"] // c or m >= ms - cfg["local"] // c}
        cand = [m for m in range(ms) if m not in fixed]
        nsc, nsg = ns[n]
        assert nsc == min(cfg["top_chunks"], len(cand))
        assert nsg == min(cfg["top_groups"], nsc * (c // g))
        selc = ci[n, :nsc].tolist()
        assert all(x == -1 for x in ci[n, nsc:]) and all(x == -1 for x in gi[n, nsg:])
        assert selc == sorted(set(selc)) and not (set(selc) & fixed)
        selg = gi[n, :nsg].tolist()
        assert selg == sorted(set(selg))
        assert all(j // (c // g) in selc for j in selg)
        assert all((j + 1) * g <= s for j in selg)
        T = oracle.token_set(cfg, b, gi[n], nsg)
        assert T.tolist() == sorted(set(T.tolist()))
        assert T.max() == s + B - 1
        expect = set(range(ms * c, s + B))   # the block's open chunk up to the block's end
        for m in fixed:
            expect |= set(range(m * c, (m + 1) * c))
        for j in selg:
            expect |= set(range(j * g, (j + 1) * g))
        assert set(T.tolist()) == expect
        assert len(T) == c * len(fixed) + g * nsg + (s + B - ms * c)


# ------------------------------------------------------------------ planted workloads
def test_planted_margins_tiny_workload():
    """The tiny fp32 workload: 4 planted groups; wherever all planted chunks are
    candidates, the kept chunks are exactly them with a score margin >= 0.5, and
    the planted groups are kept."""
    cfg = synth.config(0)
    x = synth.make_inputs(cfg)
    q, k = synth.to_f64(x["q"], "f32"), synth.to_f64(x["k"], "f32")
    ci, gi, ns, dg = oracle.route(cfg, q, k)
    planted = x["planted"][0]
    pch = sorted({j // 8 for j in planted})
    n_checked = 0
    for b in range(cfg["n_q"] // 64):
        if b - 2 >= max(pch):
            n_checked += 1
            assert ci[b].tolist() == pch
            assert dg[b, oracle.DG_GAP_C] >= 0.5
            assert set(planted) <= set(gi[b].tolist())
    assert n_checked >= 2


# ------------------------------------------------------------------ backward of step 7
def _routing(cfg, q, k):
    items = oracle.all_items(cfg)
    ci, gi, ns, _ = oracle.route(cfg, q, k, items)
    nb, hkv = cfg["n_q"] // cfg["q_block"], cfg["hkv"]
    return items, gi.reshape(nb, hkv, -1), ns[:, 1].reshape(nb, hkv)


def _forward_full(cfg, q, k, v, items, gi, ng):
    """Forward output [Hq][n_q][d] for fixed routing."""
    G, B = cfg["hq"] // cfg["hkv"], cfg["q_block"]
    flat_gi = gi.reshape(len(items), -1)
    flat_ng = ng.reshape(len(items))
    out, _ = oracle.attend(cfg, q, k, v, items, flat_gi, flat_ng)
    full = np.empty_like(q)
    for n, (b, h) in enumerate(items):
        for r in range(G):
            full[h * G + r, b * B:(b + 1) * B] = out[n, r]
    return full


@pytest.mark.parametrize("q_block,n_q", [(16, 48), (4, 36)])
def test_backward_matches_finite_differences(q_block, n_q):
    """Central differences of L = sum(dO * O) with the routing held fixed, for
    every element of Q, K and V (history keys included)."""
    cfg = tiny_cfg(L=64, n_q=n_q, hq=2, hkv=1, d=4, q_block=q_block, sink=16, local=0,
                   top_chunks=1, top_groups=2)
    q, k, v = rand_qkv(cfg, 21)
    dout = np.random.default_rng(22).standard_normal(q.shape)
    items, gi, ng = _routing(cfg, q, k)
    assert ng.max() > 0          # some block keeps routed groups
    dq, dk, dv = oracle.attend_backward(cfg, q, k, v, dout, gi, ng)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            fp = _forward_full(cfg, **{**args, name: xp}, items=items, gi=gi, ng=ng)
            fm = _forward_full(cfg, **{**args, name: xm}, items=items, gi=gi, ng=ng)
            num[idx] = ((fp - fm) * dout).sum() / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-7, err_msg=name)
    assert np.abs(dk[:, :16]).max() > 0   # the sink chunk (history) receives gradient
    # the magnitude companions bound the gradients (triangle inequality) and
    # leave the gradients themselves unchanged
    ab = oracle.attend_backward(cfg, q, k, v, dout, gi, ng, with_abs=True)
    for g, g2, a in zip((dq, dk, dv), ab[:3], ab[3:]):
        np.testing.assert_array_equal(g, g2)
        assert (a >= np.abs(g) - 1e-15).all() and a.max() > 0


def _dense_backward(cfg, q, k, v, dout):
    """Matrix-form backward of dense causal attention: P = softmax(S),
    dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = s dS K,
    dK = s dS^T Q (summed over the query heads of each KV head)."""
    G = cfg["hq"] // cfg["hkv"]
    q0 = cfg["L"] - cfg["n_q"]
    scale = 1.0 / math.sqrt(cfg["d"])
    mask = np.arange(cfg["L"])[None, :] <= np.arange(q0, cfg["L"])[:, None]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for hq in range(cfg["hq"]):
        h = hq // G
        S = np.where(mask, scale * q[hq] @ k[h].T, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = dout[hq] @ v[h].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dq[hq] = scale * dS @ k[h]
        dk[h] += scale * dS.T @ q[hq]
        dv[h] += P.T @ dout[hq]
    return dq, dk, dv


@pytest.mark.parametrize("q_block,L,n_q", [(16, 256, 224), (1, 183, 40), (8, 176, 176)])
def test_backward_dense_equivalence(q_block, L, n_q):
    """A budget covering every candidate makes the token set every earlier
    token: the gradients are those of dense causal attention."""
    cfg = tiny_cfg(L=L, n_q=n_q, hq=4, hkv=2, q_block=q_block, top_chunks=L // 16, top_groups=L // 4)
    q, k, v = rand_qkv(cfg, 23)
    dout = np.random.default_rng(24).standard_normal(q.shape)
    _, gi, ng = _routing(cfg, q, k)
    got = oracle.attend_backward(cfg, q, k, v, dout, gi, ng)
    ref = _dense_backward(cfg, q, k, v, dout)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11, err_msg=name)


def test_backward_invariants():
    """Shifting every key of a head by one vector moves each row's scores by a
    constant, so the key gradients of a head sum to zero; each row's weights
    sum to one, so the value gradients of a head sum to the output gradients
    of its query heads."""
    cfg = tiny_cfg(hq=4, hkv=2, top_chunks=2, top_groups=3)
    q, k, v = rand_qkv(cfg, 25)
    dout = np.random.default_rng(26).standard_normal(q.shape)
    _, gi, ng = _routing(cfg, q, k)
    dq, dk, dv = oracle.attend_backward(cfg, q, k, v, dout, gi, ng)
    G = cfg["hq"] // cfg["hkv"]
    for h in range(cfg["hkv"]):
        np.testing.assert_allclose(dk[h].sum(axis=0), 0.0, atol=1e-11)
        np.testing.assert_allclose(dv[h].sum(axis=0), dout[h * G:(h + 1) * G].sum(axis=(0, 1)), atol=1e-11)
    # keys after the last query and outside every token set get nothing
    assert np.abs(dq).max() > 0


# ------------------------------------------------------------------ certification bound
def test_abs_summaries_closed_form_sign_alternating():
    """Keys K[0][t][e] = (-1)^t (t + 1 + e): the mean of |K| over group j is
    g j + (g + 1) / 2 + e (likewise per chunk), while the plain mean of every
    group and chunk (of even size, starting at an even token) is -1/2: each
    pair of neighbours sums to -1."""
    cfg = tiny_cfg(L=128, n_q=64)
    L, d, g, c = cfg["L"], cfg["d"], cfg["group"], cfg["chunk"]
    t = np.arange(L)[None, :, None]
    e = np.arange(d)[None, None, :]
    k = np.where(t % 2 == 0, 1.0, -1.0) * (t + 1 + e)
    ga, ca = oracle.abs_summaries(cfg, k)
    gs, cs = oracle.summaries(cfg, k)
    j = np.arange(L // g)[None, :, None]
    m = np.arange(L // c)[None, :, None]
    np.testing.assert_array_equal(ga, g * j + (g + 1) / 2 + e + 0.0 * j)
    np.testing.assert_array_equal(ca, c * m + (c + 1) / 2 + e + 0.0 * m)
    assert np.all(gs == -0.5) and np.all(cs == -0.5)


def _alt_score(rng, qrows, krows, adversarial):
    """One decision score evaluated in another order: the block mean and the
    summary summed sequentially in a random order, the summary rounded to
    float32 (and, with adversarial = +1 / -1, moved one float32 step in the
    direction that raises / lowers the score), the dot summed in a random
    order."""
    qb = np.cumsum(qrows[rng.permutation(len(qrows))], axis=0)[-1] / len(qrows)
    s = (np.cumsum(krows[rng.permutation(len(krows))], axis=0)[-1] / len(krows)).astype(np.float32)
    if adversarial:
        s = np.nextafter(s, np.where(adversarial * qb > 0, np.float32(np.inf), np.float32(-np.inf))).astype(np.float32)
    prod = qb * s.astype(np.float64)
    return np.cumsum(prod[rng.permutation(len(prod))])[-1]


@pytest.mark.parametrize("dtype,seed", [("f32", 0), ("f32", 1), ("bf16", 2), ("bf16", 3)])
def test_eps_bounds_every_evaluation_order(dtype, seed):
    """The bound eps must cover every evaluation order of the block mean, the
    summary mean and the dot, and a float32 summary landing one step away:
    for every candidate of both stages, scores recomputed in random orders and
    with adversarially rounded summaries stay within eps of the oracle's. It
    must also not be vacuous: the adversarial one-step moves reach at least
    1/64 of it."""
    cfg = tiny_cfg(L=512, n_q=64, hq=4, hkv=2, d=16, chunk=64, group=8, q_block=64, top_chunks=2, top_groups=5,
                   sink=64, local=64)
    rng = np.random.default_rng(100 + seed)
    q, k, _ = rand_qkv(cfg, seed)
    if dtype == "bf16":
        q = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(q.astype(np.float32)))
        k = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(k.astype(np.float32)))
    else:
        q, k = q.astype(np.float32).astype(np.float64), k.astype(np.float32).astype(np.float64)
    items = oracle.all_items(cfg)
    csc, gsc, eps = oracle.route_scores(cfg, q, k, items)
    _, _, _, dg = oracle.route(cfg, q, k, items)
    G, B, c, g = cfg["hq"] // cfg["hkv"], cfg["q_block"], cfg["chunk"], cfg["group"]
    q0 = cfg["L"] - cfg["n_q"]
    for n, (b, h) in enumerate(items):
        assert eps[n, 0] >= dg[n, oracle.DG_EPS_C] and eps[n, 1] >= dg[n, oracle.DG_EPS_G]
        s = q0 + b * B
        qrows = q[h * G:(h + 1) * G, s - q0:s - q0 + B].reshape(-1, cfg["d"])
        for sc, size, e in ((csc[n], c, eps[n, 0]), (gsc[n], g, eps[n, 1])):
            idx = np.flatnonzero(~np.isnan(sc))
            assert idx.size > 0
            worst_adv = 0.0
            for i in idx:
                krows = k[h, i * size:(i + 1) * size]
                for adversarial in (0, 0, 1, -1):
                    dev = abs(_alt_score(rng, qrows, krows, adversarial) - sc[i])
                    assert dev <= e, f"item {n} candidate {i}: order moved the score by {dev} > eps {e}"
                    if adversarial:
                        worst_adv = max(worst_adv, dev)
            assert worst_adv >= e / 64, f"item {n}: eps {e} is far above any reachable move {worst_adv}"


def test_route_scores_agree_with_the_selection():
    """The score tables give the oracle's own selection back: the kept chunks
    are the top-kc candidates by (score desc, index asc), the kept groups the
    top-kg groups of the kept chunks, and the reported gaps are the gaps of
    the tables."""
    cfg = tiny_cfg(L=512, n_q=128, hq=4, hkv=2, d=16, chunk=32, group=8, q_block=32, top_chunks=3,
                   top_groups=5, sink=32, local=32)
    q, k, _ = rand_qkv(cfg, 11)
    items = oracle.all_items(cfg)
    ci, gi, ns, dg = oracle.route(cfg, q, k, items)
    csc, gsc, _ = oracle.route_scores(cfg, q, k, items)
    gpc = cfg["chunk"] // cfg["group"]
    for n in range(len(items)):
        cand = np.flatnonzero(~np.isnan(csc[n]))
        order = sorted(cand, key=lambda m: (-csc[n][m], m))
        kc = min(cfg["top_chunks"], cand.size)
        assert ci[n][:kc].tolist() == sorted(order[:kc]) and ns[n, 0] == kc
        if 0 < kc < cand.size:
            assert dg[n, oracle.DG_GAP_C] == csc[n][order[kc - 1]] - csc[n][order[kc]]
        groups = [m * gpc + u for m in ci[n][:kc] for u in range(gpc)]
        gorder = sorted(groups, key=lambda j: (-gsc[n][j], j))
        kg = min(cfg["top_groups"], len(groups))
        assert gi[n][:kg].tolist() == sorted(gorder[:kg]) and ns[n, 1] == kg


def test_valid_selection_rule():
    """Several selections are correct only inside the band of 2 eps around the
    k-th score; outside it, and for the count, the choice is forced."""
    nan = np.nan
    sc = np.array([5.0, nan, 3.0, 3.0 + 1e-9, 2.0, 1.0])
    assert oracle.valid_selection(sc, [0, 2], 2, eps=1e-6)          # within the band: either tie member
    assert oracle.valid_selection(sc, [0, 3], 2, eps=1e-6)
    assert not oracle.valid_selection(sc, [0, 2], 2, eps=1e-12)     # outside the band the order decides
    assert not oracle.valid_selection(sc, [0, 4], 2, eps=1e-6)      # 2.0 is below the band
    assert not oracle.valid_selection(sc, [2, 3], 2, eps=1e-6)      # 5.0 is above it and must be kept
    assert not oracle.valid_selection(sc, [0], 2, eps=1e-6)         # count
    assert not oracle.valid_selection(sc, [0, 1], 2, eps=1e-6)      # not a candidate
    assert not oracle.valid_selection(sc, [0, 0], 2, eps=1e-6)      # not distinct
    assert oracle.valid_selection(sc, [0, 2, 3, 4, 5], 9, eps=0.0)  # the budget covers all


def test_exact_ties_on_periodic_integer_keys():
    """Integer queries and keys that repeat every 3 chunks make many scores
    exactly equal (exact in float64): the kept sets must be the first in
    (score desc, index asc) order, which a brute force over exact rational
    scores (fractions, no floating point) gives independently."""
    from fractions import Fraction
    cfg = tiny_cfg(L=1024, n_q=128, hq=2, hkv=1, d=8, chunk=64, group=8, q_block=64, top_chunks=4,
                   top_groups=9, sink=64, local=64, dtype="f32", integer_values=(-2, 2), chunk_period=3)
    x = synth.make_inputs(cfg)
    q, k = synth.to_f64(x["q"], "f32"), synth.to_f64(x["k"], "f32")
    items = oracle.all_items(cfg)
    ci, gi, ns, dg = oracle.route(cfg, q, k, items)
    G, B, c, g, d = 2, 64, 64, 8, cfg["d"]
    ki = k.astype(np.int64)
    ties = 0
    for n, (b, h) in enumerate(items):
        s = cfg["L"] - cfg["n_q"] + b * B
        rows = q[h * G:(h + 1) * G, b * B:(b + 1) * B].reshape(-1, d).astype(np.int64)
        qbar = [Fraction(int(rows[:, e].sum()), len(rows)) for e in range(d)]

        def exact(lo, size):
            return sum(qbar[e] * Fraction(int(ki[h, lo:lo + size, e].sum()), size) for e in range(d))
        ms = s // c
        cand = [m for m in range(ms) if m >= cfg["sink"] // c and m < ms - cfg["local"] // c]
        sc = {m: exact(m * c, c) for m in cand}
        order = sorted(cand, key=lambda m: (-sc[m], m))
        kc = min(cfg["top_chunks"], len(cand))
        if kc < len(cand) and sc[order[kc - 1]] == sc[order[kc]]:
            ties += 1
        assert ci[n][:kc].tolist() == sorted(order[:kc])
        groups = [m * (c // g) + u for m in sorted(order[:kc]) for u in range(c // g)]
        gsc = {j: exact(j * g, g) for j in groups}
        gorder = sorted(groups, key=lambda j: (-gsc[j], j))
        kg = min(cfg["top_groups"], len(groups))
        if kg < len(groups) and gsc[gorder[kg - 1]] == gsc[gorder[kg]]:
            ties += 1
        assert gi[n][:kg].tolist() == sorted(gorder[:kg])
    assert ties > 0, "the periodic keys should put exact ties on some boundary"
