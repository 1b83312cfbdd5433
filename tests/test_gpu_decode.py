"""Query blocks smaller than a chunk, down to per-token decoding, on the GPU
against the oracle ("Long-Context Fine-Tuning with Limited VRAM", section 2.1:
the current query block routes over the resident summaries of the closed
chunks; the pages' generation use routes one generated token at a time).

Reading shared with the oracle: the block's own chunk is open (no summary), so
its tokens from the chunk start up to the block's last position are attended
whole and causally; windows and candidates are taken relative to that chunk.

Each case cuts a prefix of a seeded workload (its queries keep their RoPE
positions) so the sequence ends at the block's last position, and runs the
GPU path as a decoding cache would: K/V and summary buffers sized to the
workload's full length, every row past the sequence NaN, only the summaries
of the sequence's whole chunks built. Routing must match the oracle wherever
the oracle certifies the boundary and be a correct selection elsewhere; the
kept sets must in fact equal the oracle's on every item, so attention is
compared with the oracle's attention over the oracle's own routing. A
token near the start of the sequence attends a handful of tokens, so its
output is not averaged down and its own bfloat16 rounding is as large as the
mean-abs bar: bfloat16 outputs are measured beyond that rounding (see
harness.check_outputs), and the same cases run again in the float32 output
mode (HGA_BF16_F32OUT: the output before that rounding), which takes the bars
unchanged. The LSE, in float32, takes the bar unchanged in both.
"""
import numpy as np
import pytest

import oracle
import synth
from harness import bf16_round, check_outputs, check_routing, gpu_run, inputs, oracle_route

pytestmark = pytest.mark.gpu


def prefix_case(cfg_id, end, B, n_q):
    """Workload cfg_id cut to positions [0, end) with the last n_q of them
    querying in blocks of B. Returns (cfg, stored inputs, float64 inputs)."""
    full, x, f = inputs(cfg_id)
    q0_full = full["L"] - full["n_q"]
    q0 = end - n_q
    assert q0 >= q0_full and end <= full["L"] and n_q % B == 0 and q0 % B == 0
    cfg = dict(full, L=end, n_q=n_q, q_block=B, tier_split=0)
    sl = slice(q0 - q0_full, end - q0_full)
    xs = {"q": x["q"][:, sl], "k": x["k"][:, :end], "v": x["v"][:, :end]}
    fs = {"q": f["q"][:, sl], "k": f["k"][:, :end], "v": f["v"][:, :end]}
    return cfg, xs, fs, full["L"]


def check_case(cfg, x, f, capacity, fused=False, split=0, spread=False, out_f32=False):
    print(f"[decode] {cfg['name']} end={cfg['L']} n_q={cfg['n_q']} B={cfg['q_block']} fused={fused} "
          f"split={split} spread={spread} out_f32={out_f32}", flush=True)
    gpu = gpu_run(cfg, x, capacity=capacity, fused=fused, split=split, spread=spread, out_f32=out_f32)
    ref = oracle_route(cfg, f)
    n, uncert, mism = check_routing(cfg, gpu, ref, f)
    print(f"  items={n} uncertified boundaries={uncert} differing sets={mism}", flush=True)
    assert mism == 0
    items = oracle.all_items(cfg)
    ro, rl = oracle.attend(cfg, f["q"], f["k"], f["v"], items, ref[1], ref[2][:, 1])
    mx, mean, lerr = check_outputs(cfg, gpu, items, ro, rl,
                                   beyond_output_rounding=cfg["dtype"] == "bf16" and not out_f32)
    print(f"  max_abs={mx:.3g} mean_abs={mean:.3g} lse={lerr:.3g}", flush=True)
    return gpu


# one generated token at positions around chunk edges, inside the sink and
# local windows, and deep in the history
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("pos", [0, 1, 63, 64, 127, 130, 191, 1000, 2047, 4095])
def test_decode_token_qwen3_8b_4k(pos, fused):
    cfg, x, f, cap = prefix_case(1, pos + 1, 1, 1)
    check_case(cfg, x, f, cap, fused=fused)


# the same tokens with the output in float32, at the bars unchanged
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("pos", [0, 1, 63, 64, 130, 2047, 4095])
def test_decode_token_qwen3_8b_4k_f32_output(pos, fused):
    cfg, x, f, cap = prefix_case(1, pos + 1, 1, 1)
    check_case(cfg, x, f, cap, fused=fused, out_f32=True)


@pytest.mark.parametrize("pos", [14336, 15000, 16383])
def test_decode_token_segment_16k(pos):
    cfg, x, f, cap = prefix_case(2, pos + 1, 1, 1)
    check_case(cfg, x, f, cap, fused=True)


def test_decode_token_64k_device_and_host_tier():
    """G = 8 (two waves of query rows would be one for decoding), 256 kept
    groups; the same token with K/V and group summaries of the history in
    pinned host memory goes through the host-tier cache."""
    cfg, x, f, cap = prefix_case(3, 65000, 1, 1)
    a = check_case(cfg, x, f, cap)
    b = check_case(cfg, x, f, cap, split=64 * (64999 // 64))
    for name in ("chunk_idx", "group_idx", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(a[name], b[name])


# the float32 output mode through every output path (the one-workgroup
# kernel, the fused kernel, the spread kernels, the host tier): at the bars
# unchanged, and each bfloat16 output is its float32 output rounded
@pytest.mark.parametrize("path", ["attend", "fused", "spread", "host_tier", "block64_fused", "block64_g8"])
def test_float32_output_mode(path):
    if path == "host_tier":
        cfg, x, f, cap = prefix_case(3, 65000, 1, 1)
        kw = dict(split=64 * (64999 // 64))
    elif path == "block64_fused":
        cfg, x, f, cap = prefix_case(1, 4096, 64, 256)
        kw = dict(fused=True)
    elif path == "block64_g8":
        cfg, x, f, cap = prefix_case(3, 65536, 64, 128)
        kw = {}
    else:
        cfg, x, f, cap = prefix_case(1, 2048, 1, 1)
        kw = dict(fused=path == "fused", spread=path == "spread")
    a = check_case(cfg, x, f, cap, out_f32=True, **kw)
    b = gpu_run(cfg, x, capacity=cap, **kw)
    for name in ("chunk_idx", "group_idx", "n_sel", "lse"):
        np.testing.assert_array_equal(a[name], b[name])
    np.testing.assert_array_equal(bf16_round(a["out"]), b["out"])


# small blocks (speculative or chunked decoding): several blocks per call,
# ending inside a chunk; B = 32 gives the item 128 query rows (4 waves)
@pytest.mark.parametrize("B", [2, 4, 8, 16, 32])
def test_small_blocks_qwen3_8b_4k(B):
    end = 4096 - 3 * B
    cfg, x, f, cap = prefix_case(1, end, B, 16 * B)
    a = check_case(cfg, x, f, cap)
    b = check_case(cfg, x, f, cap, fused=True)
    for name in ("chunk_idx", "group_idx", "n_sel", "out", "lse"):
        np.testing.assert_array_equal(a[name], b[name])


@pytest.mark.parametrize("B,end,n_q", [(1, 1, 1), (1, 700, 1), (1, 1024, 1), (8, 1000, 64), (16, 1024, 1024)])
def test_small_blocks_float32(B, end, n_q):
    """The float32 SIMT kernel (tiny workload, one query head)."""
    cfg, x, f, cap = prefix_case(0, end, B, n_q)
    check_case(cfg, x, f, cap)


def test_decode_matches_full_block_call_where_tokens_agree():
    """The last position of a 64-token block sees the same token set as a
    one-token block at that position: the block query differs, so routing may
    differ, but with a budget covering every candidate both are dense causal
    attention; the outputs then agree to rounding."""
    full, x, f = inputs(1)
    cfg = dict(full, top_chunks=64, top_groups=512)
    wide = {"q": x["q"], "k": x["k"], "v": x["v"]}
    a = gpu_run(dict(cfg, L=1024, n_q=1024), {"q": wide["q"][:, :1024], "k": wide["k"][:, :1024],
                                            "v": wide["v"][:, :1024]})
    b = gpu_run(dict(cfg, L=1024, n_q=1, q_block=1), {"q": wide["q"][:, 1023:1024], "k": wide["k"][:, :1024],
                                                       "v": wide["v"][:, :1024]}, capacity=4096)
    np.testing.assert_allclose(b["out"][:, 0], a["out"][:, 1023], rtol=0, atol=2e-2)
    np.testing.assert_allclose(b["lse"][:, 0], a["lse"][:, 1023], rtol=0, atol=1e-3)


# Few items with the attention workspace: each item's tile list is cut into
# ranges, one workgroup each, merged per row through the LSE. Parity with the
# oracle as above; against the one-workgroup call the routing is identical.
def check_spread(cfg, x, f, cap, fused):
    a = check_case(cfg, x, f, cap, fused=fused, spread=True)
    b = gpu_run(cfg, x, capacity=cap, fused=fused)
    for name in ("chunk_idx", "group_idx", "n_sel"):
        np.testing.assert_array_equal(a[name], b[name])
    # The probabilities go to the PV product as bf16 relative to each
    # workgroup's own running maximum, so the two calls round them
    # differently (2^-9 relative each): outputs are held to the workload's
    # output bar between the two calls as well; the LSE sums float32
    # probabilities and agrees to float32 rounding.
    diff = np.abs(a["out"] - b["out"])
    print(f"  spread vs one workgroup: max {diff.max():.3g} mean {diff.mean():.3g}", flush=True)
    assert diff.max() <= 2e-2 and diff.mean() <= 1e-3
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=0, atol=1e-4)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("pos", [0, 63, 130, 2047, 4095])
def test_decode_token_spread_qwen3_8b_4k(pos, fused):
    cfg, x, f, cap = prefix_case(1, pos + 1, 1, 1)
    check_spread(cfg, x, f, cap, fused)


def test_decode_token_spread_16k_and_64k():
    """16K: 12 tiles in 3 ranges; 64K (G = 8, 256 kept groups): 36 tiles in 9
    ranges of 4 items."""
    for cfg_id, pos in ((2, 16383), (3, 65000)):
        cfg, x, f, cap = prefix_case(cfg_id, pos + 1, 1, 1)
        check_spread(cfg, x, f, cap, fused=True)


def test_small_blocks_spread():
    """16 blocks of 16 tokens (128 workgroups, two ranges each: 5 tiles at most)."""
    end = 4096 - 48
    cfg, x, f, cap = prefix_case(1, end, 16, 256)
    check_spread(cfg, x, f, cap, fused=False)


def test_block64_spread_two_workgroups_per_item():
    """G = 8 and blocks of 64: 512 rows, two workgroups per item; one block of
    the 64K workload (4 items, 8 workgroups, each item's 36 tiles in 9 ranges)."""
    cfg, x, f, cap = prefix_case(3, 65536, 64, 64)
    check_spread(cfg, x, f, cap, fused=False)
