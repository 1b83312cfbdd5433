"""The C ABI on the CPU: the library loads, exports every entry point that
include/hga.h declares, and every validation path returns its status before
anything is launched (no GPU is touched by these calls)."""
import os
import re

import pytest

import hierarchical_sparse_attention_hga_amd as hga
from hierarchical_sparse_attention_hga_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # never dereferenced: validation fails before any use


@pytest.fixture(scope="module")
def lib():
    return hga.load()


def cfg(**kw):
    base = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, top_chunks=16, top_groups=64,
                sink_tokens=64, local_tokens=128, dtype="bf16")
    base.update(kw)
    return hga.make_config(**base)


def test_every_declared_entry_point_is_exported(lib):
    header = open(os.path.join(ROOT, "include", "hga.h")).read()
    declared = set(re.findall(r"^\S[^\n;]*?\b(hga_\w+)\(", header, flags=re.M))
    assert declared == set(B.EXPORTS)
    for name in declared:
        assert hasattr(lib, name)
    assert hga.hga_version() == 110


def test_status_strings(lib):
    for st in range(5):
        assert hga.hga_status_string(st)
    assert hga.hga_status_string(99) == "unknown status"


def test_workspace_sizes():
    c = cfg()
    assert hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_ROUTE) == 0
    assert hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_ATTEND) == 0
    # few items (one decoded token: 8 items, 8 workgroups): each item's tiles
    # in ranges of four, at most 12 tiles (1 sink + 2 local chunks, 64 groups
    # of 8 in 8 tiles, the own chunk), so 3 ranges; per range 8 waves of
    # (d / 2 + 2) floats per lane
    dec = cfg(q_block=1)
    assert hga.hga_workspace_size(dec, 16384, 1, hga.HGA_WS_ATTEND) == 8 * 3 * 8 * (64 + 2) * 64 * 4
    # 64 sequences decoded together: 512 items fill the chip, no split
    assert hga.hga_workspace_size(cfg(q_block=1, n_q_heads=32 * 64, n_kv_heads=8 * 64), 16384, 1,
                                  hga.HGA_WS_ATTEND) == 0
    # host-tier cache: int32 flags and slots per (KV head, history chunk), padded to
    # 256 bytes, then K and V rows of every history chunk (history <= seq_len - n_q)
    nch = (16384 - 2048) // 64
    flags = (2 * 8 * nch * 4 + 255) // 256 * 256
    assert hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_ATTEND_TIERED) == flags + 2 * 8 * nch * 64 * 128 * 2
    assert hga.hga_workspace_size(c, 16384, 2048, 7) == 2**64 - 1
    assert hga.hga_workspace_size(cfg(head_dim=96), 16384, 2048, 0) == 2**64 - 1


def _status(fn, *args):
    with pytest.raises(hga.HgaError) as ei:
        fn(*args)
    return ei.value.status


BAD_CONFIGS = [
    (dict(n_q_heads=30), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(n_kv_heads=0), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(dtype=5), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(summary_op=3), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(top_chunks=-1), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(local_tokens=-64), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(group_size=7), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(softmax_scale=float("nan")), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(softmax_scale=-1.0), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(chunk_size=32, q_block=32), hga.HGA_ERR_UNSUPPORTED),
    (dict(q_block=128), hga.HGA_ERR_UNSUPPORTED),
    (dict(q_block=48), hga.HGA_ERR_UNSUPPORTED),       # must divide the 64-token chunk
    (dict(q_block=0), hga.HGA_ERR_INVALID_ARGUMENT),
    (dict(sink_tokens=32), hga.HGA_ERR_UNSUPPORTED),
    (dict(head_dim=96), hga.HGA_ERR_UNSUPPORTED),
    (dict(head_dim=48, dtype="f32"), hga.HGA_ERR_UNSUPPORTED),
    (dict(top_chunks=4096), hga.HGA_ERR_UNSUPPORTED),
    (dict(top_groups=5000), hga.HGA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("over,status", BAD_CONFIGS)
def test_config_validation(over, status):
    c = cfg(**over)
    assert _status(hga.hga_build_summaries, c, FAKE, 16384, FAKE, FAKE) == status
    assert _status(hga.hga_route, c, FAKE, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, FAKE) == status
    assert _status(hga.hga_attend, c, FAKE, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, FAKE) == status
    assert _status(hga.hga_route_attend, c, FAKE, 14336, 2048, 16384, *[FAKE] * 8) == status
    assert hga.hga_last_error()


@pytest.mark.parametrize("q_start,n_q,seq_len,status,q_block", [
    (14336, 2048, 16000, hga.HGA_ERR_INVALID_ARGUMENT, 64),   # q_start + n_q > seq_len
    (-64, 64, 16384, hga.HGA_ERR_INVALID_ARGUMENT, 64),
    (14300, 2048, 16384, hga.HGA_ERR_UNSUPPORTED, 64),       # not a multiple of 64
    (14336, 2000, 16384, hga.HGA_ERR_UNSUPPORTED, 64),
    (0, 64, 64 * 4097, hga.HGA_ERR_UNSUPPORTED, 64),         # too many chunk candidates
    (16382, 1, 16383, hga.HGA_ERR_UNSUPPORTED, 1),           # seq_len (the buffers' capacity) not a multiple of 64
    (14338, 4, 16384, hga.HGA_ERR_UNSUPPORTED, 4),       # q_start not a multiple of q_block
    (14336, 6, 16384, hga.HGA_ERR_UNSUPPORTED, 4),       # n_q not a multiple of q_block
])
def test_geometry_validation(q_start, n_q, seq_len, status, q_block):
    c = cfg(q_block=q_block)
    assert _status(hga.hga_route, c, FAKE, q_start, n_q, seq_len, FAKE, FAKE, FAKE, FAKE, FAKE) == status
    assert _status(hga.hga_attend, c, FAKE, q_start, n_q, seq_len, FAKE, FAKE, FAKE, FAKE, FAKE) == status
    assert _status(hga.hga_route_attend, c, FAKE, q_start, n_q, seq_len, *[FAKE] * 8) == status


def test_null_pointers():
    c = cfg()
    E = hga.HGA_ERR_INVALID_ARGUMENT
    assert _status(hga.hga_build_summaries, c, None, 16384, FAKE, FAKE) == E
    assert _status(hga.hga_route, c, None, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_route, c, FAKE, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, None) == E
    assert _status(hga.hga_route, c, FAKE, 14336, 2048, 16384, FAKE, None, FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_attend, c, FAKE, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, None) == E
    assert _status(hga.hga_attend, c, FAKE, 14336, 2048, 16384, None, FAKE, FAKE, FAKE, FAKE) == E
    # route_attend: q, chunk_sum, k, v, chunk_idx, group_idx, n_sel, out
    for i in range(8):
        args = [FAKE] * 9
        args[[0, 1, 3, 4, 5, 6, 7, 8][i]] = None
        q, cs, gs, k, v, ci, gi, ns, out = args
        assert _status(hga.hga_route_attend, c, q, 14336, 2048, 16384, cs, gs, k, v, ci, gi, ns, out) == E


def test_misaligned_pointers_are_rejected():
    """The kernels move rows 16 bytes at a time: a tensor or workspace address
    off a 16-byte boundary is refused before any launch."""
    c = cfg()
    E = hga.HGA_ERR_INVALID_ARGUMENT
    odd = FAKE + 8
    assert _status(hga.hga_build_summaries, c, odd, 16384, FAKE, FAKE) == E
    assert _status(hga.hga_build_summaries, c, FAKE, 16384, FAKE, odd) == E
    assert _status(hga.hga_route, c, odd, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_route, c, FAKE, 14336, 2048, 16384, FAKE, (odd, FAKE, 1024), FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_attend, c, FAKE, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, odd) == E
    assert _status(hga.hga_attend, c, FAKE, 14336, 2048, 16384, (FAKE, odd, 1024), FAKE, FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_attend, c, FAKE, 14336, 2048, 16384, FAKE, FAKE, FAKE, FAKE, FAKE, None, odd, 1 << 30) == E
    assert _status(hga.hga_route_attend, c, FAKE, 14336, 2048, 16384, odd, *[FAKE] * 7) == E
    assert _status(hga.hga_route_attend, c, FAKE, 14336, 2048, 16384, *[FAKE] * 8, None, odd, 1 << 30) == E
    assert "16-byte aligned" in hga.hga_last_error()
    assert _status(hga.hga_stream_forward, c, FAKE, FAKE, odd, 4096, 1024, *[FAKE] * 7) == E
    assert _status(hga.hga_attend_backward, c, FAKE, 14336, 2048, 16384, *[FAKE] * 8, odd, FAKE, FAKE,
                   1 << 30) == E


def test_tier_validation():
    c = cfg()
    E = hga.HGA_ERR_INVALID_ARGUMENT
    args = (c, FAKE, 14336, 2048, 16384)
    assert _status(hga.hga_route, *args, FAKE, (FAKE, FAKE, 14400), FAKE, FAKE, FAKE) == E   # split > q_start
    assert _status(hga.hga_route, *args, FAKE, (None, FAKE, 1024), FAKE, FAKE, FAKE) == E    # host NULL
    assert _status(hga.hga_route, *args, FAKE, (FAKE, FAKE, 1000), FAKE, FAKE, FAKE) == hga.HGA_ERR_UNSUPPORTED
    assert _status(hga.hga_attend, *args, (FAKE, FAKE, 1024), (FAKE, FAKE, 2048), FAKE, FAKE, FAKE) == E
    # tiered K/V needs the host-tier cache workspace: for a split of 1024 tokens
    # (16 chunks), flags and slots (1 KiB) and K/V of 16 chunks per KV head
    tier = (FAKE, FAKE, 1024)
    need = 1024 + 2 * 8 * 16 * 64 * 128 * 2
    assert need <= hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_ATTEND_TIERED)
    assert _status(hga.hga_attend, *args, tier, tier, FAKE, FAKE, FAKE, None, None, 0) == hga.HGA_ERR_WORKSPACE
    assert _status(hga.hga_attend, *args, tier, tier, FAKE, FAKE, FAKE, None, FAKE, need - 1) == \
        hga.HGA_ERR_WORKSPACE
    # the host-tier cache bounds the fixed windows (sink + local chunks)
    wide = cfg(sink_tokens=64 * 200, local_tokens=64 * 100)
    assert _status(hga.hga_attend, wide, FAKE, 14336, 2048, 16384, tier, tier, FAKE, FAKE, FAKE, None, FAKE,
                   need) == hga.HGA_ERR_UNSUPPORTED
    ra = (c, FAKE, 14336, 2048, 16384, FAKE)
    assert _status(hga.hga_route_attend, *ra, (FAKE, FAKE, 14400), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_route_attend, *ra, FAKE, (FAKE, FAKE, 1024), (FAKE, FAKE, 2048),
                   FAKE, FAKE, FAKE, FAKE) == E
    assert _status(hga.hga_route_attend, *ra, FAKE, tier, tier, FAKE, FAKE, FAKE, FAKE, None, None, 0) == \
        hga.HGA_ERR_WORKSPACE


def test_summary_range_and_stream_validation():
    c = cfg()
    E = hga.HGA_ERR_INVALID_ARGUMENT
    # chunk range outside [0, seq_len / 64]
    assert _status(hga.hga_build_summaries_range, c, FAKE, 16384, -1, 4, FAKE, FAKE) == E
    assert _status(hga.hga_build_summaries_range, c, FAKE, 16384, 5, 4, FAKE, FAKE) == E
    assert _status(hga.hga_build_summaries_range, c, FAKE, 16384, 0, 257, FAKE, FAKE) == E
    assert _status(hga.hga_build_summaries_range, c, None, 16384, 0, 4, FAKE, FAKE) == E
    hga.hga_build_summaries_range(c, None, 16384, 7, 7, None, None)   # empty range: no-op
    # segment must be a positive multiple of 64; pointers non-NULL
    sf = (c, FAKE, FAKE, FAKE, 4096)
    assert _status(hga.hga_stream_forward, *sf, 0, *[FAKE] * 7) == E
    assert _status(hga.hga_stream_forward, *sf, 100, *[FAKE] * 7) == E
    assert _status(hga.hga_stream_forward, c, FAKE, None, FAKE, 4096, 1024, *[FAKE] * 7) == E
    assert _status(hga.hga_stream_forward, *sf, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E
    assert _status(hga.hga_stream_forward, c, FAKE, FAKE, FAKE, 4000, 1024, *[FAKE] * 7) == \
        hga.HGA_ERR_UNSUPPORTED
    hga.hga_stream_forward(c, None, None, None, 0, 1024, *[None] * 7)   # empty sequence: no-op


def test_empty_query_range_is_a_no_op():
    c = cfg()
    hga.hga_route(c, FAKE, 16384, 0, 16384, FAKE, FAKE, FAKE, FAKE, FAKE)
    hga.hga_attend(c, FAKE, 16384, 0, 16384, FAKE, FAKE, FAKE, FAKE, FAKE)
    hga.hga_route_attend(c, FAKE, 16384, 0, 16384, *[FAKE] * 8)
    hga.hga_build_summaries(c, None, 0, None, None)
    assert hga.hga_last_error() == ""


def test_backward_validation():
    c = cfg()
    E = hga.HGA_ERR_INVALID_ARGUMENT
    geo = (14336, 2048, 16384)
    # workspace: D per query row (float32), then a 64-bit kept-token mask per
    # (block, KV head, chunk of the call's positions; at most n_q / 64 + 1)
    nb = 2048 // 64
    need = (4 * 32 * 2048 + 255) // 256 * 256 + (8 * nb * 8 * (2048 // 64 + 1) + 255) // 256 * 256
    assert hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_BACKWARD) == need
    # with a host tier, the host-tier cache follows (the forward's, for any split)
    assert hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_BACKWARD_TIERED) == \
        need + hga.hga_workspace_size(c, 16384, 2048, hga.HGA_WS_ATTEND_TIERED)
    args = [FAKE] * 11   # k, v, group_idx, n_sel, out, lse, dout, dq, dk, dv, workspace
    def call(cc, a, ws_bytes=need, g=geo):
        return _status(hga.hga_attend_backward, cc, FAKE, *g, *a[:10], a[10], ws_bytes)
    assert call(cfg(dtype="f32", head_dim=96), args) == hga.HGA_ERR_UNSUPPORTED   # head_dim not built
    for i in range(10):
        a = list(args)
        a[i] = None
        assert call(c, a) == E
    assert call(c, args[:10] + [None]) == hga.HGA_ERR_WORKSPACE
    assert call(c, args, need - 1) == hga.HGA_ERR_WORKSPACE
    assert call(c, args, need, (14300, 2048, 16384)) == hga.HGA_ERR_UNSUPPORTED
    # the float32 output mode is forward-only
    assert call(cfg(dtype="bf16_f32out"), args) == hga.HGA_ERR_UNSUPPORTED
    # tiers: same split for k and v, host memory present, workspace with the cache
    t1, t2 = (FAKE, FAKE, 1024), (FAKE, FAKE, 2048)
    assert call(c, [t1, t2] + args[2:]) == E
    assert call(c, [(None, FAKE, 1024), (None, FAKE, 1024)] + args[2:]) == E
    assert call(c, [t1, t1] + args[2:]) == hga.HGA_ERR_WORKSPACE   # the cache needs more than `need`
    # q of 4 GiB (64 heads x 262,144 rows x 256 bytes): its rows are addressed
    # by 32-bit byte offsets, so the call is refused before any device work
    big = cfg(n_q_heads=64)
    assert call(big, args, 1 << 62, (0, 262144, 262144)) == hga.HGA_ERR_UNSUPPORTED
    assert "4 GiB" in hga.hga_last_error()
    hga.hga_attend_backward(c, None, 16384, 0, 16384, *[None] * 11, 0)   # no queries: a no-op


def test_tier_cache_sizes_and_validation():
    """The persistent host-tier cache: size, fewest slots, and every
    validation path of hga_tier_cache_init and hga_route_attend_cached."""
    c = cfg()
    E = hga.HGA_ERR_INVALID_ARGUMENT
    split = 14336
    nch = split // 64
    # one call of 2,048 queries (32 blocks) can need every history chunk; one
    # block of 64 at most top_chunks + sink + local chunks (16 + 1 + 2)
    assert hga.hga_tier_cache_min_slots(c, 16384, 2048, hga.HGA_TC_KV) == nch
    assert hga.hga_tier_cache_min_slots(c, 16384, 64, hga.HGA_TC_KV) == 19
    assert hga.hga_tier_cache_min_slots(c, 16384, 64, hga.HGA_TC_GS) == 16
    # top_groups covering every group of the kept chunks: no summary is read
    assert hga.hga_tier_cache_min_slots(cfg(top_groups=128), 16384, 64, hga.HGA_TC_GS) == 0
    assert hga.hga_tier_cache_min_slots(c, 16384, 64, 7) == -1
    size = hga.hga_tier_cache_size(c, split, 64, 32)
    # counters, K/V and summary tables, then K and V rows (64 x 128 bf16 per
    # slot) and group summaries (8 x 128 float32 per slot) for 8 KV heads
    assert size >= 8 * 64 * (2 * 64 * 128 * 2) + 8 * 32 * 8 * 128 * 4
    assert size < 8 * 64 * (2 * 64 * 128 * 2) + 8 * 32 * 8 * 128 * 4 + 64 * 1024
    assert hga.hga_tier_cache_size(c, split, 0, 32) == 2**64 - 1
    assert hga.hga_tier_cache_size(c, split, 5000, 32) == 2**64 - 1
    assert hga.hga_tier_cache_size(c, 100, 64, 32) == 2**64 - 1
    ws = hga.hga_workspace_size(c, 16384, 64, hga.HGA_WS_ATTEND_CACHED)
    # per history chunk and KV head: the copied-groups word and two copy-list entries
    assert ws >= 8 * nch * (8 + 16 + 16)
    good = hga.tier_cache(FAKE * 16, size, split, 64, 32)
    assert _status(hga.hga_tier_cache_init, c, hga.tier_cache(FAKE + 16, size, split, 64, 32)) == E   # alignment
    assert _status(hga.hga_tier_cache_init, c, hga.tier_cache(FAKE * 16, size - 1, split, 64, 32)) == \
        hga.HGA_ERR_WORKSPACE
    assert _status(hga.hga_tier_cache_init, c, hga.tier_cache(FAKE * 16, size, 1000, 64, 32)) == E
    tier = (FAKE, FAKE, split)
    args = (c, FAKE, 16320, 64, 16384, FAKE, tier, tier, tier)
    tail = (FAKE, FAKE, FAKE, FAKE, None, FAKE, ws)
    assert _status(hga.hga_route_attend_cached, *args, None, *tail) == E
    assert _status(hga.hga_route_attend_cached, *args, hga.tier_cache(FAKE * 16, size, split, 18, 32), *tail) == \
        hga.HGA_ERR_UNSUPPORTED                                                 # too few K/V slots
    assert _status(hga.hga_route_attend_cached, *args, hga.tier_cache(FAKE * 16, size, split, 64, 15), *tail) == \
        hga.HGA_ERR_UNSUPPORTED                                                 # too few summary slots
    assert _status(hga.hga_route_attend_cached, c, FAKE, 16320, 64, 16384, FAKE, tier, (FAKE, FAKE, 1024), tier,
                   good, *tail) == E                                            # split differs from the cache's
    assert _status(hga.hga_route_attend_cached, *args, good, FAKE, FAKE, FAKE, FAKE, None, None, 0) == \
        hga.HGA_ERR_WORKSPACE
    assert _status(hga.hga_route_attend_cached, *args, good, *tail, FAKE * 32, FAKE * 32) == E   # one stream twice
    assert _status(hga.hga_route_attend_cached, *args, good, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1024) == \
        hga.HGA_ERR_WORKSPACE


def test_float32_output_mode_config():
    """HGA_BF16_F32OUT is a bfloat16 configuration (same shapes, limits and
    workspaces) whose output is float32."""
    a, b = cfg(), cfg(dtype="bf16_f32out")
    assert b.dtype == hga.HGA_BF16_F32OUT
    for which in (hga.HGA_WS_ATTEND, hga.HGA_WS_ATTEND_TIERED, hga.HGA_WS_ATTEND_CACHED):
        assert hga.hga_workspace_size(a, 16384, 2048, which) == hga.hga_workspace_size(b, 16384, 2048, which)
    assert hga.hga_workspace_size(cfg(dtype=3), 16384, 2048, 0) == 2**64 - 1   # unknown dtype
    # bfloat16's head sizes
    assert hga.hga_workspace_size(cfg(dtype="bf16_f32out", head_dim=96), 16384, 2048, 0) == 2**64 - 1

