"""ctypes binding of libhga.so (include/hga.h). Argument marshalling only.

Every function keeps the C entry point's name and argument order. Tensor
arguments may be torch tensors (their data_ptr() is passed), plain integer
addresses, or None for NULL. Every step of the computation runs in the HIP
kernels of libhga.so; there is no fallback: if the library is missing, the
first call raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhga.so")

HGA_OK, HGA_ERR_INVALID_ARGUMENT, HGA_ERR_UNSUPPORTED, HGA_ERR_WORKSPACE, HGA_ERR_DEVICE = range(5)
HGA_F32, HGA_BF16, HGA_BF16_F32OUT = 0, 1, 2
HGA_SUMMARY_MEAN = 0
HGA_WS_ROUTE, HGA_WS_ATTEND, HGA_WS_ATTEND_TIERED, HGA_WS_BACKWARD, HGA_WS_BACKWARD_TIERED = 0, 1, 2, 3, 4
HGA_WS_ATTEND_CACHED = 5
HGA_TC_KV, HGA_TC_GS = 0, 1
# counters at the start of a tier cache's memory (int64 each)
TC_COUNTERS = ("calls", "kv_requests", "kv_misses", "kv_bytes", "kv_evictions", "gs_requests", "gs_misses",
               "gs_bytes", "gs_evictions")
HGA_TC_COUNTERS = 16

# Every exported entry point of include/hga.h.
EXPORTS = ("hga_workspace_size", "hga_build_summaries", "hga_build_summaries_range", "hga_route", "hga_attend",
           "hga_route_attend", "hga_route_attend_noalloc", "hga_tier_cache_size", "hga_tier_cache_min_slots",
           "hga_tier_cache_init", "hga_route_attend_cached", "hga_stream_forward", "hga_attend_backward",
           "hga_status_string", "hga_last_error", "hga_version")


class HgaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class hga_config(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("chunk_size", C.c_int32), ("group_size", C.c_int32), ("q_block", C.c_int32),
                ("top_chunks", C.c_int32), ("top_groups", C.c_int32),
                ("sink_tokens", C.c_int32), ("local_tokens", C.c_int32),
                ("summary_op", C.c_int32), ("dtype", C.c_int32), ("softmax_scale", C.c_float)]


class hga_tiered(C.Structure):
    _fields_ = [("host", C.c_void_p), ("dev", C.c_void_p), ("split", C.c_int64)]


class hga_tier_cache(C.Structure):
    _fields_ = [("mem", C.c_void_p), ("bytes", C.c_size_t), ("split", C.c_int64), ("kv_slots", C.c_int32),
                ("gs_slots", C.c_int32)]


_lib = None


def load():
    """Load libhga.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with hierarchical_sparse_attention_hga_amd.build")
        lib = C.CDLL(LIB_PATH)
        P, I64, I32, SZ = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        cfgp, tierp = C.POINTER(hga_config), C.POINTER(hga_tiered)
        lib.hga_workspace_size.argtypes = [cfgp, I64, I64, I32]
        lib.hga_workspace_size.restype = SZ
        lib.hga_build_summaries.argtypes = [cfgp, P, I64, P, P, P]
        lib.hga_route.argtypes = [cfgp, P, I64, I64, I64, P, tierp, P, P, P, P, SZ, P]
        lib.hga_attend.argtypes = [cfgp, P, I64, I64, I64, tierp, tierp, P, P, P, P, P, SZ, P]
        lib.hga_route_attend.argtypes = [cfgp, P, I64, I64, I64, P, tierp, tierp, tierp, P, P, P, P, P, P, SZ, P]
        lib.hga_route_attend_noalloc.argtypes = [cfgp, P, I64, I64, I64, P, tierp, tierp, tierp, P, P, P, P, P, P]
        cachep = C.POINTER(hga_tier_cache)
        lib.hga_tier_cache_size.argtypes = [cfgp, I64, I32, I32]
        lib.hga_tier_cache_size.restype = SZ
        lib.hga_tier_cache_min_slots.argtypes = [cfgp, I64, I64, I32]
        lib.hga_tier_cache_min_slots.restype = I32
        lib.hga_tier_cache_init.argtypes = [cfgp, cachep, P]
        lib.hga_route_attend_cached.argtypes = [cfgp, P, I64, I64, I64, P, tierp, tierp, tierp, cachep, P, P, P, P,
                                                P, P, SZ, P, P]
        lib.hga_build_summaries_range.argtypes = [cfgp, P, I64, I64, I64, P, P, P]
        lib.hga_stream_forward.argtypes = [cfgp, P, P, P, I64, I64, P, P, P, P, P, P, P, P]
        lib.hga_attend_backward.argtypes = [cfgp, P, I64, I64, I64, tierp, tierp, P, P, P, P, P, P, P, P, P, SZ, P]
        for f in ("hga_build_summaries", "hga_build_summaries_range", "hga_route", "hga_attend",
                  "hga_route_attend", "hga_route_attend_noalloc", "hga_tier_cache_init", "hga_route_attend_cached",
                  "hga_stream_forward", "hga_attend_backward"):
            getattr(lib, f).restype = C.c_int
        lib.hga_status_string.argtypes = [C.c_int]
        lib.hga_status_string.restype = C.c_char_p
        lib.hga_last_error.restype = C.c_char_p
        lib.hga_version.restype = C.c_int32
        _lib = lib
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, C.c_void_p):
        return x.value
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream):
    if stream is None:
        import torch
        if torch.cuda.is_available() and torch.cuda.is_initialized():
            return torch.cuda.current_stream().cuda_stream
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _tier(t):
    """A hga_tiered from a tensor (all on device), a (host, dev, split) tuple, or a hga_tiered."""
    if isinstance(t, hga_tiered):
        return t
    if isinstance(t, tuple):
        host, dev, split = t
        return hga_tiered(_ptr(host), _ptr(dev), int(split))
    return hga_tiered(None, _ptr(t), 0)


def _check(status):
    if status != HGA_OK:
        lib = load()
        raise HgaError(status, lib.hga_last_error().decode())


def make_config(n_q_heads, n_kv_heads, head_dim, top_chunks, top_groups, sink_tokens, local_tokens,
                dtype="bf16", chunk_size=64, group_size=8, q_block=64, summary_op=HGA_SUMMARY_MEAN,
                softmax_scale=0.0) -> hga_config:
    dt = {"bf16": HGA_BF16, "f32": HGA_F32, "bf16_f32out": HGA_BF16_F32OUT}.get(dtype, dtype)
    return hga_config(n_q_heads, n_kv_heads, head_dim, chunk_size, group_size, q_block, top_chunks,
                      top_groups, sink_tokens, local_tokens, summary_op, dt, float(softmax_scale))


def hga_workspace_size(cfg, seq_len, n_q, which):
    return int(load().hga_workspace_size(C.byref(cfg), seq_len, n_q, which))


def hga_build_summaries(cfg, k, seq_len, group_sum, chunk_sum, stream=None):
    _check(load().hga_build_summaries(C.byref(cfg), _ptr(k), seq_len, _ptr(group_sum), _ptr(chunk_sum),
                                      _stream(stream)))


def hga_route(cfg, q, q_start, n_q, seq_len, chunk_sum, group_sum, chunk_idx, group_idx, n_sel,
              workspace=None, ws_bytes=0, stream=None):
    gs = _tier(group_sum)
    _check(load().hga_route(C.byref(cfg), _ptr(q), q_start, n_q, seq_len, _ptr(chunk_sum), C.byref(gs),
                            _ptr(chunk_idx), _ptr(group_idx), _ptr(n_sel), _ptr(workspace), ws_bytes,
                            _stream(stream)))


def hga_attend(cfg, q, q_start, n_q, seq_len, k, v, group_idx, n_sel, out, lse=None, workspace=None,
               ws_bytes=0, stream=None):
    kt, vt = _tier(k), _tier(v)
    _check(load().hga_attend(C.byref(cfg), _ptr(q), q_start, n_q, seq_len, C.byref(kt), C.byref(vt),
                             _ptr(group_idx), _ptr(n_sel), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                             _stream(stream)))


def hga_route_attend(cfg, q, q_start, n_q, seq_len, chunk_sum, group_sum, k, v, chunk_idx, group_idx, n_sel,
                     out, lse=None, workspace=None, ws_bytes=0, stream=None):
    gt, kt, vt = _tier(group_sum), _tier(k), _tier(v)
    _check(load().hga_route_attend(C.byref(cfg), _ptr(q), q_start, n_q, seq_len, _ptr(chunk_sum), C.byref(gt),
                                   C.byref(kt), C.byref(vt), _ptr(chunk_idx), _ptr(group_idx), _ptr(n_sel),
                                   _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def hga_route_attend_noalloc(cfg, q, q_start, n_q, seq_len, chunk_sum, group_sum, k, v, chunk_idx, group_idx,
                             n_sel, out, lse=None, stream=None):
    gt, kt, vt = _tier(group_sum), _tier(k), _tier(v)
    _check(load().hga_route_attend_noalloc(C.byref(cfg), _ptr(q), q_start, n_q, seq_len, _ptr(chunk_sum),
                                           C.byref(gt), C.byref(kt), C.byref(vt), _ptr(chunk_idx), _ptr(group_idx),
                                           _ptr(n_sel), _ptr(out), _ptr(lse), _stream(stream)))


def hga_tier_cache_size(cfg, split, kv_slots, gs_slots):
    return int(load().hga_tier_cache_size(C.byref(cfg), split, kv_slots, gs_slots))


def hga_tier_cache_min_slots(cfg, seq_len, n_q, which):
    return int(load().hga_tier_cache_min_slots(C.byref(cfg), seq_len, n_q, which))


def tier_cache(mem, nbytes, split, kv_slots, gs_slots):
    """A hga_tier_cache over device memory `mem` (a tensor or an address)."""
    return hga_tier_cache(_ptr(mem), int(nbytes), int(split), int(kv_slots), int(gs_slots))


def hga_tier_cache_init(cfg, cache, stream=None):
    _check(load().hga_tier_cache_init(C.byref(cfg), C.byref(cache), _stream(stream)))


def hga_route_attend_cached(cfg, q, q_start, n_q, seq_len, chunk_sum, group_sum, k, v, cache, chunk_idx, group_idx,
                            n_sel, out, lse=None, workspace=None, ws_bytes=0, stream=None, copy_stream=None):
    gt, kt, vt = _tier(group_sum), _tier(k), _tier(v)
    _check(load().hga_route_attend_cached(C.byref(cfg), _ptr(q), q_start, n_q, seq_len, _ptr(chunk_sum), C.byref(gt),
                                          C.byref(kt), C.byref(vt), None if cache is None else C.byref(cache),
                                          _ptr(chunk_idx), _ptr(group_idx),
                                          _ptr(n_sel), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                          _stream(stream), None if copy_stream is None else _stream(copy_stream)))


def hga_build_summaries_range(cfg, k, seq_len, chunk_begin, chunk_end, group_sum, chunk_sum, stream=None):
    _check(load().hga_build_summaries_range(C.byref(cfg), _ptr(k), seq_len, chunk_begin, chunk_end,
                                            _ptr(group_sum), _ptr(chunk_sum), _stream(stream)))


def hga_stream_forward(cfg, q, k, v, seq_len, segment, chunk_sum, group_sum, chunk_idx, group_idx, n_sel, out,
                       lse=None, stream=None):
    _check(load().hga_stream_forward(C.byref(cfg), _ptr(q), _ptr(k), _ptr(v), seq_len, segment, _ptr(chunk_sum),
                                     _ptr(group_sum), _ptr(chunk_idx), _ptr(group_idx), _ptr(n_sel), _ptr(out),
                                     _ptr(lse), _stream(stream)))


def hga_attend_backward(cfg, q, q_start, n_q, seq_len, k, v, group_idx, n_sel, out, lse, dout, dq, dk, dv,
                        workspace=None, ws_bytes=0, stream=None):
    kt, vt = _tier(k), _tier(v)
    _check(load().hga_attend_backward(C.byref(cfg), _ptr(q), q_start, n_q, seq_len, C.byref(kt), C.byref(vt),
                                      _ptr(group_idx), _ptr(n_sel), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                      _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream)))


def hga_status_string(status):
    return load().hga_status_string(status).decode()


def hga_last_error():
    return load().hga_last_error().decode()


def hga_version():
    return int(load().hga_version())
