"""Host-tier plumbing: pinned, mapped host memory for the hga_tiered layout.

hga_route and hga_attend read the host rows of a tiered tensor directly from
kernels, so those rows must live in pinned host memory mapped into the GPU's
address space (hipHostMalloc). This module allocates such memory and moves the
leading rows of a device tensor into it.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

_hip = None


def _hip_lib():
    global _hip
    if _hip is None:
        _hip = C.CDLL("libamdhip64.so")
    return _hip


class PinnedBuffer:
    """``nbytes`` of pinned host memory (hipHostMalloc, default flags: mapped
    and portable). ``dev_ptr`` is its address in the GPU's address space."""

    def __init__(self, nbytes: int):
        hip = _hip_lib()
        self.ptr = C.c_void_p()
        st = hip.hipHostMalloc(C.byref(self.ptr), C.c_size_t(max(int(nbytes), 1)), C.c_uint(0))
        if st != 0:
            raise MemoryError(f"hipHostMalloc({nbytes}) failed with HIP error {st}")
        dptr = C.c_void_p()
        st = hip.hipHostGetDevicePointer(C.byref(dptr), self.ptr, C.c_uint(0))
        if st != 0:
            hip.hipHostFree(self.ptr)
            raise RuntimeError(f"hipHostGetDevicePointer failed with HIP error {st}")
        self.dev_ptr = dptr.value
        self.nbytes = int(nbytes)

    def view(self, dtype, shape) -> np.ndarray:
        buf = (C.c_char * self.nbytes).from_address(self.ptr.value)
        return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)

    def free(self):
        if self.ptr:
            _hip_lib().hipHostFree(self.ptr)
            self.ptr = C.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def split_to_host(dev_tensor, split_rows: int):
    """Split a [H][R][w] device tensor at row ``split_rows``: rows before it go
    to a new PinnedBuffer laid out [H][split_rows][w], the rest stay on the
    device as a new contiguous tensor. Returns (pinned, device_rest, tiered),
    where ``tiered`` is the (host, dev, split) triple the binding accepts
    (``split`` counted in rows of the tensor)."""
    import torch
    H, R, w = dev_tensor.shape
    head = dev_tensor[:, :split_rows].contiguous().cpu()
    pin = PinnedBuffer(head.numel() * head.element_size())
    as_np = {torch.bfloat16: np.int16, torch.float32: np.float32}[dev_tensor.dtype]
    view_dtype = torch.int16 if dev_tensor.dtype == torch.bfloat16 else torch.float32
    pin.view(as_np, (H, split_rows, w))[...] = head.view(view_dtype).numpy()
    rest = dev_tensor[:, split_rows:].contiguous()
    return pin, rest, (pin.dev_ptr, rest, split_rows)
