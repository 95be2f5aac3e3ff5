"""PyTorch-facing entry point of the causal Based forward.

`based_forward(q, k, v, scale=None)` mirrors the signature of the page "Write a fast Based (Taylor linear
attention) forward kernel" (fields signature, returns_doc, contract_md). PyTorch only provides device
memory and the current HIP stream; every step of the computation runs in the HIP kernels of libbased.so.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.shape != k.shape:
        raise ValueError(f"q and k shapes differ: {tuple(q.shape)} vs {tuple(k.shape)}")
    if v.shape[:3] != q.shape[:3]:
        raise ValueError(f"v leading dims {tuple(v.shape[:3])} differ from q {tuple(q.shape[:3])}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _scale_arg(scale) -> float:
    return math.nan if scale is None else float(scale)


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def plan(B, T, H, K, V, segment_len: int = 0):
    """(segments, segment_len, workspace_bytes) the library uses for a shape."""
    L = _lib.lib()
    g = ctypes.c_int64()
    sl = ctypes.c_int64()
    ws = ctypes.c_size_t()
    _lib.check(L.based_forward_plan(B, T, H, K, V, segment_len, ctypes.byref(g), ctypes.byref(sl),
                                    ctypes.byref(ws)), "based_forward_plan")
    return g.value, sl.value, ws.value


def workspace_bytes(B, T, H, K, V) -> int:
    return int(_lib.lib().based_forward_workspace_bytes(B, T, H, K, V))


class Timer:
    """HIP events around every kernel launched by `based_forward(..., timer=...)`."""

    STATE, SCAN, READOUT = 0, 1, 2  # kernel ids: segment state sums, prefix scan, chunked read-out
    KERNELS = (STATE, SCAN, READOUT)

    def __init__(self, max_launches: int = 4096, kernels=None):
        self._h = ctypes.c_void_p()
        _lib.check(_lib.lib().based_timer_create(max_launches, ctypes.byref(self._h)), "based_timer_create")
        if kernels is not None:
            _lib.lib().based_timer_set_kernel_mask(self._h, sum(1 << k for k in kernels))

    @property
    def handle(self):
        return self._h

    def reset(self):
        _lib.lib().based_timer_reset(self._h)

    def read(self, kernel_id: int):
        n = ctypes.c_int()
        ms = ctypes.c_double()
        _lib.check(_lib.lib().based_timer_read(self._h, kernel_id, ctypes.byref(n), ctypes.byref(ms)),
                   "based_timer_read")
        return n.value, ms.value

    @staticmethod
    def kernel_name(kernel_id: int) -> str:
        return _lib.lib().based_kernel_name(kernel_id).decode()

    def close(self):
        if self._h:
            _lib.lib().based_timer_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def based_forward(q, k, v, scale=None, *, out=None, out_dtype=torch.bfloat16, workspace=None,
                  segment_len: int = 0, timer: Timer | None = None):
    """Causal Based forward. q, k: (B,T,H,K) bf16; v: (B,T,H,V) bf16; all contiguous on one GPU.

    scale=None means K**-0.5. Returns o of shape (B,T,H,V) in `out_dtype` (bfloat16 or float32), or writes
    into `out`. Runs on the current stream. With `workspace` (a uint8 device tensor of at least
    workspace_bytes(...) bytes) no allocation happens; without it, the library allocates stream-ordered.
    `segment_len` forces the sequence split (0 = automatic); `timer` records per-kernel HIP events.
    """
    _check_inputs(q, k, v)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if out is None:
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
        out = torch.empty((B, T, H, V), dtype=out_dtype, device=q.device)
    else:
        if out.shape != (B, T, H, V) or out.dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("out must be (B,T,H,V) bfloat16 or float32")
        if not out.is_contiguous() or out.device != q.device:
            raise ValueError("out must be contiguous on the inputs' device")
    dt = _lib.BASED_F32 if out.dtype == torch.float32 else _lib.BASED_BF16
    L = _lib.lib()
    stream = _stream_handle(q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), B, T, H, K, V, _scale_arg(scale), out.data_ptr(), dt)
    if workspace is None and segment_len == 0 and timer is None:
        _lib.check(L.based_forward(*args, stream), "based_forward")
        return out
    if workspace is None:
        _, _, need = plan(B, T, H, K, V, segment_len)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr()
    ws_bytes = workspace.numel() * workspace.element_size()
    _lib.check(L.based_forward_ex(*args, ws_ptr, ws_bytes, segment_len, timer.handle if timer else None, stream),
               "based_forward_ex")
    return out
