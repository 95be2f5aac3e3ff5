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


def feature_dim(K: int) -> int:
    """P = 1 + K + K^2, the rows of a state for feature dimension K."""
    return 1 + K + K * K


def _check_state(state, B, H, P, V, device, what):
    S, z = state
    for name, t, shape in ((f"{what}[0]", S, (B, H, P, V)), (f"{what}[1]", z, (B, H, P))):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device:
            raise TypeError(f"{name} must be a float32 tensor on {device}")
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with shape {shape}, got {tuple(t.shape)}")


def based_forward(q, k, v, scale=None, *, out=None, out_dtype=torch.bfloat16, workspace=None,
                  segment_len: int = 0, timer: Timer | None = None, initial_state=None, return_state: bool = False):
    """Causal Based forward. q, k: (B,T,H,K) bf16; v: (B,T,H,V) bf16; all contiguous on one GPU.

    scale=None means K**-0.5. Returns o of shape (B,T,H,V) in `out_dtype` (bfloat16 or float32), or writes
    into `out`. Runs on the current stream. With `workspace` (a uint8 device tensor of at least
    workspace_bytes(...) bytes) no allocation happens; without it, the library allocates stream-ordered.
    `segment_len` forces the sequence split (0 = automatic); `timer` records per-kernel HIP events.
    `initial_state` = (S, z), float32 tensors (B,H,P,V) and (B,H,P) with P = 1 + K + K^2 in the layout of the
    page's phi, stands for earlier tokens; with `return_state` the result is (o, (S, z)) with the state after
    the last token (new tensors).
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
    if initial_state is not None or return_state:
        if segment_len or timer is not None:
            raise ValueError("segment_len and timer are not available together with a state")
        P = feature_dim(K)
        s_in = z_in = None
        if initial_state is not None:
            _check_state(initial_state, B, H, P, V, q.device, "initial_state")
            s_in, z_in = initial_state[0].data_ptr(), initial_state[1].data_ptr()
        s_out = z_out = None
        if return_state:
            S = torch.empty((B, H, P, V), dtype=torch.float32, device=q.device)
            z = torch.empty((B, H, P), dtype=torch.float32, device=q.device)
            s_out, z_out = S.data_ptr(), z.data_ptr()
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        _lib.check(L.based_forward_state(*args, s_in, z_in, s_out, z_out, ws_ptr, ws_bytes, stream),
                   "based_forward_state")
        return (out, (S, z)) if return_state else out
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


def based_decode_step(q, k, v, state, scale=None, *, out=None, out_dtype=torch.bfloat16):
    """One token of the recurrence: q, k of shape (B,H,K) or (B,1,H,K), v of shape (B,H,V) or (B,1,H,V),
    bf16 contiguous; state = (S, z) float32 tensors (B,H,P,V) and (B,H,P), updated in place (the token is
    folded in first, then read out). Returns o of shape (B,H,V)."""
    if q.dim() == 4:
        q, k, v = q[:, 0], k[:, 0], v[:, 0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device.type != "cuda":
            raise TypeError(f"{name} must be a bfloat16 GPU tensor")
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with 3 dims (B, H, X)")
    B, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or v.shape[:2] != (B, H):
        raise ValueError("q, k, v shapes do not match")
    _check_state(state, B, H, feature_dim(K), V, q.device, "state")
    if out is None:
        if out_dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
        out = torch.empty((B, H, V), dtype=out_dtype, device=q.device)
    elif out.shape != (B, H, V) or out.dtype not in (torch.bfloat16, torch.float32) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B,H,V) bfloat16 or float32 tensor")
    dt = _lib.BASED_F32 if out.dtype == torch.float32 else _lib.BASED_BF16
    _lib.check(_lib.lib().based_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, K, V, _scale_arg(scale),
                                            state[0].data_ptr(), state[1].data_ptr(), out.data_ptr(), dt,
                                            _stream_handle(q.device)), "based_decode_step")
    return out
