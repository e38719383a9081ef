"""Thin Python binding of ``libq1.so`` (see ``include/q1.h`` and ``include/q1_measure.h``).

Argument marshalling only: torch tensors provide device memory and the current
stream; every operation runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback -- if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq1.so")

Q1_F32, Q1_F16, Q1_BF16 = 0, 1, 2
Q1_WS_RESERVED_BYTES = 16384  # reserved counter block at the start of every workspace
_TORCH_TO_Q1 = {torch.float32: Q1_F32, torch.float16: Q1_F16, torch.bfloat16: Q1_BF16}
_STATUS = {0: "Q1_OK", -1: "Q1_ERR_INVALID_ARG", -2: "Q1_ERR_UNSUPPORTED", -3: "Q1_ERR_WORKSPACE", -4: "Q1_ERR_HIP"}
Q1_ERR_INVALID_ARG, Q1_ERR_UNSUPPORTED, Q1_ERR_WORKSPACE, Q1_ERR_HIP = -1, -2, -3, -4


class Q1Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class _Weight(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("meta_dtype", ctypes.c_int32), ("symmetric", ctypes.c_int32), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("group_size", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()

EXPORTS = ["q1_qmm", "q1_qmm_noalloc", "q1_qmm_workspace_bytes", "q1_dequantize", "q1_embed_rows", "q1_ffn", "q1_ffn_workspace_bytes",
           "q1_check_symmetric", "q1_pack_signs", "q1_stream_read", "q1_set_max_packed_rows", "q1_device_supported", "q1_last_error",
           "q1_version"]


def load_library(path: str = LIB_PATH):
    """Load ``libq1.so`` and declare the C signatures.  Raises if missing."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m gemm_decode_q1_amd.build` "
                               "(or __graft_entry__.build()) first -- there is no fallback path")
        L = ctypes.CDLL(path)
        W = ctypes.POINTER(_Weight)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "q1_qmm": (i32, [vp, i32, i64, W, vp, i32, vp, sz, vp]),
            "q1_qmm_noalloc": (i32, [vp, i32, i64, W, vp, i32, vp]),
            "q1_qmm_workspace_bytes": (sz, [i64, W]),
            "q1_dequantize": (i32, [W, vp, i32, vp]),
            "q1_embed_rows": (i32, [vp, i32, i64, W, vp, i32, vp]),
            "q1_ffn": (i32, [vp, i64, W, W, W, vp, vp, sz, vp]),
            "q1_ffn_workspace_bytes": (sz, [i64, W, W, W]),
            "q1_check_symmetric": (i32, [W, vp, vp]),
            "q1_pack_signs": (i32, [vp, i32, i64, i64, vp, vp, i32, vp, vp]),
            "q1_stream_read": (i32, [vp, sz, vp, vp]),
            "q1_set_max_packed_rows": (ctypes.c_int, [ctypes.c_int]),
            "q1_device_supported": (i32, [ctypes.c_int]),
            "q1_last_error": (ctypes.c_char_p, []),
            "q1_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
        return L


def _check(status: int):
    if status != 0:
        raise Q1Error(status, load_library().q1_last_error().decode())


@dataclass
class PackedQ1:
    """One packed Q1 matrix held in device tensors.

    packed: int32 [N, K/32] (the uint32 words, bit pattern preserved);
    scales: float16 or bfloat16 [N, K/128]; biases: same or None (symmetric).
    """
    packed: torch.Tensor
    scales: torch.Tensor
    biases: Optional[torch.Tensor]
    N: int
    K: int

    @property
    def symmetric(self) -> bool:
        return self.biases is None

    def desc(self) -> _Weight:
        """The C descriptor (rebuilt only when a tensor or shape changed)."""
        key = (self.packed.data_ptr(), self.scales.data_ptr(),
               None if self.biases is None else self.biases.data_ptr(), self.scales.dtype, self.N, self.K)
        cached = self.__dict__.get("_desc_cache")
        if cached is not None and cached[0] == key:
            return cached[1]
        meta = _TORCH_TO_Q1.get(self.scales.dtype)
        d = _Weight(key[0], key[1], key[2], -1 if meta is None else meta, 1 if self.biases is None else 0,
                    self.N, self.K, 128, 0)
        self.__dict__["_desc_cache"] = (key, d)
        return d

    @staticmethod
    def from_host(w, device="cuda") -> "PackedQ1":
        """From a host weight with numpy fields packed (uint32), scales/biases
        (uint16 bit patterns) and meta ("f16" | "bf16")."""
        import numpy as np
        dt = torch.float16 if w.meta == "f16" else torch.bfloat16
        packed = torch.from_numpy(np.ascontiguousarray(w.packed).view(np.int32)).to(device)
        scales = torch.from_numpy(np.ascontiguousarray(w.scales).view(np.int16)).view(dt).to(device)
        biases = None
        if w.biases is not None:
            biases = torch.from_numpy(np.ascontiguousarray(w.biases).view(np.int16)).view(dt).to(device)
        return PackedQ1(packed, scales, biases, int(w.N), int(w.K))


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device=None) -> ctypes.c_void_p:
    """The current HIP stream of `device` (default: the current device)."""
    if _raw_stream is not None:
        idx = torch.cuda.current_device() if device is None else device.index
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _Workspaces:
    """Zero-filled device workspaces, one per (device, stream), grown on demand.
    The library leaves the zero-required part zero after every call."""

    def __init__(self):
        self._ws = {}

    def get(self, nbytes: int, device: torch.device) -> torch.Tensor:
        key = (device.index, _stream(device).value)
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._ws[key] = t
        return t


_WS = _Workspaces()


def _check_tensor(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def q1_qmm_workspace_bytes(M: int, w: PackedQ1) -> int:
    d = w.desc()
    n = load_library().q1_qmm_workspace_bytes(M, ctypes.byref(d))
    if n == 0 and load_library().q1_last_error():
        msg = load_library().q1_last_error().decode()
        if msg:
            raise Q1Error(Q1_ERR_INVALID_ARG, msg)
    return n


_need_cache = {}


def _qmm_need(L, M: int, w: PackedQ1, d: _Weight) -> int:
    # (the kernel choices follow Q1_WIDE_KERNEL and Q1_PACKED_KERNEL, which
    # the library reads on every call, so they are part of the key)
    key = (M, w.N, w.K, d.meta_dtype, d.symmetric, os.environ.get("Q1_WIDE_KERNEL"),
           os.environ.get("Q1_PACKED_KERNEL"))
    n = _need_cache.get(key)
    if n is None:
        n = L.q1_qmm_workspace_bytes(M, ctypes.byref(d))
        if n == 0 and L.q1_last_error():
            # the call itself fails the same way, before any launch, and
            # reports the library's own status
            return 0
        _need_cache[key] = n
    return n


def q1_qmm(x: torch.Tensor, w: PackedQ1, out_dtype: torch.dtype = torch.bfloat16,
           y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``y[..., N] = x[..., K] @ W^T``; x bf16, leading dims flattened to M rows."""
    _check_tensor(x, "x")
    if x.shape[-1] != w.K:
        raise ValueError(f"x has {x.shape[-1]} features, weight has K={w.K}")
    lead = tuple(x.shape[:-1])
    M = math.prod(lead)
    if y is None:
        y = torch.empty(*lead, w.N, dtype=out_dtype, device=x.device)
    _check_tensor(y, "y")
    L = load_library()
    d = w.desc()
    need = _qmm_need(L, M, w, d) if M > 0 else 0
    ws = workspace if workspace is not None else (_WS.get(need, x.device) if need else None)
    _check(L.q1_qmm(ctypes.c_void_p(x.data_ptr()), _TORCH_TO_Q1.get(x.dtype, -1), M, ctypes.byref(d),
                    ctypes.c_void_p(y.data_ptr()), _TORCH_TO_Q1.get(y.dtype, -1),
                    None if ws is None else ctypes.c_void_p(ws.data_ptr()), 0 if ws is None else ws.numel(),
                    _stream(x.device)))
    return y


def q1_qmm_noalloc(x: torch.Tensor, w: PackedQ1, out_dtype: torch.dtype = torch.bfloat16,
                   y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``q1_qmm`` without a workspace: temporaries live in the library's own
    device scratch (for callers that cannot allocate)."""
    _check_tensor(x, "x")
    if x.shape[-1] != w.K:
        raise ValueError(f"x has {x.shape[-1]} features, weight has K={w.K}")
    lead = tuple(x.shape[:-1])
    M = math.prod(lead)
    if y is None:
        y = torch.empty(*lead, w.N, dtype=out_dtype, device=x.device)
    _check_tensor(y, "y")
    d = w.desc()
    _check(load_library().q1_qmm_noalloc(ctypes.c_void_p(x.data_ptr()), _TORCH_TO_Q1.get(x.dtype, -1), M,
                                         ctypes.byref(d), ctypes.c_void_p(y.data_ptr()),
                                         _TORCH_TO_Q1.get(y.dtype, -1), _stream(x.device)))
    return y


def q1_dequantize(w: PackedQ1, out_dtype: torch.dtype = torch.bfloat16,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty(w.N, w.K, dtype=out_dtype, device=w.packed.device)
    _check_tensor(out, "out")
    d = w.desc()
    _check(load_library().q1_dequantize(ctypes.byref(d), ctypes.c_void_p(out.data_ptr()),
                                        _TORCH_TO_Q1.get(out.dtype, -1), _stream(out.device)))
    return out


def q1_embed_rows(ids: torch.Tensor, table: PackedQ1, out_dtype: torch.dtype = torch.bfloat16,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _check_tensor(ids, "ids")
    if ids.dtype not in (torch.int32, torch.int64):
        raise ValueError("ids must be int32 or int64")
    T = ids.numel()
    if out is None:
        out = torch.empty(*ids.shape, table.K, dtype=out_dtype, device=ids.device)
    _check_tensor(out, "out")
    d = table.desc()
    _check(load_library().q1_embed_rows(ctypes.c_void_p(ids.data_ptr()), 1 if ids.dtype == torch.int64 else 0, T,
                                        ctypes.byref(d), ctypes.c_void_p(out.data_ptr()),
                                        _TORCH_TO_Q1.get(out.dtype, -1), _stream(out.device)))
    return out


def q1_ffn_workspace_bytes(M: int, gate: PackedQ1, up: PackedQ1, down: PackedQ1) -> int:
    g, u, d = gate.desc(), up.desc(), down.desc()
    return load_library().q1_ffn_workspace_bytes(M, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d))


def q1_ffn(x: torch.Tensor, gate: PackedQ1, up: PackedQ1, down: PackedQ1, y: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, return_hidden: bool = False):
    """Fused dense FFN; x bf16 ``[..., H]`` -> y bf16 ``[..., H_out]``.  With
    ``return_hidden`` also returns the bf16 hidden activation ``h [..., I]``
    that the library leaves in the workspace after the counter region."""
    _check_tensor(x, "x")
    lead = tuple(x.shape[:-1])
    M = math.prod(lead)
    if y is None:
        y = torch.empty(*lead, down.N, dtype=torch.bfloat16, device=x.device)
    _check_tensor(y, "y")
    L = load_library()
    g, u, d = gate.desc(), up.desc(), down.desc()
    need = L.q1_ffn_workspace_bytes(M, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d))
    ws = workspace if workspace is not None else _WS.get(need, x.device)
    _check(L.q1_ffn(ctypes.c_void_p(x.data_ptr()), M, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                    ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(x.device)))
    if return_hidden:
        off = Q1_WS_RESERVED_BYTES
        h = ws[off:off + M * gate.N * 2].view(torch.bfloat16).view(*lead, gate.N).clone()
        return y, h
    return y


def q1_check_symmetric(w: PackedQ1, count: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Device int32 [1]: groups of the affine tensor ``w`` whose bias cannot be
    replaced by -scale/2 (0 means the tensor can drop its biases)."""
    if w.biases is None:
        raise ValueError("w is already symmetric")
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=w.scales.device)
    _check_tensor(count, "count")
    d = w.desc()
    _check(load_library().q1_check_symmetric(ctypes.byref(d), ctypes.c_void_p(count.data_ptr()),
                                             _stream(count.device)))
    return count


def q1_pack_signs(dense: torch.Tensor, meta_dtype: torch.dtype = torch.float16):
    """Pack dense [N, K] bf16/fp16 weights into a symmetric ``PackedQ1``
    (scale = 2 max|w| per group of 128, bit = w > 0).  Returns (weight,
    inexact) with ``inexact`` a device int32 [1]: groups that do not
    round-trip bit for bit through ``q1_dequantize``."""
    _check_tensor(dense, "dense")
    if dense.dim() != 2:
        raise ValueError("dense must be [N, K]")
    N, K = dense.shape
    packed = torch.empty(N, K // 32, dtype=torch.int32, device=dense.device)
    scales = torch.empty(N, K // 128, dtype=meta_dtype, device=dense.device)
    inexact = torch.empty(1, dtype=torch.int32, device=dense.device)
    _check(load_library().q1_pack_signs(ctypes.c_void_p(dense.data_ptr()), _TORCH_TO_Q1.get(dense.dtype, -1), N, K,
                                        ctypes.c_void_p(packed.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                        _TORCH_TO_Q1.get(meta_dtype, -1), ctypes.c_void_p(inexact.data_ptr()),
                                        _stream(dense.device)))
    return PackedQ1(packed, scales, None, int(N), int(K)), inexact


def q1_stream_read(data: torch.Tensor, sink: torch.Tensor) -> None:
    """One read pass over ``data`` (measurement aid: the single-launch read
    ceiling for that many bytes).  ``sink`` is a device int32 [1]."""
    _check_tensor(data, "data")
    _check_tensor(sink, "sink")
    _check(load_library().q1_stream_read(ctypes.c_void_p(data.data_ptr()), data.numel() * data.element_size(),
                                         ctypes.c_void_p(sink.data_ptr()), _stream(data.device)))


def q1_set_max_packed_rows(rows: int) -> int:
    _need_cache.clear()  # the routing, and with it the workspace sizes, change
    return load_library().q1_set_max_packed_rows(rows)


def q1_device_supported(device: int = 0) -> bool:
    return load_library().q1_device_supported(device) == 0


def q1_last_error() -> str:
    return load_library().q1_last_error().decode()


def q1_version() -> str:
    return load_library().q1_version().decode()
