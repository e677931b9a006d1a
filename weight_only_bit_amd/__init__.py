"""weight_only_bit_amd -- Python binding of libwq.so (include/wq.h).

Argument marshalling only: every computation runs in the library's HIP kernels on the GPU.
PyTorch provides device memory and the current HIP stream.  If the library has not been
built, importing works but every call raises (there is no CPU fallback).

Names follow the C ABI: ``wq_dequantize``, ``wq_gemm``, ``wq_moe_route``, ``wq_moe_ffn``,
``wq_moe_workspace_bytes``, ``wq_pack_int4``, ``wq_unpack_int4``, ``wq_packed_size``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

WQ_OK = 0
WQ_ERR_ARG = -1
WQ_ERR_UNSUPPORTED = -2
WQ_ERR_ALIGN = -3
WQ_ERR_RANGE = -4
WQ_ERR_WORKSPACE = -5
WQ_ERR_HIP = -6

FMT_INT4, FMT_INT2_AFFINE, FMT_CCQ2, FMT_CCQ432, FMT_CCQ_HYBRID, FMT_INT8 = 1, 2, 3, 4, 5, 6

# Every symbol include/wq.h declares.
EXPORTS = ("wq_dequantize", "wq_gemm", "wq_moe_workspace_bytes", "wq_moe_route", "wq_moe_ffn",
           "wq_moe_gate_up", "wq_moe_down", "wq_moe_combine", "wq_pack_int4", "wq_unpack_int4",
           "wq_packed_size", "wq_status_string", "wq_last_error", "wq_quantize_ccq")


class WqError(RuntimeError):
    pass


class _CWeight(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("experts", ctypes.c_int64),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("zeros", ctypes.c_void_p),
        ("qscale", ctypes.c_void_p),
        ("super_scale", ctypes.c_void_p),
        ("code_scale", ctypes.c_void_p),
        ("code_zero", ctypes.c_void_p),
        ("zp", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libwq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise WqError(f"{LIB_PATH} is missing: build it with weight_only_bit_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        W = ctypes.POINTER(_CWeight)
        sig = {
            "wq_dequantize": (i32, [W, vp, vp]),
            "wq_gemm": (i32, [vp, i64, W, vp, vp]),
            "wq_moe_workspace_bytes": (sz, [i64, i32, i32, i64, i64]),
            "wq_moe_route": (i32, [vp, i64, i32, i32, vp, vp, vp, sz, vp]),
            "wq_moe_ffn": (i32, [vp, i64, i64, vp, vp, i32, W, W, W, vp, vp, sz, vp]),
            "wq_moe_gate_up": (i32, [vp, i64, vp, vp, i32, W, W, vp, vp]),
            "wq_moe_down": (i32, [vp, i64, i32, vp, vp, W, vp, vp]),
            "wq_moe_combine": (i32, [vp, vp, i64, i32, i64, vp, vp]),
            "wq_quantize_ccq": (i32, [vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp]),
            "wq_pack_int4": (i32, [vp, i64, vp]),
            "wq_unpack_int4": (i32, [vp, i64, vp]),
            "wq_packed_size": (i64, [i64, i32]),
            "wq_status_string": (ctypes.c_char_p, [i32]),
            "wq_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st == WQ_OK:
        return
    L = lib()
    name = L.wq_status_string(st).decode()
    detail = L.wq_last_error().decode()
    msg = f"{what}: {name}: {detail}"
    if st in (WQ_ERR_ARG, WQ_ERR_UNSUPPORTED, WQ_ERR_ALIGN, WQ_ERR_RANGE, WQ_ERR_WORKSPACE):
        raise ValueError(msg)
    raise WqError(msg)


def _stream():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class PackedWeight:
    """Device tensors of a packed weight [experts, n, k] (see include/wq.h for layouts)."""
    format: int
    n: int
    k: int
    experts: int = 1
    group: int = 64
    codes: object = None
    scales: object = None
    zeros: object = None
    qscale: object = None
    super_scale: object = None
    code_scale: object = None
    code_zero: object = None
    zp: int = 32
    _c: object = field(default=None, repr=False)

    def cstruct(self) -> _CWeight:
        self._c = _CWeight(self.format, self.group, self.experts, self.n, self.k,
                           *[None if getattr(self, f) is None else getattr(self, f).data_ptr()
                             for f in ("codes", "scales", "zeros", "qscale", "super_scale",
                                       "code_scale", "code_zero")],
                           self.zp)
        return self._c

    def nbytes(self) -> int:
        return sum(getattr(self, f).numel() * getattr(self, f).element_size()
                   for f in ("codes", "scales", "zeros", "qscale", "super_scale", "code_scale",
                             "code_zero") if getattr(self, f) is not None)

    @staticmethod
    def from_arrays(fmt: int, experts: int, n: int, k: int, arrays: dict, group: int = 64,
                    zp: int = 32, device="cuda") -> "PackedWeight":
        """Upload host (numpy) or wrap device (torch) arrays named as in include/wq.h."""
        import torch

        def dev(a):
            if a is None:
                return None
            if isinstance(a, torch.Tensor):
                return a.to(device).contiguous()
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                a = a.view(np.int16)
            return torch.from_numpy(a).to(device)

        return PackedWeight(fmt, n, k, experts, group, *(dev(arrays.get(f)) for f in (
            "codes", "scales", "zeros", "qscale", "super_scale", "code_scale", "code_zero")), zp)


# ---------------------------------------------------------------------------------------------
# Compute calls (device tensors in, device tensors out, on torch's current stream)
# ---------------------------------------------------------------------------------------------

def wq_dequantize(w: PackedWeight, out=None):
    """All weights decoded to bf16, shape [experts, n, k] (int16 tensor of bf16 bits)."""
    import torch

    if out is None:
        out = torch.empty((w.experts, w.n, w.k), dtype=torch.int16, device=w.codes.device)
    _check(lib().wq_dequantize(ctypes.byref(w.cstruct()), _ptr(out), _stream()), "wq_dequantize")
    return out


def wq_gemm(x, w: PackedWeight, y=None):
    """y = bf16(x @ dequant(W)^T); x is [m, k] bf16 (torch.bfloat16 or int16 bits)."""
    import torch

    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.bfloat16, device=x.device)
    _check(lib().wq_gemm(_ptr(x), m, ctypes.byref(w.cstruct()), _ptr(y), _stream()), "wq_gemm")
    return y


def wq_moe_workspace_bytes(t: int, topk: int, experts: int, hidden: int, inter: int) -> int:
    return int(lib().wq_moe_workspace_bytes(t, topk, experts, hidden, inter))


def wq_moe_route(topk_ids, experts: int):
    """(expert_offsets int32 [E+1], sorted_pairs int32 [t*topk]) on the device."""
    import torch

    t, topk = topk_ids.shape
    off = torch.empty(experts + 1, dtype=torch.int32, device=topk_ids.device)
    pairs = torch.empty(t * topk, dtype=torch.int32, device=topk_ids.device)
    _check(lib().wq_moe_route(_ptr(topk_ids), t, topk, experts, _ptr(off), _ptr(pairs), None, 0,
                              _stream()), "wq_moe_route")
    return off, pairs


def wq_moe_ffn(x, topk_ids, topk_weights, gate: PackedWeight, up: PackedWeight,
               down: PackedWeight, y=None, ws=None):
    """MoE expert FFN; x [t, hidden] bf16, topk_ids int32 [t, topk], topk_weights f32."""
    import torch

    t, hidden = x.shape
    topk = topk_ids.shape[1]
    if y is None:
        y = torch.empty((t, hidden), dtype=torch.bfloat16, device=x.device)
    need = wq_moe_workspace_bytes(t, topk, gate.experts, hidden, gate.n)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib().wq_moe_ffn(_ptr(x), t, hidden, _ptr(topk_ids), _ptr(topk_weights), topk,
                            ctypes.byref(gate.cstruct()), ctypes.byref(up.cstruct()),
                            ctypes.byref(down.cstruct()), _ptr(y), _ptr(ws), ws.numel(),
                            _stream()), "wq_moe_ffn")
    return y


def wq_moe_gate_up(x, offsets, sorted_pairs, topk: int, gate: PackedWeight, up: PackedWeight,
                   h=None):
    """h [t*topk, inter] bf16 (rows in expert-sorted order) = SiLU(gate x) * (up x)."""
    import torch

    t = x.shape[0]
    if h is None:
        h = torch.empty((t * topk, gate.n), dtype=torch.bfloat16, device=x.device)
    _check(lib().wq_moe_gate_up(_ptr(x), t, _ptr(offsets), _ptr(sorted_pairs), topk,
                                ctypes.byref(gate.cstruct()), ctypes.byref(up.cstruct()), _ptr(h),
                                _stream()), "wq_moe_gate_up")
    return h


def wq_moe_down(h, t: int, topk: int, offsets, sorted_pairs, down: PackedWeight, d=None):
    """d [t*topk, hidden] f32 (row = pair id) = down h."""
    import torch

    if d is None:
        d = torch.empty((t * topk, down.n), dtype=torch.float32, device=h.device)
    _check(lib().wq_moe_down(_ptr(h), t, topk, _ptr(offsets), _ptr(sorted_pairs),
                             ctypes.byref(down.cstruct()), _ptr(d), _stream()), "wq_moe_down")
    return d


def wq_moe_combine(d, topk_weights, y=None):
    """y [t, hidden] bf16 = sum_j topk_weights[t, j] * d[t*topk + j]."""
    import torch

    t, topk = topk_weights.shape
    hidden = d.shape[1]
    if y is None:
        y = torch.empty((t, hidden), dtype=torch.bfloat16, device=d.device)
    _check(lib().wq_moe_combine(_ptr(d), _ptr(topk_weights), t, topk, hidden, _ptr(y), _stream()),
           "wq_moe_combine")
    return y


def wq_quantize_ccq(w, zp: int = 32, refine: bool = True) -> PackedWeight:
    """CCQ (6,4,3) code-cluster encoding of fp32 weights [n, k] or [E, n, k] on the GPU."""
    import torch

    if w.dim() == 2:
        w = w.unsqueeze(0)
    E, n, k = w.shape
    w = w.contiguous().float()
    dev = w.device
    rows = E * n
    G = k // 64
    codes = torch.empty((E, n, k // 4), dtype=torch.uint8, device=dev)
    qscale = torch.empty((E, n, (G + 1) // 2), dtype=torch.uint8, device=dev)
    sup = torch.empty((E, n), dtype=torch.float32, device=dev)
    cs = torch.empty((E, n), dtype=torch.float32, device=dev)
    cz = torch.empty((E, n), dtype=torch.float32, device=dev)
    _check(lib().wq_quantize_ccq(_ptr(w), rows, k, zp, int(bool(refine)), _ptr(codes), _ptr(qscale),
                                 _ptr(sup), _ptr(cs), _ptr(cz), _stream()), "wq_quantize_ccq")
    return PackedWeight(FMT_CCQ2, n, k, E, 64, codes, None, None, qscale, sup, cs, cz, zp)


# ---------------------------------------------------------------------------------------------
# Host helpers
# ---------------------------------------------------------------------------------------------

def wq_pack_int4(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.int32).ravel()
    out = np.zeros((c.size + 1) // 2, np.uint8)
    _check(lib().wq_pack_int4(c.ctypes.data, c.size, out.ctypes.data), "wq_pack_int4")
    return out


def wq_unpack_int4(data, n: int) -> np.ndarray:
    d = np.ascontiguousarray(data, dtype=np.uint8).ravel()
    if n > 2 * d.size:
        raise ValueError("wq_unpack_int4: not enough bytes")
    out = np.empty(n, np.int32)
    _check(lib().wq_unpack_int4(d.ctypes.data, n, out.ctypes.data), "wq_unpack_int4")
    return out


def wq_packed_size(n_codes: int, bits: int = 4) -> int:
    return int(lib().wq_packed_size(n_codes, bits))
