"""Causal streaming attention for MI355X (gfx950), head width 64.

A thin Python binding of the HIP library ``libsa.so`` (built from ``csrc/`` by
``causal_streaming_attention_amd.build``).  The functions named ``sa_*`` are the
C ABI of ``include/sa.h`` with the same names and argument order; they only
turn torch tensors into device pointers, pass the current torch stream unless
one is given, and raise :class:`SaError` on a non-zero status.  Every step of
the computation runs in the library's kernels; there is no fallback.  If the
library is missing, the first call raises.

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")
_lib = None

(SA_OK, SA_ERR_SHAPE, SA_ERR_NULL, SA_ERR_ALIGN, SA_ERR_WORKSPACE, SA_ERR_ARGUMENT, SA_ERR_DEVICE,
 SA_ERR_TOO_LARGE) = range(8)
SA_STATIC_SCRATCH_BYTES = 64 << 20


class SaShape(ctypes.Structure):
    """``sa_shape`` of include/sa.h."""
    _fields_ = [("batch", ctypes.c_int), ("T", ctypes.c_int), ("heads", ctypes.c_int),
                ("kv_heads", ctypes.c_int), ("causal", ctypes.c_int), ("seqlens", ctypes.c_void_p),
                ("block_order", ctypes.c_int), ("v_rows", ctypes.c_int)]


class SaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({sa_status_string(status)})")


_V = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_SP = ctypes.POINTER(SaShape)

_SIGS = {
    "sa_check_shape": (_I, [_SP]),
    "sa_forward": (_I, [_V, _V, _V, _V, _V, _F, _I, _I, _I, _V]),
    "sa_forward_ex": (_I, [_SP, _V, _V, _V, _V, _V, _F, _V]),
    "sa_backward_workspace_bytes": (_Z, [_SP]),
    "sa_backward": (_I, [_V, _V, _V, _V, _V, _Z, _V, _V, _V, _F, _F, _I, _I, _I, _V, _V, _V, _V]),
    "sa_backward_ex": (_I, [_SP, _V, _V, _V, _V, _V, _Z, _V, _V, _V, _F, _F, _V, _V, _V, _V]),
    "sa_row_terms": (_I, [_SP, _V, _V, _V, _V]),
    "sa_key_pass": (_I, [_SP, _V, _V, _V, _V, _V, _V, _V, _Z, _F, _F, _V, _V, _V]),
    "sa_dq_pass": (_I, [_SP, _V, _V, _Z, _F, _V, _V]),
    "sa_dq_pass_rotated": (_I, [_SP, _V, _V, _Z, _F, _V, _V, _V, _I, _V]),
    "sa_backward_projection": (_I, [_SP, _V, _V, _V, _V, _V, _Z, _V, _V, _V, _F, _F, _V, _V, _V, _V, _V, _V, _I,
                                    _V]),
    "sa_backward_two_pass_projection": (_I, [_SP, _V, _V, _V, _V, _V, _V, _V, _F, _F, _V, _V, _V, _V, _V, _V, _I,
                                             _V]),
    "sa_query_pass": (_I, [_SP, _V, _V, _V, _V, _V, _V, _F, _F, _V, _V, _V]),
    "sa_backward_two_pass": (_I, [_SP, _V, _V, _V, _V, _V, _V, _V, _F, _F, _V, _V, _V, _V]),
    "sa_backward_static": (_I, [_SP, _V, _V, _V, _V, _V, _V, _V, _F, _F, _V, _V, _V, _V]),
    "sa_backward_chunked": (_I, [_SP, _V, _V, _V, _V, _V, _Z, _V, _V, _V, _F, _F, _V, _V, _V, _V]),
    "sa_backward_chunked_min_bytes": (_Z, [_SP]),
    "sa_status_string": (ctypes.c_char_p, [_I]),
}


def native():
    """The loaded libsa.so (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m causal_streaming_attention_amd.build`")
        from . import build as _build
        try:
            with open(_build.HASH_FILE) as f:
                built = f.read().strip()
        except OSError:
            built = None
        if built != _build.source_hash():
            raise RuntimeError(f"{LIB_PATH} was not built from the sources beside it (source hash "
                               f"{built} against {_build.source_hash()}): rebuild it with "
                               "`python -m causal_streaming_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGS)


def base2_scale(s: float) -> float:
    """The binary32 nearest s / ln 2 (the forward's score factor c)."""
    return float(np.float32(s / math.log(2.0)))


def make_shape(batch, T, heads, kv_heads, causal=True, seqlens=None, block_order=0, v_rows=0) -> SaShape:
    """An sa_shape; `seqlens` is a device int32 tensor (kept alive by the shape) or None.
    v_rows=1: the V operand is V [B][KV][T][64] (and dV comes back as [B][KV][T][64])."""
    sh = SaShape(batch, T, heads, kv_heads, int(bool(causal)), _ptr(seqlens), block_order, v_rows)
    sh._keep = seqlens
    return sh


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != SA_OK:
        raise SaError(status, where)


def sa_status_string(status: int) -> str:
    return native().sa_status_string(int(status)).decode()


def sa_check_shape(shape: SaShape) -> int:
    return native().sa_check_shape(ctypes.byref(shape))


def sa_forward(Q, K, Vt, O, L, c, T, heads, kv_heads, stream=None):
    _check(native().sa_forward(_ptr(Q), _ptr(K), _ptr(Vt), _ptr(O), _ptr(L), c, T, heads, kv_heads,
                               _stream(stream)), "sa_forward")


def sa_forward_ex(shape, Q, K, Vt, O, L, c, stream=None):
    _check(native().sa_forward_ex(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(Vt), _ptr(O), _ptr(L), c,
                                  _stream(stream)), "sa_forward_ex")


def sa_backward_workspace_bytes(shape) -> int:
    return int(native().sa_backward_workspace_bytes(ctypes.byref(shape)))


def sa_backward(dO, O, L, D, dS, dS_bytes, Q, K, Vt, c, s, T, heads, kv_heads, dQ, dK, dVt, stream=None):
    _check(native().sa_backward(_ptr(dO), _ptr(O), _ptr(L), _ptr(D), _ptr(dS), dS_bytes, _ptr(Q), _ptr(K),
                                _ptr(Vt), c, s, T, heads, kv_heads, _ptr(dQ), _ptr(dK), _ptr(dVt),
                                _stream(stream)), "sa_backward")


def sa_backward_ex(shape, dO, O, L, D, dS, dS_bytes, Q, K, Vt, c, s, dQ, dK, dVt, stream=None):
    _check(native().sa_backward_ex(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(D), _ptr(dS),
                                   dS_bytes, _ptr(Q), _ptr(K), _ptr(Vt), c, s, _ptr(dQ), _ptr(dK), _ptr(dVt),
                                   _stream(stream)), "sa_backward_ex")


def sa_backward_chunked(shape, dO, O, L, D, dS, dS_bytes, Q, K, Vt, c, s, dQ, dK, dVt, stream=None):
    _check(native().sa_backward_chunked(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(D), _ptr(dS),
                                        dS_bytes, _ptr(Q), _ptr(K), _ptr(Vt), c, s, _ptr(dQ), _ptr(dK), _ptr(dVt),
                                        _stream(stream)), "sa_backward_chunked")


def sa_backward_chunked_min_bytes(shape) -> int:
    return int(native().sa_backward_chunked_min_bytes(ctypes.byref(shape)))


def sa_backward_static(shape, dO, O, L, D, Q, K, Vt, c, s, dQ, dK, dVt, stream=None):
    """The split backward with the library's static dS scratch (no workspace argument, nothing allocated)."""
    _check(native().sa_backward_static(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(D), _ptr(Q), _ptr(K),
                                       _ptr(Vt), c, s, _ptr(dQ), _ptr(dK), _ptr(dVt), _stream(stream)),
           "sa_backward_static")


def sa_row_terms(shape, dO, O, D, stream=None):
    _check(native().sa_row_terms(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(D), _stream(stream)),
           "sa_row_terms")


def sa_key_pass(shape, Q, K, Vt, dO, L, D, dS, dS_bytes, c, s, dK, dVt, stream=None):
    _check(native().sa_key_pass(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(Vt), _ptr(dO), _ptr(L), _ptr(D),
                                _ptr(dS), dS_bytes, c, s, _ptr(dK), _ptr(dVt), _stream(stream)), "sa_key_pass")


def sa_dq_pass(shape, K, dS, dS_bytes, s, dQ, stream=None):
    _check(native().sa_dq_pass(ctypes.byref(shape), _ptr(K), _ptr(dS), dS_bytes, s, _ptr(dQ),
                               _stream(stream)), "sa_dq_pass")


def sa_dq_pass_rotated(shape, K, dS, dS_bytes, s, cos, sin, dqkv, width, stream=None):
    _check(native().sa_dq_pass_rotated(ctypes.byref(shape), _ptr(K), _ptr(dS), dS_bytes, s, _ptr(cos), _ptr(sin),
                                       _ptr(dqkv), width, _stream(stream)), "sa_dq_pass_rotated")


def sa_backward_projection(shape, dO, O, L, D, dS, dS_bytes, Q, K, Vt, c, s, dQ32, dQ16, dK32, dK16, dV32, dV16,
                           width, stream=None):
    """The pointer arguments may be torch tensors (their start) or plain device addresses (ints), so a
    column slice of a shared [B][T][width] buffer can be named by its first element's address."""
    _check(native().sa_backward_projection(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(D), _ptr(dS),
                                           dS_bytes, _ptr(Q), _ptr(K), _ptr(Vt), c, s, _ptr(dQ32), _ptr(dQ16),
                                           _ptr(dK32), _ptr(dK16), _ptr(dV32), _ptr(dV16), width, _stream(stream)),
           "sa_backward_projection")


def sa_backward_two_pass_projection(shape, dO, O, L, D, Q, K, Vt, c, s, dQ32, dQ16, dK32, dK16, dV32, dV16, width,
                                    stream=None):
    _check(native().sa_backward_two_pass_projection(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(D),
                                                    _ptr(Q), _ptr(K), _ptr(Vt), c, s, _ptr(dQ32), _ptr(dQ16),
                                                    _ptr(dK32), _ptr(dK16), _ptr(dV32), _ptr(dV16), width,
                                                    _stream(stream)),
           "sa_backward_two_pass_projection")


def sa_query_pass(shape, dO, O, L, Q, K, Vt, c, s, D, dQ, stream=None):
    _check(native().sa_query_pass(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(Q), _ptr(K), _ptr(Vt),
                                  c, s, _ptr(D), _ptr(dQ), _stream(stream)), "sa_query_pass")


def sa_backward_two_pass(shape, dO, O, L, D, Q, K, Vt, c, s, dQ, dK, dVt, stream=None):
    _check(native().sa_backward_two_pass(ctypes.byref(shape), _ptr(dO), _ptr(O), _ptr(L), _ptr(D), _ptr(Q),
                                         _ptr(K), _ptr(Vt), c, s, _ptr(dQ), _ptr(dK), _ptr(dVt),
                                         _stream(stream)), "sa_backward_two_pass")


class Buffers:
    """Device tensors for one problem (torch allocations; the library allocates nothing).

    Inputs are copied from the float16 numpy arrays of ``workloads.make_inputs``;
    outputs and the dS workspace are allocated empty.  With ``v_rows`` the V
    operand (attribute ``Vt``) holds V as rows [B][KV][T][64] and ``dVt``
    receives dV in that layout."""

    def __init__(self, inputs: dict, causal: bool, device="cuda", block_order=0, v_rows=False):
        import torch
        Q = inputs["Q"]
        B, H, T, _ = Q.shape
        KV = inputs["K"].shape[1]
        self.B, self.H, self.T, self.KV = B, H, T, KV
        dev = torch.device(device)
        def put(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(dev)
        v = inputs["Vt"].transpose(0, 1, 3, 2) if v_rows else inputs["Vt"]
        self.Q, self.K, self.Vt, self.dO = put(Q), put(inputs["K"]), put(v), put(inputs["dO"])
        sl = inputs.get("seqlens")
        self.seqlens = None if sl is None else torch.from_numpy(np.asarray(sl, dtype=np.int32)).to(dev)
        self.v_rows = bool(v_rows)
        self.shape = make_shape(B, T, H, KV, causal, self.seqlens, block_order, int(self.v_rows))
        f16, f32 = torch.float16, torch.float32
        self.O = torch.empty((B, T, H * 64), dtype=f16, device=dev)
        self.L = torch.empty((B, H, T), dtype=f32, device=dev)
        self.D = torch.empty((B, H, T), dtype=f32, device=dev)
        self.dQ = torch.empty((B, H, T, 64), dtype=f32, device=dev)
        self.dK = torch.empty((B, KV, T, 64), dtype=f32, device=dev)
        self.dVt = torch.empty((B, KV, T, 64) if v_rows else (B, KV, 64, T), dtype=f32, device=dev)
        self.ws_bytes = sa_backward_workspace_bytes(self.shape)
        self.dS = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)

    def forward(self, c, stream=None):
        sa_forward_ex(self.shape, self.Q, self.K, self.Vt, self.O, self.L, c, stream)

    def backward(self, c, s, stream=None):
        sa_backward_ex(self.shape, self.dO, self.O, self.L, self.D, self.dS, self.ws_bytes, self.Q, self.K,
                       self.Vt, c, s, self.dQ, self.dK, self.dVt, stream)

    def backward_two_pass(self, c, s, stream=None):
        sa_backward_two_pass(self.shape, self.dO, self.O, self.L, self.D, self.Q, self.K, self.Vt, c, s,
                             self.dQ, self.dK, self.dVt, stream)
