"""Reference oracle for causal streaming attention (binary64, CPU).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the library
itself never does.  It shares no code with the HIP path.

The arithmetic lives in ``sa_oracle.c`` (plain C, OpenMP over independent rows
or key columns).  This module only builds it with gcc, loads it with ctypes
and marshals numpy arrays.  What each function computes, with its citation of
the pages, is stated in ``sa_oracle.c``:

* forward rows: StreamingAttentionSM86 page, banner "Causal attention as a
  streaming normalised sum" (softmax in base-2 units, O and the base-2
  log-sum-exp L);
* backward rows and key columns: same page, banner "The backward pass,
  deterministic and in two launches" (D, dP, dS, dQ, dK, dV);
* length masks and zero output for fully masked rows: the variable-length
  gist page (``self_attn_fwd``);
* ``rotated_dq_slice`` (plain numpy, binary64): dQ turned back by the inverse
  half-split rotation and laid out as the Q slice of a token-major projection
  gradient, as the same page's query pass stores it in its rotated variant
  (the "dQ = s (the sum), turned back by the inverse half-split rotation"
  epilogue);
* ``projection_slices`` (plain numpy): dQ, dK and dV laid out as the Q, K and
  V column slices of a fused projection's token-major gradient, as the same
  page's query and key launches store them in their projection variants.

Array layouts follow the library: Q, dO ``[B][H][T][64]``; K ``[B][KV][T][64]``;
Vt ``[B][KV][64][T]``; the outputs are float64.  Inputs may be float16 (the
exact values are used) or float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sa_oracle.c")
_LIB = os.path.join(_HERE, "libsa_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile sa_oracle.c into libsa_oracle.so next to it (gcc, OpenMP)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    common = [_dp, _dp, _dp]
    shape = [ctypes.c_int] * 5 + [_ip, ctypes.c_double]
    lib.oracle_forward_rows.argtypes = common + shape + [_lp, ctypes.c_int64, _dp, _dp]
    lib.oracle_backward_rows.argtypes = common + [_dp] + shape + [_lp, ctypes.c_int64, _dp, _dp, _dp, _dp]
    lib.oracle_backward_cols.argtypes = common + [_dp] + shape + [_lp, ctypes.c_int64, _dp, _dp]
    for f in (lib.oracle_forward_rows, lib.oracle_backward_rows, lib.oracle_backward_cols):
        f.restype = ctypes.c_int
    lib.oracle_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle uses."""
    return int(_load().oracle_threads())


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a, t=_dp):
    return a.ctypes.data_as(t) if a is not None else None


class _Problem:
    def __init__(self, Q, K, Vt, dO, causal, seqlens, s):
        self.Q, self.K, self.Vt = _f64(Q), _f64(K), _f64(Vt)
        self.dO = _f64(dO) if dO is not None else None
        B, H, T, d = self.Q.shape
        KV = self.K.shape[1]
        if d != 64 or self.K.shape != (B, KV, T, 64) or self.Vt.shape != (B, KV, 64, T):
            raise ValueError("oracle: shapes must be Q[B,H,T,64], K[B,KV,T,64], Vt[B,KV,64,T]")
        if self.dO is not None and self.dO.shape != self.Q.shape:
            raise ValueError("oracle: dO must have Q's shape")
        self.B, self.H, self.T, self.KV = B, H, T, KV
        self.causal = int(bool(causal))
        self.seqlens = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
        if self.seqlens is not None and self.seqlens.shape != (B,):
            raise ValueError("oracle: seqlens must have shape [B]")
        self.s = float(s)

    def shape_args(self):
        return [self.B, self.T, self.H, self.KV, self.causal, _ptr(self.seqlens, _ip), self.s]


def _ids(ids, n):
    ids = np.arange(n, dtype=np.int64) if ids is None else np.ascontiguousarray(ids, dtype=np.int64)
    return ids


def forward_rows(Q, K, Vt, *, s, causal, seqlens=None, rows=None):
    """O [n,64] and L [n] for row ids (b*H + h)*T + i (all rows if None)."""
    p = _Problem(Q, K, Vt, None, causal, seqlens, s)
    rows = _ids(rows, p.B * p.H * p.T)
    O = np.empty((rows.size, 64))
    L = np.empty(rows.size)
    rc = _load().oracle_forward_rows(_ptr(p.Q), _ptr(p.K), _ptr(p.Vt), *p.shape_args(),
                                     _ptr(rows, _lp), rows.size, _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError("oracle_forward_rows: bad shape or row id")
    return O, L


def backward_rows(Q, K, Vt, dO, *, s, causal, seqlens=None, rows=None):
    """D [n], dQ [n,64], O [n,64], L [n] for row ids (b*H + h)*T + i."""
    p = _Problem(Q, K, Vt, dO, causal, seqlens, s)
    rows = _ids(rows, p.B * p.H * p.T)
    D = np.empty(rows.size)
    dQ = np.empty((rows.size, 64))
    O = np.empty((rows.size, 64))
    L = np.empty(rows.size)
    rc = _load().oracle_backward_rows(_ptr(p.Q), _ptr(p.K), _ptr(p.Vt), _ptr(p.dO), *p.shape_args(),
                                      _ptr(rows, _lp), rows.size, _ptr(D), _ptr(dQ), _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError("oracle_backward_rows: bad shape or row id")
    return D, dQ, O, L


def backward_cols(Q, K, Vt, dO, *, s, causal, seqlens=None, cols=None):
    """dK [n,64], dV [n,64] for key column ids (b*KV + kv)*T + j."""
    p = _Problem(Q, K, Vt, dO, causal, seqlens, s)
    cols = _ids(cols, p.B * p.KV * p.T)
    dK = np.empty((cols.size, 64))
    dV = np.empty((cols.size, 64))
    rc = _load().oracle_backward_cols(_ptr(p.Q), _ptr(p.K), _ptr(p.Vt), _ptr(p.dO), *p.shape_args(),
                                      _ptr(cols, _lp), cols.size, _ptr(dK), _ptr(dV))
    if rc != 0:
        raise ValueError("oracle_backward_cols: bad shape or column id")
    return dK, dV


def forward(Q, K, Vt, *, s, causal, seqlens=None):
    """Full forward: O [B,H,T,64] (head-major) and L [B,H,T]."""
    B, H, T, _ = np.shape(Q)
    O, L = forward_rows(Q, K, Vt, s=s, causal=causal, seqlens=seqlens)
    return O.reshape(B, H, T, 64), L.reshape(B, H, T)


def backward(Q, K, Vt, dO, *, s, causal, seqlens=None):
    """Full backward: dict with O, L, D, dQ (head-major), dK [B,KV,T,64], dVt [B,KV,64,T]."""
    B, H, T, _ = np.shape(Q)
    KV = np.shape(K)[1]
    D, dQ, O, L = backward_rows(Q, K, Vt, dO, s=s, causal=causal, seqlens=seqlens)
    dK, dV = backward_cols(Q, K, Vt, dO, s=s, causal=causal, seqlens=seqlens)
    return {
        "O": O.reshape(B, H, T, 64), "L": L.reshape(B, H, T), "D": D.reshape(B, H, T),
        "dQ": dQ.reshape(B, H, T, 64), "dK": dK.reshape(B, KV, T, 64),
        "dVt": dV.reshape(B, KV, T, 64).transpose(0, 1, 3, 2).copy(),
    }


def rotated_dq_slice(dQ, cos, sin, width):
    """The Q slice of a token-major projection gradient [B][T][width] (binary64).

    StreamingAttentionSM86 page, the query pass's rotated epilogue: dQ
    [B][H][T][64] (already scaled by s) is turned back by the inverse of the
    half-split rotation, whose tables cos and sin are [T][32] (position p,
    column pair c < 32), and row p, column c of head h lands at (p, 64 h + c):
        out[64 h + c]      = dQ[c] cos[p][c] + dQ[c + 32] sin[p][c]
        out[64 h + c + 32] = dQ[c + 32] cos[p][c] - dQ[c] sin[p][c]
    Columns at or past 64 H are zero here (the library leaves them untouched).
    """
    dQ = np.asarray(dQ, dtype=np.float64)
    B, H, T, d = dQ.shape
    assert d == 64 and width >= 64 * H
    c = np.asarray(cos, dtype=np.float64)[None, None, :, :]   # [1,1,T,32]
    s_ = np.asarray(sin, dtype=np.float64)[None, None, :, :]
    x1, x2 = dQ[..., :32], dQ[..., 32:]
    rot = np.concatenate([x1 * c + x2 * s_, x2 * c - x1 * s_], axis=-1)   # [B,H,T,64]
    out = np.zeros((B, T, width))
    out[:, :, :64 * H] = rot.transpose(0, 2, 1, 3).reshape(B, T, 64 * H)
    return out


def projection_slices(dQ, dK, dVt, width, q_col, k_col, v_col):
    """dQ [B][H][T][64], dK [B][KV][T][64] and dVt [B][KV][64][T] laid out in one token-major [B][T][width]
    gradient (binary64): row t holds head h's dQ at columns q_col + 64 h + c, K/V head kv's dK at
    k_col + 64 kv + c and dV at v_col + 64 kv + c (StreamingAttentionSM86 page, the query and key launches'
    projection epilogues: dQ, dK and dV "stored straight into a fused projection's gradient").  Other
    columns are zero."""
    dQ, dK, dVt = (np.asarray(a, dtype=np.float64) for a in (dQ, dK, dVt))
    B, H, T, _ = dQ.shape
    KV = dK.shape[1]
    out = np.zeros((B, T, width))
    out[:, :, q_col:q_col + 64 * H] = dQ.transpose(0, 2, 1, 3).reshape(B, T, 64 * H)
    out[:, :, k_col:k_col + 64 * KV] = dK.transpose(0, 2, 1, 3).reshape(B, T, 64 * KV)
    out[:, :, v_col:v_col + 64 * KV] = dVt.transpose(0, 3, 1, 2).reshape(B, T, 64 * KV)
    return out
