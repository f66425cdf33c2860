"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the binary64 oracle on the same seeded inputs.

Tolerances (the stated bar for this path): O max abs error <= 2e-3, L max
abs error <= 1e-3 on rows with an admitted key (masked rows exactly O = 0 and
L = -inf), dQ / dK / dV relative L2 error <= 1e-2."""
import math
import sys

import numpy as np

import causal_streaming_attention_amd as sa
from causal_streaming_attention_amd.workloads import SCALE

O_ATOL = 2e-3
L_ATOL = 1e-3
GRAD_RTOL_L2 = 1e-2
C = sa.base2_scale(SCALE)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(inputs, causal, block_order=0, backward=True, path="split", v_rows=False):
    """Forward (and backward) on cuda:0; returns the buffers object and numpy copies.
    path "split" is the three-launch backward through the dS workspace,
    "two_pass" the two-launch backward that stores no dS.  v_rows: V goes in
    as rows [B][KV][T][64]; dV comes back in that layout and is returned
    transposed, as dVt, like the V^T path's."""
    import torch
    buf = sa.Buffers(inputs, causal, block_order=block_order, v_rows=v_rows)
    buf.forward(C)
    if backward and path == "split":
        buf.backward(C, SCALE)
    elif backward:
        assert path == "two_pass", path
        buf.backward_two_pass(C, SCALE)
    torch.cuda.synchronize()
    B, H, T = buf.B, buf.H, buf.T
    out = {
        "O": buf.O.view(B, T, H, 64).permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64),
        "L": buf.L.cpu().numpy().astype(np.float64),
    }
    if backward:
        out.update({k: getattr(buf, k).cpu().numpy().astype(np.float64) for k in ("D", "dQ", "dK", "dVt")})
        if v_rows:
            out["dVt"] = np.ascontiguousarray(out["dVt"].transpose(0, 1, 3, 2))
    return buf, out


def rel_l2(got, want):
    num = float(np.linalg.norm((got - want).ravel()))
    den = float(np.linalg.norm(want.ravel()))
    return num / den if den > 0 else num


def check_forward(got_O, got_L, ref_O, ref_L, where=""):
    """O and L within tolerance; masked rows (ref L = -inf) exactly O = 0, L = -inf."""
    masked = np.isneginf(ref_L)
    assert np.array_equal(np.isneginf(got_L), masked), f"{where}: masked-row pattern of L differs"
    assert np.all(got_O[masked] == 0.0), f"{where}: masked rows of O not zero"
    err_o = np.abs(got_O - ref_O)
    i = np.unravel_index(np.argmax(err_o), err_o.shape)
    assert err_o[i] <= O_ATOL, f"{where}: O max abs err {err_o[i]:.3e} at {i} (|O|={abs(ref_O[i]):.3f})"
    live = ~masked
    if live.any():
        err_l = float(np.max(np.abs(got_L[live] - ref_L[live])))
        assert err_l <= L_ATOL, f"{where}: L max abs err {err_l:.3e}"
    return float(err_o[i])


def check_grad(name, got, want, where=""):
    e = rel_l2(got, want)
    assert e <= GRAD_RTOL_L2, f"{where}: {name} relative L2 error {e:.3e}"
    return e


def full_reference(inputs, causal):
    import oracle
    return oracle.backward(inputs["Q"], inputs["K"], inputs["Vt"], inputs["dO"], s=SCALE, causal=causal,
                           seqlens=inputs["seqlens"])


def sample_rows(B, H, T, n, seed, seqlens=None):
    """Row ids (b*H + h)*T + i: tile edges plus random rows."""
    rng = np.random.default_rng(seed)
    ids = set()
    edges = [0, 1, 63, 64, 127, 128, T // 2, T - 65, T - 64, T - 1]
    for b in range(B):
        for h in (0, H - 1):
            for i in edges:
                if 0 <= i < T:
                    ids.add((b * H + h) * T + i)
    while len(ids) < n:
        ids.add(int(rng.integers(0, B * H * T)))
    return np.array(sorted(ids), dtype=np.int64)


def sample_cols(B, KV, T, n, seed, kv_list=None, lo=0):
    """Key column ids (b*KV + kv)*T + j with j >= lo."""
    rng = np.random.default_rng(seed)
    kv_list = list(range(KV)) if kv_list is None else kv_list
    ids = set()
    for b in range(B):
        for kv in kv_list:
            for j in (lo, lo + 1, lo + 63, lo + 64, T - 64, T - 1):
                if lo <= j < T:
                    ids.add((b * KV + kv) * T + j)
    while len(ids) < n:
        b = int(rng.integers(0, B))
        kv = kv_list[int(rng.integers(0, len(kv_list)))]
        ids.add((b * KV + kv) * T + int(rng.integers(lo, T)))
    return np.array(sorted(ids), dtype=np.int64)
