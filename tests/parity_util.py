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


# The oracle's results for the named workloads, computed once per process and
# shared by the split and two-launch tests (the oracle is deterministic).
_REFERENCE = {}


def workload_reference(w, x):
    """Every output of the oracle (full forward and backward) for a workload small enough to take whole."""
    if w.name not in _REFERENCE:
        say(f"case {w.name}: oracle, every row and key column")
        _REFERENCE[w.name] = full_reference(x, w.causal)
    return _REFERENCE[w.name]


def long_context_reference(w, x, kv_heads, n_rows):
    """For the long-context workload: sampled rows (O, L, D, dQ) and the whole sequence's dK / dV columns of
    the given K/V heads (key tile 0, the longest reduction, and every boosted key among them)."""
    import oracle
    key = (w.name, tuple(kv_heads), n_rows)
    if key not in _REFERENCE:
        B, H, T, KV = w.batch, w.heads, w.T, w.kv_heads
        rows = sample_rows(B, H, T, n_rows, seed=w.seed)
        say(f"case {w.name}: oracle rows {rows.size}")
        D, dQ, O, L = oracle.backward_rows(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=w.causal,
                                           seqlens=x["seqlens"], rows=rows)
        cols = np.concatenate([np.arange((b * KV + kv) * T, (b * KV + kv + 1) * T, dtype=np.int64)
                               for b in range(B) for kv in kv_heads])
        say(f"case {w.name}: oracle key columns {cols.size} (K/V heads {list(kv_heads)}, whole sequence)")
        dK, dV = oracle.backward_cols(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=w.causal,
                                      seqlens=x["seqlens"], cols=cols)
        _REFERENCE[key] = {"rows": rows, "D": D, "dQ": dQ, "O": O, "L": L, "cols": cols, "dK": dK, "dV": dV}
    return _REFERENCE[key]


def check_workload_full(w, x, got, where):
    """Every O / L / D / dQ row and every dK / dV column against the oracle, padded rows and keys exactly 0."""
    ref = workload_reference(w, x)
    check_forward(got["O"], got["L"], ref["O"], ref["L"], where)
    errs = {k: check_grad(k, got[k], ref[k], where) for k in ("dQ", "dK", "dVt")}
    d_err = rel_l2(got["D"], ref["D"])
    assert d_err <= 1e-2, f"{where}: D rel L2 {d_err:.2e}"
    # each K/V head's columns on their own too, so that an error confined to one head is not averaged away
    for b in range(w.batch):
        for kv in range(w.kv_heads):
            if np.linalg.norm(ref["dK"][b, kv]) > 0:
                check_grad("dK", got["dK"][b, kv], ref["dK"][b, kv], f"{where} b={b} kv={kv}")
                check_grad("dV", got["dVt"][b, kv], ref["dVt"][b, kv], f"{where} b={b} kv={kv}")
    if x["seqlens"] is not None:
        for b, n in enumerate(x["seqlens"]):
            assert np.all(got["D"][b, :, n:] == 0) and np.all(got["dQ"][b, :, n:] == 0), where
            assert np.all(got["dK"][b, :, n:] == 0) and np.all(got["dVt"][b, :, :, n:] == 0), where
    say(f"{where}: full tensors: dQ {errs['dQ']:.2e} dK {errs['dK']:.2e} dV {errs['dVt']:.2e} D {d_err:.2e}")


def check_long_context(w, x, got, where, kv_heads=(0, 5), n_rows=1024):
    """Long-context workload: sampled rows, and the whole sequence of two K/V heads' dK / dV columns."""
    ref = long_context_reference(w, x, kv_heads, n_rows)
    rows = ref["rows"]
    check_forward(got["O"].reshape(-1, 64)[rows], got["L"].reshape(-1)[rows], ref["O"], ref["L"], where)
    check_grad("dQ", got["dQ"].reshape(-1, 64)[rows], ref["dQ"], where)
    assert rel_l2(got["D"].reshape(-1)[rows], ref["D"]) <= 1e-2, where
    cols = ref["cols"]
    gK = got["dK"].reshape(-1, 64)[cols]
    gV = np.swapaxes(got["dVt"], -1, -2).reshape(-1, 64)[cols]
    T = w.T
    for i, kv in enumerate(kv_heads):
        part = slice(i * T, (i + 1) * T)
        check_grad("dK", gK[part], ref["dK"][part], f"{where} kv={kv}")
        check_grad("dV", gV[part], ref["dV"][part], f"{where} kv={kv}")
        # key tile 0 (the longest walk, scheduled first) on its own
        check_grad("dK", gK[part][:64], ref["dK"][part][:64], f"{where} kv={kv} key tile 0")
        check_grad("dV", gV[part][:64], ref["dV"][part][:64], f"{where} kv={kv} key tile 0")
    # every boosted key of the first head: the rows whose norm stands out (the boost is x8)
    K0 = x["K"][0, kv_heads[0]].astype(np.float64)
    norms = np.linalg.norm(K0, axis=1)
    boosted = np.nonzero(norms > 4.0 * np.median(norms))[0]
    assert boosted.size == int(round(w.boost_frac * T)), boosted.size
    check_grad("dK", gK[:T][boosted], ref["dK"][:T][boosted], f"{where} boosted keys")
    check_grad("dV", gV[:T][boosted], ref["dV"][:T][boosted], f"{where} boosted keys")
    say(f"{where}: rows {rows.size}, whole-sequence dK/dV of K/V heads {list(kv_heads)}, "
        f"{boosted.size} boosted keys")
