"""GPU parity over a seeded sweep of small shapes: batch 1-3, T a multiple of
64 up to 640 (odd tile counts included), 1-3 K/V heads with 1-8 query heads
each (so one, two, three and four wave pairs per key-pass workgroup, and wave
slots that walk several heads), causal or not, random length masks (zero and
full lengths included), both backwards, V as rows or V^T, both block orders.
Every output against the oracle; for the split backward, also the chunked
backward with its smallest workspace (one 128-row block per chunk): D and dQ
bitwise the split backward's, dK and dV within rounding.  Needs an
MI355X."""
import numpy as np
import pytest

from causal_streaming_attention_amd.workloads import make_inputs
import causal_streaming_attention_amd as sa
from parity_util import check_forward, check_grad, full_reference, rel_l2, run_gpu, say
from test_gpu_chunked import _chunked

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        T = 64 * int(rng.integers(1, 11))
        KV = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 5, 6, 8]))
        causal = bool(rng.random() < 0.6)
        seqlens = None
        if rng.random() < 0.4:
            seqlens = [int(v) for v in rng.integers(0, T + 1, size=B)]
            seqlens[int(rng.integers(0, B))] = int(rng.choice([0, T, 1, T - 1]))
        path = "two_pass" if i % 3 == 2 else "split"
        v_rows = bool(i % 4 == 1)
        order = int(i % 5 == 3)
        out.append((f"s{i:02d}_b{B}_t{T}_h{KV * G}_kv{KV}_{'c' if causal else 'f'}"
                    f"{'_var' if seqlens else ''}_{path}{'_vrows' if v_rows else ''}{'_plain' if order else ''}",
                    B, T, KV * G, KV, causal, seqlens, path, v_rows, order))
    return out


CASES = _cases()


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens,path,v_rows,order", CASES, ids=[c[0] for c in CASES])
def test_sweep(name, B, T, H, KV, causal, seqlens, path, v_rows, order):
    say(f"case sweep {name}")
    x = make_inputs(B, T, H, KV, seed=3000 + B * 7 + T + H, seqlens=seqlens)
    buf, got = run_gpu(x, causal, block_order=order, path=path, v_rows=v_rows)
    ref = full_reference(x, causal)
    check_forward(got["O"], got["L"], ref["O"], ref["L"], name)
    for k in ("dQ", "dK", "dVt"):
        check_grad(k, got[k], ref[k], name)
    assert rel_l2(got["D"], ref["D"]) <= 1e-2, name
    if seqlens is not None:
        for b, n in enumerate(seqlens):
            assert np.all(got["dQ"][b, :, n:] == 0) and np.all(got["D"][b, :, n:] == 0), name
            assert np.all(got["dK"][b, :, n:] == 0) and np.all(got["dVt"][b, :, :, n:] == 0), name
    if path == "split":
        ch = _chunked(buf, sa.sa_backward_chunked_min_bytes(buf.shape))
        for k in ("D", "dQ"):
            assert np.array_equal(ch[k], got[k]), f"{name}: chunked {k} differs from the split backward"
        for k in ("dK", "dVt"):
            assert rel_l2(ch[k], got[k]) <= 1e-5, f"{name}: chunked {k} differs from the split backward"
