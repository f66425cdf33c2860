"""GPU parity of the V-as-rows operand layout (shape v_rows = 1, StreamingAttentionSM86
page, the shared forward with V as rows): V is passed as [B][KV][T][64] like K, the
forward reads P V's operand transposed from the staged V tile, the key pass loads V's
rows as its dP operand, and dV comes back as [B][KV][T][64].

The same values reach the same MFMA lanes in the same order as on the V^T path, so every
output must be bitwise identical to that path's (dV transposed); the small cases are also
checked against the binary64 oracle."""
import numpy as np
import pytest

from causal_streaming_attention_amd.workloads import WORKLOADS, generate, make_inputs
from parity_util import check_forward, check_grad, full_reference, run_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, T, H, KV, causal, seqlens
    ("gqa2_t320_causal_odd_tiles", 2, 320, 4, 2, True, None),
    ("mha_t128_full", 1, 128, 2, 2, False, None),
    ("varlen_causal_b4_t192", 4, 192, 4, 2, True, [65, 64, 130, 191]),
    ("varlen_gqa4_full_b2_t384", 2, 384, 4, 1, False, [383, 97]),
]


def _same(rows, cols, where):
    for k in cols:
        assert np.array_equal(rows[k], cols[k], equal_nan=True), f"{where}: {k} differs from the V^T path"


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", CASES, ids=[c[0] for c in CASES])
def test_v_rows_small(name, B, T, H, KV, causal, seqlens):
    say(f"case v_rows {name}")
    x = make_inputs(B, T, H, KV, seed=300 + T + H, seqlens=seqlens)
    buf_r, rows = run_gpu(x, causal, v_rows=True)
    buf_c, cols = run_gpu(x, causal)
    _same(rows, cols, name)
    if seqlens is None:
        # (with lengths, tiles past a sequence's end are neither written nor read)
        assert bool((buf_r.dS == buf_c.dS).all()), f"{name}: dS workspace differs"
    ref = full_reference(x, causal)
    check_forward(rows["O"], rows["L"], ref["O"], ref["L"], name)
    for k in ("dQ", "dK", "dVt"):
        check_grad(k, rows[k], ref[k], name)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_v_rows_structured_scores_bitwise(causal):
    """The rising and stepped score recipes (the forward's exponent maximum moves tile after tile, or on
    lane sums of P): the V-rows instantiation takes the same growth steps, bit for bit."""
    from test_gpu_parity import _structured_scores
    for name, x in (("rising", _structured_scores(512, 2, [0.0] * 8, seed=901, slope=6.0 / 64.0, noise=0.3)),
                    ("stepped", _structured_scores(256, 2, [0.0, 4.0, 6.0, 9.5], seed=902))):
        say(f"case v_rows {name}_scores causal={causal}")
        _, rows = run_gpu(x, causal, v_rows=True)
        _, cols = run_gpu(x, causal)
        _same(rows, cols, f"{name}_scores_{causal}")


def test_v_rows_causal_gqa_t4096_bitwise():
    """The benchmark's shape and launch configuration (its V^T path is parity-tested
    against the oracle in the workload tests)."""
    w = WORKLOADS["causal_gqa_t4096"]
    say(f"case v_rows {w.name}")
    x = generate(w)
    _, rows = run_gpu(x, w.causal, v_rows=True)
    _, cols = run_gpu(x, w.causal)
    _same(rows, cols, w.name)


def test_v_rows_padding_garbage_does_not_leak():
    say("case v_rows padding-garbage")
    lens = [100, 37, 192]
    x = make_inputs(3, 192, 4, 2, seed=323, seqlens=lens)
    for causal in (False, True):
        _, clean = run_gpu(x, causal, v_rows=True)
        dirty = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        rng = np.random.default_rng(1)
        for b, n in enumerate(lens):
            for k in ("Q", "K", "dO"):
                pad = dirty[k][b, :, n:]
                pad[...] = rng.choice([-65504.0, 65504.0], size=pad.shape).astype(np.float16)
            pad = dirty["Vt"][b, :, :, n:]   # V's padded rows, once transposed to rows
            pad[...] = rng.choice([-65504.0, 65504.0], size=pad.shape).astype(np.float16)
        _, got = run_gpu(dirty, causal, v_rows=True)
        for k in clean:
            assert np.array_equal(clean[k], got[k]), (causal, k)


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", CASES, ids=[c[0] for c in CASES])
def test_v_rows_two_pass_backward(name, B, T, H, KV, causal, seqlens):
    """The two-launch backward (query pass + key pass without dS) with V as rows."""
    say(f"case v_rows two-pass {name}")
    x = make_inputs(B, T, H, KV, seed=400 + T + H, seqlens=seqlens)
    _, rows = run_gpu(x, causal, path="two_pass", v_rows=True)
    _, cols = run_gpu(x, causal, path="two_pass")
    _same(rows, cols, name)
    ref = full_reference(x, causal)
    for k in ("dQ", "dK", "dVt"):
        check_grad(k, rows[k], ref[k], name)
