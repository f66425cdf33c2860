"""GPU parity of the two-launch backward (query pass for D and dQ, then the
key pass without a dS store), through the C ABI, against the binary64
oracle: the same tolerances, cases and invariants as the three-launch path.
Every test here needs an MI355X."""
import numpy as np
import pytest

from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate, make_inputs
from parity_util import (check_forward, check_grad, check_long_context, check_workload_full, full_reference,
                         rel_l2, run_gpu, say)
from test_gpu_parity import SMALL, _gradient_sums, _structured_scores

pytestmark = pytest.mark.gpu
PATH = "two_pass"


def _check_all(inputs, causal, where):
    _, got = run_gpu(inputs, causal, path=PATH)
    ref = full_reference(inputs, causal)
    check_forward(got["O"], got["L"], ref["O"], ref["L"], where)
    errs = {k: check_grad(k, got[k], ref[k], where) for k in ("dQ", "dK", "dVt")}
    if inputs["seqlens"] is not None:
        for b, n in enumerate(inputs["seqlens"]):
            assert np.all(got["D"][b, :, n:] == 0) and np.all(got["dQ"][b, :, n:] == 0), where
            assert np.all(got["dK"][b, :, n:] == 0) and np.all(got["dVt"][b, :, :, n:] == 0), where
    assert rel_l2(got["D"], ref["D"]) <= 1e-2, where
    say(f"{where} (two-pass): dQ {errs['dQ']:.2e} dK {errs['dK']:.2e} dV {errs['dVt']:.2e}")
    return got


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", SMALL, ids=[c[0] for c in SMALL])
def test_two_pass_small_full_parity(name, B, T, H, KV, causal, seqlens):
    say(f"case two-pass {name}")
    x = make_inputs(B, T, H, KV, seed=100 + T + H, seqlens=seqlens)
    _check_all(x, causal, name)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_two_pass_structured_scores(causal):
    """The split path's rising and stepped score recipes (the forward's exponent maximum moves tile after
    tile, or on lane sums of P): the query pass recomputes P from the forward's L on these rows too."""
    for name, x in (("rising", _structured_scores(512, 2, [0.0] * 8, seed=901, slope=6.0 / 64.0, noise=0.3)),
                    ("stepped", _structured_scores(256, 2, [0.0, 4.0, 6.0, 9.5], seed=902))):
        say(f"case {name}_scores two-pass causal={causal}")
        _check_all(x, causal, f"{name}_scores_{causal}")


def test_two_pass_causal_mha_t1024_workload():
    w = WORKLOADS["causal_mha_t1024"]
    say(f"case two-pass {w.name}")
    _check_all(generate(w), w.causal, w.name)


@pytest.mark.timeout(900)
def test_two_pass_causal_gqa_t4096_workload_full():
    w = WORKLOADS["causal_gqa_t4096"]
    x = generate(w)
    say(f"case two-pass {w.name}: gpu")
    _, got = run_gpu(x, w.causal, path=PATH)
    check_workload_full(w, x, got, f"{w.name} two-pass")
    _gradient_sums(x, got, w)


@pytest.mark.timeout(900)
def test_two_pass_varlen_b16_t2048_workload_full():
    w = WORKLOADS["varlen_b16_t2048"]
    x = generate(w)
    say(f"case two-pass {w.name}: gpu")
    _, got = run_gpu(x, w.causal, path=PATH)
    check_workload_full(w, x, got, f"{w.name} two-pass")
    _gradient_sums(x, got, w)


@pytest.mark.timeout(900)
def test_two_pass_long_causal_gqa_t16384_workload():
    """The two-launch backward exists to give long context O(T) memory: at T = 16384 with boosted keys,
    the same rows and whole-sequence key columns as the split path's test."""
    w = WORKLOADS["long_causal_gqa_t16384"]
    x = generate(w)
    say(f"case two-pass {w.name}: gpu")
    _, got = run_gpu(x, w.causal, path=PATH)
    check_long_context(w, x, got, f"{w.name} two-pass")
    _gradient_sums(x, got, w)


def test_two_pass_agrees_with_the_split_backward():
    """Both paths compute the same gradients; they differ only in rounding."""
    w = WORKLOADS["causal_gqa_t4096"]
    say("case two-pass vs split")
    x = generate(w)
    _, a = run_gpu(x, True, path="split")
    _, b = run_gpu(x, True, path=PATH)
    for k in ("dQ", "dK", "dVt"):
        e = rel_l2(b[k], a[k])
        say(f"  {k}: rel L2 {e:.2e}")
        assert e <= 1e-2, k
    assert rel_l2(b["D"], a["D"]) <= 1e-5


def test_two_pass_determinism_and_block_order():
    w = WORKLOADS["causal_gqa_t4096"]
    say("case two-pass determinism")
    x = generate(w)
    _, a = run_gpu(x, True, block_order=0, path=PATH)
    _, b = run_gpu(x, True, block_order=0, path=PATH)
    _, c = run_gpu(x, True, block_order=1, path=PATH)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), f"{k} differs between repeats"
        assert np.array_equal(a[k], c[k], equal_nan=True), f"{k} differs between block orders"


def test_two_pass_padding_garbage_does_not_leak():
    say("case two-pass padding-garbage")
    lens = [100, 37, 192]
    x = make_inputs(3, 192, 4, 2, seed=23, seqlens=lens)
    for causal in (False, True):
        _, clean = run_gpu(x, causal, path=PATH)
        dirty = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        rng = np.random.default_rng(1)
        for b, n in enumerate(lens):
            for k in ("Q", "K", "dO"):
                pad = dirty[k][b, :, n:]
                pad[...] = rng.choice([-65504.0, 65504.0], size=pad.shape).astype(np.float16)
            pad = dirty["Vt"][b, :, :, n:]
            pad[...] = rng.choice([-65504.0, 65504.0], size=pad.shape).astype(np.float16)
        _, got = run_gpu(dirty, causal, path=PATH)
        for k in clean:
            assert np.array_equal(clean[k], got[k]), (causal, k)


def test_two_pass_row_terms_from_the_forward_output():
    """The query pass's D is rowsum(dO * O) of the forward's own fp16 O."""
    say("case two-pass row-terms")
    x = make_inputs(2, 256, 4, 4, seed=24, seqlens=[256, 77])
    buf, got = run_gpu(x, True, path=PATH)
    O16 = buf.O.view(2, 256, 4, 64).permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64)
    want = np.sum(x["dO"].astype(np.float64) * O16, axis=-1)
    want[1, :, 77:] = 0.0
    assert np.max(np.abs(got["D"] - want)) <= 1e-5 * max(1.0, np.max(np.abs(want)))
