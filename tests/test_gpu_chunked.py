"""GPU parity of the chunked split backward (sa_backward_chunked): the key and dQ
passes taken in query-row chunks over a dS workspace smaller than the whole
problem's, dK and dV summed across chunks in a fixed order.  Against the oracle
(every output), against the one-chunk backward (D and dQ bitwise: each row's dQ
is the same walk; dK and dV within rounding), bitwise repeatable, and bitwise
the one-chunk backward when the workspace holds the whole dS.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import causal_streaming_attention_amd as sa
from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate, make_inputs
from parity_util import C, check_workload_full, full_reference, check_forward, check_grad, rel_l2, run_gpu, say
from test_gpu_parity import SMALL, _gradient_sums

pytestmark = pytest.mark.gpu


def _chunked(buf, ws_bytes):
    out = {k: torch.full_like(getattr(buf, k), -3.0) for k in ("D", "dQ", "dK", "dVt")}
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    sa.sa_backward_chunked(buf.shape, buf.dO, buf.O, buf.L, out["D"], ws, ws_bytes, buf.Q, buf.K, buf.Vt, C, SCALE,
                           out["dQ"], out["dK"], out["dVt"])
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    if buf.v_rows:
        got["dVt"] = np.ascontiguousarray(got["dVt"].transpose(0, 1, 3, 2))
    return got


def _against_one_chunk(got, one, where):
    assert np.array_equal(got["D"], one["D"]), f"{where}: D differs from the one-chunk backward"
    assert np.array_equal(got["dQ"], one["dQ"]), f"{where}: dQ differs from the one-chunk backward"
    for k in ("dK", "dVt"):
        e = rel_l2(got[k], one[k])
        assert e <= 1e-5, f"{where}: {k} rel L2 {e:.2e} from the one-chunk backward"


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", SMALL, ids=[c[0] for c in SMALL])
def test_chunked_small_with_the_smallest_workspace(name, B, T, H, KV, causal, seqlens):
    """One 128-row block per chunk (the most chunks), against the oracle and the one-chunk backward."""
    say(f"case chunked {name}")
    x = make_inputs(B, T, H, KV, seed=100 + T + H, seqlens=seqlens)
    buf, one = run_gpu(x, causal)
    least = sa.sa_backward_chunked_min_bytes(buf.shape)
    got = _chunked(buf, least)
    ref = full_reference(x, causal)
    for k in ("dQ", "dK", "dVt"):
        check_grad(k, got[k], ref[k], name)
    _against_one_chunk(got, one, name)
    if seqlens is not None:
        for b, n in enumerate(seqlens):
            assert np.all(got["dK"][b, :, n:] == 0) and np.all(got["dVt"][b, :, :, n:] == 0), name
    # a workspace holding the whole dS is one chunk: bitwise the split backward
    whole = _chunked(buf, buf.ws_bytes)
    for k in ("D", "dQ", "dK", "dVt"):
        assert np.array_equal(whole[k], one[k]), f"{name}: {k} with one chunk differs from sa_backward_ex"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mib", [64, 160])
def test_chunked_causal_gqa_t4096_workload(mib):
    """The benchmark's workload with a 64 MiB and a 160 MiB workspace (9 and 4 chunks of its 545 MB of dS):
    every output against the oracle, against the one-chunk backward, and bitwise repeatable."""
    w = WORKLOADS["causal_gqa_t4096"]
    x = generate(w)
    say(f"case chunked {w.name} {mib} MiB")
    buf, one = run_gpu(x, True)
    got = _chunked(buf, mib << 20)
    again = _chunked(buf, mib << 20)
    for k in got:
        assert np.array_equal(got[k], again[k]), f"{k} differs between repeats"
    _against_one_chunk(got, one, f"{w.name} {mib} MiB")
    check_workload_full(w, x, dict(one, **got), f"{w.name} chunked {mib} MiB")
    _gradient_sums(x, dict(one, **got), w)


@pytest.mark.timeout(900)
def test_chunked_varlen_b16_t2048_workload():
    w = WORKLOADS["varlen_b16_t2048"]
    x = generate(w)
    say(f"case chunked {w.name}")
    buf, one = run_gpu(x, w.causal)
    # the full squares of 16 sequences: one 128-row block is 134 MB of dS; two blocks per chunk
    got = _chunked(buf, 2 * sa.sa_backward_chunked_min_bytes(buf.shape))
    _against_one_chunk(got, one, w.name)
    check_workload_full(w, x, dict(one, **got), f"{w.name} chunked")
    _gradient_sums(x, dict(one, **got), w)


def test_chunked_v_rows_matches_v_transposed():
    say("case chunked v_rows")
    B, T, H, KV = 2, 384, 4, 2
    x = make_inputs(B, T, H, KV, seed=451, seqlens=[384, 130])
    outs = []
    for v_rows in (False, True):
        buf, _ = run_gpu(x, True, v_rows=v_rows)
        outs.append(_chunked(buf, sa.sa_backward_chunked_min_bytes(buf.shape)))
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k
