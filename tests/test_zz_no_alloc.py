"""The backward that allocates nothing (sa_backward_static): its dS workspace is
the library's static device array, taken in query-row chunks when the problem's
dS is larger.  Called through the C ABI on three problems in a row, each smaller
than the one before: the benchmark's workload (545 MB of dS, chunked) matches
sa_backward_ex (D and dQ bitwise, dK and dV within rounding); the two that fit
whole give exactly sa_backward_ex's bits, and the smallest also matches the
oracle.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import causal_streaming_attention_amd as sa
from causal_streaming_attention_amd.workloads import SCALE, make_inputs
from parity_util import C, check_forward, check_grad, full_reference, rel_l2, run_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # B, T, H, KV, causal, seqlens: 545 MB of dS (chunked), then 34.6 MB, then 0.8 MB
    (1, 4096, 32, 8, True, None),
    (1, 2048, 8, 2, True, None),
    (3, 256, 4, 2, False, [256, 77, 0]),
]


def _static_backward(buf):
    f32 = torch.float32
    out = {"D": torch.full_like(buf.D, -3.0), "dQ": torch.full_like(buf.dQ, -3.0),
           "dK": torch.full_like(buf.dK, -3.0), "dVt": torch.full_like(buf.dVt, -3.0)}
    assert all(t.dtype == f32 for t in out.values())
    sa.sa_backward_static(buf.shape, buf.dO, buf.O, buf.L, out["D"], buf.Q, buf.K, buf.Vt, C, SCALE, out["dQ"],
                          out["dK"], out["dVt"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


def test_static_scratch_backward_two_calls_in_a_row():
    assert sa.SA_STATIC_SCRATCH_BYTES == 64 << 20
    for i, (B, T, H, KV, causal, seqlens) in enumerate(CASES):
        say(f"case static-scratch backward call {i}: B={B} T={T} H={H} KV={KV} causal={causal}")
        x = make_inputs(B, T, H, KV, seed=700 + i, seqlens=seqlens)
        buf, want = run_gpu(x, causal)          # forward + sa_backward_ex with its own workspace
        got = _static_backward(buf)
        if buf.ws_bytes > sa.SA_STATIC_SCRATCH_BYTES:
            for k in ("D", "dQ"):
                assert np.array_equal(got[k], want[k]), f"call {i}: {k} differs from sa_backward_ex"
            for k in ("dK", "dVt"):
                e = rel_l2(got[k], want[k])
                assert e <= 1e-5, f"call {i}: {k} rel L2 {e:.2e} from sa_backward_ex"
        else:
            for k in ("D", "dQ", "dK", "dVt"):
                assert np.array_equal(got[k], want[k]), f"call {i}: {k} differs from sa_backward_ex"
        if i == len(CASES) - 1:
            ref = full_reference(x, causal)
            check_forward(want["O"], want["L"], ref["O"], ref["L"], "static scratch")
            for k in ("dQ", "dK", "dVt"):
                check_grad(k, got[k], ref[k], "static scratch")


def test_static_scratch_refuses_a_problem_beyond_its_size():
    """T = 16384 with 32 heads needs 134 MB of dS for a single 128-row block: refused before any launch,
    outputs untouched."""
    say("case static-scratch too large")
    T, H, KV = 16384, 32, 8
    shape = sa.make_shape(1, T, H, KV, True)
    assert sa.sa_backward_chunked_min_bytes(shape) > sa.SA_STATIC_SCRATCH_BYTES
    f16, f32 = torch.float16, torch.float32
    t = lambda *s, d=f16: torch.zeros(*s, dtype=d, device="cuda")
    dQ = torch.full((1, H, T, 64), 5.0, dtype=f32, device="cuda")
    with pytest.raises(sa.SaError) as e:
        sa.sa_backward_static(shape, t(1, H, T, 64), t(1, T, H * 64), t(1, H, T, d=f32), t(1, H, T, d=f32),
                              t(1, H, T, 64), t(1, KV, T, 64), t(1, KV, 64, T), C, SCALE, dQ,
                              t(1, KV, T, 64, d=f32), t(1, KV, 64, T, d=f32))
    assert e.value.status == sa.SA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool(torch.all(dQ == 5.0))


def test_static_scratch_backward_under_hip_graph_capture():
    """The case it is for: captured into a HIP graph (no allocation inside the capture), replayed five
    times with eager work and host synchronisations between replays, every replay bitwise equal to the
    eager call."""
    say("case static-scratch backward in a HIP graph")
    B, T, H, KV = 1, 1024, 8, 2
    x = make_inputs(B, T, H, KV, seed=710)
    buf, _ = run_gpu(x, True)
    outs = {k: torch.empty_like(getattr(buf, k)) for k in ("D", "dQ", "dK", "dVt")}

    def call():
        sa.sa_backward_static(buf.shape, buf.dO, buf.O, buf.L, outs["D"], buf.Q, buf.K, buf.Vt, C, SCALE,
                              outs["dQ"], outs["dK"], outs["dVt"])

    call()                                   # eager, first call on this device outside the capture
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.synchronize()
    for r in range(5):
        for v in outs.values():
            v.fill_(float(r + 7))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], want[k]), f"replay {r}: {k} differs from the eager call"
