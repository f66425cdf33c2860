"""GPU parity of the backward that stores dQ, dK and dV straight into a fused
QKV projection's token-major gradient (sa_backward_projection): the binary32
slices equal the split path's dQ, dK, dV bitwise (same arithmetic), the
bfloat16 copies equal torch's own bfloat16 conversion of them bit for bit, the slices
match the oracle's layout of its own gradients, columns outside the slices are
untouched, and padded rows are zero."""
import numpy as np
import pytest
import torch

import causal_streaming_attention_amd as sa
import oracle
from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate, make_inputs
from parity_util import C, check_grad, run_gpu, say

pytestmark = pytest.mark.gpu

SENT32 = -7.25
SENT16 = 0x3FC0      # bfloat16 1.5
EXTRA = 16           # columns past the three slices, never written


def _torch_bf16(x32):
    """torch's own float32 -> bfloat16 conversion (round to nearest even), as raw bits."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _projection(buf, H, KV, two_pass=False):
    B, T = buf.B, buf.T
    width = 64 * (H + 2 * KV) + EXTRA
    g32 = torch.full((B, T, width), SENT32, dtype=torch.float32, device="cuda")
    g16 = torch.full((B, T, width), SENT16, dtype=torch.int16, device="cuda")
    qc, kc, vc = 0, 64 * H, 64 * (H + KV)
    p32, p16 = g32.data_ptr(), g16.data_ptr()
    slices = (p32 + 4 * qc, p16 + 2 * qc, p32 + 4 * kc, p16 + 2 * kc, p32 + 4 * vc, p16 + 2 * vc)
    if two_pass:
        sa.sa_backward_two_pass_projection(buf.shape, buf.dO, buf.O, buf.L, buf.D, buf.Q, buf.K, buf.Vt, C, SCALE,
                                           *slices, width)
    else:
        sa.sa_backward_projection(buf.shape, buf.dO, buf.O, buf.L, buf.D, buf.dS, buf.ws_bytes, buf.Q, buf.K,
                                  buf.Vt, C, SCALE, *slices, width)
    torch.cuda.synchronize()
    return g32.cpu().numpy(), g16.cpu().numpy().view(np.uint16), width, (qc, kc, vc)


CASES = [
    # name, B, T, H, KV, causal, seqlens
    ("mha_t128_causal", 1, 128, 2, 2, True, None),
    ("gqa2_t320_causal", 2, 320, 4, 2, True, None),
    ("varlen_gqa2_full_b3_t256", 3, 256, 4, 2, False, [256, 77, 0]),
    ("varlen_causal_b2_t192", 2, 192, 2, 1, True, [130, 191]),
]


def _check(x, causal, H, KV, name, with_oracle=True):
    buf, got = run_gpu(x, causal)                       # the split path: dQ, dK, dVt planes
    g32, g16, width, (qc, kc, vc) = _projection(buf, H, KV)
    # the same values, laid out, bitwise
    want32 = oracle.projection_slices(got["dQ"], got["dK"], got["dVt"], width, qc, kc, vc).astype(np.float32)
    used = slice(0, vc + 64 * KV)
    assert np.array_equal(g32[:, :, used], want32[:, :, used]), f"{name}: binary32 slices differ from the planes"
    assert np.array_equal(g16[:, :, used], _torch_bf16(g32[:, :, used])), f"{name}: bfloat16 copies not RNE"
    assert np.all(g32[:, :, vc + 64 * KV:] == SENT32) and np.all(g16[:, :, vc + 64 * KV:] == SENT16), \
        f"{name}: columns past the slices were written"
    if x["seqlens"] is not None:
        for b, n in enumerate(x["seqlens"]):
            assert np.all(g32[b, n:, used] == 0.0), f"{name}: padded rows not zero"
    if with_oracle:
        ref = oracle.backward(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=causal, seqlens=x["seqlens"])
        want = oracle.projection_slices(ref["dQ"], ref["dK"], ref["dVt"], width, qc, kc, vc)
        for nm, sl in (("dQ", slice(qc, kc)), ("dK", slice(kc, vc)), ("dV", slice(vc, vc + 64 * KV))):
            check_grad(nm, g32[:, :, sl].astype(np.float64), want[:, :, sl], name)


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", CASES, ids=[c[0] for c in CASES])
def test_projection_small(name, B, T, H, KV, causal, seqlens):
    say(f"case projection {name}")
    _check(make_inputs(B, T, H, KV, seed=400 + T + H, seqlens=seqlens), causal, H, KV, name)


def test_projection_causal_gqa_t4096_workload():
    w = WORKLOADS["causal_gqa_t4096"]
    say(f"case projection {w.name}")
    _check(generate(w), w.causal, w.heads, w.kv_heads, w.name, with_oracle=False)


def test_projection_v_rows_matches_v_transposed():
    """With V passed as rows, the key pass loads V's rows directly; the slices are bitwise the V^T path's."""
    say("case projection v_rows")
    B, T, H, KV = 2, 256, 4, 2
    x = make_inputs(B, T, H, KV, seed=451, seqlens=[256, 130])
    outs = []
    for v_rows in (False, True):
        buf, _ = run_gpu(x, True, v_rows=v_rows)
        g32, g16, _, _ = _projection(buf, H, KV)
        outs.append((g32, g16))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", CASES, ids=[c[0] for c in CASES])
def test_two_pass_projection_small(name, B, T, H, KV, causal, seqlens):
    """The two-launch backward's projection variant: bitwise the two-launch planes, RNE copies, untouched
    columns, zero padding."""
    say(f"case two-pass projection {name}")
    x = make_inputs(B, T, H, KV, seed=500 + T + H, seqlens=seqlens)
    buf, got = run_gpu(x, causal, path="two_pass")
    g32, g16, width, (qc, kc, vc) = _projection(buf, H, KV, two_pass=True)
    want32 = oracle.projection_slices(got["dQ"], got["dK"], got["dVt"], width, qc, kc, vc).astype(np.float32)
    used = slice(0, vc + 64 * KV)
    assert np.array_equal(g32[:, :, used], want32[:, :, used]), f"{name}: binary32 slices differ from the planes"
    assert np.array_equal(g16[:, :, used], _torch_bf16(g32[:, :, used])), f"{name}: bfloat16 copies not RNE"
    assert np.all(g32[:, :, vc + 64 * KV:] == SENT32) and np.all(g16[:, :, vc + 64 * KV:] == SENT16)
    if seqlens is not None:
        for b, n in enumerate(seqlens):
            assert np.all(g32[b, n:, used] == 0.0), f"{name}: padded rows not zero"


def test_projection_and_rotated_outputs_equal_across_block_orders():
    """Block order 1 (one tile per block, plain order) gives the same bits as the paired, XCD-grouped order."""
    say("case projection block orders")
    B, T, H, KV = 1, 512, 8, 2
    x = make_inputs(B, T, H, KV, seed=470)
    theta = np.random.default_rng(471).uniform(-np.pi, np.pi, size=(T, 32))
    cos_t = torch.from_numpy(np.cos(theta).astype(np.float32)).cuda()
    sin_t = torch.from_numpy(np.sin(theta).astype(np.float32)).cuda()
    outs = []
    for order in (0, 1):
        buf, _ = run_gpu(x, True, block_order=order)
        g32, g16, width, _ = _projection(buf, H, KV)
        rot = torch.zeros((B, T, width), dtype=torch.int16, device="cuda")
        sa.sa_dq_pass_rotated(buf.shape, buf.K, buf.dS, buf.ws_bytes, SCALE, cos_t, sin_t, rot, width)
        torch.cuda.synchronize()
        outs.append((g32, g16, rot.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
