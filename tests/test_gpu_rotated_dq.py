"""GPU parity of the dQ pass's rotated epilogue (sa_dq_pass_rotated): dQ turned
back by the inverse half-split rotation and stored as the bfloat16 Q slice of a
token-major projection gradient.  Checked against the oracle (the relative L2
bar of dQ), against the library's own fp32 dQ rotated in binary64 (within one
bfloat16 ulp, which pins the epilogue's layout, signs and rounding), for
untouched columns outside the Q slice and for zero padded rows."""
import numpy as np
import pytest
import torch

import causal_streaming_attention_amd as sa
import oracle
from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate, make_inputs
from parity_util import check_grad, run_gpu, sample_rows, say

pytestmark = pytest.mark.gpu

SENTINEL = 0x3FC0  # bfloat16 1.5, left in every column the pass must not write


def _tables(T, seed):
    theta = np.random.default_rng(seed).uniform(-np.pi, np.pi, size=(T, 32))
    return np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)


def _bf16_to_f64(bits_u16):
    return (bits_u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _run_rotated(buf, cos, sin, width):
    dqkv = torch.full((buf.B, buf.T, width), SENTINEL, dtype=torch.int16, device="cuda")
    ct, st = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    sa.sa_dq_pass_rotated(buf.shape, buf.K, buf.dS, buf.ws_bytes, SCALE, ct, st, dqkv, width)
    torch.cuda.synchronize()
    return dqkv.cpu().numpy().view(np.uint16)


def _check_epilogue(bits, dq_gpu, cos, sin, width, H, where):
    """Against the library's fp32 dQ rotated in binary64: within one bfloat16 ulp of the result, plus
    the binary32 rounding of the two products, which dominates where they nearly cancel."""
    c64, s64 = cos.astype(np.float64), sin.astype(np.float64)
    want = oracle.rotated_dq_slice(dq_gpu, c64, s64, width)[:, :, :64 * H]
    a = np.abs(dq_gpu)
    mag = oracle.rotated_dq_slice(np.concatenate([a[..., :32], a[..., 32:]], axis=-1), np.abs(c64), np.abs(s64),
                                  width)[:, :, :64 * H]
    mag2 = oracle.rotated_dq_slice(np.concatenate([a[..., 32:], a[..., :32]], axis=-1), np.abs(c64), np.abs(s64),
                                   width)[:, :, :64 * H]
    # mag: |x1| |cos| + |x2| |sin| in the first 32 columns of each head; mag2 the same with x1 and x2
    # swapped, i.e. |x2| |cos| + |x1| |sin|, in the first 32, which is the second half's magnitude
    B, T = want.shape[:2]
    m = mag.reshape(B, T, H, 64)
    m2 = mag2.reshape(B, T, H, 64)
    bound_mag = np.concatenate([m[..., :32], m2[..., :32]], axis=-1).reshape(B, T, 64 * H)
    got = _bf16_to_f64(bits)
    q = got[:, :, :64 * H]
    tol = np.abs(want) * 2.0 ** -7 + bound_mag * 2.0 ** -20
    bad = np.abs(q - want) > tol
    assert not bad.any(), f"{where}: {int(bad.sum())} values beyond one bfloat16 ulp of the rotated fp32 dQ"
    assert np.all(bits[:, :, 64 * H:] == SENTINEL), f"{where}: columns outside the Q slice were written"
    return got


CASES = [
    # name, B, T, H, KV, causal, seqlens, extra columns past the Q slice
    ("mha_t128_causal", 1, 128, 2, 2, True, None, 0),
    ("gqa2_t320_causal_qkv_width", 2, 320, 4, 2, True, None, 2 * 2 * 64),
    ("varlen_gqa2_full_b3_t256", 3, 256, 4, 2, False, [256, 77, 0], 64),
    ("varlen_causal_b2_t192", 2, 192, 2, 1, True, [130, 191], 8),
]


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens,extra", CASES, ids=[c[0] for c in CASES])
def test_rotated_dq_small(name, B, T, H, KV, causal, seqlens, extra):
    say(f"case rotated {name}")
    x = make_inputs(B, T, H, KV, seed=200 + T + H, seqlens=seqlens)
    cos, sin = _tables(T, 300 + T)
    width = 64 * H + extra
    buf, got = run_gpu(x, causal)
    bits = _run_rotated(buf, cos, sin, width)
    rot = _check_epilogue(bits, got["dQ"], cos, sin, width, H, name)
    ref = oracle.backward(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=causal, seqlens=x["seqlens"])
    want = oracle.rotated_dq_slice(ref["dQ"], cos.astype(np.float64), sin.astype(np.float64), width)
    check_grad("rotated dQ", rot[:, :, :64 * H], want[:, :, :64 * H], name)
    if seqlens is not None:
        for b, n in enumerate(seqlens):
            assert np.all(rot[b, n:, :64 * H] == 0.0), f"{name}: padded rows not zero"


def test_rotated_dq_causal_gqa_t4096_workload():
    w = WORKLOADS["causal_gqa_t4096"]
    say(f"case rotated {w.name}")
    x = generate(w)
    cos, sin = _tables(w.T, 7)
    width = (w.heads + 2 * w.kv_heads) * 64    # a fused QKV projection's width
    buf, got = run_gpu(x, w.causal)
    bits = _run_rotated(buf, cos, sin, width)
    rot = _check_epilogue(bits, got["dQ"], cos, sin, width, w.heads, w.name)
    rows = sample_rows(w.batch, w.heads, w.T, 192, seed=w.seed)
    say(f"case rotated {w.name}: oracle rows {rows.size}")
    _, dQ, _, _ = oracle.backward_rows(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=w.causal,
                                       seqlens=x["seqlens"], rows=rows)
    # the sampled rows' dQ, rotated by the oracle, against the same rows of the slice
    h_idx, t_idx = (rows // w.T) % w.heads, rows % w.T
    c64, s64 = cos.astype(np.float64)[t_idx], sin.astype(np.float64)[t_idx]
    want = np.concatenate([dQ[:, :32] * c64 + dQ[:, 32:] * s64, dQ[:, 32:] * c64 - dQ[:, :32] * s64], axis=1)
    gotr = np.stack([rot[0, t, 64 * h:64 * h + 64] for h, t in zip(h_idx, t_idx)])
    check_grad("rotated dQ (sampled rows)", gotr, want, w.name)
