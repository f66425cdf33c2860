"""GPU parity: the HIP path (through the C ABI) against the binary64 oracle.

Small problems compare every output; the five named workloads run at their
full sizes in the launch configuration the benchmark times.  Up to the
variable-length batch every output row and key column is compared; the
long-context workload compares 1024 sampled rows and the whole sequence of
two K/V heads' dK / dV columns, plus properties that hold at any size.  Also: bitwise determinism across repeats and block orders, grouped
heads against repeated heads, variable length against per-sequence runs, and
padding that holds garbage."""
import numpy as np
import pytest

import oracle
from causal_streaming_attention_amd.workloads import SCALE, WORKLOADS, generate, make_inputs
from parity_util import (check_forward, check_grad, check_long_context, check_workload_full, full_reference,
                         rel_l2, run_gpu, sample_cols, sample_rows, say)

pytestmark = pytest.mark.gpu


def _check_all(inputs, causal, where, block_order=0):
    _, got = run_gpu(inputs, causal, block_order=block_order)
    ref = full_reference(inputs, causal)
    check_forward(got["O"], got["L"], ref["O"], ref["L"], where)
    errs = {k: check_grad(k, got[k], ref[k], where) for k in ("dQ", "dK", "dVt")}
    # padded rows / keys are exact zeros
    if inputs["seqlens"] is not None:
        for b, n in enumerate(inputs["seqlens"]):
            assert np.all(got["D"][b, :, n:] == 0) and np.all(got["dQ"][b, :, n:] == 0), where
            assert np.all(got["dK"][b, :, n:] == 0) and np.all(got["dVt"][b, :, :, n:] == 0), where
    d_err = rel_l2(got["D"], ref["D"])
    assert d_err <= 1e-2, f"{where}: D rel L2 {d_err:.2e}"
    say(f"{where}: dQ {errs['dQ']:.2e} dK {errs['dK']:.2e} dV {errs['dVt']:.2e}")
    return got


SMALL = [
    # name, B, T, H, KV, causal, seqlens
    ("mha_t128_causal", 1, 128, 1, 1, True, None),
    ("gqa2_t320_causal_odd_tiles", 2, 320, 4, 2, True, None),
    ("gqa2_t320_b4_causal_xcd_groups", 4, 320, 4, 2, True, None),
    ("gqa3_t192_causal", 1, 192, 6, 2, True, None),
    ("gqa8_t256_causal", 1, 256, 8, 1, True, None),
    ("mha_t128_full", 1, 128, 2, 2, False, None),
    ("varlen_full_b3_t256", 3, 256, 2, 2, False, [0, 1, 200]),
    ("varlen_causal_b4_t192", 4, 192, 4, 2, True, [65, 64, 130, 191]),
    ("varlen_gqa4_full_b2_t384", 2, 384, 4, 1, False, [383, 97]),
    # edge cases: a single 64-key tile, lengths inside it and of zero, every
    # sequence empty, and 16 query heads per K/V head (each wave slot walks
    # four heads in turn)
    ("single_tile_t64_causal", 2, 64, 2, 1, True, None),
    ("single_tile_t64_varlen_full", 3, 64, 2, 2, False, [0, 17, 64]),
    ("all_empty_varlen_causal", 2, 128, 2, 1, True, [0, 0]),
    ("gqa16_t128_causal", 1, 128, 16, 1, True, None),
    # grids too small for the chip: groups of one or two heads walk their
    # sub-tiles in interleaved phases (4 / G wave pairs per head)
    ("gqa2_t768_causal_split_walk", 1, 768, 2, 1, True, None),
    ("mha_t512_b2_full_split_walk", 2, 512, 3, 3, False, None),
    ("varlen_mha_t640_causal_split_walk", 2, 640, 2, 2, True, [640, 201]),
]


@pytest.mark.parametrize("name,B,T,H,KV,causal,seqlens", SMALL, ids=[c[0] for c in SMALL])
def test_small_full_parity(name, B, T, H, KV, causal, seqlens):
    say(f"case {name}")
    x = make_inputs(B, T, H, KV, seed=100 + T + H, seqlens=seqlens)
    _check_all(x, causal, name)


def _structured_scores(T, H, tile_offsets, seed, slope=0.0, noise=0.1):
    """Q rows along one +-1 direction u, K row j = g_j u, both plus Gaussian noise, so that the base-2
    score of key j is close to the same g_j c |u|^2 for every query: tile k's keys sit tile_offsets[k]
    above tile 0's, and `slope` adds a rise per key.  The noise keeps the softmax from collapsing onto
    one key, where dP - D cancels and the fp16 O inside D (the pages' reading) alone would cost dQ
    about 1% relative L2; with these settings that share stays under 0.4% in binary64 estimates."""
    rng = np.random.default_rng(seed)
    c = SCALE / np.log(2.0)
    u = rng.choice([-1.0, 1.0], size=64)
    g = np.array([0.5 + (tile_offsets[j // 64] + slope * j) / (c * 64.0) for j in range(T)])
    Q = (u[None, None, :] + noise * rng.standard_normal((1, H, T, 64))).astype(np.float16)
    K = (g[None, None, :, None] * u[None, None, None, :]
         + noise * rng.standard_normal((1, 1, T, 64))).astype(np.float16)
    V = rng.standard_normal((1, 1, T, 64)).astype(np.float16)
    dO = rng.standard_normal((1, H, T, 64)).astype(np.float16)
    return {"Q": Q, "K": K, "Vt": np.ascontiguousarray(V.transpose(0, 1, 3, 2)), "dO": dO, "seqlens": None}


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_scores_rising_tile_after_tile(causal):
    """Base-2 scores rising by about 6 per 64-key tile: under the old maximum a lane's 32 P of a new tile
    sum past 2^8 on most tiles, so the exponents' maximum moves and O and l are rescaled tile after tile."""
    say(f"case rising_scores causal={causal}")
    x = _structured_scores(512, 2, [0.0] * 8, seed=901, slope=6.0 / 64.0, noise=0.3)
    _check_all(x, causal, f"rising_scores_{causal}")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_scores_stepping_up_by_less_than_eight(causal):
    """Whole tiles 4, then 2 more, then 3.5 more above the first: no single P exceeds 2^8 under the old
    maximum, but 32 keys of 2^4 (or 2^3.5) sum past 2^8 in a lane and move it, while 32 of 2^2 do not."""
    say(f"case stepped_scores causal={causal}")
    x = _structured_scores(256, 2, [0.0, 4.0, 6.0, 9.5], seed=902)
    _check_all(x, causal, f"stepped_scores_{causal}")


def test_tiny_causal_t128_workload():
    w = WORKLOADS["tiny_causal_t128"]
    say(f"case {w.name}")
    _check_all(generate(w), w.causal, w.name)


def test_causal_mha_t1024_workload():
    w = WORKLOADS["causal_mha_t1024"]
    say(f"case {w.name}")
    _check_all(generate(w), w.causal, w.name)


def _gradient_sums(x, got, w):
    """sum_j dK_j = 0 and sum_j dV_j = sum of the group's admitted dO rows, at full size."""
    dO = x["dO"].astype(np.float64)
    G = w.heads // w.kv_heads
    lens = x["seqlens"] if x["seqlens"] is not None else [w.T] * w.batch
    for b in range(w.batch):
        n = int(lens[b])
        for kv in range(w.kv_heads):
            want = dO[b, kv * G:(kv + 1) * G, :n].sum(axis=(0, 1))
            got_v = got["dVt"][b, kv].sum(axis=1)
            assert np.max(np.abs(got_v - want)) <= 1e-2 * max(1.0, np.max(np.abs(want))), (b, kv)
            dk = got["dK"][b, kv]          # [T, 64]; sum over keys vanishes up to rounding
            assert np.all(np.abs(dk.sum(axis=0)) <= 1e-2 * np.sqrt(np.sum(dk * dk, axis=0)) + 1e-6), (b, kv)


@pytest.mark.timeout(900)
def test_causal_gqa_t4096_workload_full():
    """The benchmark's workload at full size, in the benchmark's launch configuration: every output row and
    key column against the oracle."""
    w = WORKLOADS["causal_gqa_t4096"]
    x = generate(w)
    say(f"case {w.name}: gpu")
    _, got = run_gpu(x, w.causal)
    check_workload_full(w, x, got, w.name)
    _gradient_sums(x, got, w)


@pytest.mark.timeout(900)
def test_varlen_b16_t2048_workload_full():
    w = WORKLOADS["varlen_b16_t2048"]
    x = generate(w)
    say(f"case {w.name}: gpu")
    _, got = run_gpu(x, w.causal)
    for b, n in enumerate(x["seqlens"]):
        assert np.all(got["O"][b, :, n:] == 0) and np.all(np.isneginf(got["L"][b, :, n:]))
    check_workload_full(w, x, got, w.name)
    _gradient_sums(x, got, w)


@pytest.mark.timeout(900)
def test_long_causal_gqa_t16384_workload():
    """Long context with boosted keys: 1024 sampled rows, and dK / dV over the whole sequence of two K/V
    heads (key tile 0 and every boosted key of the first among them) against the oracle."""
    w = WORKLOADS["long_causal_gqa_t16384"]
    x = generate(w)
    say(f"case {w.name}: gpu")
    _, got = run_gpu(x, w.causal)
    check_long_context(w, x, got, w.name)
    _gradient_sums(x, got, w)


def test_the_pages_calls_batch1_causal():
    """sa_forward and sa_backward, the pages' own argument lists (batch 1, causal), against the oracle on
    the causal_mha_t1024 workload and bitwise against the general entry points, with grouped heads too."""
    import torch
    import causal_streaming_attention_amd as sa
    from parity_util import C
    for name in ("causal_mha_t1024", "causal_gqa_t4096"):
        w = WORKLOADS[name]
        x = generate(w)
        say(f"case pages' calls {w.name}")
        buf, via_ex = run_gpu(x, True)
        T, H, KV = w.T, w.heads, w.kv_heads
        f16, f32 = torch.float16, torch.float32
        O = torch.empty((1, T, H * 64), dtype=f16, device="cuda")
        L = torch.empty((1, H, T), dtype=f32, device="cuda")
        D = torch.empty((1, H, T), dtype=f32, device="cuda")
        dQ = torch.empty((1, H, T, 64), dtype=f32, device="cuda")
        dK = torch.empty((1, KV, T, 64), dtype=f32, device="cuda")
        dVt = torch.empty((1, KV, 64, T), dtype=f32, device="cuda")
        dS = torch.empty(buf.ws_bytes, dtype=torch.uint8, device="cuda")
        sa.sa_forward(buf.Q, buf.K, buf.Vt, O, L, C, T, H, KV)
        sa.sa_backward(buf.dO, O, L, D, dS, buf.ws_bytes, buf.Q, buf.K, buf.Vt, C, SCALE, T, H, KV, dQ, dK, dVt)
        torch.cuda.synchronize()
        got = {"O": O.view(1, T, H, 64).permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64),
               "L": L.cpu().numpy().astype(np.float64), "D": D.cpu().numpy().astype(np.float64),
               "dQ": dQ.cpu().numpy().astype(np.float64), "dK": dK.cpu().numpy().astype(np.float64),
               "dVt": dVt.cpu().numpy().astype(np.float64)}
        for k in got:
            assert np.array_equal(got[k], via_ex[k]), f"{name}: {k} differs from the general entry point"
        if name == "causal_mha_t1024":
            check_workload_full(w, x, got, f"{name} (pages' calls)")


def test_determinism_and_block_order():
    w = WORKLOADS["causal_gqa_t4096"]
    say("case determinism")
    x = generate(w)
    _, a = run_gpu(x, True, block_order=0)
    _, b = run_gpu(x, True, block_order=0)
    _, c = run_gpu(x, True, block_order=1)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), f"{k} differs between repeats"
        assert np.array_equal(a[k], c[k], equal_nan=True), f"{k} differs between block orders"


@pytest.mark.parametrize("B,T,H,KV,causal,seqlens", [
    (1, 1024, 8, 8, True, None),          # the T = 1024 workload's shape: one tile per block, longest first
    (2, 320, 4, 2, True, [320, 77]),
    (3, 256, 2, 2, False, [0, 200, 256]),
])
def test_block_orders_agree_bitwise_on_small_grids(B, T, H, KV, causal, seqlens):
    """Grids small enough to fit the chip at once take one tile per block, longest first; the plain order
    gives the same bits, for the split and the two-launch backward."""
    say(f"case block orders B={B} T={T} H={H} KV={KV} causal={causal}")
    x = make_inputs(B, T, H, KV, seed=40 + T, seqlens=seqlens)
    for path in ("split", "two_pass"):
        _, a = run_gpu(x, causal, block_order=0, path=path)
        _, b = run_gpu(x, causal, block_order=1, path=path)
        for k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), f"{path}: {k} differs between block orders"


@pytest.mark.parametrize("B,T,H,KV", [
    (1, 2112, 32, 8),    # 33 key tiles x 8 K/V heads: 16 pairs and the middle tile alone; 4 wave pairs per group
    (1, 2560, 32, 16),   # 40 key tiles x 16 K/V heads, 2 wave pairs per group
])
def test_key_tile_pairs_against_the_oracle_and_the_plain_order(B, T, H, KV):
    """Where single key tiles need between one and two rounds of the chip, each key-pass workgroup takes key
    tiles p and nkt - 1 - p one after the other: every output against the oracle, and bitwise the plain
    order (one tile per workgroup)."""
    say(f"case key tile pairs B={B} T={T} H={H} KV={KV}")
    x = make_inputs(B, T, H, KV, seed=60 + T)
    got = _check_all(x, True, f"key tile pairs T={T} KV={KV}")
    _, plain = run_gpu(x, True, block_order=1)
    for k in got:
        assert np.array_equal(got[k], plain[k], equal_nan=True), f"{k} differs from the plain order"


def test_grouped_heads_equal_repeated_heads():
    say("case gqa-vs-mha")
    x = make_inputs(1, 256, 8, 2, seed=21)
    G = 4
    xm = dict(x, K=np.repeat(x["K"], G, axis=1), Vt=np.repeat(x["Vt"], G, axis=1))
    _, g = run_gpu(x, True)
    _, m = run_gpu(xm, True)
    for k in ("O", "L", "D", "dQ"):
        assert np.array_equal(g[k], m[k]), k
    for k in ("dK", "dVt"):
        summed = m[k].reshape(1, 2, G, *m[k].shape[2:]).sum(axis=2)
        assert rel_l2(g[k], summed) <= 1e-5, k


def test_varlen_equals_per_sequence_runs():
    say("case varlen-vs-single")
    lens = [130, 64, 1, 250]
    x = make_inputs(4, 256, 4, 2, seed=22, seqlens=lens)
    for causal in (False, True):
        _, got = run_gpu(x, causal)
        for b, n in enumerate(lens):
            Tp = ((n + 63) // 64) * 64
            one = {k: x[k][b:b + 1, :, :Tp] for k in ("Q", "K", "dO")}
            one["Vt"] = x["Vt"][b:b + 1, :, :, :Tp]
            one["seqlens"] = np.array([n], dtype=np.int32)
            _, r = run_gpu(one, causal)
            for k in ("O", "L", "D", "dQ", "dK"):
                assert np.array_equal(got[k][b:b + 1, :, :Tp], r[k]), (causal, b, k)
            assert np.array_equal(got["dVt"][b:b + 1, :, :, :Tp], r["dVt"]), (causal, b)


def test_padding_garbage_does_not_leak():
    say("case padding-garbage")
    lens = [100, 37, 192]
    x = make_inputs(3, 192, 4, 2, seed=23, seqlens=lens)
    for causal in (False, True):
        _, clean = run_gpu(x, causal)
        dirty = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in x.items()}
        rng = np.random.default_rng(0)
        for b, n in enumerate(lens):
            for k in ("Q", "K", "dO"):
                pad = dirty[k][b, :, n:]
                pad[...] = rng.choice([-65504.0, 65504.0], size=pad.shape).astype(np.float16)
            pad = dirty["Vt"][b, :, :, n:]
            pad[...] = rng.choice([-65504.0, 65504.0], size=pad.shape).astype(np.float16)
        _, got = run_gpu(dirty, causal)
        for k in clean:
            assert np.array_equal(clean[k], got[k]), (causal, k)


def test_row_terms_from_the_forward_output():
    """D is rowsum(dO * O) of the forward's own fp16 O, to binary32 accuracy."""
    say("case row-terms")
    x = make_inputs(2, 256, 4, 4, seed=24, seqlens=[256, 77])
    buf, got = run_gpu(x, True)
    O16 = buf.O.view(2, 256, 4, 64).permute(0, 2, 1, 3).float().cpu().numpy().astype(np.float64)
    want = np.sum(x["dO"].astype(np.float64) * O16, axis=-1)
    want[1, :, 77:] = 0.0
    assert np.max(np.abs(got["D"] - want)) <= 1e-5 * max(1.0, np.max(np.abs(want)))


def test_long_sequence_t65536_sampled():
    """T = 65536 with two query heads on one K/V head: the dS workspace alone
    is 8.6 GB, and every in-kernel offset and buffer-resource size is 4x the
    long-context workload's.  Sampled rows (tile edges included) and the last
    1024 key columns against the oracle."""
    T, H, KV = 65536, 2, 1
    say(f"case long_causal_t{T}")
    x = make_inputs(1, T, H, KV, seed=31)
    _, got = run_gpu(x, True)
    rows = sample_rows(1, H, T, 96, seed=31)
    say(f"case long_causal_t{T}: oracle rows {rows.size}")
    D, dQ, O, L = oracle.backward_rows(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=True, seqlens=None,
                                       rows=rows)
    check_forward(got["O"].reshape(-1, 64)[rows], got["L"].reshape(-1)[rows], O, L, "t65536")
    check_grad("dQ", got["dQ"].reshape(-1, 64)[rows], dQ, "t65536")
    assert rel_l2(got["D"].reshape(-1)[rows], D) <= 1e-2
    cols = sample_cols(1, KV, T, 48, seed=32, lo=T - 1024)
    say(f"case long_causal_t{T}: oracle cols {cols.size}")
    dK, dV = oracle.backward_cols(x["Q"], x["K"], x["Vt"], x["dO"], s=SCALE, causal=True, seqlens=None, cols=cols)
    check_grad("dK", got["dK"].reshape(-1, 64)[cols], dK, "t65536")
    check_grad("dV", np.swapaxes(got["dVt"], -1, -2).reshape(-1, 64)[cols], dV, "t65536")
