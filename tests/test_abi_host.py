"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every function include/sa.h declares, and rejects bad shapes, pointers,
workspace sizes and scales with the documented status before launching
anything.  Only error paths are called here; no call reaches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

import causal_streaming_attention_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.LIB_PATH):
        from causal_streaming_attention_amd import build
        build.build()
    return sa.native()


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(sa.exported_symbols())


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (sa_\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_plain_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "sa.h"\nint main(void) { sa_shape s = {1, 64, 1, 1, 1, 0, 0, 0};'
                   ' return (int)sa_backward_workspace_bytes(&s) == 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-c", str(src), "-I", os.path.join(ROOT, "include"),
                        "-o", str(tmp_path / "use.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def shape(batch=1, T=128, heads=4, kv=2, causal=1, order=0, seqlens=None, v_rows=0):
    return sa.SaShape(batch, T, heads, kv, causal, seqlens, order, v_rows)


@pytest.mark.parametrize("kw,ok", [
    ({}, True),
    ({"T": 64}, True),
    ({"T": 0}, False),
    ({"T": 96}, False),
    ({"T": 100}, False),
    ({"T": 1 << 21}, False),
    ({"batch": 0}, False),
    ({"heads": 0}, False),
    ({"kv": 0}, False),
    ({"heads": 6, "kv": 4}, False),
    ({"heads": 65536, "kv": 1}, False),
    ({"heads": 32, "kv": 8}, True),
    ({"causal": 2}, False),
    ({"v_rows": 1}, True),
    ({"v_rows": 2}, False),
    ({"v_rows": -1}, False),
    ({"order": 2}, False),
    ({"order": 1}, True),
    ({"batch": 1 << 20, "heads": 32, "kv": 8}, False),
])
def test_admission(lib, kw, ok):
    st = sa.sa_check_shape(shape(**kw))
    assert st == (sa.SA_OK if ok else sa.SA_ERR_SHAPE), sa.sa_status_string(st)


def test_admission_null_and_misaligned_seqlens(lib):
    assert lib.sa_check_shape(None) == sa.SA_ERR_NULL
    assert sa.sa_check_shape(shape(seqlens=0x1002)) == sa.SA_ERR_ALIGN


def test_workspace_bytes(lib):
    nt = 4096 // 64
    assert sa.sa_backward_workspace_bytes(shape(1, 4096, 32, 8, 1)) == 32 * nt * (nt + 1) // 2 * 8192
    assert sa.sa_backward_workspace_bytes(shape(16, 2048, 16, 16, 0)) == 16 * 16 * 32 * 32 * 8192
    assert sa.sa_backward_workspace_bytes(shape(T=96)) == 0


FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails first


def test_forward_rejects_null_misaligned_and_bad_scale(lib):
    s = shape()
    args = [FAKE] * 5
    for i in range(5):
        bad = list(args)
        bad[i] = None
        assert lib.sa_forward_ex(ctypes.byref(s), *bad, 0.18, None) == sa.SA_ERR_NULL
        bad[i] = FAKE + 8
        assert lib.sa_forward_ex(ctypes.byref(s), *bad, 0.18, None) == sa.SA_ERR_ALIGN
    for c in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.sa_forward_ex(ctypes.byref(s), *args, c, None) == sa.SA_ERR_ARGUMENT
    assert lib.sa_forward(*args, 0.18, 96, 4, 2, None) == sa.SA_ERR_SHAPE
    assert lib.sa_forward(None, *args[1:], 0.18, 128, 4, 2, None) == sa.SA_ERR_NULL


def test_backward_rejects_bad_arguments(lib):
    s = shape()
    need = sa.sa_backward_workspace_bytes(s)
    ptrs = [FAKE] * 11   # dO O L D dS Q K Vt dQ dK dVt

    def call(p, ws=need, c=0.18, sc=0.125, sh=s):
        return lib.sa_backward_ex(ctypes.byref(sh), p[0], p[1], p[2], p[3], p[4], ws, p[5], p[6], p[7], c, sc,
                                  p[8], p[9], p[10], None)

    for i in range(11):
        bad = list(ptrs)
        bad[i] = None
        assert call(bad) == sa.SA_ERR_NULL
        bad[i] = FAKE + 4
        assert call(bad) == sa.SA_ERR_ALIGN
    assert call(ptrs, ws=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ptrs, sc=0.0) == sa.SA_ERR_ARGUMENT
    assert call(ptrs, c=float("nan")) == sa.SA_ERR_ARGUMENT
    assert call(ptrs, sh=shape(heads=3, kv=2)) == sa.SA_ERR_SHAPE
    assert lib.sa_backward(*ptrs[:5], need, *ptrs[5:8], 0.18, 0.125, 100, 4, 2, *ptrs[8:], None) == sa.SA_ERR_SHAPE


def test_stage_entry_points_reject_bad_arguments(lib):
    s = shape()
    need = sa.sa_backward_workspace_bytes(s)
    assert lib.sa_row_terms(ctypes.byref(s), FAKE, None, FAKE, None) == sa.SA_ERR_NULL
    assert lib.sa_key_pass(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 2, 0.18, 0.125,
                           FAKE, FAKE, None) == sa.SA_ERR_WORKSPACE
    # dS may be NULL (no store): the workspace size is then not checked, the rest still is
    assert lib.sa_key_pass(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0.18, -0.125,
                           FAKE, FAKE, None) == sa.SA_ERR_ARGUMENT
    assert lib.sa_key_pass(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, 0.18, 0.125,
                           FAKE, FAKE, None) == sa.SA_ERR_NULL
    assert lib.sa_key_pass(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, need, 0.18, 0.125,
                           FAKE, FAKE, None) == sa.SA_ERR_ALIGN
    assert lib.sa_dq_pass(ctypes.byref(s), FAKE, FAKE, need, -0.125, FAKE, None) == sa.SA_ERR_ARGUMENT
    assert lib.sa_dq_pass(ctypes.byref(s), FAKE, FAKE + 1, need, 0.125, FAKE, None) == sa.SA_ERR_ALIGN


def test_two_pass_entry_points_reject_bad_arguments(lib):
    s = shape()
    q_ptrs = [FAKE] * 8   # dO O L Q K Vt D dQ

    def query(p, c=0.18, sc=0.125, sh=s):
        return lib.sa_query_pass(ctypes.byref(sh), p[0], p[1], p[2], p[3], p[4], p[5], c, sc, p[6], p[7], None)

    for i in range(8):
        bad = list(q_ptrs)
        bad[i] = None
        assert query(bad) == sa.SA_ERR_NULL
        bad[i] = FAKE + 2
        assert query(bad) == sa.SA_ERR_ALIGN
    assert query(q_ptrs, c=0.0) == sa.SA_ERR_ARGUMENT
    assert query(q_ptrs, sc=float("inf")) == sa.SA_ERR_ARGUMENT
    assert query(q_ptrs, sh=shape(T=100)) == sa.SA_ERR_SHAPE

    b_ptrs = [FAKE] * 10  # dO O L D Q K Vt dQ dK dVt

    def two_pass(p, c=0.18, sc=0.125, sh=s):
        return lib.sa_backward_two_pass(ctypes.byref(sh), *p[:7], c, sc, *p[7:], None)

    for i in range(10):
        bad = list(b_ptrs)
        bad[i] = None
        assert two_pass(bad) == sa.SA_ERR_NULL
        bad[i] = FAKE + 8
        assert two_pass(bad) == sa.SA_ERR_ALIGN
    assert two_pass(b_ptrs, sc=-1.0) == sa.SA_ERR_ARGUMENT
    assert two_pass(b_ptrs, sh=shape(heads=6, kv=4)) == sa.SA_ERR_SHAPE
    assert lib.sa_backward_two_pass(None, *b_ptrs[:7], 0.18, 0.125, *b_ptrs[7:], None) == sa.SA_ERR_NULL


def test_status_strings(lib):
    for st in range(7):
        assert sa.sa_status_string(st) != "unknown status"
    assert sa.sa_status_string(99) == "unknown status"


def test_base2_scale_is_the_nearest_binary32():
    import struct
    c = sa.base2_scale(0.125)
    assert struct.pack(">f", c).hex() == "3e38aa3b"


def test_rotated_dq_pass_rejects_bad_arguments(lib):
    s = shape()
    need = sa.sa_backward_workspace_bytes(s)
    W = 64 * s.heads

    def call(p, ws=need, sc=0.125, width=W):
        return lib.sa_dq_pass_rotated(ctypes.byref(s), p[0], p[1], ws, sc, p[2], p[3], p[4], width, None)

    ptrs = [FAKE] * 5   # K dS cos sin dqkv
    for i in range(5):
        bad = list(ptrs)
        bad[i] = None
        assert call(bad) == sa.SA_ERR_NULL
        bad[i] = FAKE + 8
        assert call(bad) == sa.SA_ERR_ALIGN
    assert call(ptrs, ws=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ptrs, sc=float("inf")) == sa.SA_ERR_ARGUMENT
    assert call(ptrs, width=W - 8) == sa.SA_ERR_ARGUMENT      # narrower than the Q slice
    assert call(ptrs, width=W + 4) == sa.SA_ERR_ARGUMENT      # not a multiple of 8


def test_projection_backward_rejects_bad_arguments(lib):
    s = shape()
    need = sa.sa_backward_workspace_bytes(s)
    W = 64 * (s.heads + 2 * s.kv_heads)

    def call(p, ws=need, c=0.18, sc=0.125, width=W):
        return lib.sa_backward_projection(ctypes.byref(s), p[0], p[1], p[2], p[3], p[4], ws, p[5], p[6], p[7], c,
                                          sc, p[8], p[9], p[10], p[11], p[12], p[13], width, None)

    ptrs = [FAKE] * 14   # dO O L D dS Q K Vt dQ32 dQ16 dK32 dK16 dV32 dV16
    for i in range(14):
        bad = list(ptrs)
        bad[i] = None
        assert call(bad) == sa.SA_ERR_NULL
        bad[i] = FAKE + 8
        assert call(bad) == sa.SA_ERR_ALIGN
    assert call(ptrs, ws=need - 1) == sa.SA_ERR_WORKSPACE
    assert call(ptrs, c=-1.0) == sa.SA_ERR_ARGUMENT
    assert call(ptrs, width=64 * s.heads - 8) == sa.SA_ERR_ARGUMENT
    assert call(ptrs, width=W + 2) == sa.SA_ERR_ARGUMENT


def test_two_pass_projection_backward_rejects_bad_arguments(lib):
    s = shape()
    W = 64 * (s.heads + 2 * s.kv_heads)

    def call(p, c=0.18, sc=0.125, width=W):
        return lib.sa_backward_two_pass_projection(ctypes.byref(s), p[0], p[1], p[2], p[3], p[4], p[5], p[6], c, sc,
                                                   p[7], p[8], p[9], p[10], p[11], p[12], width, None)

    ptrs = [FAKE] * 13   # dO O L D Q K Vt dQ32 dQ16 dK32 dK16 dV32 dV16
    for i in range(13):
        bad = list(ptrs)
        bad[i] = None
        assert call(bad) == sa.SA_ERR_NULL
        bad[i] = FAKE + 8
        assert call(bad) == sa.SA_ERR_ALIGN
    assert call(ptrs, sc=float("nan")) == sa.SA_ERR_ARGUMENT
    assert call(ptrs, width=W - 4) == sa.SA_ERR_ARGUMENT


def test_a_library_built_from_other_sources_is_refused(monkeypatch):
    """The binding loads libsa.so only if the source hash it was built from matches the sources beside it."""
    from causal_streaming_attention_amd import build
    monkeypatch.setattr(sa, "_lib", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0000000000000000")
    with pytest.raises(RuntimeError, match="not built from the sources"):
        sa.native()


def test_static_scratch_backward_rejects_before_touching_the_gpu(lib):
    """sa_backward_static checks shape, pointers, scales and its size limit before any HIP call."""
    fits = shape(batch=1, T=8192, heads=32, kv=8)
    assert sa.sa_backward_chunked_min_bytes(fits) <= sa.SA_STATIC_SCRATCH_BYTES
    P = 256
    big = shape(batch=1, T=16384, heads=32, kv=8)          # one 128-row block alone needs 134 MB of dS
    assert sa.sa_backward_chunked_min_bytes(big) > sa.SA_STATIC_SCRATCH_BYTES
    args = [P] * 7 + [sa.base2_scale(0.125), 0.125] + [P] * 3 + [None]
    f = lib.sa_backward_static
    assert f(ctypes.byref(big), *args) == sa.SA_ERR_TOO_LARGE
    assert f(ctypes.byref(shape(T=100)), *args) == sa.SA_ERR_SHAPE
    bad = list(args)
    bad[0] = None
    assert f(ctypes.byref(shape()), *bad) == sa.SA_ERR_NULL
    bad[0] = P + 8
    assert f(ctypes.byref(shape()), *bad) == sa.SA_ERR_ALIGN
    bad = list(args)
    bad[7] = float("nan")
    assert f(ctypes.byref(shape()), *bad) == sa.SA_ERR_ARGUMENT
    assert "static scratch" in sa.sa_status_string(sa.SA_ERR_TOO_LARGE)


def test_chunked_backward_minimum_workspace(lib):
    """The chunked backward needs one 128-row block's dS at least: the block with the most tiles."""
    tile = 64 * 64 * 2
    # causal T = 320 (5 tiles): blocks hold rows {0,1}, {2,3}, {4}: 1+2, 3+4, 5 tiles; the most is 7
    assert sa.sa_backward_chunked_min_bytes(shape(batch=2, T=320, heads=4, kv=2)) == 2 * 4 * 7 * tile
    # full square T = 320: two rows of 5 tiles
    assert sa.sa_backward_chunked_min_bytes(shape(batch=1, T=320, heads=2, kv=2, causal=0)) == 2 * 10 * tile
    assert sa.sa_backward_chunked_min_bytes(shape(T=100)) == 0
    P = 256
    sh = shape(batch=1, T=256, heads=2, kv=1)
    need = sa.sa_backward_chunked_min_bytes(sh)
    args = [P] * 5 + [need - 16] + [P] * 3 + [sa.base2_scale(0.125), 0.125] + [P] * 3 + [None]
    assert lib.sa_backward_chunked(ctypes.byref(sh), *args) == sa.SA_ERR_WORKSPACE
    args[4] = None
    assert lib.sa_backward_chunked(ctypes.byref(sh), *args) == sa.SA_ERR_NULL
