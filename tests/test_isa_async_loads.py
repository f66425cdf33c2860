"""The kernels issue some loads as inline assembly the compiler does not track
(non-temporal dS loads in the dQ pass, transposed LDS reads in the key pass) and
wait for them with an s_waitcnt that ties the result registers.  The compiler may
still copy such registers, e.g. for a loop-carried value, right after the load and
before the wait, which reads stale data.  This test compiles the kernels for gfx950
and checks, along each function's instruction stream, that no instruction outside
the inline assembly reads an untracked load's destination before a wait on that
load's counter.  (A conservative linear scan: any wait on the counter ends the
window, and uses across a loop's back edge are not followed.)"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_streaming_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _vregs(tok):
    m = re.fullmatch(r"-?v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"-?v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _scan(asm_text):
    problems = []
    pending = {"vm": {}, "lgkm": {}}
    in_asm = False
    fn = None
    for n, line in enumerate(asm_text.splitlines()):
        s = line.strip()
        if re.match(r"^_Z\S*:", s):
            fn, pending = s.split(":")[0], {"vm": {}, "lgkm": {}}
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith("."):
            continue
        ops = s.replace(",", " ").split()
        op = ops[0]
        if op == "s_waitcnt":
            if "vmcnt" in s:
                pending["vm"] = {}
            if "lgkmcnt" in s:
                pending["lgkm"] = {}
            continue
        if in_asm:
            if op == "global_load_dwordx4" and len(ops) > 1:
                for r in _vregs(ops[1]):
                    pending["vm"][r] = n
            elif op.startswith("ds_read") and len(ops) > 1:
                for r in _vregs(ops[1]):
                    pending["lgkm"][r] = n
            continue
        srcs = set()
        for tok in ops[2:] if not op.startswith(("ds_write", "global_store", "buffer_store")) else ops[1:]:
            srcs |= _vregs(tok)
        for kind in ("vm", "lgkm"):
            hit = srcs & set(pending[kind])
            if hit:
                problems.append(f"{fn}: line {n}: '{s}' reads v{sorted(hit)[0]} of an untracked {kind} load "
                                f"issued at line {pending[kind][sorted(hit)[0]]} before any wait")
    return problems


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["sa_backward.hip", "sa_forward.hip", "sa_query.hip"])
def test_untracked_loads_are_waited_for_before_use(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-fno-honor-nans", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    problems = _scan(out.read_text())
    assert not problems, "\n".join(problems[:10])


def test_the_scan_flags_a_copy_before_the_wait():
    """The scan itself: a register copy between an untracked load and its wait is flagged,
    a use after the wait is not."""
    bad = """_Zk:
\t;;#ASMSTART
\tds_read_b64_tr_b16 v[66:67], v1 offset:0x800
\t;;#ASMEND
\tv_bfi_b32 v148, s77, v66, v66
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
"""
    good = bad.replace("\tv_bfi_b32 v148, s77, v66, v66\n", "") + "\tv_mov_b32 v148, v66\n"
    assert _scan(bad) and not _scan(good)
