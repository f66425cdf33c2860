"""Waits for the loads the compiler does not track, checked on the gfx950 assembly.

The kernels issue some loads as inline assembly the compiler does not see
(non-temporal dS loads into registers in the dQ pass, transposed LDS reads in
the key pass and the dQ pass) and wait for them with hand-counted s_waitcnt
immediates.  The compiler may still read such a register (a copy for a
loop-carried value), or reuse it for a value of its own, while the load is in
flight, and a hand-counted immediate may be one short.  Either is a race that
tests on the GPU only catch by chance.

This test compiles the kernels for gfx950 and runs a dataflow analysis over
each kernel's control-flow graph (branches and loop back edges included):

* every untracked load's destination registers are pending, with the least
  number, over all paths, of vector-memory (vmcnt) or LDS (lgkmcnt)
  instructions issued after it;
* an s_waitcnt vmcnt(N) retires a pending load only if at least N later
  vector-memory instructions were issued on every path (gfx9 counts loads and
  stores in one in-order counter); lgkmcnt(N) likewise with LDS instructions
  only (scalar loads return out of order);
* any instruction other than the waits that reads or writes a register of a
  still-pending load is reported.

The same analysis is also run over every load, so that the compiler's own
waits are checked the same way.  For the dQ pass it also checks the K tiles' LDS DMA: after every hand-written
s_waitcnt vmcnt(22) at most six DMA instructions (three tiles' worth, two per
tile) may still be in flight on any path, so the tile the next step reads has
landed."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_streaming_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CAP = 64  # vmcnt and lgkmcnt immediates stay below this

_VREG = re.compile(r"(?<![\w\[])v\[(\d+):(\d+)\]|(?<![\w\[])v(\d+)\b")


def _vregs(text):
    regs = set()
    for m in _VREG.finditer(text):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


class Insn:
    __slots__ = ("text", "op", "args", "in_asm", "line")

    def __init__(self, text, in_asm, line):
        self.text, self.in_asm, self.line = text, in_asm, line
        parts = text.split(None, 1)
        self.op = parts[0]
        self.args = parts[1] if len(parts) > 1 else ""


def _functions(asm_text):
    """{kernel name: [("label", name) | ("insn", Insn)]} in program order."""
    fns, cur, in_asm = {}, None, False
    for n, line in enumerate(asm_text.splitlines(), 1):
        s = line.split(";;#")[0] if not line.strip().startswith(";;#") else line.strip()
        s = s.strip()
        if re.match(r"^_Z\S*:", s):
            cur = fns.setdefault(s.split(":")[0], [])
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if cur is None:
            continue
        s = s.split(";")[0].strip()
        if not s:
            continue
        if re.match(r"^\.LBB\w+:", s):
            cur.append(("label", s[:-1]))
            continue
        if s.startswith("."):
            if s.startswith(".Lfunc_end"):
                cur = None
            continue
        cur.append(("insn", Insn(s, in_asm, n)))
    return fns


def _blocks(items):
    """Basic blocks [insns] of one function and their successor indices."""
    blocks, labels = [], {}
    cur, label, started = [], None, False
    for kind, x in items:
        if kind == "label":
            if started:
                blocks.append((label, cur))
            cur, label, started = [], x, True
            continue
        cur.append(x)
        started = True
        if x.op.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append((label, cur))
            cur, label, started = [], None, False
    if started:
        blocks.append((label, cur))
    labels = {lab: i for i, (lab, _) in enumerate(blocks) if lab is not None}
    succ = []
    for i, (_, insns) in enumerate(blocks):
        last = insns[-1] if insns else None
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last is None:
            succ.append(nxt)
        elif last.op == "s_branch":
            succ.append([labels[last.args.strip()]])
        elif last.op.startswith("s_cbranch"):
            succ.append([labels[last.args.strip()]] + nxt)
        elif last.op.startswith(("s_endpgm", "s_setpc")):
            succ.append([])
        else:
            succ.append(nxt)
    return [b for _, b in blocks], succ


def _is_vmem(op):
    return op.startswith(("global_", "buffer_", "flat_", "scratch_"))


def _is_dma(insn):
    return insn.op.startswith("global_load_lds") or (insn.op.startswith("buffer_load") and
                                                     re.search(r"\blds\b", insn.args) is not None)


def _waitcnt(insn):
    """(vmcnt, lgkmcnt) of an s_waitcnt, None for a field it leaves alone."""
    if insn.op != "s_waitcnt":
        return None, None
    vm = re.search(r"vmcnt\((\d+)\)", insn.args)
    lg = re.search(r"lgkmcnt\((\d+)\)", insn.args)
    return (int(vm.group(1)) if vm else None), (int(lg.group(1)) if lg else None)


def _merge(a, b):
    vm = dict(a[0])
    for r, y in b[0].items():
        vm[r] = min(y, vm.get(r, CAP))
    lg = dict(a[1])
    for r, y in b[1].items():
        lg[r] = min(y, lg.get(r, CAP))
    return (vm, lg, a[2] | b[2])


def _age(d, n=1):
    return {r: min(y + n, CAP) for r, y in d.items()}


def _transfer(insns, state, problems, fn, dma_waits, all_loads=False):
    vm, lg, dma = dict(state[0]), dict(state[1]), set(state[2])
    for x in insns:
        wvm, wlg = _waitcnt(x)
        if wvm is not None or wlg is not None:
            if wvm is not None:
                vm = {r: y for r, y in vm.items() if y < wvm}
                dma = {tuple(y for y in t if y < wvm) for t in dma}
                if x.in_asm and wvm > 0:
                    dma_waits.append((x.line, wvm, max((len(t) for t in dma), default=0)))
            if wlg is not None:
                lg = {r: y for r, y in lg.items() if y < wlg}
            continue
        untracked_vm = (x.in_asm or all_loads) and x.op.startswith(("global_load", "buffer_load")) and not _is_dma(x)
        untracked_lg = (x.in_asm or all_loads) and x.op.startswith("ds_read")
        if untracked_vm or untracked_lg:
            dst, _, rest = x.args.partition(",")
            dst_regs, src_regs = _vregs(dst), _vregs(rest)
        else:
            dst_regs, src_regs = set(), _vregs(x.args)
        touched = (src_regs | dst_regs) if not (untracked_vm or untracked_lg) else src_regs
        for kind, pend in (("vm", vm), ("lgkm", lg)):
            hit = touched & set(pend)
            if (untracked_vm and kind == "lgkm") or (untracked_lg and kind == "vm"):
                # a load into a register another counter's load may still fill
                # (loads on one counter return in order: their order is kept)
                hit |= dst_regs & set(pend)
            if hit:
                problems.add(f"{fn}: line {x.line}: '{x.text}' uses v{min(hit)} of an untracked {kind} "
                             f"load that may still be in flight")
        if _is_vmem(x.op):
            vm = _age(vm)
            dma = {tuple(min(y + 1, CAP) for y in t) for t in dma}
            if _is_dma(x):
                dma = {t + (0,) for t in dma}
        if x.op.startswith("ds_"):
            lg = _age(lg)
        if untracked_vm:
            for r in dst_regs:
                vm[r] = 0
        if untracked_lg:
            for r in dst_regs:
                lg[r] = 0
        # a tuple of in-flight DMAs longer than the counter's range is capped:
        # entries at CAP are retired by any wait
        dma = {tuple(y for y in t if y < CAP) for t in dma}
    return (vm, lg, frozenset(dma))


def analyse(asm_text, only=None, all_loads=False):
    """(problems, {kernel: [(line, N, most DMAs in flight after that hand-written vmcnt(N))]})."""
    problems, dma_report = set(), {}
    for fn, items in _functions(asm_text).items():
        if only and only not in fn:
            continue
        blocks, succ = _blocks(items)
        if not blocks:
            continue
        entry = ({}, {}, frozenset({()}))
        state_in = {0: entry}
        work = [0]
        while work:
            i = work.pop()
            waits = []
            out = _transfer(blocks[i], state_in[i], problems, fn, waits, all_loads)
            for j in succ[i]:
                new = out if j not in state_in else _merge(state_in[j], out)
                if j not in state_in or new != state_in[j]:
                    state_in[j] = new
                    work.append(j)
        waits = []
        for i in state_in:
            _transfer(blocks[i], state_in[i], set(), fn, waits, all_loads)
        if waits:
            dma_report[fn] = sorted(set(waits))
    return sorted(problems), dma_report


def _compile(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-fno-honor-nans", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src", ["sa_backward.hip", "sa_forward.hip", "sa_query.hip"])
def test_untracked_loads_are_waited_for_before_use(tmp_path, src):
    asm = _compile(tmp_path, src)
    problems, dma = analyse(asm)
    assert not problems, "\n".join(problems[:10])
    # The same check over every load, the compiler's own included: its waits
    # must hold up too (a load into a register that a load on the other
    # counter may still fill is flagged as well).
    problems_all, _ = analyse(asm, all_loads=True)
    assert not problems_all, "\n".join(problems_all[:10])
    if src == "sa_backward.hip":
        dq = {fn: w for fn, w in dma.items() if "sa_dq_kernel" in fn}
        assert len(dq) == 12, sorted(dma)   # causal x varlen x three epilogues
        for fn, waits in dq.items():
            assert waits, fn
            k_waits = [(line, n) for line, cnt, n in waits if cnt == 22]
            assert k_waits, fn
            for line, n in k_waits:
                assert n <= 6, f"{fn}: line {line}: {n} K-tile DMAs may be in flight after vmcnt(22)"


def _kernel(body):
    return "_Zk:\n" + body + "\ts_endpgm\n.Lfunc_end0:\n"


def test_the_scan_flags_a_copy_before_the_wait():
    """A register copy between an untracked load and its wait is flagged, a use after the wait is not."""
    bad = _kernel("""\t;;#ASMSTART
\tds_read_b64_tr_b16 v[66:67], v1 offset:0x800
\t;;#ASMEND
\tv_bfi_b32 v148, s77, v66, v66
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
""")
    good = bad.replace("\tv_bfi_b32 v148, s77, v66, v66\n", "").replace("\ts_endpgm", "\tv_mov_b32 v148, v66\n\ts_endpgm")
    assert analyse(bad)[0] and not analyse(good)[0]


def test_the_scan_flags_a_register_reused_while_a_load_is_in_flight():
    """The compiler reusing an in-flight load's destination for its own value (an address here) is flagged."""
    bad = _kernel("""\t;;#ASMSTART
\tglobal_load_dwordx4 v[4:7], v[8:9], off nt
\t;;#ASMEND
\tv_mov_b32 v4, s2
\tglobal_store_dwordx4 v[4:5], v[10:13], off
""")
    assert analyse(bad)[0]
    drained = bad.replace("\tv_mov_b32 v4, s2", "\ts_waitcnt vmcnt(0)\n\tv_mov_b32 v4, s2")
    assert not analyse(drained)[0]


def test_the_scan_counts_younger_memory_instructions_on_every_path():
    """vmcnt(N) retires a load only with N younger vector-memory instructions on every path into the wait:
    one path issuing a single younger load leaves it in flight for vmcnt(2), and across a loop's back
    edge the count is the least over the iterations."""
    two_paths = _kernel("""\t;;#ASMSTART
\tglobal_load_dwordx4 v[4:7], v[8:9], off nt
\t;;#ASMEND
\tglobal_load_dword v20, v[8:9], off
\ts_cbranch_scc1 .LBB0_2
\tglobal_load_dword v21, v[8:9], off
.LBB0_2:
\t;;#ASMSTART
\ts_waitcnt vmcnt(2)
\t;;#ASMEND
\tv_mov_b32 v30, v4
""")
    assert analyse(two_paths)[0]
    assert not analyse(two_paths.replace("vmcnt(2)", "vmcnt(1)"))[0]
    loop = _kernel("""\t;;#ASMSTART
\tglobal_load_dwordx4 v[4:7], v[8:9], off nt
\t;;#ASMEND
.LBB0_1:
\tglobal_load_dword v20, v[8:9], off
\t;;#ASMSTART
\ts_waitcnt vmcnt(1)
\t;;#ASMEND
\tv_mov_b32 v30, v4
\t;;#ASMSTART
\tglobal_load_dwordx4 v[4:7], v[8:9], off nt
\t;;#ASMEND
\ts_cbranch_scc1 .LBB0_1
""")
    assert not analyse(loop)[0]
    assert analyse(loop.replace("vmcnt(1)", "vmcnt(2)"))[0]


def test_the_dma_count_after_a_vmcnt22_wait():
    """Three loop steps of (two DMAs, then four other loads) after the DMA in question leave 22 younger
    instructions: vmcnt(22) retires it, and the DMAs still in flight are the last three steps' six."""
    step = "\tglobal_load_lds_dwordx4 v[4:5], off\n\tglobal_load_lds_dwordx4 v[4:5], off\n" + \
           "\tglobal_load_dword v20, v[8:9], off\n" * 4
    body = step * 4 + "\t;;#ASMSTART\n\ts_waitcnt vmcnt(22)\n\t;;#ASMEND\n"
    _, dma = analyse(_kernel(body))
    assert dma["_Zk"] == [(27, 22, 6)]
    _, dma = analyse(_kernel(body.replace("vmcnt(22)", "vmcnt(23)")))
    assert dma["_Zk"] == [(27, 23, 7)]
