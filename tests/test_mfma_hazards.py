"""Matrix-core hazard check of the compiled contraction kernels (CPU only).

The bf16 main loop issues its v_mfma instructions through inline assembly, so that
every accumulator is updated in place; the compiler does not track wait states for
inline assembly.  This test compiles the kernel source to gfx950 assembly with the
library's own flags and checks, along every control-flow path, the dependency rules
of the matrix-core pipeline (CDNA3/CDNA4 instruction set reference, "dependency
resolution: required independent instructions" for XDL operations), with generous
windows:

* after an MFMA, no instruction reads or writes its result registers for 11 wait
  states (a 4-pass operation such as v_mfma_f32_16x16x32_bf16 needs 7; 11 is the
  figure for 8 passes), except another MFMA that uses the same registers as its
  accumulator input and output;
* before an MFMA, no VALU instruction writes any of its operand registers within 3
  wait states (2 are required), and no MFMA writes its A/B operands within 11;
* after an MFMA, no VALU instruction overwrites its A/B operands within 6 wait
  states.

The fp8 main loop's v_mfma_f32_16x16x128_f8f6f4 takes 8 passes with fp8 operands;
for it the windows are those of a 16-pass operation (19 wait states after, 11 for
its A/B operands), above what 8 passes require.

Only MFMAs issued from inline assembly are checked (the listing brackets them with
ASMSTART / ASMEND markers), but against every instruction around them, the
compiler's included: for its builtin MFMAs the compiler inserts the wait states
itself.

Wait states are counted as one per instruction (an MFMA too) and N + 1 per s_nop N,
which undercounts real time and so errs on the safe side.  Loads that write operand
registers are ordered by s_waitcnt, which the compiler inserts for inline assembly
operands as for any other use, and are not checked here.
"""

import os
import re
import shutil
import subprocess

import pytest

from entropy_block_sparse_amd import build as B

W_AFTER = 11
W_BEFORE_VALU = 3
W_AB_WAR = 6
# windows per MFMA mnemonic where they differ from the 4-pass defaults
LONG_MFMA = {"v_mfma_f32_16x16x128_f8f6f4": (19, 11)}


def windows(op):
    return LONG_MFMA.get(op, (W_AFTER, W_AB_WAR))

REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def regs(text):
    out = set()
    for m in REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


class Inst:
    def __init__(self, text, from_asm=False):
        self.text = text
        self.from_asm = from_asm
        parts = text.split(None, 1)
        self.op = parts[0]
        ops = [o.strip() for o in (parts[1].split(",") if len(parts) > 1 else [])]
        self.operands = ops
        self.is_mfma = self.op.startswith("v_mfma")
        self.is_valu = self.op.startswith("v_") and not self.is_mfma
        self.nop = int(ops[0], 0) + 1 if self.op == "s_nop" and ops else 0
        self.reads, self.writes = set(), set()
        if self.op.startswith("v_"):
            if self.op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
                self.reads = regs(",".join(ops[1:]))
            elif ops:
                self.writes = regs(ops[0])
                self.reads = regs(",".join(ops[1:]))
        elif self.op.startswith(("ds_read", "buffer_load", "global_load", "scratch_load", "flat_load")):
            if " lds" in text or text.rstrip().endswith("lds"):
                self.reads = regs(",".join(ops))
            elif ops:
                self.writes = regs(ops[0])
                self.reads = regs(",".join(ops[1:]))
        elif self.op.startswith(("ds_", "buffer_", "global_", "scratch_", "flat_")):
            self.reads = regs(",".join(ops))
        if self.is_mfma:
            self.dst = regs(ops[0])
            self.src_ab = regs(ops[1]) | regs(ops[2])
            self.src_c = regs(ops[3])

    @property
    def wait(self):
        return self.nop if self.op == "s_nop" else 1


def parse_kernels(asm):
    """{kernel name: (blocks, order)}; blocks[label] = list of Inst, plus successor labels."""
    kernels = {}
    cur_k = None
    for line in asm.splitlines():
        m = re.match(r"^(_ZN3flh\S*):", line)
        if m:
            cur_k = m.group(1)
            kernels[cur_k] = []
            continue
        if cur_k is None:
            continue
        if line.startswith(".Lfunc_end"):
            cur_k = None
            continue
        kernels[cur_k].append(line)
    out = {}
    for name, lines in kernels.items():
        blocks, order, label = {}, [], "entry"
        blocks[label] = []
        order.append(label)
        in_asm = False
        for line in lines:
            if "ASMSTART" in line:
                in_asm = True
                continue
            if "ASMEND" in line:
                in_asm = False
                continue
            m = re.match(r"^(\.LBB\S+):", line)
            if m:
                label = m.group(1)
                blocks[label] = []
                order.append(label)
                continue
            s = line.split(";")[0].strip()
            if not s or s.startswith(".") or s.endswith(":"):
                continue
            blocks[label].append(Inst(s, in_asm))
        succ = {}
        for i, lb in enumerate(order):
            ss = []
            insts = blocks[lb]
            last = insts[-1] if insts else None
            for ins in insts:
                if ins.op.startswith("s_cbranch") or ins.op == "s_branch":
                    ss.append(ins.operands[0])
            if not (last is not None and (last.op == "s_branch" or last.op == "s_endpgm")) and i + 1 < len(order):
                ss.append(order[i + 1])
            succ[lb] = ss
        pred = {lb: [] for lb in order}
        for lb, ss in succ.items():
            for t in ss:
                if t in pred:
                    pred[t].append(lb)
        out[name] = (blocks, order, succ, pred)
    return out


def walk_forward(blocks, succ, lb, idx, window):
    """Instructions within `window` wait states after blocks[lb][idx], on every path."""
    seen = {}
    stack = [(lb, idx + 1, 0)]
    while stack:
        b, i, ws = stack.pop()
        insts = blocks[b]
        while i < len(insts):
            if ws >= window:
                break
            yield insts[i], ws
            ws += insts[i].wait
            i += 1
        else:
            for t in succ[b]:
                if t in blocks and seen.get(t, 1 << 30) > ws:
                    seen[t] = ws
                    stack.append((t, 0, ws))


def walk_backward(blocks, pred, lb, idx, window):
    seen = {}
    stack = [(lb, idx - 1, 0)]
    while stack:
        b, i, ws = stack.pop()
        insts = blocks[b]
        while i >= 0:
            if ws >= window:
                break
            yield insts[i], ws
            ws += insts[i].wait
            i -= 1
        else:
            for t in pred[b]:
                if seen.get(t, 1 << 30) > ws:
                    seen[t] = ws
                    stack.append((t, len(blocks[t]) - 1, ws))


def check(asm, kernel_filter=None):
    problems = []
    for name, (blocks, order, succ, pred) in parse_kernels(asm).items():
        if kernel_filter and not kernel_filter(name):
            continue
        for lb in order:
            for idx, m in enumerate(blocks[lb]):
                if not (m.is_mfma and m.from_asm):
                    continue
                w_after, w_war = windows(m.op)
                for ins, ws in walk_forward(blocks, succ, lb, idx, w_after):
                    if ins.is_mfma and ins.dst == m.dst and ins.src_c == m.dst and not (ins.src_ab & m.dst):
                        continue
                    if (ins.reads | ins.writes) & m.dst:
                        problems.append((name, lb, m.text, ins.text, ws, "result used too early"))
                for ins, ws in walk_forward(blocks, succ, lb, idx, w_war):
                    if ins.is_valu and ins.writes & m.src_ab:
                        problems.append((name, lb, m.text, ins.text, ws, "A/B operand overwritten too early"))
                for ins, ws in walk_backward(blocks, pred, lb, idx, max(W_AFTER, *(w[0] for w in LONG_MFMA.values()))):
                    if ins.is_valu and ws < W_BEFORE_VALU and ins.writes & (m.src_ab | m.src_c):
                        problems.append((name, lb, m.text, ins.text, ws, "operand written by VALU too late"))
                    if ins.is_mfma and ins.writes & m.src_ab and ws < windows(ins.op)[0]:
                        problems.append((name, lb, m.text, ins.text, ws, "A/B operand written by MFMA too late"))
    return problems


def compile_to_asm(src, out):
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-I", B.INCLUDE, "-I", B.CSRC,
           *B.DEVICE_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    if shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "flh_gemm.s"
    return compile_to_asm(os.path.join(B.CSRC, "flh_gemm.hip"), str(out))


def test_contraction_kernels_respect_matrix_core_wait_states(kernel_asm):
    problems = check(kernel_asm)
    n_asm = sum(i.is_mfma and i.from_asm for blocks, *_ in parse_kernels(kernel_asm).values()
                for b in blocks.values() for i in b)
    assert n_asm > 0, "expected the bf16 main loop to issue its MFMAs from inline assembly"
    n_f8 = sum(i.is_mfma and i.from_asm and i.op == "v_mfma_f32_16x16x128_f8f6f4"
               for blocks, *_ in parse_kernels(kernel_asm).values() for b in blocks.values() for i in b)
    assert n_f8 > 0, "expected the fp8 main loop to issue its MFMAs from inline assembly"
    assert not problems, "\n".join(f"{n[-40:]} {lb}: {m}  ->  {i}  (after {ws} wait states: {why})"
                                   for n, lb, m, i, ws, why in problems[:20])


def test_checker_flags_a_planted_hazard():
    """The checker itself: an accumulator read one wait state after the MFMA that wrote
    it, and an operand written by a VALU right before the MFMA, are both reported; the
    same code with enough s_nop is clean."""
    bad = """_ZN3flhX:
\tv_accvgpr_write_b32 a3, 0
\t;;#ASMSTART
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]
\t;;#ASMEND
\ts_nop 0
\tv_accvgpr_read_b32 v20, a2
\ts_endpgm
.Lfunc_end0:
"""
    kinds = {p[5] for p in check(bad)}
    assert kinds == {"result used too early", "operand written by VALU too late"}
    good = """_ZN3flhX:
\tv_accvgpr_write_b32 a3, 0
\ts_nop 4
\t;;#ASMSTART
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]
\t;;#ASMEND
\ts_nop 7
\ts_nop 7
\ts_nop 2
\tv_accvgpr_read_b32 v20, a2
\ts_endpgm
.Lfunc_end0:
"""
    assert check(good) == []
    # a loop back edge is followed: the read at the top of the loop is one wait state
    # after the MFMA at its bottom
    loop = """_ZN3flhX:
.LBB0_1:
\tv_accvgpr_read_b32 v20, a2
\ts_nop 7
\ts_nop 7
\ts_nop 7
\t;;#ASMSTART
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]
\t;;#ASMEND
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
.Lfunc_end0:
"""
    assert {p[5] for p in check(loop)} == {"result used too early"}
