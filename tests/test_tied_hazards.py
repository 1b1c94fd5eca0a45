"""Hazard check of the built kernels whose MFMAs are written out with tied
accumulators (the one-wave-per-SIMD tile kernels, mma16<true>, and the
128-byte-row MX kernels, mma_mx_tied and mma16_mx_tied).

The compiler inserts the wait states an MFMA needs only around MFMAs it
generated itself; around a written-out one the kernel keeps them: a vector
ALU write of any MFMA operand needs two wait states before the MFMA issues,
and an MFMA's result must not be read or overwritten by another kind of
instruction for the instruction's result latency (checked against 19 wait
states for the 16x16 forms and 24 for the 16-pass 32x32 ones, more than
either needs). This test disassembles the device
code of the in-tree libtile_gemm.so (ROCm's own llvm tools on code built here)
and walks back from every MFMA of those kernels, across branches, counting
wait states (one per instruction, N + 1 for s_nop N).
"""

import os
import re
import shutil
import subprocess

import pytest

from tile_partitioned_dense_amd import binding

LLVM = "/opt/rocm/llvm/bin"
TIED_KERNEL = re.compile(r"^_ZN2tg(?:1[68]tile(16|64)|17mx128|16mx16)_gemm_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")
REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\d))")
VALU_WRITE_BEFORE_MFMA = 2
MFMA_RESULT_LATENCY = {"16x16": 19, "32x32": 24}


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _regs(text):
    out = set()
    for kind, lo, hi, one in REG.findall(text):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return out


def _disassemble(lib, workdir):
    """Disassembly text of every device code object in the library."""
    fat = os.path.join(workdir, "fatbin.bin")
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib,
                    os.path.join(workdir, "host.o")], check=True, capture_output=True)
    data = open(fat, "rb").read()
    offs = [m.start() for m in re.finditer(rb"__CLANG_OFFLOAD_BUNDLE__", data)] + [len(data)]
    texts = []
    for i in range(len(offs) - 1):
        b = os.path.join(workdir, f"b{i}.bin")
        co = os.path.join(workdir, f"co{i}.o")
        open(b, "wb").write(data[offs[i]:offs[i + 1]])
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={b}", f"--output={co}"],
                       check=True, capture_output=True)
        r = subprocess.run([_tool("llvm-objdump"), "-d", "--symbolize-operands", "--mcpu=gfx950", co],
                           check=True, capture_output=True, text=True)
        texts.append(r.stdout)
    return texts


def _functions(text):
    """{symbol: [(kind, payload)]} with kind 'label' (name) or 'insn' (text)."""
    funcs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <([^>]+)>:$", line)
        if m:
            name = m.group(1)
            if name.startswith("_Z"):
                cur = funcs.setdefault(name, [])
            elif cur is not None:
                cur.append(("label", name))
            continue
        if cur is not None and line.startswith("\t"):
            cur.append(("insn", line.split("//")[0].strip()))
    return funcs


class _Insn:
    __slots__ = ("op", "ops", "ws", "labels_before", "target")

    def __init__(self, text, labels_before):
        parts = text.split(None, 1)
        self.op = parts[0]
        self.ops = parts[1] if len(parts) > 1 else ""
        self.ws = int(self.ops.split(",")[0], 0) + 1 if self.op == "s_nop" else 1
        self.labels_before = labels_before
        self.target = self.ops.split()[0] if self.op.startswith(("s_branch", "s_cbranch")) else None

    @property
    def is_mfma(self):
        return self.op.startswith("v_mfma")

    @property
    def valu_dest(self):
        if not self.op.startswith("v_") or self.is_mfma:
            return set()
        first = self.ops.split(",")[0]
        return _regs(first)

    def operands(self):
        names = [x.strip() for x in self.ops.split(",")]
        return names


def _check_function(name, items):
    insns, pending = [], []
    for kind, payload in items:
        if kind == "label":
            pending.append(payload)
        else:
            insns.append(_Insn(payload, pending))
            pending = []
    label_at = {}
    for i, ins in enumerate(insns):
        for lb in ins.labels_before:
            label_at[lb] = i
    preds = {i: [] for i in range(len(insns))}  # extra predecessors (branch sources) of label heads
    for i, ins in enumerate(insns):
        if ins.target in label_at:
            preds[label_at[ins.target]].append(i)

    def walk_back(i, budget, visit, seen):
        """Call visit(insn, distance) for instructions that can precede insn i
        within `budget` wait states, over fall-through and branch edges."""
        stack = [(i, 0)]
        while stack:
            j, dist = stack.pop()
            if (j, dist) in seen:
                continue
            seen.add((j, dist))
            # predecessors of instruction j
            cands = []
            if j > 0 and insns[j - 1].op not in ("s_branch", "s_endpgm", "s_setpc_b64"):
                cands.append(j - 1)
            if insns[j].labels_before:
                cands.extend(preds[j])
            for p in cands:
                visit(insns[p], dist)
                nd = dist + insns[p].ws
                if nd < budget:
                    stack.append((p, nd))

    problems = []
    for i, ins in enumerate(insns):
        if not ins.is_mfma:
            continue
        o = ins.operands()
        dst, srcs = _regs(o[0]), set().union(*(_regs(x) for x in o[1:4]))

        def valu_check(p, dist, srcs=srcs, i=i):
            hit = p.valu_dest & srcs
            if hit:
                problems.append(f"{name}: '{p.op} {p.ops}' writes an operand of MFMA #{i} "
                                f"'{ins.op} {ins.ops}' {dist} wait states before it")

        walk_back(i, VALU_WRITE_BEFORE_MFMA, valu_check, set())

    # forward: nothing but an accumulating MFMA on the same registers touches an
    # MFMA's result within its latency (checked as: walking back from every
    # non-MFMA instruction that names such a register)
    for i, ins in enumerate(insns):
        if ins.is_mfma:
            continue
        regs = _regs(ins.ops)
        if not regs:
            continue

        def res_check(p, dist, regs=regs, i=i):
            if p.is_mfma and dist < MFMA_RESULT_LATENCY["32x32" if "32x32" in p.op else "16x16"]:
                hit = _regs(p.operands()[0]) & regs
                if hit:
                    problems.append(f"{name}: '{ins.op} {ins.ops}' touches the result of "
                                    f"'{p.op} {p.ops}' {dist} wait states after it")

        walk_back(i, max(MFMA_RESULT_LATENCY.values()), res_check, set())
    return problems


@pytest.fixture(scope="module")
def tied_functions(tmp_path_factory):
    lib = binding.library_path()
    if not os.path.exists(lib):
        pytest.skip("libtile_gemm.so is not built")
    for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump"):
        if _tool(t) is None:
            pytest.skip(f"{t} not available")
    work = tmp_path_factory.mktemp("disasm")
    found = {}
    for text in _disassemble(lib, str(work)):
        for name, items in _functions(text).items():
            m = TIED_KERNEL.match(name)
            if m and int(m.group(4)) * int(m.group(5)) == 4:
                found[name] = items
    return found


def test_tied_kernels_are_present(tied_functions):
    # the one-wave-per-SIMD configurations of both tile kernels and the
    # 128-byte-row MX kernel, every variant
    bits = {n.split("kernel")[0] for n in tied_functions}
    assert all(any(k in b for b in bits) for k in ("tile16", "tile64", "mx128", "mx16_")), sorted(tied_functions)


def test_tied_kernels_keep_mfma_hazards(tied_functions):
    problems = []
    for name, items in tied_functions.items():
        problems += _check_function(name, items)
    assert not problems, "\n".join(problems[:20])


def test_checker_finds_a_planted_hazard():
    """The walk sees a vector write right before an MFMA, also across a loop's
    back edge, and a read of an MFMA's result too soon."""
    body = [("insn", "v_mov_b32_e32 v4, 0"),
            ("insn", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]")]
    assert _check_function("straight", body)
    loop = [("label", "L0"),
            ("insn", "s_nop 1"),
            ("insn", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]"),
            ("insn", "v_accvgpr_write_b32 a2, 0"),
            ("insn", "s_cbranch_scc1 L0")]
    # a write one wait state before the back edge's branch, then s_nop 1 at
    # the head: 1 + 2 wait states, enough
    assert not [p for p in _check_function("loop", loop) if "writes an operand" in p]
    loop_bad = [("label", "L0"),
                ("insn", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]"),
                ("insn", "s_nop 7"), ("insn", "s_nop 7"), ("insn", "s_nop 7"),
                ("insn", "v_accvgpr_write_b32 a2, 0"),
                ("insn", "s_cbranch_scc1 L0")]
    assert [p for p in _check_function("loop_bad", loop_bad) if "writes an operand" in p]
    early_read = [("insn", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]"),
                  ("insn", "s_nop 7"),
                  ("insn", "v_accvgpr_read_b32 v0, a1")]
    assert [p for p in _check_function("early", early_read) if "touches the result" in p]
    chained = [("insn", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]"),
               ("insn", "v_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]")]
    assert not _check_function("chained", chained)
