"""The built gfx950 code object honours the DPP read rule on every path.

A VALU instruction that writes a VGPR must be followed by two wait states
(independent instructions, or s_nop N counting N + 1) before a DPP
instruction reads that VGPR as its DPP source; the hardware does not
interlock this and a read that comes too early sees the stale value. The
compiler inserts these wait states for the DPP operations it emits itself,
but not for DPP instructions written inside asm statements (the row
transpose-reduce and the broadcast-fmac of the gradient), whose guarantees
rest on where the compiler places the surrounding code. This test reads the
machine code of the library as built here (the gfx950 code object unbundled
from the shared library and disassembled with llvm-objdump) and checks every
DPP instruction against every predecessor path, loop back-edges included.
No GPU is involved."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
WAIT_STATES = 2

# instructions after which control never falls through
UNCONDITIONAL = ("s_branch", "s_endpgm", "s_setpc_b64", "s_endpgm_saved")
# instructions whose first operand is a VGPR they write
WRITERS = ("v_", "ds_read", "ds_load", "buffer_load", "global_load", "flat_load", "scratch_load")


def regs(tok):
    tok = tok.rstrip(",")
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return {"v%d" % k for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {tok} if re.fullmatch(r"v\d+", tok) else set()


class Ins:
    def __init__(self, addr, text):
        self.addr = addr
        self.text = text
        parts = text.split()
        self.op = parts[0]
        self.ops = parts[1:]
        self.writes = set()
        if self.op.startswith(WRITERS) and self.ops:
            self.writes = regs(self.ops[0])
            if self.op.startswith(("v_permlane", "v_swap")) and len(self.ops) > 1:
                self.writes |= regs(self.ops[1])
        self.wait = int(self.ops[0], 0) + 1 if self.op == "s_nop" else 1
        self.dpp_src = None
        if self.op.startswith("v_") and self.op.endswith("_dpp") and len(self.ops) > 1:
            self.dpp_src = regs(self.ops[1])
        self.target = None


def disassemble(lib):
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin")
        co = os.path.join(d, "co.o")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fat,
                        lib, os.path.join(d, "lib_copy.so")], check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--input=" + fat,
                        "--output=" + co], check=True, capture_output=True)
        out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                             check=True, capture_output=True, text=True).stdout
    funcs = {}
    cur = None
    for line in out.split("\n"):
        m = re.match(r"^([0-9a-f]+) <([^>]+)>:$", line)
        if m:
            cur = funcs.setdefault(m.group(2), {"start": int(m.group(1), 16), "ins": []})
            continue
        m = re.match(r"^\s+(\S.*?)\s*// ([0-9A-F]+):", line)
        if m and cur is not None:
            ins = Ins(int(m.group(2), 16), m.group(1))
            t = re.search(r"<([^>+]+)\+0x([0-9a-f]+)>", line)
            if ins.op.startswith(("s_branch", "s_cbranch")) and t:
                ins.target = (t.group(1), int(t.group(2), 16))
            cur["ins"].append(ins)
    return funcs


def violations(funcs):
    bad = []
    checked = 0
    for name, f in funcs.items():
        ins = f["ins"]
        index = {x.addr: k for k, x in enumerate(ins)}
        preds = [[] for _ in ins]
        for k, x in enumerate(ins):
            if k + 1 < len(ins) and not x.op.startswith(UNCONDITIONAL):
                preds[k + 1].append(k)
            if x.target is not None:
                assert x.target[0] == name, (name, x.text)
                tgt = f["start"] + x.target[1]
                assert tgt in index, (name, x.text)
                preds[index[tgt]].append(k)

        def clear(k, src, need, seen):
            # every path into instruction k leaves `need` wait states free of writes to src
            for p in preds[k]:
                if (p, need) in seen:
                    continue
                seen.add((p, need))
                if ins[p].writes & src:
                    return ins[p]
                if ins[p].wait < need:
                    hit = clear(p, src, need - ins[p].wait, seen)
                    if hit is not None:
                        return hit
            return None

        for k, x in enumerate(ins):
            if x.dpp_src:
                checked += 1
                hit = clear(k, x.dpp_src, WAIT_STATES, set())
                if hit is not None:
                    bad.append("%s: '%s' reads %s written by '%s'" % (name[:60], x.text, x.ops[1], hit.text))
    return bad, checked


def test_the_checker_sees_a_hazard():
    """Planted listings: a write right before the read, a write one s_nop 0
    before it, a write across a loop back-edge, and clean cases."""
    def fn(lines, targets=None):
        f = {"start": 0, "ins": []}
        for k, text in enumerate(lines):
            x = Ins(4 * k, text)
            if targets and k in targets:
                x.target = ("f", 4 * targets[k])
            f["ins"].append(x)
        return {"f": f}
    dpp = "v_fmac_f32_dpp v2, v5, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf"
    assert violations(fn(["v_mov_b32_e32 v5, v1", dpp]))[0]
    assert violations(fn(["v_mov_b32_e32 v5, v1", "s_nop 0", dpp]))[0]
    assert not violations(fn(["v_mov_b32_e32 v5, v1", "s_nop 1", dpp]))[0]
    assert not violations(fn(["v_mov_b32_e32 v5, v1", "v_mul_f32_e32 v6, v1, v1",
                              "v_mul_f32_e32 v7, v1, v1", dpp]))[0]
    # loop: the DPP read opens the body, the write closes it
    loop = [dpp, "v_mul_f32_e32 v8, v1, v1", "v_mov_b32_e32 v5, v8", "s_cbranch_scc1 0"]
    assert violations(fn(loop, targets={3: 0}))[0]
    assert not violations(fn(["s_nop 1"] + loop[:3] + ["s_nop 1", "s_cbranch_scc1 0"],
                             targets={5: 1}))[0]


def test_library_code_object_has_no_dpp_read_hazard():
    from vision_mamba_selective_amd import _native
    lib = _native.LIB_PATH
    assert os.path.exists(lib), "build the library first (__graft_entry__.build())"
    for tool in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip("ROCm LLVM tool %s not installed" % tool)
    funcs = disassemble(lib)
    bad, checked = violations(funcs)
    # the gradient kernel's broadcast-fmac and the row transpose are present
    assert checked > 1000
    assert any("rowgrad" in n for n in funcs)
    assert not bad, "\n".join(bad[:20])
