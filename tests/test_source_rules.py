"""Rules for the HIP sources that the compiler does not enforce (CPU only).

Inline-asm register loads: the compiler takes the output of an asm statement
as written when the statement ends, although the hardware writes it only when
the load lands.  A use of the value may then be scheduled above a bare
`s_waitcnt`, and the destination register handed to other work while the load
is still in flight.  Every asm register load in the library is therefore
waited for by an asm statement that names its destination as a "+v" operand.
This test scans the kernel sources for that pattern, and checks on planted
snippets that the scan catches the mistakes it is meant to catch.
"""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_integer_amd", "csrc")


def _strip_comments(text):
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return re.sub(r"//[^\n]*", " ", text)


def asm_statements(text):
    """The argument text of every `asm`/`__asm__` statement, with its offset."""
    text = _strip_comments(text)
    out = []
    for mt in re.finditer(r"\b(?:asm|__asm__)\s*(?:volatile|__volatile__)?\s*\(", text):
        i, depth, in_str = mt.end(), 1, False
        while i < len(text) and depth:
            c = text[i]
            if in_str:
                if c == "\\":
                    i += 1
                elif c == '"':
                    in_str = False
            elif c == '"':
                in_str = True
            elif c == "(":
                depth += 1
            elif c == ")":
                depth -= 1
            i += 1
        out.append((mt.start(), text[mt.end(): i - 1]))
    return out


def _template(body):
    """The instruction text: the leading string literals of the statement."""
    m = re.match(r'\s*((?:"(?:[^"\\]|\\.)*"\s*)+)', body)
    return "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', m.group(1))) if m else ""


def _operands(body, constraint):
    """Base names of the operands bound to `constraint` (e.g. "=v", "+v")."""
    names = re.findall(r'"%s"\s*\(\s*([A-Za-z_]\w*)' % re.escape(constraint), body)
    return set(names)


REG_LOAD = re.compile(r"\b(?:global|buffer|flat|scratch)_load_(?!lds)\w+")


def violations(text):
    """Register loads (asm, with a "=v" destination) whose destination is
    named by no asm s_waitcnt statement as a "+v" operand."""
    loads, waited = [], set()
    for pos, body in asm_statements(text):
        tmpl = _template(body)
        if REG_LOAD.search(tmpl):
            dst = _operands(body, "=v")
            if not dst:
                loads.append((pos, "<register load without a named \"=v\" destination>"))
            loads.extend((pos, d) for d in dst)
        if "s_waitcnt" in tmpl:
            waited |= _operands(body, "+v")
    return [(pos, d) for pos, d in loads if d not in waited]


def test_kernel_sources_wait_for_asm_register_loads_by_name():
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")))
    assert files
    bad = []
    for f in files:
        with open(f) as fh:
            for pos, name in violations(fh.read()):
                bad.append("%s: asm register load into %s" % (os.path.basename(f), name))
    assert not bad, "asm register loads not waited for through their registers:\n" + "\n".join(bad)


def test_scan_catches_planted_mistakes():
    good = '''
      uint32_t a;
      asm volatile("global_load_ushort %0, %1, off" : "=v"(a) : "v"(p) : "memory");
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(a) :: "memory");
    '''
    assert violations(good) == []
    # a bare wait does not name the register
    bare = good.replace('asm volatile("s_waitcnt vmcnt(0)" : "+v"(a) :: "memory");',
                        '__builtin_amdgcn_s_waitcnt(0);')
    assert [d for _, d in violations(bare)] == ["a"]
    # a wait that names a different register
    other = good.replace('"+v"(a) ::', '"+v"(b) ::')
    assert [d for _, d in violations(other)] == ["a"]
    # a wave-wide load into two registers, only one of them waited for
    two = '''
      asm volatile("global_load_ushort %0, %2, off\\n\\tglobal_load_ushort %1, %3, off"
                   : "=v"(x), "=v"(y) : "v"(p), "v"(q) : "memory");
      asm volatile("s_waitcnt vmcnt(0)" : "+v"(x) :: "memory");
    '''
    assert [d for _, d in violations(two)] == ["y"]
    # direct-to-LDS loads write no register and need no named wait
    dma = 'asm volatile("s_nop 0\\n\\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(b) : "memory");'
    assert violations(dma) == []
    # commented-out code is ignored
    assert violations("// " + bare.replace("\n", "\n// ")) == []


# ---------------------------------------------------------------------------
# The same rule on the compiled code: between an asm register load and the
# asm wait that names its destination, no instruction may read or overwrite
# the destination register (the compiler may copy an asm output as soon as
# the asm statement ends, e.g. to reconcile registers across a loop, and such
# a copy reads the register before the load has written it).
# ---------------------------------------------------------------------------

import shutil
import subprocess

import pytest

HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _compile_to_asm(src):
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
             "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), src, "-o", "-"]
    r = subprocess.run([HIPCC] + flags, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    assert r.returncode == 0, "hipcc failed on %s" % src
    return r.stdout


def _vregs(code):
    """Numbers of the vector registers an instruction line mentions
    (single registers such as v52 and ranges such as v[52:55])."""
    regs = set()
    for lo, hi in re.findall(r"\bv\[(\d+):(\d+)\]", code):
        regs.update(range(int(lo), int(hi) + 1))
    regs.update(int(r) for r in re.findall(r"\bv(\d+)\b", code))
    return regs


LOAD_LINE = re.compile(r"(?:global|buffer|flat|scratch)_load_(?!lds)\w+\s+(v\[\d+:\d+\]|v\d+)")


def asm_load_violations(text):
    """Scan compiled GCN assembly in program order: for each register load
    emitted from inline asm, the lines up to the next inline-asm s_waitcnt
    must not mention any register the load writes."""
    bad = []
    in_asm = False
    pending = {}  # register number -> line of its load
    for i, line in enumerate(text.splitlines()):
        code = line.split(";")[0].strip()
        if line.strip().startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.strip().startswith(";;#ASMEND"):
            in_asm = False
            continue
        if in_asm:
            if "s_waitcnt" in code:
                pending.clear()
            m = LOAD_LINE.match(code)
            if m:
                for r in _vregs(m.group(1)):
                    pending[r] = i
            continue
        if not code or not pending:
            continue
        hit = _vregs(code) & set(pending)
        for r in sorted(hit):
            bad.append("line %d uses v%d loaded at line %d: %s" % (i + 1, r, pending.pop(r) + 1, code))
    return bad


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_compiled_kernels_leave_asm_loaded_registers_alone_until_the_wait():
    checked = 0
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        with open(f) as fh:
            src = fh.read()
        if not any(REG_LOAD.search(_template(b)) for _, b in asm_statements(src)):
            continue
        bad = asm_load_violations(_compile_to_asm(f))
        assert not bad, "%s:\n%s" % (os.path.basename(f), "\n".join(bad[:10]))
        checked += 1
    assert checked >= 1


def test_asm_scan_catches_a_copy_before_the_wait():
    good = """
	;;#ASMSTART
	global_load_ushort v52, v1, s[2:3]
	;;#ASMEND
	v_add_u32_e32 v3, 4, v2
	;;#ASMSTART
	s_waitcnt vmcnt(0)
	;;#ASMEND
	v_cvt_f32_f16_e32 v4, v52
"""
    assert asm_load_violations(good) == []
    bad = good.replace("v_add_u32_e32 v3, 4, v2", "v_mov_b32_e32 v103, v52")
    assert len(asm_load_violations(bad)) == 1
    # a wide load and a use through a register range that overlaps it
    wide = good.replace("global_load_ushort v52", "global_load_dwordx2 v[52:53]")
    assert asm_load_violations(wide) == []
    assert len(asm_load_violations(wide.replace("v_add_u32_e32 v3, 4, v2",
                                                "v_pk_mov_b32 v[60:61], v[53:54], v[53:54] op_sel:[0,1]"))) == 1
    # registers that merely share digits are not the loaded one
    assert asm_load_violations(good.replace("v_add_u32_e32 v3, 4, v2", "v_add_u32_e32 v152, v5, v520")) == []
