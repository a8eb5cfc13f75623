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
