"""Static check of the gfx950 assembly of the library's kernels for one hazard.

A vector-memory or LDS load must not write a VGPR that an MFMA issued before it
still reads: the product may not have read its operands when the load's data
lands.  The compiler does not always keep such registers apart (a chunk-scan
variant whose loads followed the products it feeds lost parity this way).
`load_over_mfma_operands(asm_text)` lists every load whose destination overlaps
an operand (A, B or C) of an MFMA whose result no instruction has read yet,
within one basic block.

A second rule: no MFMA may take as its accumulator (C operand) a register
whose last writer is an MFMA of another instruction shape.  On gfx950 the
compiler can leave too few wait states between a 16x16x32 product and a
16x16x16 product that reads its result as C (measured: stale rows in the
result).  `mfma_cross_shape_chains(asm_text)` lists every such pair; a chain
within one shape, or one that passes through a VALU instruction, is allowed.

Host-side test tooling only: the kernels never use it.
"""
import re

_REG = re.compile(r'v\[(\d+):(\d+)\]|\bv(\d+)\b')
_AREG = re.compile(r'a\[(\d+):(\d+)\]|\ba(\d+)\b')
_LOADS = ("ds_read", "global_load", "buffer_load")


def _regs(tok):
    out = set()
    for m in _REG.finditer(tok):
        if m.group(1):
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
        else:
            out.add(int(m.group(3)))
    return out


def _check_function(lines):
    found = []
    inflight = []  # (line number, destination VGPRs, operand VGPRs)
    for no, ln in lines:
        s = ln.strip()
        if not s or s.startswith(";") or s.startswith("."):
            if s.endswith(":"):
                inflight = []
            continue
        if s.endswith(":"):
            inflight = []
            continue
        op = s.split()[0]
        args = s[len(op):].split(",")
        if op.startswith("v_mfma"):
            dst, src = _regs(args[0]), set()
            for a in args[1:4]:
                src |= _regs(a)
            inflight = [x for x in inflight if not (x[1] & src)]  # chained on a pending result
            inflight.append((no, dst, src))
            continue
        if op.startswith(_LOADS) and "lds" not in op:
            dst = _regs(args[0])
            for mno, _, msrc in inflight:
                if dst & msrc:
                    found.append((no, s, mno))
            continue
        used = set()
        for a in args[1:]:
            used |= _regs(a)
        if op.startswith(("ds_write", "global_store", "buffer_store")):
            used |= _regs(args[0])
        inflight = [x for x in inflight if not (x[1] & used)]
    return found


def load_over_mfma_operands(asm_text):
    """[(function, line number, load instruction, line number of the MFMA)]"""
    out, name, cur = [], None, []
    for i, ln in enumerate(asm_text.splitlines(), 1):
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            if name:
                out += [(name, *f) for f in _check_function(cur)]
            name, cur = m.group(1), []
        elif name:
            cur.append((i, ln))
    if name:
        out += [(name, *f) for f in _check_function(cur)]
    return out


def _regs_any(tok):
    """VGPRs as ("v", n) and AGPRs as ("a", n)."""
    out = {("v", r) for r in _regs(tok)}
    for m in _AREG.finditer(tok):
        if m.group(1):
            out |= {("a", r) for r in range(int(m.group(1)), int(m.group(2)) + 1)}
        else:
            out.add(("a", int(m.group(3))))
    return out


def _cross_shape(lines):
    """Walks the function twice (the second pass sees what the end of the
    first left behind, which stands in for loop back edges); reports on the
    second pass only."""
    found = []
    writer = {}  # register -> mnemonic of the MFMA that last wrote it (None: other)
    for pass_ in range(2):
        for no, ln in lines:
            s = ln.strip()
            if not s or s.startswith((";", ".")) or s.endswith(":"):
                continue
            op = s.split()[0]
            args = s[len(op):].split(",")
            if not args or not args[0].strip():
                continue
            if op.startswith("v_mfma"):
                if len(args) >= 4:
                    for r in _regs_any(args[3]):
                        w = writer.get(r)
                        if w is not None and w != op and pass_ == 1:
                            found.append((no, s, w))
                            break
                for r in _regs_any(args[0]):
                    writer[r] = op
                continue
            # any other instruction writing a register (first operand) ends the chain
            if op.startswith(("v_", "ds_read", "global_load", "buffer_load", "flat_load",
                              "scratch_load")) and "store" not in op and "write" not in op:
                for r in _regs_any(args[0]):
                    writer[r] = None
    return found


def mfma_cross_shape_chains(asm_text):
    """[(function, line number, MFMA instruction, mnemonic of the MFMA that
    wrote its accumulator)]"""
    out, name, cur = [], None, []
    for i, ln in enumerate(asm_text.splitlines(), 1):
        m = re.match(r"^(_Z\S+):", ln)
        if m:
            if name:
                out += [(name, *f) for f in _cross_shape(cur)]
            name, cur = m.group(1), []
        elif name:
            cur.append((i, ln))
    if name:
        out += [(name, *f) for f in _cross_shape(cur)]
    return out
