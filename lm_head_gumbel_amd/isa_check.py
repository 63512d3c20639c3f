"""Build-time check of hand-counted memory waits in gfx950 assembly.

Some kernels issue global loads from inline assembly, which the compiler does
not track, and wait for them with explicit `s_waitcnt vmcnt(N)`.  The
compiler still owns the destination registers of such a load: it believes
them written when the instruction issues, so it may copy, spill or reuse them
before the data has arrived.  Any of these corrupts results, and a reused
address register can turn into a memory fault.  This module proves, on the
assembly the compiler actually emitted, that no instruction touches a
register of an untracked load before a wait retires that load.

The analysis is a forward data-flow pass over each kernel's control-flow
graph.  The state is the set of untracked loads in flight, each with the
smallest number of vector-memory loads issued after it on any path.  Rules:

* a load from an inline-assembly block (between ;;#ASMSTART and ;;#ASMEND)
  enters the set;
* every vector-memory load (global_, buffer_, scratch_ loads, tracked or not)
  adds one to the count of each older entry.  Stores do not count: they may
  complete out of order with loads, so they never help retire one;
* `s_waitcnt vmcnt(N)` retires every entry with count >= N (loads return in
  order);
* any other use or definition of a register of an entry in flight is an
  error, and so are flat memory instructions (they count in two counters
  and may complete out of order), calls, and instructions that write M0.
  The compiler's long jumps (s_getpc_b64, s_add_u32 of the label offset,
  s_setpc_b64) are branches.

Usage:  python -m lm_head_gumbel_amd.isa_check file.s [...]
"""
import re
import sys

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_FUNC = re.compile(r"^([A-Za-z_][\w.$]*):")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")
_CAP = 64   # vmcnt never exceeds 63 on gfx9: a count of 64 is retired by any wait


def _regs(text):
    """Set of ('v'|'a', index) named in an operand string."""
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


class Instr:
    __slots__ = ("line", "op", "args", "asm")

    def __init__(self, line, op, args, asm):
        self.line, self.op, self.args, self.asm = line, op, args, asm


def _functions(lines):
    """(name, [(label or None, [Instr])]) per function in an assembly file."""
    funcs = []
    cur = None
    in_asm = False
    for no, raw in enumerate(lines, 1):
        text = raw.split(";", 1)[0].rstrip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        if raw.strip().startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.strip().startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not text.strip():
            continue
        m = _FUNC.match(text)
        if m and not text.startswith(".") and cur is None or (m and m.group(1).startswith("_Z")):
            if m.group(1).startswith("_Z"):
                cur = (m.group(1), [(None, [])])
                funcs.append(cur)
                continue
        if cur is None:
            continue
        if text.startswith(".Lfunc_end"):
            cur = None
            continue
        lm = _LABEL.match(text)
        if lm:
            cur[1].append((lm.group(1), []))
            continue
        s = text.strip()
        if s.startswith("."):
            continue   # directive
        parts = s.split(None, 1)
        cur[1][-1][1].append(Instr(no, parts[0], parts[1] if len(parts) > 1 else "", in_asm))
    return funcs


_LONG = re.compile(r"\((\.LBB\d+_\d+)-\.Lpost_getpc\d+\)")


def _long_jump_target(instrs, i):
    """Target of the long jump s_getpc_b64 / s_add_u32 (label - .Lpost_getpc)
    / s_addc_u32 / s_setpc_b64 that ends at instrs[i], or None."""
    for back in range(i - 1, max(-1, i - 4), -1):
        m = _LONG.search(instrs[back].args)
        if m and instrs[back].op == "s_add_u32":
            return m.group(1)
    return None


def _ends_block(instrs, i):
    op = instrs[i].op
    return (op.startswith("s_branch") or op.startswith("s_cbranch") or op == "s_endpgm"
            or (op == "s_setpc_b64" and _long_jump_target(instrs, i) is not None))


def _blocks(body):
    """Basic blocks: (name, instrs, successors), split after branches."""
    blocks = []
    for label, instrs in body:
        name = label or "<entry>"
        cur = []
        k = 0
        for i, ins in enumerate(instrs):
            cur.append(ins)
            if _ends_block(instrs, i):
                blocks.append([name if k == 0 else "%s+%d" % (name, k), cur])
                cur = []
                k += 1
        if cur or k == 0:
            blocks.append([name if k == 0 else "%s+%d" % (name, k), cur])
    out = []
    for i, (name, instrs) in enumerate(blocks):
        succ = []
        last = instrs[-1] if instrs else None
        nxt = blocks[i + 1][0] if i + 1 < len(blocks) else None
        if last is None:
            if nxt:
                succ.append(nxt)
        elif last.op == "s_endpgm":
            pass
        elif last.op.startswith("s_branch"):
            succ.append(last.args.split()[0])
        elif last.op == "s_setpc_b64":
            succ.append(_long_jump_target(instrs, len(instrs) - 1))
        elif last.op.startswith("s_cbranch"):
            succ.append(last.args.split()[0])
            if nxt:
                succ.append(nxt)
        elif nxt:
            succ.append(nxt)
        out.append((name, instrs, succ))
    return out


def _is_vm_load(op):
    return (op.startswith("global_load") or op.startswith("buffer_load")
            or op.startswith("scratch_load"))


def _is_vm(op):
    return op.startswith(("global_", "buffer_", "scratch_"))


def _transfer(state, instrs, errors, fname):
    """Apply a block to the state {load line: (regs, count)}; append errors."""
    st = dict(state)
    for ins in instrs:
        op = ins.op
        if op.startswith("flat_"):
            errors.append("%s line %d: flat memory instruction %s" % (fname, ins.line, op))
        if op in ("s_swappc_b64", "s_call_b64") or (
                op == "s_setpc_b64" and ins is not instrs[-1]):
            errors.append("%s line %d: call %s" % (fname, ins.line, op))
        if not ins.asm and re.match(r"^\s*m0\b", ins.args) and op.startswith("s_"):
            errors.append("%s line %d: writes m0" % (fname, ins.line))
        if op.startswith("s_waitcnt"):
            if op != "s_waitcnt":
                errors.append("%s line %d: unhandled wait %s" % (fname, ins.line, op))
                continue
            m = _VMCNT.search(ins.args)
            if m:
                n = int(m.group(1))
                st = {k: v for k, v in st.items() if v[1] < n}
            continue
        used = _regs(ins.args)
        untracked_load = ins.asm and _is_vm_load(op)
        dest = set()
        if untracked_load:
            first = ins.args.split(",", 1)[0]
            dest = _regs(first)
            used = _regs(ins.args.split(",", 1)[1]) if "," in ins.args else set()
        for key, (regs, _) in st.items():
            clash = (used | dest) & regs
            if clash:
                errors.append("%s line %d: %s %s touches a register of the load from line %d "
                              "still in flight (%s)" % (fname, ins.line, op, ins.args, key,
                                                       ",".join("%s%d" % r for r in sorted(clash))))
        if _is_vm_load(op):
            st = {k: (r, min(c + 1, _CAP)) for k, (r, c) in st.items()}
        if untracked_load:
            st[ins.line] = (frozenset(dest), 0)
        elif ins.asm and _is_vm(op):
            errors.append("%s line %d: untracked %s (only loads are handled)" % (fname, ins.line, op))
    return st


def _merge(a, b):
    out = dict(a)
    for k, (r, c) in b.items():
        out[k] = (r, min(c, out[k][1])) if k in out else (r, c)
    return out


def check_function(name, body):
    """Errors (strings) for one function; empty if every untracked load is
    retired before its registers are touched."""
    blocks = _blocks(body)
    index = {b[0]: i for i, b in enumerate(blocks)}
    entry = [None] * len(blocks)
    entry[0] = {}
    work = [0]
    errors = []
    while work:
        i = work.pop()
        name_b, instrs, succ = blocks[i]
        out = _transfer(entry[i], instrs, [], name)
        for s in succ:
            if s not in index:
                errors.append("%s: branch to unknown label %s" % (name, s))
                continue
            j = index[s]
            new = out if entry[j] is None else _merge(entry[j], out)
            if new != entry[j]:
                entry[j] = new
                work.append(j)
    for i, (name_b, instrs, _) in enumerate(blocks):
        if entry[i] is not None:
            _transfer(entry[i], instrs, errors, name)
    return sorted(set(errors))


def check_text(text, require_untracked=False):
    """Errors for every function of an assembly listing.  With
    require_untracked, a listing without any untracked load is an error too
    (the check would be vacuous)."""
    lines = text.splitlines()
    errors = []
    seen = 0
    for name, body in _functions(lines):
        seen += sum(1 for _, ins in body for i in ins if i.asm and _is_vm_load(i.op))
        errors += check_function(name, body)
    if require_untracked and seen == 0:
        errors.append("no untracked loads found")
    return errors


def main(argv):
    bad = 0
    for path in argv:
        with open(path) as f:
            errs = check_text(f.read())
        for e in errs:
            print(path + ": " + e)
        bad += len(errs)
    print("%d problem(s)" % bad)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
