"""Static check of hand-placed memory waits in a kernel's gfx950 assembly.

Some decode kernels issue their vector-memory loads and LDS reads as inline
assembly and wait for them with explicit s_waitcnt counts, so the compiler
does not see when a load's destination registers are filled.  Were it to
copy, spill or reuse such a register before the wait, the kernel would read
stale data without any error.  This checker walks the kernel's control-flow
graph and tracks, for every path, the loads still in flight:

* vector-memory operations (buffer_, global_, flat_, scratch_) complete in
  issue order, so ``s_waitcnt vmcnt(N)`` leaves only the last N in flight;
* LDS and scalar-memory operations likewise, through ``lgkmcnt(N)`` (the
  compiler never waits with N > 0 while a scalar load is outstanding);

and reports every instruction other than a wait that names a VGPR a load in
flight has yet to fill.  Test infrastructure only.
"""

import collections
import re


def _vgprs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def kernels(asm: str, pattern: str):
    """Symbols of the kernels in `asm` whose name contains `pattern`."""
    return [m.group(1) for m in re.finditer(r"^(_Z\w+):", asm, re.M) if pattern in m.group(1)]


def _blocks(asm_lines, name):
    st = next(i for i, line in enumerate(asm_lines) if line.startswith(name + ":"))
    en = next(i for i in range(st, len(asm_lines)) if asm_lines[i].startswith(".Lfunc_end"))
    blocks, order, cur = {"entry": []}, ["entry"], "entry"
    for line in asm_lines[st + 1:en]:
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            cur = m.group(1)
            blocks[cur] = []
            order.append(cur)
            continue
        t = line.split(";")[0].strip()
        if t and not t.startswith("."):
            blocks[cur].append(t)
    return blocks, order


def _successors(blocks, order, b):
    i = order.index(b)
    nxt = order[i + 1] if i + 1 < len(order) else None
    ins = blocks[b]
    if ins:
        last = ins[-1]
        op = last.split()[0]
        if op == "s_branch":
            return [last.split()[1]]
        if op.startswith("s_cbranch"):
            return [last.split()[1]] + ([nxt] if nxt else [])
        if op in ("s_endpgm", "s_setpc_b64"):
            return []
    return [nxt] if nxt else []


def _step(state, t, issues, where):
    vmq, lgq = state
    op = t.split()[0]
    if op == "s_waitcnt":
        m = re.search(r"vmcnt\((\d+)\)", t)
        if m:
            n = int(m.group(1))
            vmq = vmq[len(vmq) - n:] if 0 < n < len(vmq) else (() if n == 0 else vmq)
        m = re.search(r"lgkmcnt\((\d+)\)", t)
        if m:
            n = int(m.group(1))
            lgq = lgq[len(lgq) - n:] if 0 < n < len(lgq) else (() if n == 0 else lgq)
        return vmq, lgq
    pending = set()
    for e in vmq + lgq:
        pending |= e
    hit = _vgprs(t) & pending
    if hit:
        issues.append((where, t, sorted(hit)))
    first = t.split(",")[0]
    if op.startswith(("buffer_", "global_", "flat_", "scratch_")):
        dest = set()
        if ("_load" in op and " lds" not in t) or ("_atomic" in op and " glc" in t):
            dest = _vgprs(first)
        vmq = vmq + (frozenset(dest),)
        if op.startswith("flat_"):
            lgq = lgq + (frozenset(dest),)
    elif op.startswith(("ds_read", "ds_load")) or "_rtn" in op or op.startswith(("ds_swizzle", "ds_bpermute", "ds_permute")):
        lgq = lgq + (frozenset(_vgprs(first)),)
    elif op.startswith(("ds_", "s_load", "s_buffer_load")):
        lgq = lgq + (frozenset(),)
    return vmq[-64:], lgq[-64:]


def check(asm: str, name: str, max_states: int = 400):
    """[(block+index, instruction, registers)] of every early use in kernel `name`."""
    blocks, order = _blocks(asm.split("\n"), name)
    seen = collections.defaultdict(set)
    work = [("entry", ((), ()))]
    issues = []
    while work:
        b, state = work.pop()
        if state in seen[b]:
            continue
        seen[b].add(state)
        if len(seen[b]) > max_states:
            raise RuntimeError(f"{name}: too many wait states at {b}")
        for i, t in enumerate(blocks[b]):
            state = _step(state, t, issues, f"{b}+{i}")
        for s2 in _successors(blocks, order, b):
            work.append((s2, state))
    return issues
