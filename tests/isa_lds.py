"""A check over the gfx950 assembly of the library's own kernels: every path from an LDS read
(ds_read*) to an instruction that uses the read's destination registers must pass an
`s_waitcnt lgkmcnt(N)` that covers the read.

The kernels issue LDS reads in inline assembly and wait for them in separate statements that name
the destination registers, often a whole step later (behind MFMAs or a rescale).  Nothing in the
compiler knows that such an output is still in flight: a register copy it inserts before the wait
(at a loop back-edge, say) would read stale data.  This scan follows every branch of the kernel,
including loop back-edges, with the set of LDS reads still outstanding, and reports each
instruction that reads or overwrites one of their registers.  LDS returns complete in issue order,
so `lgkmcnt(N)` leaves the N most recent reads outstanding (the kernels have no scalar memory loads
in flight when they wait, which would break that order; `s_load` is not tracked).
"""
import re


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return frozenset(out)


def kernel_names(asm):
    """Mangled names of the kernels defined in an assembly listing."""
    return re.findall(r"^(_Z\S+):", asm, flags=re.M)


def _body(asm, name):
    ins, labels, on = [], {}, False
    for line in asm.split("\n"):
        if line.startswith(name + ":"):
            on = True
            continue
        if on and line.startswith(".Lfunc_end"):
            break
        if not on:
            continue
        t = line.split(";")[0].strip()
        if t.endswith(":"):
            labels[t[:-1]] = len(ins)
            continue
        if not t or t.startswith("."):
            continue
        ins.append(t)
    return ins, labels


def hazards(asm, name, depth=48):
    """[(instruction, the LDS read it races)] for kernel `name` of an assembly listing: an
    instruction that names (reads or writes) a register an outstanding LDS read will write."""
    ins, labels = _body(asm, name)
    seen, work, bad = set(), [(0, ())], set()
    while work:
        i, pend = work.pop()
        while i < len(ins):
            if (i, pend) in seen:
                break
            seen.add((i, pend))
            t = ins[i]
            op = t.split()[0]
            args = t[len(op):]
            wait = re.match(r"s_waitcnt\b.*lgkmcnt\((\d+)\)", t)
            if wait:
                n = int(wait.group(1))
                pend = pend[-n:] if n else ()
            elif op.startswith(("ds_read", "ds_load")):
                parts = args.split(",", 1)
                bad.update((i, o) for s, o in pend if _regs(args) & s)
                pend = (pend + ((_regs(parts[0]), i),))[-depth:]
            elif not op.startswith("s_"):
                # any operand: a read races the return, a write is overwritten by it
                used = _regs(args)
                bad.update((i, o) for s, o in pend if used & s)
            if op == "s_branch" or op.startswith("s_cbranch"):
                target = args.strip().split(",")[-1].strip()
                if target in labels:
                    work.append((labels[target], pend))
                if op == "s_branch":
                    break
            if op == "s_endpgm":
                break
            i += 1
    return [(ins[i], ins[o]) for i, o in sorted(bad)]
