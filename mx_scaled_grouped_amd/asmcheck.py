"""Wait-state checks on the GEMM kernels' device assembly.

Two rules the compiler cannot be left to keep, checked on the built code:
the wait states before the inline-asm direct-to-LDS copies (below), and the
distance between an MFMA and a non-MFMA read of its result (further down).

The GEMM kernels issue their global->LDS copies (``buffer_load_* ... lds``,
``global_load_lds_*``) through inline asm, so that the compiler inserts no
``s_waitcnt`` for them. The price is that the compiler's hazard recognizer
does not know these are vector-memory instructions and pads none of the
wait states that the CDNA3/CDNA4 ISA requires before them:

* a VALU write of an SGPR (``v_readlane``, ``v_readfirstlane``, a VOP3
  compare or carry-out) followed by a vector-memory read of that SGPR (the
  buffer resource, the soffset, or M0 for the LDS address) needs 5 wait
  states; the compiler reloads spilled SGPRs with ``v_readlane`` right before
  their use, so whether this happens depends on register allocation;
* an SALU write of M0 followed by an LDS DMA needs 1 wait state (LLVM
  applies this to every GFX9 target).

The copy helpers cover what they can themselves (an SALU copy of the soffset
and a ``s_nop 0`` inside the asm); this check proves the rest on the built
code: every path into every copy is walked backwards through labels and
branches, counting ``s_nop N`` as N+1 wait states and any other instruction
as one, and any write of an SGPR the copy reads that comes too close is
reported. ``python -m mx_scaled_grouped_amd.asmcheck file.s`` prints them.
"""
from __future__ import annotations

import re
import sys
from dataclasses import dataclass

VALU_SGPR_WAIT = 5   # VALU writes an SGPR -> VMEM reads it
SALU_M0_WAIT = 1     # SALU writes M0 -> LDS DMA reads it

# VOP3b encodings whose second operand is an SGPR (carry or condition) output
_VOP3B = re.compile(r"^v_(add|sub|subrev|addc|subb|subbrev)_co_|^v_div_scale_|^v_mad_[iu]64_[iu]32")
_BRANCH = re.compile(r"^s_(c?branch\w*|cbranch_\w+)\s+(\S+)")
_NO_FALLTHROUGH = re.compile(r"^s_(branch|endpgm|setpc_b64|trap)\b")


@dataclass
class Finding:
    kernel: str
    copy: str        # the copy instruction
    writer: str      # the instruction that writes a register it reads
    reg: str
    distance: int    # wait states between them
    needed: int

    def __str__(self) -> str:
        return (f"{self.kernel}: '{self.writer}' writes {self.reg} {self.distance} wait state(s) "
                f"before '{self.copy}' (needs {self.needed})")


def sgprs(tok: str) -> set:
    """SGPR names in one operand token: s7, s[4:7], m0, vcc, vcc_lo, vcc_hi."""
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    if re.fullmatch(r"s\d+", tok) or tok == "m0":
        return {tok}
    if tok == "vcc":
        return {"vcc_lo", "vcc_hi"}
    if tok in ("vcc_lo", "vcc_hi"):
        return {tok}
    return set()


def operands(ins: str) -> list:
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def is_lds_copy(ins: str) -> bool:
    op = ins.split(None, 1)[0]
    if op.startswith("global_load_lds_"):
        return True
    return op.startswith("buffer_load_") and re.search(r"\blds\b", ins) is not None


def copy_reads(ins: str) -> set:
    """SGPRs an LDS copy reads: its scalar operands, and M0 (the LDS address)."""
    regs = {"m0"}
    for o in operands(ins):
        for w in o.split():
            regs |= sgprs(w)
    return regs


def written_sgprs(ins: str) -> tuple:
    """(kind, SGPRs written) for an instruction; kind is 'valu', 'salu' or ''."""
    op = ins.split(None, 1)[0]
    ops = operands(ins)
    if not ops:
        return "", set()
    if op.startswith("v_"):
        out = set()
        for w in ops[0].split():
            out |= sgprs(w)
        if _VOP3B.match(op) and len(ops) > 1:
            out |= sgprs(ops[1].split()[0])
        if op.startswith("v_cmp") and "_e32" in op:
            out |= {"vcc_lo", "vcc_hi"}
        return "valu", out
    if op.startswith("s_") and not op.startswith(("s_nop", "s_waitcnt", "s_barrier", "s_branch", "s_cbranch",
                                                  "s_endpgm", "s_setprio", "s_sleep", "s_sendmsg")):
        out = set()
        for w in ops[0].split():
            out |= sgprs(w)
        return "salu", out
    return "", set()


def wait_states(ins: str) -> int:
    m = re.match(r"s_nop\s+(\w+)", ins)
    return int(m.group(1), 0) + 1 if m else 1


def split_kernels(text: str):
    """Yield (name, [lines]) for each function body in a device .s file."""
    tops = [m for m in re.finditer(r"^([A-Za-z_$][\w.$]*):\s*(?:;.*)?$", text, re.M)]
    for n, m in enumerate(tops):
        end = tops[n + 1].start() if n + 1 < len(tops) else len(text)
        fe = text.find(".Lfunc_end", m.end(), end)
        yield m.group(1), text[m.end():fe if fe >= 0 else end].split("\n")


def _body(lines):
    """Instructions and labels of one function: [('L', name) | ('I', text)]."""
    out = []
    for raw in lines:
        s = raw.split(";", 1)[0].strip()
        if not s:
            continue
        m = re.fullmatch(r"([.\w$]+):", s)
        if m:
            out.append(("L", m.group(1)))
        elif not s.startswith("."):
            out.append(("I", s))
    return out


def check_function(name: str, lines) -> list:
    body = _body(lines)
    label_at = {v: i for i, (k, v) in enumerate(body) if k == "L"}
    jumps = {}
    for i, (k, v) in enumerate(body):
        if k == "I":
            m = _BRANCH.match(v)
            if m and m.group(2) in label_at:
                jumps.setdefault(m.group(2), []).append(i)
    findings = []

    def walk(pos, copy, reads, dist, seen):
        # examine the instructions before position pos, `dist` wait states away
        i = pos - 1
        while i >= 0:
            k, v = body[i]
            if k == "L":
                for j in jumps.get(v, ()):
                    if (j, dist) not in seen:  # the branch itself is one wait state
                        seen.add((j, dist))
                        walk(j, copy, reads, dist + 1, seen)
                if i > 0 and body[i - 1][0] == "I" and _NO_FALLTHROUGH.match(body[i - 1][1]):
                    return
                i -= 1
                continue
            if dist >= VALU_SGPR_WAIT:
                return
            kind, regs = written_sgprs(v)
            hit = regs & reads
            if kind == "valu" and hit:
                findings.append(Finding(name, copy, v, sorted(hit)[0], dist, VALU_SGPR_WAIT))
            elif kind == "salu" and "m0" in hit and dist < SALU_M0_WAIT:
                findings.append(Finding(name, copy, v, "m0", dist, SALU_M0_WAIT))
            if hit:
                reads = reads - hit  # an older write of the same register is superseded
                if not reads:
                    return
            dist += wait_states(v)
            i -= 1

    for i, (k, v) in enumerate(body):
        if k == "I" and is_lds_copy(v):
            walk(i, v, copy_reads(v), 0, set())
    return findings


# ---- reads of MFMA results -------------------------------------------------
#
# The compiler's own wait states after v_mfma_scale were seen to be too few
# for a VALU or LDS read of the result (stale values), so the kernels keep a
# stricter rule of their own: a non-MFMA instruction reads an MFMA's
# destination only after at least two further MFMAs have issued (each of
# them occupies the matrix pipe for its full latency) or after MFMA_READ_WAIT
# wait states (explicit s_nop padding). This part checks that rule on the
# built code, along every path, as for the copies above.

MFMA_READ_WAIT = 40
MFMA_BEHIND = 2


def vregs(tok: str) -> set:
    """VGPR/AGPR names in one operand token: v7, v[4:7], a3, a[0:15]."""
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {f"{m.group(1)}{k}" for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    if re.fullmatch(r"[va]\d+", tok):
        return {tok}
    return set()


_STORE = re.compile(r"^(ds_write|ds_store|global_store|buffer_store|flat_store|scratch_store|global_atomic|buffer_atomic|ds_add|ds_max|ds_min)")


def vector_reads(ins: str) -> set:
    """VGPRs/AGPRs an instruction reads (its sources; all operands of a store or LDS copy)."""
    op = ins.split(None, 1)[0]
    ops = operands(ins)
    if op.startswith("s_") or not ops:
        return set()
    first = 0 if (_STORE.match(op) or is_lds_copy(ins)) else 1
    if _VOP3B.match(op):
        first = 2
    out = set()
    for o in ops[first:]:
        for w in o.split():
            out |= vregs(w)
    return out


def vector_writes(ins: str) -> set:
    """VGPRs/AGPRs a non-store instruction writes (its first operand)."""
    op = ins.split(None, 1)[0]
    ops = operands(ins)
    if op.startswith("s_") or not ops or _STORE.match(op) or is_lds_copy(ins):
        return set()
    return vregs(ops[0].split()[0])


def mfma_dest(ins: str) -> set:
    if not ins.startswith("v_mfma"):
        return set()
    ops = operands(ins)
    return vregs(ops[0].split()[0]) if ops else set()


def check_mfma_reads(name: str, lines) -> list:
    body = _body(lines)
    written = set()
    for k, v in body:
        if k == "I":
            written |= mfma_dest(v)
    if not written:
        return []
    label_at = {v: i for i, (k, v) in enumerate(body) if k == "L"}
    jumps = {}
    for i, (k, v) in enumerate(body):
        if k == "I":
            m = _BRANCH.match(v)
            if m and m.group(2) in label_at:
                jumps.setdefault(m.group(2), []).append(i)
    findings = []

    def walk(pos, reader, reads, dist, behind, seen):
        i = pos - 1
        while i >= 0:
            k, v = body[i]
            if k == "L":
                for j in jumps.get(v, ()):
                    if (j, dist, behind) not in seen:
                        seen.add((j, dist, behind))
                        walk(j, reader, reads, dist + 1, behind, seen)
                if i > 0 and body[i - 1][0] == "I" and _NO_FALLTHROUGH.match(body[i - 1][1]):
                    return
                i -= 1
                continue
            if dist >= MFMA_READ_WAIT:
                return
            if v.startswith("v_mfma"):
                hit = mfma_dest(v) & reads
                if hit:
                    findings.append(Finding(name, reader, v, sorted(hit)[0], dist, MFMA_READ_WAIT))
                    return
                behind += 1
                if behind >= MFMA_BEHIND:
                    return
            else:
                reads = reads - vector_writes(v)  # the read sees this later write
                if not reads:
                    return
            dist += wait_states(v)
            i -= 1

    for i, (k, v) in enumerate(body):
        if k != "I" or v.startswith("v_mfma"):
            continue
        reads = vector_reads(v) & written
        if reads:
            walk(i, v, reads, 0, 0, set())
    return findings


def check_text(text: str) -> list:
    out = []
    for name, lines in split_kernels(text):
        out.extend(check_function(name, lines))
        out.extend(check_mfma_reads(name, lines))
    return out


def main(argv) -> int:
    bad = 0
    for path in argv:
        with open(path) as f:
            found = check_text(f.read())
        for x in found:
            print(f"{path}: {x}")
        bad += len(found)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
