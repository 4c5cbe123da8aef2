"""Static check of the library's gfx950 assembly for a scalar select that
reads a stale SCC flag.

A select of data (s_cselect with operands other than the -1/0 carry mask),
an s_cmov or an s_cbranch_scc reads SCC, which almost every SALU instruction
rewrites.  A select whose reaching SCC writer, followed back through the
predecessor blocks, is an add/sub with carry computes from that carry, not
from a comparison: a hipcc of this toolchain produced one for a 64-bit
min() whose branch had been taken on VCC (a tail-window length that came
out as the full window).  The check lists every such site."""
import re

_WRITER = re.compile(
    r"^\s+(s_(add|addc|sub|subb)_u32|s_(add|sub)_i32|s_lshl_b(32|64)|s_lshr_b(32|64)|s_ashr_i(32|64)|"
    r"s_and_b(32|64)|s_or_b(32|64)|s_xor_b(32|64)|s_andn2_b(32|64)|s_orn2_b(32|64)|s_nand_b\d+|s_nor_b\d+|"
    r"s_xnor_b\d+|s_not_b(32|64)|s_bfe_\w+|s_cmp\w*|s_bitcmp\w*|s_min_\w+|s_max_\w+|s_\w+_saveexec_b64|"
    r"s_mul_i32|s_lshl\d_add_u32|s_abs\w*|s_bcnt\w*|s_absdiff\w*)\b")
_LABEL = re.compile(r"^(\.LBB\w+):")
_FUNC = re.compile(r"^(_Z\w+):")
_BRANCH = re.compile(r"^\s+s_(cbranch_\w+|branch)\s+(\.LBB\w+)")
_NOFALL = re.compile(r"^\s+(s_branch|s_endpgm|s_setpc_b64)\b")
_CARRY = ("s_add_u32", "s_addc_u32", "s_sub_u32", "s_subb_u32")


def stale_scc_selects(asm: str):
    """[(function, line, instruction, writer line, writer)] of SCC readers
    whose reaching SCC writer is a carry-producing add/sub."""
    lines = asm.splitlines()
    branches = {}
    for i, line in enumerate(lines):
        m = _BRANCH.match(line)
        if m:
            branches.setdefault(m.group(2), []).append(i)

    def reaching(i, seen):
        j = i - 1
        while j >= 0:
            line = lines[j]
            if _WRITER.match(line):
                return [j]
            if _FUNC.match(line):
                return []
            m = _LABEL.match(line)
            if m:
                lab = m.group(1)
                if lab in seen:
                    return []
                seen.add(lab)
                preds = list(branches.get(lab, []))
                k = j - 1
                while k >= 0 and not lines[k].startswith("\t") and not _LABEL.match(lines[k]) and not _FUNC.match(lines[k]):
                    k -= 1
                if k >= 0 and not _NOFALL.match(lines[k]):
                    preds.append(j)
                out = []
                for p in preds:
                    out += reaching(p, seen)
                return out
            j -= 1
        return []

    found = []
    func = None
    for i, line in enumerate(lines):
        m = _FUNC.match(line)
        if m:
            func = m.group(1)
        t = line.strip()
        data_select = t.startswith("s_cselect") and not re.search(r", (-1, 0|0, -1)$", t)
        if data_select or t.startswith("s_cbranch_scc") or t.startswith("s_cmov"):
            for j in reaching(i, set()):
                if lines[j].split()[0] in _CARRY:
                    found.append((func, i + 1, t, j + 1, lines[j].strip()))
    return found
