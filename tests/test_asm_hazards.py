"""Wait states around the kernels' inline asm (CPU: compiles to gfx950 assembly and reads it).

The compiler inserts the wait states that CDNA requires between dependent instructions only
where it knows both ends.  Two cases involve the encoder's inline asm (the lane-mask compares
and their consumers in quantize.hip):

* an MFMA writes VGPRs that a VALU instruction reads: the read must come several wait states
  later (up to 19 for a 16-pass XDL op).  The compiler does not count an asm statement as
  such a reader, so an asm compare issued right after the MFMA reads the old accumulator.
  This happened once: the comparison read a partial sum and a QJL sign came out wrong.
* a VALU instruction writes an SGPR (a compare's lane mask) that a VALU instruction reads as
  a mask or carry: the compiler keeps at least one wait state between them when it emits the
  writer as asm, but not when it emits the writer itself and the reader is asm.

The scan below walks every kernel of every source that holds inline asm and checks, for each
VALU instruction inside an asm block, the issue distance from the last writer of each register
it reads (an instruction counts one wait state, s_nop N counts N + 1).  Branches reset the
record, which is exact for the straight-line tile code that holds the asm.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from kv_cache_embedding_amd import build as tq_build

MFMA_TO_VALU = 19       # the longest XDL write -> VALU read requirement (16-pass ops)
VALU_SGPR_TO_VALU = 1   # what the compiler itself keeps between such a pair


def _regs(tok: str) -> set[tuple[str, int]]:
    tok = tok.strip().strip("|").lstrip("-")
    m = re.fullmatch(r"([vs])(\d+)", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    m = re.fullmatch(r"([vs])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    return set()


def scan(lines: list[str]) -> list[tuple[str, int, str]]:
    """Violations in one kernel's assembly: (kind, distance, instruction)."""
    in_asm = False
    last: dict[tuple[str, int], tuple[str, int]] = {}
    pos = 0
    bad = []
    for raw in lines:
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        op = t.split()[0]
        if op == "s_nop":
            pos += int(t.split()[1], 0) + 1
            continue
        if op.startswith(("s_cbranch", "s_branch", "s_setpc", "s_swappc")):
            last.clear()
        args = [a.split()[0] for a in t[len(op):].split(",") if a.strip()]
        if in_asm and op.startswith("v_"):
            found = {}
            for a in args[1:]:
                for r in _regs(a):
                    if r not in last:
                        continue
                    kind, p = last[r]
                    if r[0] == "v" and kind == "mfma" and pos - p < MFMA_TO_VALU:
                        found["mfma->asm"] = min(found.get("mfma->asm", pos - p), pos - p)
                    if r[0] == "s" and kind == "valu" and pos - p <= VALU_SGPR_TO_VALU:
                        found["valu sgpr->asm"] = min(found.get("valu sgpr->asm", pos - p), pos - p)
            bad.extend((k, d, t) for k, d in found.items())
        written = _regs(args[0]) if args else set()
        # v_addc/v_add_co/v_sub_co in VOP3 form: the second operand is the carry-out pair
        if op.startswith(("v_addc", "v_add_co", "v_sub_co", "v_subb")) and op.endswith("_e64") and len(args) > 1:
            written |= _regs(args[1])
        kind = "mfma" if op.startswith(("v_mfma", "v_smfmac")) else ("valu" if op.startswith("v_") else "other")
        for r in written:
            last[r] = (kind, pos)
        pos += 1
    return bad


def kernels(asm_text: str) -> dict[str, list[str]]:
    out, name, body = {}, None, []
    for line in asm_text.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            if line.strip().startswith("s_endpgm"):
                out[name] = body
                name = None
            else:
                body.append(line)
    return out


def test_scan_finds_planted_hazards():
    close = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
             ";;#ASMSTART", "v_cmp_ge_f32_e64 s[6:7], |v15|, v30", ";;#ASMEND"]
    assert [k for k, _, _ in scan(close)] == ["mfma->asm"]
    far = close[:1] + ["s_nop 7", "s_nop 7", "s_nop 2"] + close[1:]
    assert scan(far) == []
    mask = ["v_cmp_ge_f32_e64 s[6:7], |v1|, v2", ";;#ASMSTART",
            "v_addc_co_u32_e64 v3, s[8:9], v3, v3, s[6:7]", ";;#ASMEND"]
    assert [k for k, _, _ in scan(mask)] == ["valu sgpr->asm"]
    assert scan(mask[:1] + ["s_nop 0"] + mask[1:]) == []


def _asm_sources() -> list[str]:
    srcs = []
    for s in tq_build.sources():
        if s.endswith(".hip") and re.search(r"\basm\s*(volatile\s*)?\(\s*\"[^\"]", open(s).read()):
            srcs.append(s)
    return srcs


@pytest.mark.skipif(not os.path.exists(tq_build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
@pytest.mark.parametrize("src", [os.path.basename(s) for s in _asm_sources()])
def test_inline_asm_keeps_wait_states(src, tmp_path):
    path = os.path.join(tq_build.CSRC, src)
    out = tmp_path / (src + ".s")
    cmd = [tq_build.HIPCC, *tq_build.COMMON, "-x", "hip", "--cuda-device-only", "-S", path, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    ks = kernels(out.read_text())
    assert ks, "no kernels found in the assembly"
    report = {name: scan(body) for name, body in ks.items()}
    bad = {name: v[:3] for name, v in report.items() if v}
    assert not bad, f"{len(bad)} of {len(ks)} kernels read too early from inline asm: {bad}"
