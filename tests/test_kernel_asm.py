"""CPU check of the generated gfx950 code (no GPU needed; hipcc cross-compiles).

The operand copies global -> LDS are written as inline assembly that loads M0 with
the LDS destination right before each global_load_lds instruction.  M0 is a
register the compiler reserves for itself, so the assembly cannot declare it
clobbered; the design is sound only while the compiler keeps no value of its own
in M0 across those copies.  This test compiles the kernels and requires that no
kernel touches M0 anywhere else.
"""
import os
import re
import subprocess

import pytest

from fp8_rowwise_scaled_amd import build as B


def device_asm(tmp_path, source):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(source) + ".s")
    cmd = [hipcc, *B.COMMON, "--cuda-device-only", "-S", source, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


# Instructions that read M0 without naming it: indexed register moves, GWS, messages,
# interpolation, and LDS-DMA copies (allowed only right after the copy's own
# 's_mov_b32 m0').  The compiler's own GPR-indexing mode is accepted as a closed
# bracket: 's_set_gpr_idx_on' loads M0 from a scalar register itself, the indexed
# moves follow and 's_set_gpr_idx_off' ends it, so it depends on no earlier M0 value
# as long as nothing else writes M0 inside the bracket.
IMPLICIT_M0 = ("v_movrel", "s_movrel", "s_set_gpr_idx", "ds_gws", "s_sendmsg", "v_interp")


def m0_uses_outside_lds_copies(asm):
    """(kernel, instruction) pairs that read or write M0 other than the
    's_mov_b32 m0, ...' that directly precedes a global_load_lds copy and that copy."""
    found = []
    kernel = None
    lines = [l.split(";")[0].strip() for l in asm.splitlines()]
    skip_to = -1
    for i, text in enumerate(lines):
        if i <= skip_to:
            continue
        if text.startswith("s_set_gpr_idx_on"):
            end = next((j for j in range(i + 1, min(i + 16, len(lines))) if lines[j].startswith("s_set_gpr_idx_off")),
                       None)
            inside = lines[i + 1:end] if end is not None else []
            if end is None or any(re.search(r"\bm0\b", t) or "_lds" in t or t.startswith("s_set_gpr_idx_on")
                                  for t in inside):
                found.append((kernel, text))
            else:
                skip_to = end
            continue
        m = re.match(r"^(_Z\S+):", text)
        if m:
            kernel = m.group(1)
            continue
        if text.startswith("global_load_lds") or re.match(r"buffer_load\S*.*\blds\b", text):
            if not any(p.startswith("s_mov_b32 m0,") for p in lines[max(0, i - 2):i]):
                found.append((kernel, text))
            continue
        if text.startswith(IMPLICIT_M0):
            found.append((kernel, text))
            continue
        if not re.search(r"\bm0\b", text):
            continue
        if text.startswith("s_mov_b32 m0,") and any(f.startswith("global_load_lds") for f in lines[i + 1:i + 3]):
            continue
        found.append((kernel, text))
    return found


def test_kernels_use_m0_only_for_the_lds_copies(tmp_path):
    for src in ("fp8gg_kernels.hip", "fp8gg_quantize.hip"):
        asm = device_asm(tmp_path, os.path.join(B.CSRC, src))
        assert "global_load_lds" in asm or src == "fp8gg_quantize.hip"
        uses = m0_uses_outside_lds_copies(asm)
        assert not uses, f"{src}: M0 used outside the LDS copies: {uses[:5]}"


def test_the_scan_flags_other_m0_uses():
    """The scan itself: the copy sequence passes, any other M0 access is reported."""
    ok = "_Zk:\n\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v[2:3], off\n"
    assert m0_uses_outside_lds_copies(ok) == []
    bad = ok + "\ts_mov_b32 m0, -1\n\tds_read_b32 v1, v2\n\tv_movrels_b32 v0, v4\n\tglobal_load_lds_dword v[4:5], off\n"
    uses = m0_uses_outside_lds_copies(bad)
    assert [u[1] for u in uses] == ["s_mov_b32 m0, -1", "v_movrels_b32 v0, v4", "global_load_lds_dword v[4:5], off"]
    assert m0_uses_outside_lds_copies("_Zk:\n\ts_add_u32 m0, m0, 4\n") == [("_Zk", "s_add_u32 m0, m0, 4")]
    bracket = "_Zk:\n\ts_set_gpr_idx_on s24, gpr_idx(SRC0)\n\tv_mov_b32_e32 v5, v3\n\ts_set_gpr_idx_off\n"
    assert m0_uses_outside_lds_copies(bracket) == []
    broken = bracket.replace("\tv_mov_b32_e32 v5, v3\n", "\tv_mov_b32_e32 v5, v3\n\ts_mov_b32 m0, s4\n")
    assert m0_uses_outside_lds_copies(broken)[0] == ("_Zk", "s_set_gpr_idx_on s24, gpr_idx(SRC0)")
    unclosed = "_Zk:\n\ts_set_gpr_idx_on s24, gpr_idx(SRC0)\n\tv_mov_b32_e32 v5, v3\n"
    assert m0_uses_outside_lds_copies(unclosed) == [("_Zk", "s_set_gpr_idx_on s24, gpr_idx(SRC0)")]
