"""Checks on the gfx950 assembly of the GEMM kernels (CPU only: hipcc
cross-compiles).  The main loops rely on properties the compiler could
silently take away, each of which has cost 10-30 % when it went missing:

* no register spills in the bf16 GEMM kernels (a spill puts scratch traffic
  and waits into the loop);
* between the direct-to-LDS copies of the next k-tile and the fragment reads
  of the current one there is no wait on the vector-memory counter (such a
  wait serialises copies and MFMAs);
* no such wait sits between two copies either: the compiler does not count
  the copies (inline assembly), so a wait it places for a load of its own
  (a spill reload, an index) also waits for every copy already issued, and
  the copies of a k-tile then go out one at a time;
* M0, which the copies set, is written by nothing else.
"""

import os
import re
import shutil
import subprocess

import pytest

from token_dispatch_expert_amd import build_lib

CSRC = os.path.join(build_lib.HERE, "csrc")
GEMMS = ("f1_gather_glu", "f2_down_combine", "b1_dgrad_glu", "b0_dw2", "b2_dw13", "b3_dx")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        hipcc = build_lib.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "ffn.s")
    flags = [f for f in build_lib.common_flags() if f != "-fPIC"]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, "ffn.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _kernels(asm_text):
    names = re.findall(r"^(_ZN3moe[A-Za-z0-9_]*):", asm_text, re.M)
    out = {}
    for n in names:
        i = asm_text.index(n + ":")
        j = asm_text.index(".Lfunc_end", i)
        out[n] = [l.strip() for l in asm_text[i:j].split("\n")]
    return out


def _bf16_gemms(kernels):
    return {n: b for n, b in kernels.items()
            if "bf16" in n and any(g in n for g in GEMMS)}


def test_bf16_gemm_kernels_do_not_spill(asm):
    """No bf16 GEMM kernel holds spilled registers, in either G mode (with
    MOE_FLAG_RECOMPUTE_G the second GEMMs read G from a piece formed ahead
    of them, through the same loaders)."""
    meta = re.findall(r"- \.agpr_count:.*?\.vgpr_spill_count:\s*\d+", asm, re.S)
    seen = 0
    for blk in meta:
        name = re.search(r"\.name:\s+(\S+)", blk).group(1)
        if "bf16" in name and any(g in name for g in GEMMS):
            seen += 1
            spill = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", blk).group(1))
            assert spill == 0, f"{name} spills {spill} VGPRs"
    assert seen >= 2 * len(GEMMS)


def test_no_copy_wait_before_fragment_reads(asm):
    """Once a k-tile's copies (global_load_lds) are out, no LDS read or MFMA
    may follow a vmcnt wait in the same basic block before the barrier that
    ends the k-tile: the copies only have to land by that barrier (the loop's
    own waits sit at the end of a block that branches to the barrier)."""
    checked = 0
    for name, body in _bf16_gemms(_kernels(asm)).items():
        inflight = waited = False
        for line in body:
            if line.startswith("global_load_lds"):
                inflight, waited = True, False
            elif line.startswith("s_barrier"):
                inflight = waited = False
            elif line.startswith((".LBB", "s_branch", "s_cbranch")):
                waited = False          # a new basic block
            elif inflight and line.startswith("s_waitcnt") and "vmcnt" in line:
                waited = True
            elif inflight and line.startswith(("ds_read", "v_mfma")):
                assert not waited, f"{name}: vmcnt wait between the copies and {line.split()[0]}"
                checked += 1
    assert checked >= len(GEMMS)


def test_no_wait_between_copies(asm):
    """Inside one basic block, no vmcnt wait separates two direct-to-LDS
    copies in any GEMM kernel (bf16 and float32, every mode)."""
    copies = 0
    for name, body in _kernels(asm).items():
        if not any(g in name for g in GEMMS):
            continue
        after_copy = waited = False
        for line in body:
            if line.startswith("global_load_lds"):
                assert not (after_copy and waited), f"{name}: vmcnt wait between two copies"
                after_copy, waited = True, False
                copies += 1
            elif line.startswith((".LBB", "s_branch", "s_cbranch", "s_barrier")):
                after_copy = waited = False
            elif after_copy and line.startswith("s_waitcnt") and "vmcnt" in line:
                waited = True
    assert copies >= 8 * len(GEMMS)


def test_m0_written_only_by_the_copies(asm):
    lines = asm.split("\n")
    for k, line in enumerate(lines):
        t = line.strip()
        if t.startswith((";", ".")) or not re.search(r"\bm0\b", t):
            continue
        assert t.startswith("s_mov_b32 m0,"), f"unexpected use of m0: {t}"
        nxt = [l.strip() for l in lines[k + 1:k + 4]]
        assert any(l.startswith("global_load_lds") for l in nxt), f"m0 set without a copy: {t}"
