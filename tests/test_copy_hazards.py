"""Wait states before the library's HBM -> LDS copies (host only; needs hipcc).

The copies (global_load_lds_dwordx4) are inline asm, so the compiler's hazard
pass cannot see that they are LDS-DMA loads.  On this GPU family a VMEM
instruction that reads an SGPR written by a VALU instruction needs 5 wait
states in between, and an LDS-DMA load needs 1 after a scalar write of M0, its
LDS address.  A copy whose SGPR base was written by v_readfirstlane just before
it read a stale base and faulted the GPU; the copy helpers now carry the wait
states in the asm.  This test compiles every kernel source to gfx950 assembly
and checks, at every copy, the wait states since the last write of each SGPR
it reads (its base pair and M0), counting s_nop N as N + 1; a block boundary
reached before enough wait states counts as a violation.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_flash_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
VALU_SGPR_WAIT, SALU_M0_WAIT = 5, 1


def sgprs(tok):
    # an operand, possibly followed by cache-policy modifiers ("s[4:5] nt")
    tok = (tok.split() or [""])[0].rstrip(",")
    if tok == "m0":
        return {"m0"}
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return {"s%d" % r for r in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"s(\d+)$", tok)
    return {"s" + m.group(1)} if m else set()


def violations(asm):
    bad = []
    for name in re.findall(r"^(_Z\S*kernel\S*):", asm, re.M):
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        lines = []
        for ln in asm[i:j].splitlines():
            if re.match(r"^\.LBB\d+_\d+:", ln):
                lines.append("LABEL")
            elif ln.startswith("\t") and not ln.strip().startswith((".", ";")):
                lines.append(ln.strip())
        for k, ln in enumerate(lines):
            if not ln.startswith("global_load_lds"):
                continue
            ops = ln.split(None, 1)[1].split(",")
            pending = {"m0"} | (sgprs(ops[1]) if len(ops) > 1 else set())
            ws = 0
            for back in range(k - 1, -1, -1):
                if not pending:
                    break
                p = lines[back]
                if p == "LABEL" or p.startswith(("s_branch", "s_cbranch")):
                    if ws < VALU_SGPR_WAIT:
                        bad.append("%s: %s -- block boundary after %d wait states, %s unresolved"
                                   % (name[:60], ln, ws, sorted(pending)))
                    break
                op, _, rest = p.partition(" ")
                dst = sgprs(rest.split(",")[0]) if rest else set()
                hit = dst & pending
                if hit:
                    need = VALU_SGPR_WAIT if op.startswith("v_") else (SALU_M0_WAIT if hit == {"m0"} else 0)
                    if ws < need:
                        bad.append("%s: %s -- %s writes %s %d wait states before"
                                   % (name[:60], ln, op, sorted(hit), ws))
                    pending -= hit
                m = re.match(r"s_nop\s+(\d+)", p)
                ws += int(m.group(1)) + 1 if m else 1
    return bad


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["decode.hip", "prefill.hip", "mla.hip"])
def test_copies_have_their_wait_states(src, tmp_path):
    out = str(tmp_path / (src + ".s"))
    subprocess.check_call([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    asm = open(out).read()
    copies = asm.count("global_load_lds_dwordx4")
    assert copies > 0
    bad = violations(asm)
    assert not bad, "%d of %d copies lack wait states, e.g.:\n%s" % (len(bad), copies, "\n".join(bad[:10]))


def _kernel(body):
    return "_Zcopy_kernel:\n" + "".join("\t%s\n" % ln for ln in body) + ".Lfunc_end0:\n"


@pytest.mark.parametrize("policy", ["", " nt"])
def test_checker_sees_the_base_pair_with_any_cache_policy(policy):
    copy = "global_load_lds_dwordx4 v1, s[4:5]" + policy
    early = _kernel(["s_mov_b32 m0, s9", "s_nop 0", "v_readfirstlane_b32 s5, v2", "s_nop 2", copy])
    assert violations(early) and "s5" in violations(early)[0]
    assert not violations(_kernel(["v_readfirstlane_b32 s5, v2", "s_mov_b32 m0, s9", "s_nop 4", copy]))
    assert violations(_kernel(["s_mov_b32 m0, s9", copy]))  # M0 written right before the copy
