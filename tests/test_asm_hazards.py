"""Device-code check of the inline-asm MFMAs (CPU only: hipcc cross-compiles).

On gfx950 an MFMA that reads a VGPR written by a VALU instruction needs 2
wait states in between.  The compiler inserts them before its own MFMAs but
not before inline asm, and the S^T MFMAs of the decode kernels are inline
asm (their accumulator must stay in VGPRs).  An operand written by the VALU
right before such an MFMA is read stale: the logits come out wrong with no
error (whole heads turned NaN in a variant that widened its operands just
before the MFMA).  The other direction holds as well: the MFMA's result
may be read by another instruction only after its passes (the kernels wait
18 states; the compiler's own rule for this 8-pass MFMA is 11).  This test
compiles the kernels to gfx950 assembly and checks every inline-asm MFMA
against the VALU writes before it and the reads of its result after it.
"""

import os
import re
import subprocess

import pytest

from sparse_mla_decode_gather_amd import build as B

WAIT_STATES = 2          # VALU write of an operand -> MFMA read
RESULT_WAIT_STATES = 11  # 8-pass MFMA result -> read by a non-MFMA instruction


def _vgprs(tok: str) -> set:
    tok = tok.strip()
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def scan(asm: str) -> tuple[int, list]:
    """Returns (inline-asm MFMAs seen, violations), in program order,
    counting one wait state per instruction and N+1 per s_nop N: (1) walking
    back from each inline-asm MFMA, no VALU write of a VGPR it reads within
    WAIT_STATES; (2) going forward from it, no non-MFMA instruction reading
    its result within RESULT_WAIT_STATES (MFMAs may chain on it)."""
    seen, bad = 0, []
    in_asm = False
    hist = []                      # (opcode, written VGPRs, wait states it adds)
    pending = []                   # [result VGPRs, wait states still needed, MFMA text]
    func = "?"
    for line in asm.splitlines():
        t = line.strip()
        if re.match(r"^_Z\S+:", t):
            func, hist, pending = t.split(":")[0], [], []
            continue
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        op = t.split()[0]
        args = [a.strip() for a in t[len(op):].split(",")]
        if not op.startswith(("v_mfma", "s_")):
            first = 0 if ("store" in op or op.startswith("ds_write")) else 1
            reads = set()
            for a in args[first:]:
                reads |= _vgprs(a.split()[0]) if a else set()
            for dst, need, mf in pending:
                if need > 0 and dst & reads:
                    bad.append(f"{func}: {mf} then {t} with {RESULT_WAIT_STATES - need} "
                               f"wait state(s)")
        if op.startswith("v_mfma") and in_asm:
            seen += 1
            srcs = set()
            for a in args[1:4]:
                srcs |= _vgprs(a.split()[0]) if a else set()
            ws = 0
            for pop, dst, w in reversed(hist):
                if ws >= WAIT_STATES:
                    break
                if dst & srcs and not pop.startswith("v_mfma"):
                    bad.append(f"{func}: {pop} then {t} after {ws} wait state(s)")
                    break
                ws += w
        step = (int(args[0]) + 1 if args and args[0].isdigit() else 1) if op == "s_nop" else 1
        pending = [[d, n - step, m] for d, n, m in pending if n - step > 0]
        if op.startswith("v_mfma") and in_asm:
            pending.append([_vgprs(args[0].split()[0]), RESULT_WAIT_STATES, t])
        if op == "s_nop":
            n = int(args[0]) if args and args[0].isdigit() else 0
            hist.append((op, set(), n + 1))
        else:
            dst = set()
            if op.startswith("v_") and not op.startswith(("v_cmp", "v_readfirstlane",
                                                          "v_readlane")):
                dst = _vgprs(args[0].split()[0]) if args and args[0] else set()
            hist.append((op, dst, 1))
        hist = hist[-16:]
    return seen, bad


def test_scanner_flags_a_valu_written_operand():
    snippet = "\n".join([
        "_Zfake:",
        "\tv_cvt_scalef32_pk_bf16_fp8 v10, v2, 1.0",
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]",
        "\t;;#ASMEND",
        "\tv_mov_b32_e32 v11, v40",
        "\t;;#ASMSTART",
        "\ts_nop 1",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[10:13], v[20:23], v[0:15]",
        "\t;;#ASMEND",
    ])
    seen, bad = scan(snippet)
    assert seen == 2 and len(bad) == 1 and "v_cvt_scalef32" in bad[0]


def test_scanner_flags_an_early_read_of_an_mfma_result():
    snippet = "\n".join([
        "_Zfake:",
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]",
        "\ts_nop 7",
        "\t;;#ASMEND",
        "\tv_max_f32_e32 v30, v1, v2",
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]",
        "\ts_nop 7",
        "\ts_nop 7",
        "\t;;#ASMEND",
        "\tv_max_f32_e32 v30, v1, v2",
    ])
    seen, bad = scan(snippet)
    assert seen == 2 and len(bad) == 1 and "v_max_f32" in bad[0]


def test_inline_asm_mfma_operands_have_their_wait_states(tmp_path):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / "kernels.s"
    cmd = [cc, f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-fPIC",
           f"-I{B.INCLUDE}", f"-I{B.CSRC}", *B.DEVICE_FLAGS, "--cuda-device-only",
           "-S", os.path.join(B.CSRC, "kernels.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    seen, bad = scan(out.read_text())
    assert seen > 0, "no inline-asm MFMA found"
    assert not bad, "\n".join(bad[:10])
