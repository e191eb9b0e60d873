"""Wait states around the hand-written MFMAs of the decode kernels.

The score chains of the 16-bit MFMA decode are inline asm, so the compiler's
hazard recognizer does not see them as MFMAs (the 8-bit decode issues every
MFMA as a builtin, so it has no inline-asm MFMA to check; it is compiled here
for the stage-loop scratch check below).  gfx950 needs
  - 2 wait states between a VALU write of a VGPR and an MFMA that reads it
    (A, B or C operand): the kernels place an ``s_nop 1`` only where such a
    write can precede a chain;
  - passes + 3 wait states between an MFMA's result and a VALU that reads or
    writes it: 11 for the 8-pass 32x32x16 bf16/f16 MFMA, 19 for the 16-pass
    32x32x64 8-bit one.
This test compiles the kernels to gfx950 assembly and checks every inline-asm
MFMA against the instructions before it (within 2 wait states, an ``s_nop N``
counting N + 1 and any other instruction 1, no VALU instruction may write one
of its source registers, and no label may start the window, since a jump into
it could bring a VALU write the scan does not see, unless the MFMA has a nop)
and after it (within its result latency no VALU may touch its destination;
the scan stops at a branch or label, which no chain ends in).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_07_amd", "csrc")
SOURCES = ["decode_mfma.hip", "decode_f8w8.hip"]
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

WINDOW = 2
_REG = re.compile(r"v\[(\d+):(\d+)\]|\bv(\d+)\b")


def regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def instr(line):
    """(mnemonic, operand text) of an instruction line, or None."""
    t = line.split(";")[0].strip()
    if not t or t.startswith(".") or t.endswith(":"):
        return None
    parts = t.split(None, 1)
    return parts[0], (parts[1] if len(parts) > 1 else "")


def check_asm(lines):
    """Violations: (line number, mfma text, offending text)."""
    bad = []
    in_asm = False
    for n, line in enumerate(lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        ins = instr(line)
        if not (in_asm and ins and ins[0].startswith("v_mfma")):
            continue
        ops = [o.strip() for o in ins[1].split(",")]
        srcs = set()
        for o in ops[1:]:
            srcs |= regs(o)
        waits = 0
        k = n - 1
        while k >= 0 and waits < WINDOW:
            prev = lines[k]
            ps = prev.strip()
            if re.match(r"^[.\w]+:", ps):                 # a label: another path may enter here
                bad.append((n + 1, s, "label " + ps.split(":")[0]))
                break
            p = instr(prev)
            k -= 1
            if p is None:
                continue
            mn, args = p
            if mn == "s_nop":
                waits += int(args.strip(), 0) + 1
                continue
            if mn.startswith("v_") and not mn.startswith("v_mfma"):
                dst = args.split(",")[0]
                if regs(dst) & srcs:
                    bad.append((n + 1, s, ps))
            waits += 1
    return bad


def result_latency(mnemonic):
    """Wait states from an MFMA's result to a VALU access of it."""
    return 19 if "32x32x64" in mnemonic else 11


def check_results(lines):
    """Violations of the MFMA-result -> VALU latency: (line, mfma, offending)."""
    bad = []
    in_asm = False
    for n, line in enumerate(lines):
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        ins = instr(line)
        if not (in_asm and ins and ins[0].startswith("v_mfma")):
            continue
        dst = regs(ins[1].split(",")[0])
        need = result_latency(ins[0])
        waits = 0
        k = n + 1
        while k < len(lines) and waits < need:
            ps = lines[k].strip()
            k += 1
            if re.match(r"^[.\w]+:", ps):
                break
            p = instr(ps)
            if p is None:
                continue
            mn, args = p
            if mn.startswith("s_cbranch") or mn.startswith("s_branch") or mn.startswith("s_setpc"):
                break
            if mn == "s_nop":
                waits += int(args.strip(), 0) + 1
                continue
            if mn.startswith("v_") and not mn.startswith("v_mfma") and regs(args) & dst:
                bad.append((n + 1, s, ps))
            waits += 1
    return bad


@pytest.fixture(scope="module", params=SOURCES)
def decode_asm(request, tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    src = os.path.join(CSRC, request.param)
    out = tmp_path_factory.mktemp("asm") / (request.param + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", str(out), src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


def test_checker_flags_a_planted_hazard():
    planted = ["\tv_mul_f32_e32 v20, v1, v2", ";;#ASMSTART",
               "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]", ";;#ASMEND"]
    assert check_asm(planted)
    covered = ["\tv_mul_f32_e32 v20, v1, v2", ";;#ASMSTART", "\ts_nop 1",
               "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]", ";;#ASMEND"]
    assert not check_asm(covered)
    acc = ["\tv_mul_f32_e32 v3, v1, v2", "\ts_waitcnt lgkmcnt(0)", ";;#ASMSTART",
           "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]", ";;#ASMEND"]
    assert check_asm(acc)
    late = [";;#ASMSTART", "\tv_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v40, v41",
            ";;#ASMEND", "\ts_nop 15", "\tv_mul_f32_e32 v3, v3, v50"]
    assert check_results(late)
    late_ok = late[:3] + ["\ts_nop 15", "\ts_nop 3", "\tv_mul_f32_e32 v3, v3, v50"]
    assert not check_results(late_ok)
    bf16_ok = [";;#ASMSTART", "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], v[0:15]",
               ";;#ASMEND", "\ts_nop 15", "\tv_mul_f32_e32 v3, v3, v50"]
    assert not check_results(bf16_ok)


def test_score_chain_wait_states(decode_asm):
    n_mfma = sum(1 for l in decode_asm if re.match(r"\s+v_mfma", l))
    assert n_mfma > 40
    bad = check_asm(decode_asm)
    assert not bad, "\n".join(f"line {a}: {b} <- {c}" for a, b, c in bad[:20])


def test_score_chain_result_latency(decode_asm):
    bad = check_results(decode_asm)
    assert not bad, "\n".join(f"line {a}: {b} -> {c}" for a, b, c in bad[:20])


def kernel_bodies(lines):
    """{kernel symbol: its instruction lines} of a gfx950 assembly listing."""
    out = {}
    for n, line in enumerate(lines):
        m = re.match(r"^(_Z\w*(decode_mfma_kernel|decode_f8w8_kernel)\w*):", line)
        if m:
            end = next(k for k in range(n, len(lines)) if "s_endpgm" in lines[k])
            out[m.group(1)] = lines[n:end]
    return out


def test_no_scratch_access_in_the_stage_loop(decode_asm):
    """A spill reload inside the stage loop is a vector-memory load the
    compiler waits for with vmcnt(0), which also waits for every stage copy
    in flight (the copies are inline asm, invisible to its counting): one
    such reload per iteration drains the copy pipeline.  The stage loop runs
    from the first MFMA after the prologue to the last MFMA of the kernel
    (the 16-bit kernel scores stage 0 in its prologue with 36 MFMAs; the
    8-bit kernel has none before its loop).  The 8-bit kernel runs two waves
    per SIMD within 256 registers, where this is easy to break."""
    bodies = kernel_bodies(decode_asm)
    assert bodies
    for name, body in bodies.items():
        mf = [i for i, l in enumerate(body) if re.match(r"\s+v_mfma", l)]
        skip = 36 if "decode_mfma_kernel" in name else 0
        lo, hi = mf[skip], mf[-1]
        bad = [body[i].strip() for i in range(lo, hi) if "scratch_" in body[i]]
        assert not bad, f"{name}: {bad[:4]}"
