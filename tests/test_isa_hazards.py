"""Static check of the generated gfx950 ISA for the one hazard the compiler
cannot see: the inline-asm v_mul_f32_dpp / v_fmac_f32_dpp read their DPP
source (src0) through a cross-lane broadcast, and gfx9 requires two wait
states between a VALU write of a VGPR and a DPP read of it.  The kernels
keep those sources load-only; this test compiles the forward and backward
kernels to assembly (CPU only) and fails if any VALU instruction writes the
source of any DPP instruction within the two instructions before it, or if
standalone broadcasts (v_mov_b32_dpp, one extra instruction per state-step)
appear.  It also checks that no kernel writes through the scalar data cache
(scalar stores or atomics, cache write-back or discard): every store of the
library is a vector store."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_ssm_amd", "csrc")

pytestmark = pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")


SOURCES = ["ssm_fwd.hip", "ssm_bwd.hip", "ssm_step.hip", "ssm_proj.hip", "affine_scan.hip"]


def _compile(tmp_dir, src):
    out = tmp_dir / (src + ".s")
    cmd = ["/opt/rocm/bin/hipcc", "-O3", "--offload-arch=gfx950", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def all_isa(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")
    return {src: _compile(d, src) for src in SOURCES}


@pytest.fixture(scope="module", params=["ssm_fwd.hip", "ssm_bwd.hip"])
def isa(request, all_isa):
    return all_isa[request.param]


def _instructions(text):
    """(mnemonic, operand string) per instruction line, labels and directives dropped."""
    out = []
    for line in text.splitlines():
        line = line.split(";")[0].strip()
        if not line or line.endswith(":") or line.startswith(".") or line.startswith("#"):
            continue
        parts = line.split(None, 1)
        out.append((parts[0], parts[1] if len(parts) > 1 else ""))
    return out


def _regs(operand):
    """VGPR indices named by one operand (v7 or v[4:7])."""
    m = re.fullmatch(r"v(\d+)", operand)
    if m:
        return {int(m.group(1))}
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def test_dpp_sources_not_written_by_valu_just_before(isa):
    ins = _instructions(isa)
    checked = 0
    for i, (op, args) in enumerate(ins):
        if not op.endswith("_dpp") or "row_newbcast" not in args:
            continue
        src0 = args.split(",")[1].strip()
        regs = _regs(src0)
        assert regs, args
        # the two instructions before (s_nop n counts as n+1 wait states)
        waits = 0
        j = i - 1
        while j >= 0 and waits < 2:
            pop, pargs = ins[j]
            if pop == "s_nop":
                waits += int(pargs.strip() or 0) + 1
                j -= 1
                continue
            if pop.startswith("v_") and not pop.startswith("v_cmp") and not pop.startswith("v_readlane") \
                    and not pop.startswith("v_readfirstlane"):
                dst = pargs.split(",")[0].strip()
                assert not (_regs(dst) & regs), f"VALU write of DPP source {src0} right before: {pop} {pargs}"
            waits += 1
            j -= 1
        checked += 1
    assert checked > 0


def test_row_broadcasts_are_fused(isa):
    """Almost every per-step B/C broadcast is an operand of the consuming
    v_mul/v_fmac; a stray standalone broadcast costs one instruction."""
    ins = _instructions(isa)
    fused = sum(1 for op, a in ins if "row_newbcast" in a and op != "v_mov_b32_dpp")
    loose = sum(1 for op, a in ins if "row_newbcast" in a and op == "v_mov_b32_dpp")
    assert fused > 0 and loose == 0, (fused, loose)


def test_no_scalar_cache_writes(all_isa):
    bad = re.compile(r"^(s_store|s_buffer_store|s_scratch_store|s_atomic|s_buffer_atomic|s_dcache_wb|s_dcache_discard)")
    for src, text in all_isa.items():
        for op, args in _instructions(text):
            assert not bad.match(op), f"{src}: scalar-cache write {op} {args}"


def test_lds_dma_m0_writes_and_waits(all_isa):
    """The projection's bfloat16 kernel loads its operands straight into LDS
    with inline-asm buffer loads whose LDS address is in M0.  In its
    generated code: every such load is preceded by its own M0 write and one
    wait state (s_nop), nothing else reads or writes M0, and the only full
    vmcnt(0) wait is the drain before the workgroup ends (a compiler-inserted
    wait inside the loop would serialize the pipeline)."""
    text = all_isa["ssm_proj.hip"]
    kernels = re.findall(r"^(_Z\w*ssm_proj_dma_kernel\w*):", text, flags=re.M)
    assert kernels, "no DMA kernel in ssm_proj.hip"
    for k in kernels:
        body = text.split(k + ":", 1)[1].split("s_endpgm", 1)[0]
        ins = _instructions(body)
        loads = [i for i, (op, a) in enumerate(ins) if op.startswith("buffer_load") and a.rstrip().endswith("lds")]
        assert loads, k
        for i in loads:
            assert ins[i - 1][0] == "s_nop", (k, ins[i - 1])
            assert ins[i - 2][0] == "s_mov_b32" and ins[i - 2][1].startswith("m0,"), (k, ins[i - 2])
        m0 = [i for i, (op, a) in enumerate(ins) if re.search(r"\bm0\b", a)]
        assert set(m0) == {i - 2 for i in loads}, (k, [ins[i] for i in m0 if i + 2 not in loads])
        full = [i for i, (op, a) in enumerate(ins) if op == "s_waitcnt" and "vmcnt(0)" in a]
        assert len(full) == 1 and full[0] > max(loads), (k, len(full))
