"""The persistent grouped GEMM issues its weight and activation loads from inline asm and
awaits them with one explicit vmcnt wait per stage; compile it and check the generated
gfx950 code keeps that contract (no use or copy of an in-flight register, no scratch)."""
import os
import re
import shutil

import pytest

from tests.asm_check import compile_to_asm, kernel_bodies, untracked_load_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_gemm_amd", "csrc")


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not installed")
def test_persistent_gemm_has_no_untracked_load_hazard(tmp_path):
    asm = compile_to_asm(os.path.join(CSRC, "gemm_stream.hip"), os.path.join(ROOT, "include"),
                         str(tmp_path / "gemm_stream.s"))
    bodies = kernel_bodies(asm, "gemm_stream_kernel")
    # one row half: plain, SwiGLU, SwiGLU backward; two row halves: plain, SwiGLU
    assert len(bodies) == 5, sorted(bodies)
    for name, body in bodies.items():
        nbw, xbm, rs, rh, mode = (int(v) for v in re.findall(r"Li(\d+)E", name)[:5])
        # the two-row-half shape has half the registers per wave and spills a few loop
        # invariants; scratch operations only add to the in-order vector-memory count, so
        # they can only make the explicit waits stricter (the hazard below is a copy or
        # spill of a register an untracked load has not filled yet)
        if rh == 1:
            assert "scratch_" not in body, f"{name} spills to scratch"
        hz = untracked_load_hazards(body)
        assert not hz, f"{name}: {hz[:3]}"
        # one explicit wait per stage of the RS-stage unrolled loop, with the count the
        # stage's later loads allow: PER ops per stage (activation loads XBM, weight loads
        # 4 NBW), the weights RS - 1 stages ahead, the activations 3 stages ahead
        per = xbm + 4 * nbw
        waitn = min((rs - 1) * per, 4 * nbw + 2 * per)
        assert body.count(f"s_waitcnt vmcnt({waitn})") == rs, (name, waitn)


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not installed")
def test_split_router_logits_have_no_untracked_load_hazard(tmp_path):
    """The split-K router logits (many experts) load the packed router rows into registers
    from inline asm and the token rows into LDS, with one explicit wait per stage: four
    stages of router rows and three of token rows ahead, 12 loads a stage, so the wait
    allows 32 later loads; the stage loop is unrolled four times."""
    asm = compile_to_asm(os.path.join(CSRC, "route.hip"), os.path.join(ROOT, "include"),
                         str(tmp_path / "route.s"))
    bodies = kernel_bodies(asm, "logits_split_kernel")
    assert len(bodies) == 1, sorted(bodies)
    for name, body in bodies.items():
        assert "scratch_" not in body, f"{name} spills to scratch"
        hz = untracked_load_hazards(body)
        assert not hz, f"{name}: {hz[:3]}"
        assert body.count("s_waitcnt vmcnt(32)") == 4, name


@pytest.mark.skipif(shutil.which("/opt/rocm/bin/hipcc") is None, reason="hipcc not installed")
@pytest.mark.parametrize("src", ["gemm_stream.hip", "gemm.hip", "gemm_packed.hip", "backward.hip",
                                 "route.hip"])
def test_m0_is_only_set_for_direct_to_lds_loads(src, tmp_path):
    """The direct-to-LDS loads set M0 in inline asm and list it as clobbered. M0 is a
    reserved register the compiler does not preserve around such asm, so that is only
    safe while the compiler itself never uses M0 in these kernels: every instruction
    that names m0 must be one of the asm statements' own s_mov_b32 m0, s<n>."""
    asm = compile_to_asm(os.path.join(CSRC, src), os.path.join(ROOT, "include"),
                         str(tmp_path / (src + ".s")))
    bad = []
    for line in asm.split("\n"):
        t = line.strip()
        if not t or t.startswith(";") or t.startswith("."):
            continue
        code = t.split(";")[0]
        if re.search(r"\bm0\b", code) and not re.match(r"s_mov_b32 m0, s\d+$", code.strip()):
            bad.append(t)
    assert not bad, bad[:5]
