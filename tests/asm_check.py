"""Checks of compiled gfx950 assembly for the kernels whose loads the compiler does not
track (inline-asm global loads into registers, completion awaited only by explicit
s_waitcnt vmcnt): no instruction may read or overwrite a destination register of such a
load before a vmcnt wait, and the kernel may not spill to scratch (scratch traffic would
change the vector-memory counts those waits rely on)."""
import re
import subprocess

HIPCC = "/opt/rocm/bin/hipcc"


def compile_to_asm(src: str, include: str, out: str) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", include, src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return open(out).read()


def kernel_bodies(asm: str, name_part: str) -> dict:
    """Text of every kernel whose symbol contains `name_part`, keyed by symbol."""
    out = {}
    for m in re.finditer(r"^(_Z\S*" + re.escape(name_part) + r"\S*):", asm, flags=re.M):
        start = m.end()
        end = asm.find(".Lfunc_end", start)  # a kernel may hold several s_endpgm (early exits)
        out[m.group(1)] = asm[start:end]
    return out


def _regs(text: str) -> set:
    r = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", text):
        r.update(range(int(a), int(b) + 1))
    for a in re.findall(r"\bv(\d+)\b", text):
        r.add(int(a))
    return r


def untracked_load_hazards(body: str) -> list:
    """Instructions that touch a register loaded by an inline-asm global load before any
    later s_waitcnt vmcnt (each wait is taken to complete every earlier load: the check
    aims at copies and spills the compiler might place right after such a load)."""
    pending = {}
    in_asm = False
    hazards = []
    for line in body.split("\n"):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        op, _, rest = t.partition(" ")
        if in_asm and op.startswith("global_load_dword") and not op.startswith("global_load_lds"):
            dst = rest.split(",")[0]
            for r in _regs(dst):
                pending[r] = t
            continue
        if op == "s_waitcnt" and "vmcnt" in rest:
            pending.clear()
            continue
        touched = _regs(rest)
        hit = [r for r in touched if r in pending]
        if hit:
            hazards.append((t, pending[hit[0]]))
    return hazards
