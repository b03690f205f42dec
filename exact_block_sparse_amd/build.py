"""Build libfa.so in place: hipcc for gfx950, one object per source, then one link.

Usage: python exact_block_sparse_amd/build.py  (or call build()); run as a file, since importing
the package needs the library it builds.
The library lands next to this file; build products go to _build/ at the repo root.

Every compiler message is printed, also when the build succeeds. Besides the objects, the
device code of each HIP source is compiled to gfx950 assembly (_build/<source>.s), and the
build fails unless that assembly keeps the M0 invariant the loads into LDS rely on
(`check_m0`).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code (see the package documentation).
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# The host pass does not know the device-only target feature above and says so; that note
# is expected and not shown.
_HOST_FEATURE_NOTE = re.compile(r"'-packed-fp32-ops' is not a recognized feature")


class BuildError(RuntimeError):
    pass


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise BuildError("hipcc not found; the HIP library cannot be built")


def _messages(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if l.strip() and not _HOST_FEATURE_NOTE.search(l))


def _run(cmd: list[str], what: str) -> str:
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = _messages(r.stdout + r.stderr)
    if r.returncode != 0:
        raise BuildError(f"{what} failed: {' '.join(cmd)}\n{msg}")
    return msg


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    return obj, _run(cmd, f"compile {src}")


def _assemble(src: str) -> tuple[str, str]:
    out = os.path.join(BUILD, os.path.basename(src) + ".s")
    # (hipcc adds a link flag the assembly-only compile does not use)
    cmd = [hipcc(), *HIP_FLAGS, "-Wno-unused-command-line-argument", "--offload-device-only", "-S", "-I", INCLUDE, "-I", CSRC,
           os.path.join(CSRC, src), "-o", out]
    return out, _run(cmd, f"device assembly of {src}")


# Instructions that read or write M0 without naming it in the assembly text.
_IMPLICIT_M0 = re.compile(r"\b(s_movrel\w*|v_movrel\w*|s_sendmsg\w*|ds_gws\w*|ds_ordered\w*|s_set_gpr_idx\w*|"
                          r"v_interp\w*|global_load_lds\w*|scratch_load_lds\w*)\b")
_LDS_LOAD = re.compile(r"\bbuffer_load_\w+\b.*\blds\b")
_M0 = re.compile(r"\bm0\b")


def check_m0(asm: str) -> list[str]:
    """Problems with the M0 invariant in gfx950 assembly text (empty list: it holds).

    The loads into LDS set M0 inside their own inline-assembly block and use it at once.
    That is sound only if the compiler keeps nothing in M0 across such a block, i.e. if no
    compiler-generated instruction touches M0: every line naming M0 and every buffer load
    into LDS must sit between an ;;#ASMSTART / ;;#ASMEND pair, each such load must follow an
    M0 move in the same block, and no instruction may use M0 implicitly.
    """
    problems = []
    inside = False
    m0_set = False
    for n, raw in enumerate(asm.splitlines(), 1):
        line = raw.split(";", 1)[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
        if line.startswith(";;#ASMSTART"):
            inside, m0_set = True, False
            continue
        if line.startswith(";;#ASMEND"):
            inside = False
            continue
        if not line or line.startswith(".") or line.endswith(":"):
            continue
        if _IMPLICIT_M0.search(line):
            problems.append(f"line {n}: instruction that uses M0 implicitly: {line}")
        if _M0.search(line):
            if not inside:
                problems.append(f"line {n}: compiler-generated use of M0: {line}")
            elif re.match(r"s_mov_b32\s+m0\s*,", line):
                m0_set = True
            else:
                problems.append(f"line {n}: unexpected M0 use inside an asm block: {line}")
        if _LDS_LOAD.search(line):
            if not inside:
                problems.append(f"line {n}: load into LDS outside an asm block: {line}")
            elif not m0_set:
                problems.append(f"line {n}: load into LDS without an M0 move before it: {line}")
    return problems


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hip_sources = [s for s in SOURCES if s.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        fo = [ex.submit(_compile, s) for s in SOURCES]
        fa = [ex.submit(_assemble, s) for s in hip_sources]
        objs = [f.result() for f in fo]
        asms = [f.result() for f in fa]
    for src, (_, msg) in list(zip(SOURCES, objs)) + list(zip(hip_sources, asms)):
        if msg:
            print(f"[build] {src}:\n{msg}", file=sys.stderr, flush=True)
    for src, (path, _) in zip(hip_sources, asms):
        with open(path) as f:
            problems = check_m0(f.read())
        if problems:
            raise BuildError(f"{src}: the M0 invariant of the loads into LDS does not hold:\n" +
                             "\n".join(problems[:20]))
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *(o for o, _ in objs)], "link")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
