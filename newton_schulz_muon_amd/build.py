"""Builds libmuon_hip.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m newton_schulz_muon_amd.build

Each .hip source is compiled to an object in parallel, then linked into
newton_schulz_muon_amd/libmuon_hip.so (replaced atomically).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmuon_hip.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["muon_api.hip", "muon_elementwise.hip", "ns_gemm.hip", "ns_schedule.cpp", "small_ns.hip", "adamw.hip"]

# -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32 (the host pass warns that
# it does not know the feature; that is harmless).
COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source flags.  ns_gemm.hip: the atomic optimizer would turn the
# persistent loop's queue claim into an atomic followed by an immediate wait;
# its kernels' resource usage is reported so that the build can reject
# scratch use (its hand-counted vmcnt waits assume no compiler-placed vector
# memory operation, and scratch accesses are such operations).
SOURCE_FLAGS = {"ns_gemm.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                                "-Rpass-analysis=kernel-resource-usage"]}
NO_SCRATCH_SOURCES = ("ns_gemm.hip",)


def _kernels_with_scratch(out: str):
    """Kernels whose resource remarks in `out` report a private segment."""
    name = None
    seen = 0
    found = []
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m:
            seen += 1
            if int(m.group(1)) != 0:
                found.append(name)
    if seen == 0:
        raise RuntimeError("no kernel resource report in the compiler output")
    return found


def _check_no_scratch(src: str, out: str, cc: str, flags) -> None:
    """Raises if a kernel of `src` accesses scratch memory.  A kernel may
    reserve a private segment that its code never touches (the register
    allocator's emergency slot beside SGPR spills to VGPR lanes); such a
    kernel is accepted only when its generated code holds no scratch access."""
    found = _kernels_with_scratch(out)
    if not found:
        return
    asm = subprocess.run([cc, *flags, "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)],
                         stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    if asm.returncode != 0:
        raise RuntimeError(f"{src}: device assembly failed")
    for name in found:
        body = asm.stdout.split(f"\n{name}:", 1)
        if len(body) < 2:
            raise RuntimeError(f"{src}: kernel {name} not found in the device assembly")
        code = body[1].split("s_endpgm", 1)[0]
        if re.search(r"\bscratch_|\bbuffer_\w+ [^\n]*s\[0:3\]|flat_\w+", code):
            raise RuntimeError(f"{src}: kernel {name} accesses scratch memory")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 4) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, cmds))
    for src, out in zip(SOURCES, outs):
        if src in NO_SCRATCH_SOURCES:
            _check_no_scratch(src, out, cc, [f for f in COMMON_FLAGS + SOURCE_FLAGS.get(src, [])
                                             if not f.startswith("-Rpass")])
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB_PATH + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    build_test_kernels(cc)
    return LIB_PATH


def build_test_kernels(cc: str) -> None:
    """Test-only HIP kernels (tests/kernels/*.hip), each its own shared library
    beside the tests; the library above does not contain them."""
    src_dir = os.path.join(ROOT, "tests", "kernels")
    if not os.path.isdir(src_dir):
        return
    for src in sorted(os.listdir(src_dir)):
        if not src.endswith(".hip"):
            continue
        out = os.path.join(ROOT, "tests", "lib" + os.path.splitext(src)[0] + ".so")
        _run([cc, *COMMON_FLAGS, "-shared", os.path.join(src_dir, src), "-o", out + ".tmp"])
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
