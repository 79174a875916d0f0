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
# memory operation, and scratch accesses are such operations).  Its device
# assembly is also scanned for LDS DMA hazards (dma_sgpr_hazards).
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


def _device_asm(src: str, cc: str, flags) -> str:
    """The gfx950 assembly that `src` compiles to."""
    asm = subprocess.run([cc, *flags, "--cuda-device-only", "-S", "-o", "-", os.path.join(CSRC, src)],
                         stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    if asm.returncode != 0:
        raise RuntimeError(f"{src}: device assembly failed")
    return asm.stdout


def _check_no_scratch(src: str, out: str, asm: str) -> None:
    """Raises if a kernel of `src` accesses scratch memory.  A kernel may
    reserve a private segment that its code never touches (the register
    allocator's emergency slot beside SGPR spills to VGPR lanes); such a
    kernel is accepted only when its generated code holds no scratch access."""
    found = _kernels_with_scratch(out)
    if not found:
        return
    for name in found:
        body = asm.split(f"\n{name}:", 1)
        if len(body) < 2:
            raise RuntimeError(f"{src}: kernel {name} not found in the device assembly")
        code = body[1].split("s_endpgm", 1)[0]
        if re.search(r"\bscratch_|\bbuffer_\w+ [^\n]*s\[0:3\]|flat_\w+", code):
            raise RuntimeError(f"{src}: kernel {name} accesses scratch memory")


# Wait states required between a VALU write of an SGPR and a vector memory
# instruction that reads it: five, the figure documented for gfx9 (on gfx950
# tests/test_gpu_dma_hazard.py finds loads one instruction after the write
# using the old value, and none from two on).
VMEM_SGPR_WAIT_STATES = 5


def _sgprs(tok: str):
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"s(\d+)", tok)
    if m:
        return {int(m.group(1))}
    if tok in ("vcc", "vcc_lo", "vcc_hi"):
        return {106, 107} if tok == "vcc" else ({106} if tok == "vcc_lo" else {107})
    return set()


def _valu_sgpr_defs(inst: str):
    """SGPRs written by the VALU instruction `inst` (empty if none)."""
    parts = inst.replace(",", " ").split()
    op = parts[0]
    defs = _sgprs(parts[1]) if len(parts) > 1 else set()
    if op.startswith(("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
                      "v_mad_u64_u32", "v_mad_i64_i32", "v_div_scale_")) and len(parts) > 2:
        defs |= _sgprs(parts[2])
    if op.endswith("_e32") and (op.startswith(("v_cmp", "v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_",
                                               "v_subb_co_", "v_subbrev_co_"))):
        defs |= {106, 107}                                       # implicit VCC
    return defs


def dma_sgpr_hazards(asm: str, need: int = VMEM_SGPR_WAIT_STATES):
    """LDS DMA instructions (buffer_load ... lds, written as inline assembly,
    which the compiler's hazard recognizer does not see) that read an SGPR
    written by a VALU instruction fewer than `need` wait states before, or
    that follow a branch target within that distance.  Each instruction
    counts one wait state, s_nop N counts N + 1."""
    insts = []
    for line in asm.splitlines():
        t = line.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):
            insts.append(("label", t))
        elif not t.startswith("."):
            insts.append(("inst", t))
    found = []
    for i, (kind, text) in enumerate(insts):
        if kind != "inst":
            continue
        m = re.match(r"buffer_load_\w+\s+\S+,\s+(s\[\d+:\d+\]),\s+(\S+)\s+offen\s+lds", text)
        if not m:
            continue
        regs = _sgprs(m.group(1)) | _sgprs(m.group(2))
        ws = 0
        j = i - 1
        while j >= 0 and ws < need:
            pkind, ptext = insts[j]
            if pkind == "label":
                found.append(f"{text}: branch target {ptext} {ws} wait states before")
                break
            op = ptext.split()[0]
            if op.startswith("s_nop"):
                ws += int(ptext.split()[1], 0) + 1
            else:
                if op.startswith("v_") and _valu_sgpr_defs(ptext) & regs:
                    found.append(f"{text}: {ws} wait states after {ptext}")
                ws += 1
            j -= 1
    return found


def _check_dma_hazards(src: str, asm: str) -> None:
    found = dma_sgpr_hazards(asm)
    if not any(re.search(r"buffer_load_\w+\s[^\n]*\slds", l) for l in asm.splitlines()):
        raise RuntimeError(f"{src}: no LDS DMA instruction found in the device assembly")
    if found:
        raise RuntimeError(f"{src}: LDS DMA reads an SGPR too soon after a VALU write:\n  " + "\n  ".join(found[:10]))


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
            asm = _device_asm(src, cc, [f for f in COMMON_FLAGS + SOURCE_FLAGS.get(src, [])
                                        if not f.startswith("-Rpass")])
            _check_no_scratch(src, out, asm)
            _check_dma_hazards(src, asm)
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
