"""Build libq8.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Every source is compiled for gfx950 only, with:
  -ffp-contract=off     no implicit fused multiply-adds: the kernels spell out
                        every fma they use, so results never depend on the
                        compiler's contraction choices;
  -packed-fp32-ops off  no v_pk_{add,mul,fma}_f32 (scalar fp32 VALU only);
  mfma-vgpr-form        MFMA results land in ordinary VGPRs, which the epilogue
                        reads directly (no accumulator-register copies);
  default HIP division  fp32 '/' is correctly rounded (the quantizer relies on
                        it); no -ffast-math, no denormal flushing.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libq8.so")
ARCH = "gfx950"

HIP_SOURCES = ["quantize.hip", "repack.hip", "gemv.hip", "gemv_seq.hip", "gemm.hip", "norm.hip", "moe.hip", "kv.hip", "measure.hip"]
HOST_SOURCES = ["api.cpp", "plan.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def source_digest() -> str:
    """sha256 over every file the library is built from (the kernel and host
    sources, their headers, include/q8.h) and the compile flags, without
    absolute paths, so the same tree gives the same digest on any machine.
    build() compiles it into the library (q8_build_digest), and the binding
    refuses a library whose digest differs from the tree's."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp", ".cpp", ".h", ".inc")))
    for name in files:
        h.update(name.encode() + b"\0")
        h.update(open(os.path.join(CSRC, name), "rb").read())
    h.update(b"include/q8.h\0")
    h.update(open(os.path.join(ROOT, "include", "q8.h"), "rb").read())
    h.update(" ".join(a for a in COMMON + DEVICE if not os.path.isabs(a) and a != "-I").encode())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    out = subprocess.run(cmd, capture_output=True, text=True)
    if out.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out.stdout + out.stderr)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    return "\n".join(l for l in (out.stdout + out.stderr).splitlines() if noise not in l)


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libq8.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    digest = source_digest()
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        rocm_inc = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(cc))), "include")
        cmds.append([cc, *COMMON, "-D__HIP_PLATFORM_AMD__", f'-DQ8_BUILD_DIGEST="{digest}"', "-I", rocm_inc,
                     "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    logs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
