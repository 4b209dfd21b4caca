"""Build libqmm.so (the HIP kernels + C-ABI) for gfx950, in-tree.

    python -m gemv_prefill_decode_amd.build        # or __graft_entry__.build()

Each translation unit is compiled with hipcc in parallel, then linked into
gemv_prefill_decode_amd/libqmm.so.  Packed-f32 VALU instructions are disabled
(-packed-fp32-ops) for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libqmm.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["gemv.hip", "moe.hip", "gemm_mfma.hip", "gemm_lds.hip", "noalloc.hip", "qmm_api.cpp"]
ARCH = os.environ.get("QMM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fno-gpu-rdc",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: with the default AGPR form the register
        # allocator shuffles the prefill kernel's 64 accumulators between the
        # two unrolled halves of its k loop on every iteration
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# ---------------------------------------------------------------- sanitized host build
# The host side of every translation unit (argument validation, planning,
# launch set-up) compiled with AddressSanitizer and UndefinedBehaviorSanitizer,
# linked with the code-object bundles of the regular build (device code is
# not recompiled or instrumented): the boundary tests run against it on the
# CPU.
SAN_DIR = os.path.join(PKG, "_build", "san")
SAN_OUT = os.path.join(SAN_DIR, "libqmm_san.so")
# -Xarch_host before each sanitizer flag: host code only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libsan", "-g", "-O1"]


def _compile_san(src: str) -> str:
    obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
    flags = [f for f in _flags() if f != "-O3"]
    host_only = ["--cuda-host-only"] if src.endswith(".hip") else []
    cmd = [hipcc()] + flags + host_only + SAN_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
        raise RuntimeError(f"sanitized compile failed for {src}:\n" + "\n".join(msgs))
    return obj


def _fatbin_stub(src: str, host_obj: str) -> str:
    """An object defining the code-object bundle that a host-only object of
    `src` refers to (__hip_fatbin_<id>), with the bytes of the regular build's
    bundle for the same source: the sanitized library then registers the same
    kernels as libqmm.so."""
    r = subprocess.run(["nm", host_obj], capture_output=True, text=True, check=True)
    names = [ln.split()[-1] for ln in r.stdout.splitlines()
             if ln.split()[-1].startswith("__hip_fatbin_") and ln.split()[0] == "U"]
    if not names:
        return ""
    regular = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if not os.path.exists(regular):
        raise RuntimeError(f"{regular} missing: run build() first")
    blob = os.path.join(SAN_DIR, os.path.basename(src) + ".fatbin")
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", regular, blob], check=True)
    asm = os.path.join(SAN_DIR, os.path.basename(src) + ".fatbin.s")
    with open(asm, "w") as f:
        f.write('.section .hip_fatbin,"a",@progbits\n.p2align 12\n')
        for nm in names:
            f.write(f".globl {nm}\n{nm}:\n")
        f.write(f'.incbin "{blob}"\n')
    obj = asm[:-2] + ".o"
    subprocess.run([hipcc(), "-c", asm, "-o", obj], check=True, capture_output=True)
    return obj


def build_sanitized() -> str:
    """Build the ASan + UBSan host library (kernels from the regular build's
    objects); returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile_san, SOURCES))
    stubs = [o for o in (_fatbin_stub(src, obj) for src, obj in zip(SOURCES, objs)) if o]
    cmd = [hipcc(), "-shared", "-fPIC", "-shared-libsan", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", SAN_OUT] + objs + stubs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stdout + r.stderr)
    return SAN_OUT


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (preloaded into the test process)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or clang
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found: " + r.stdout + r.stderr)
    return path


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized())
    else:
        build(verbose=True)
