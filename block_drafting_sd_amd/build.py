"""Build the step's shared library (HIP C++ for gfx950) in-tree.

``python -m block_drafting_sd_amd.build`` compiles every ``csrc/*.hip`` with
hipcc into ``block_drafting_sd_amd/libsd_amd.so``.  hipcc cross-compiles for
gfx950 on a machine without a GPU.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsd_amd.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32 from
# ordinary float code (the host pass warns that it does not know the
# feature; that is harmless).
HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Extra flags for single sources.  The attention and summary kernels keep their MFMA
# accumulators in ordinary VGPRs: the softmax reads every score and rescales
# the output accumulators, which would otherwise cost a copy out of (and back
# into) the accumulation registers per tile.
FILE_FLAGS = {
    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "summary.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Host-side sanitizers for a checking build of the C ABI's validation layer:
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
# (-Xarch_host before each -fsanitize=; the device code is built as usual).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host",
                  "-fno-sanitize-recover=undefined"]
SANITIZED_LIB_PATH = os.path.join(PKG, "libsd_amd_sanitized.so")


def clangxx() -> str:
    c = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin",
                     "clang++")
    for cand in (c, "/opt/rocm/lib/llvm/bin/clang++"):
        if os.path.exists(cand):
            return cand
    raise RuntimeError("ROCm's clang++ not found")


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime a host process preloads to run
    the sanitized library."""
    return subprocess.run([clangxx(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True, check=True).stdout.strip()


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every source and link ``libsd_amd.so`` (or, with
    ``sanitize``, the host-sanitized ``libsd_amd_sanitized.so``); returns its
    path."""
    cc = hipcc()
    srcs = sources()
    out_path = SANITIZED_LIB_PATH if sanitize else LIB_PATH
    extra = SANITIZE_FLAGS if sanitize else []
    with tempfile.TemporaryDirectory(prefix="sd_amd_build_") as tmp:
        objs, procs = [], []
        for s in srcs:
            o = os.path.join(tmp, os.path.basename(s) + ".o")
            cmd = [cc, *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), *extra,
                   f"-I{INCLUDE}", f"-I{CSRC}", "-c", s, "-o", o]
            if verbose:
                print(" ".join(cmd), flush=True)
            # compiler output goes to a file: a pipe nobody reads while
            # waiting for another job would stall a chatty compile
            log = open(o + ".log", "w+")
            procs.append((s, subprocess.Popen(cmd, stdout=log, stderr=subprocess.STDOUT,
                                              text=True), log))
            objs.append(o)
            while len([p for _, p, _ in procs if p.poll() is None]) >= jobs:
                next(p for _, p, _ in procs if p.poll() is None).wait()
        for s, p, log in procs:
            p.wait()
            log.seek(0)
            out = log.read()
            log.close()
            keep = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
            if p.returncode != 0:
                raise RuntimeError(f"hipcc failed on {s}:\n" + "\n".join(keep))
            if keep and verbose:
                print("\n".join(keep))
        tmp_lib = os.path.join(tmp, os.path.basename(out_path))
        if sanitize:
            # host link with the sanitizer runtimes as shared libraries
            rocm_lib = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "lib")
            cmd = [clangxx(), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan",
                   *objs, f"-L{rocm_lib}", "-lamdhip64", "-o", tmp_lib]
        else:
            cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        shutil.copyfile(tmp_lib, out_path + ".tmp")
        os.replace(out_path + ".tmp", out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
