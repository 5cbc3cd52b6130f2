"""Builds libkda.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library lands next to this file, inside the package, so the Python binding,
the tests and the bench all load the in-tree build.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["kda_api.hip", "kda_backward.hip", "kda_decode.hip", "kda_dplr.hip", "kda_norm.hip", "kda_prefill.hip", "kda_seg.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build_library(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into one shared library. Packed fp32 instructions
    are disabled on the device side; the host pass warns that it does not know the
    feature, which is harmless."""
    out_tmp = LIB + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: the kernels post-process accumulators with VALU
        # instructions, which would otherwise need AGPR<->VGPR copies
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        *extra_flags,
        "-o", out_tmp,
        *[os.path.join(CSRC, s) for s in SOURCES],
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libkda.so")
    if verbose and res.stderr:
        noise = "is not a recognized feature for this target"
        msgs = [ln for ln in res.stderr.splitlines() if noise not in ln]
        if msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(out_tmp, LIB)
    return LIB


# host-side AddressSanitizer and UndefinedBehaviorSanitizer; every -fsanitize goes to
# the host pass only (the device code is built as usual and never run by these checks)
SANITIZE_HOST_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                       "-shared-libsan")


def sanitizer_runtime_dir() -> str:
    """Directory of the ROCm LLVM sanitizer runtimes a host-sanitized build links to."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True, check=True)
    return os.path.join(res.stdout.strip(), "lib", "linux")


def build_host_sanitized(out_path: str, verbose: bool = False) -> str:
    """The same library with the host code (the C ABI, argument checks, workspace
    sizing, launch set-up) built under AddressSanitizer and UndefinedBehaviorSanitizer,
    written to ``out_path``; the in-tree libkda.so is left alone."""
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-mllvm", "-amdgpu-mfma-vgpr-form=1", *SANITIZE_HOST_FLAGS,
        "-o", out_path + ".tmp", *[os.path.join(CSRC, s) for s in SOURCES],
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build the host-sanitized library")
    os.replace(out_path + ".tmp", out_path)
    return out_path


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--sanitize-host":
        build_host_sanitized(sys.argv[2], verbose=True)
    else:
        build_library(verbose=True)
