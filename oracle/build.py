"""Builds ``liboracle.so`` from ``kda_oracle.c`` with gcc (plain C, OpenMP, fp64).

Test infrastructure: the GPU library never links this.
"""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def oracle_lib_path() -> str:
    return _LIB


def oracle_source_path() -> str:
    return _SRC


def build_oracle(verbose: bool = False) -> str:
    """Compile the oracle. FP contraction is off so the arithmetic is the plain
    sequence of fp64 multiplies and adds written in the source."""
    cmd = [
        "gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
        "-fopenmp", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


SANITIZE_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer")


def build_sanitized_program(driver_c: str, out_path: str, verbose: bool = False) -> str:
    """Links a C driver with the oracle's source into an executable built under gcc's
    AddressSanitizer and UndefinedBehaviorSanitizer (the oracle's C checked for
    out-of-bounds access, leaks and undefined behaviour)."""
    cmd = ["gcc", "-O1", "-g", *SANITIZE_FLAGS, "-ffp-contract=off", "-fopenmp", "-o", out_path, driver_c, _SRC,
           "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out_path
