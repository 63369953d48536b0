"""Build the CPU oracle library (test infrastructure only).

Compiled with gcc, IEEE binary32 semantics: no fused multiply-add
contraction and no fast-math, so that fp32 decisions match the method's
definition bit for bit.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nvfp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source
# (clang, so that it shares one sanitizer runtime with the HIP library's
# sanitized host code in the same process); selected at load time with
# NVFP4_ORACLE_LIB.
LIB_SAN = os.path.join(HERE, "liboracle_san.so")
CLANG = os.environ.get("CLANG", "/opt/rocm/llvm/bin/clang")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    if sanitize:
        cmd = [CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c11", "-fPIC", "-shared",
               "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-shared-libasan", "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
               "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
