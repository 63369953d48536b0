"""Run the CPU checks of the oracle and of the C ABI's host validation under
AddressSanitizer + UndefinedBehaviorSanitizer.

Builds the oracle (oracle/build.py --sanitize) and the HIP library with
sanitized host code (quantize_precision_gemm_amd/build.py --sanitize), then
runs the CPU tests that exercise them -- the oracle's pins and the C-ABI
export, status and argument-validation tests -- in a child process with the
sanitizer runtime preloaded (the Python interpreter itself is not
instrumented).  Any sanitizer report aborts the run.  Exit status: pytest's.

    python tests/run_sanitized.py [extra pytest args]
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

TESTS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py", "tests/test_oracle_philox.py",
         "tests/test_oracle_rht_gemm.py", "tests/test_oracle_rht_sized.py", "tests/test_oracle_mx.py",
         "tests/test_abi.py", "tests/test_binding_checks.py"]


def main():
    from oracle import build as orc_build
    from quantize_precision_gemm_amd import build as hip_build

    orc = orc_build.build(verbose=True, sanitize=True)
    hip = hip_build.build(verbose=True, sanitize=True)
    clang = os.environ.get("CLANG", "/opt/rocm/llvm/bin/clang")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "NVFP4_ORACLE_LIB": orc,
        "NVFP4_LIB": hip,
        # the interpreter and torch are not instrumented: no leak report at exit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"] + \
        TESTS + sys.argv[1:]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    sys.exit(main())
