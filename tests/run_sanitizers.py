"""CPU sanitizer run: the oracle's C code and the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer, then the CPU tests that exercise
them (tests/test_oracle.py and tests/test_abi.py).  Needs no GPU.

Usage (from the repository root):  python tests/run_sanitizers.py

The oracle is built with gcc and runs against gcc's sanitizer runtimes; the HIP
library's host pass is built with hipcc (clang) and runs against clang's shared
ASan runtime (which carries UBSan too).  Each set of tests runs in its own
process with its runtime preloaded, since an uninstrumented Python has to load
the runtime first.  Leak checking is off (the interpreter itself keeps memory
until exit); any other report aborts the run.
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def gcc_runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()


def clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's shared ASan runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def run(tests, env_extra, label):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *tests]
    print(f"[sanitizers] {label}: {' '.join(cmd)}", flush=True)
    res = subprocess.run(cmd, cwd=ROOT, env=env)
    print(f"[sanitizers] {label}: exit {res.returncode}", flush=True)
    return res.returncode


def main():
    # Instrumented builds.
    env = dict(os.environ, EVO_ORACLE_SANITIZE="1")
    subprocess.run([sys.executable, "-c", "import oracle; print(oracle.build(force=True))"], cwd=ROOT, env=env,
                   check=True)
    sys.path.insert(0, ROOT)
    from af3_attention_amd import build as libbuild
    san_lib = libbuild.build(sanitize=True)
    print("[sanitizers] built", san_lib, flush=True)

    gcc_rt = ":".join(gcc_runtime(n) for n in ("libasan.so", "libubsan.so"))
    rc1 = run(["tests/test_oracle.py"], {"EVO_ORACLE_SANITIZE": "1", "LD_PRELOAD": gcc_rt},
              "oracle (gcc ASan+UBSan)")
    rc2 = run(["tests/test_abi.py"], {"EVOATTN_LIB": san_lib, "LD_PRELOAD": clang_asan_runtime()},
              "library host code (clang ASan+UBSan)")
    ok = rc1 == 0 and rc2 == 0
    print("[sanitizers] " + ("clean" if ok else "FAILED"), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
