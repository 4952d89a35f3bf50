"""Build libatlas.so (all HIP sources, gfx950) in-tree with hipcc."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libatlas.so")
SAN_LIB = os.path.join(HERE, "libatlas_san.so")

SOURCES = ["api.hip", "decode.hip", "decode_mfma.hip", "prefill.hip", "inspect.hip",
           "kv_write.hip", "residency.cpp"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # keep the compiler from forming packed-f32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer build (the device
# code is built as usual): the host argument checks, size arithmetic and the
# residency runtime run instrumented.  Load it with ATLAS_LIBRARY=<SAN_LIB> and
# the clang ASan runtime preloaded (sanitize_env() gives the environment).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
             "-fno-omit-frame-pointer", "-g"]


def sanitize_env() -> dict:
    """Environment for running the CPU tests against the sanitizer build."""
    rt = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                        stdout=subprocess.PIPE, text=True).stdout.strip()
    env = dict(os.environ)
    env.update(ATLAS_LIBRARY=SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every HIP source into kv_cache_runtime_amd/libatlas.so (or,
    with sanitize, the host-sanitizer build libatlas_san.so)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    target = SAN_LIB if sanitize else LIB
    tmp = target + ".tmp"
    cmd = [hipcc, *FLAGS, *(SAN_FLAGS if sanitize else []), "-I", INCLUDE, "-I", CSRC, *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host-pass notice about the feature flag
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        # build, then run the host-side tests under the sanitizers
        print(build(verbose="-v" in sys.argv, sanitize=True), flush=True)
        tests = [os.path.join(ROOT, "tests", t) for t in ("test_residency.py", "test_abi.py")]
        res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", *tests],
                             env=sanitize_env(), cwd=ROOT)
        sys.exit(res.returncode)
    build(verbose="-v" in sys.argv)
    print(LIB)
