"""Build libatlas.so (all HIP sources, gfx950) in-tree with hipcc."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

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


def build(verbose: bool = False, sanitize: bool = False, incremental: bool = False) -> str:
    """Compile every HIP source into kv_cache_runtime_amd/libatlas.so (or,
    with sanitize, the host-sanitizer build libatlas_san.so).

    Each source is compiled to its own object in parallel (no relocatable
    device code: every kernel and its launch live in one file), then the
    objects are linked into the shared library.  With incremental, a source
    whose object is newer than it and than every header is not recompiled."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    target = SAN_LIB if sanitize else LIB
    tmp = target + ".tmp"
    objdir = os.path.join(HERE, "_build", "san" if sanitize else "rel")
    os.makedirs(objdir, exist_ok=True)
    extra = SAN_FLAGS if sanitize else []

    headers = [os.path.join(d, f) for d in (CSRC, INCLUDE) for f in os.listdir(d)
               if f.endswith(".h")]
    newest_header = max(os.path.getmtime(h) for h in headers)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        if (incremental and os.path.exists(obj) and
                os.path.getmtime(obj) > max(os.path.getmtime(src), newest_header)):
            return obj, subprocess.CompletedProcess([], 0, "")
        cmd = [hipcc, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        return obj, res

    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as pool:
        results = list(pool.map(compile_one, srcs))
    for _, res in results:
        out = "\n".join(l for l in res.stdout.splitlines()
                        if "packed-fp32-ops" not in l)  # host-pass notice about the feature flag
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
        if verbose and out.strip():
            print(out)
    cmd = [hipcc, *FLAGS, *extra, *[o for o, _ in results], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{res.stdout}")
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
    build(verbose="-v" in sys.argv, incremental="-i" in sys.argv)
    print(LIB)
