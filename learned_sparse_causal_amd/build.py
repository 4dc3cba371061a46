"""Compile the gfx950 library libmono.so in-tree with hipcc.

    python -m learned_sparse_causal_amd.build [--incremental]

Every HIP source is compiled for gfx950 with fp contraction off (the routing
arithmetic is specified operation by operation) and packed fp32 ops disabled,
then linked into learned_sparse_causal_amd/libmono.so.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmono.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["capi.cpp", "build_index.hip", "route.hip", "attention.hip", "decode.hip", "calibrate.hip", "gemm.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _stale(src, obj):
    """An object is stale if it is missing or older than its source or any
    header of the source directory or include/."""
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src)]
    deps += [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith((".hpp", ".h"))]
    deps += [os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))]
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src, incremental=False):
    obj = os.path.join(BUILD_DIR, src + ".o")
    if incremental and not _stale(src, obj):
        return obj, ""
    cmd = ["hipcc", *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    return obj, err


def build(verbose=False, incremental=False):
    """Compile every source (only the stale ones with incremental=True) and
    link libmono.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, incremental), SOURCES))
    if verbose:
        for obj, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    return OUT


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
# layer (argument validation, workspace layout, dispatch), for the sanitizer
# run of the host tests.  Only the host pass of capi.cpp is instrumented (each
# sanitizer flag applies to the host through -Xarch_host); the kernels' objects
# are the normal build's.  Loaded through MONO_LIBRARY with clang's ASan runtime
# preloaded.
SAN_OUT = os.path.join(BUILD_DIR, "libmono_san.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized_host():
    """Compile capi.cpp with host sanitizers and link it with the normal
    build's kernel objects into _build/libmono_san.so."""
    objs = [os.path.join(BUILD_DIR, src + ".o") for src in SOURCES if src != "capi.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError("build the library first: %s" % missing[0])
    san_obj = os.path.join(BUILD_DIR, "capi_san.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run(["hipcc", *flags, *SAN_HOST, "-x", "hip", "-c",
                    os.path.join(CSRC, "capi.cpp"), "-o", san_obj],
                   check=True, capture_output=True, text=True)
    tmp = SAN_OUT + ".tmp%d" % os.getpid()
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_HOST,
                    "-Xarch_host", "-shared-libsan", "-o", tmp, san_obj, *objs],
                   check=True, capture_output=True, text=True)
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv[1:]))
