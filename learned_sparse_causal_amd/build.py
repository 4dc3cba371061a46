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


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv[1:]))
