"""Build libgemmf16.so in-tree with hipcc for gfx950 (cross-compiles without
a GPU).  Each csrc/*.hip translation unit is compiled in parallel, then all
are linked into one shared library.

    python dense_tiled_gemm_fp16_amd/build.py [-v] [--incremental]

--incremental recompiles only the units older than their source or any
header under csrc/ or include/ (build() from the entry point always
compiles everything).
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libgemmf16.so")
OBJDIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms stay disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _obj(src):
    return os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")


def _stale(src):
    obj = _obj(src)
    if not os.path.exists(obj):
        return True
    deps = [src] + glob.glob(os.path.join(HERE, "csrc", "*.hpp")) + \
        glob.glob(os.path.join(HERE, "..", "include", "*.h"))
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def _compile(src, verbose):
    obj = _obj(src)
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return obj, res


def build(verbose=False, jobs=None, incremental=False):
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or max(1, min(16, len(os.sched_getaffinity(0))))
    objs = [_obj(s) for s in sources()]
    todo = [s for s in sources() if not incremental or _stale(s)]
    failed = []
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for obj, res in ex.map(lambda s: _compile(s, verbose), todo):
            if res.returncode != 0:
                failed.append(res.stdout + res.stderr)
    if failed:
        sys.stderr.write("\n".join(failed))
        raise RuntimeError("hipcc failed to compile libgemmf16")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to link libgemmf16.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
