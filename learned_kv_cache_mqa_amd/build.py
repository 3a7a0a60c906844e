"""Build libkvmem.so in-tree with hipcc for gfx950.

    python -m learned_kv_cache_mqa_amd.build [--jobs N] [--verbose] [--asan]

Every csrc/*.hip file is compiled to an object under _build/ and linked into
learned_kv_cache_mqa_amd/libkvmem.so.  Always recompiles (the build is the check).
"""
import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvmem.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (p.stdout + p.stderr).splitlines() if _NOISE not in line)
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


# Host-only AddressSanitizer build (the device code is built as usual): every -fsanitize
# flag sits behind -Xarch_host, so it never reaches the GPU compilation.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_DIR = os.path.join(BUILD, "asan")


def build(jobs=None, verbose=False, asan=False):
    """Compile every csrc/*.hip and link libkvmem.so (in the package; with asan=True the
    host-sanitized library goes to _build/asan/ instead).  Returns the library's path."""
    out_dir = ASAN_DIR if asan else BUILD
    lib = os.path.join(ASAN_DIR, "libkvmem.so") if asan else LIB
    os.makedirs(out_dir, exist_ok=True)
    extra = ASAN_FLAGS if asan else []
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [HIPCC, *FLAGS, *extra, "-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)
    return lib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--asan", action="store_true", help="host AddressSanitizer build into _build/asan/")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, a.asan))


if __name__ == "__main__":
    sys.exit(main())
