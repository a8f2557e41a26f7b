"""Build libpagedkv.so (gfx950) in-tree with hipcc.

Every HIP source under ``csrc/`` is compiled to an object in parallel and
linked into ``paged_kv_cache_mapping_amd/libpagedkv.so``; ``csrc/probe``
(the streaming-read probe that bench.py measures the ceiling with) becomes
``libpkvprobe.so``.  hipcc
cross-compiles, so this runs on a machine without a GPU.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
PROBE_LIB = os.path.join(PKG, "libpkvprobe.so")
PROBE_SOURCES = [os.path.join(CSRC, "probe", "stream_read.hip")]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-fvisibility=hidden",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    """Every .hip source; the heavy instantiation units first, so that the
    parallel build does not end on a long one started late."""
    def weight(f):
        return (0 if f.startswith("decode_multi_d") else 1 if f.startswith("decode_d") else 2, f)
    return [os.path.join(CSRC, f) for f in sorted((f for f in os.listdir(CSRC) if f.endswith(".hip")),
                                                  key=weight)]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose=True, jobs=None):
    """Compile every source, link the shared library and the streaming-read
    probe's library (csrc/probe, used by bench.py only); returns the
    library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources() + PROBE_SOURCES
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    n = len(srcs) - len(PROBE_SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


# Host-side sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer)
# for the CPU tests of argument checks, plans and sizing: the flags reach
# the host compilation only; the device code is built as usual.
SANITIZE_DIR = os.path.join(BUILD, "host_sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libpagedkv.so")
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined"]
CLANG = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")


def _compile_host_sanitized(src):
    obj = os.path.join(SANITIZE_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = ([HIPCC] + COMMON_FLAGS + ["-Xarch_host", "-O1", "-Xarch_host", "-g", "-Xarch_host",
                                     "-fno-omit-frame-pointer"]
           + SANITIZE_FLAGS + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def sanitizer_runtime():
    """The shared AddressSanitizer runtime the sanitized library needs
    preloaded into the Python process."""
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    return r.stdout.strip()


def build_host_sanitized(jobs=None):
    """Build SANITIZE_LIB unless it is newer than every source; returns its
    path."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    srcs = sources()
    deps = srcs + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)] + [os.path.abspath(__file__)]
    if os.path.exists(SANITIZE_LIB) and os.path.getmtime(SANITIZE_LIB) > max(map(os.path.getmtime, deps)):
        return SANITIZE_LIB
    jobs = jobs or max(1, min(8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile_host_sanitized, srcs))
    tmp = SANITIZE_LIB + ".tmp"
    cmd = ([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-shared-libsan"] + SANITIZE_FLAGS
           + ["-o", tmp] + objs)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, SANITIZE_LIB)
    return SANITIZE_LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
