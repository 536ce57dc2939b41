"""Build the HIP library libkvq.so in-tree for gfx950 (MI355X).

Compiles every source under csrc/ with hipcc and links one shared library next to
this file. Run `python -m bit_asymmetric_kv_amd.build_lib` (or call build()).

`--incremental` recompiles only sources newer than their objects (or than the
shared header), for quick rebuilds. `--sanitize` also links libkvq_san.so: the
host code (argument checks, layout, bookkeeping) built with AddressSanitizer and
UndefinedBehaviorSanitizer, the device code unchanged; it is meant for CPU-only
checks of the C ABI (load it with the sanitizer runtime preloaded).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libkvq.so")
SAN_OUT = os.path.join(HERE, "libkvq_san.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["kvq_host.cpp", "append.hip", "decode.hip", "baseline.hip"]
HEADERS = [os.path.join(CSRC, "kvq_internal.h"), os.path.join(ROOT, "include", "kvq.h")]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR copies around the softmax rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
]

# host-only sanitizers: each -fsanitize= applies to the host pass alone
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(cc, src, obj, extra=(), verbose=False):
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [cc] + HIP_FLAGS + list(extra) + lang + ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stderr}")


def _stale(src, obj):
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(p) > t for p in [os.path.join(CSRC, src)] + HEADERS)


def _link(cc, objs, out, extra=()):
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC"] + list(extra) + ["-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, incremental: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cc = hipcc()
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        if not incremental or _stale(src, obj):
            _compile(cc, src, obj, verbose=verbose)
        objs.append(obj)
    _link(cc, objs, OUT)
    if sanitize:
        san_obj = os.path.join(BUILD_DIR, "kvq_host_san.o")
        _compile(cc, "kvq_host.cpp", san_obj, SAN_FLAGS, verbose=verbose)
        _link(cc, [san_obj] + objs[1:], SAN_OUT, ["-Xarch_host", "-shared-libsan"] + SAN_FLAGS)
    return OUT


def sanitizer_runtime() -> str | None:
    """Path of clang's shared AddressSanitizer runtime (to preload), if present."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv,
                sanitize="--sanitize" in sys.argv))
