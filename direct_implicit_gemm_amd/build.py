"""Build libconv.so (HIP, gfx950) in-tree.

    python -m direct_implicit_gemm_amd.build [--sanitize]

Compiles each source with hipcc for gfx950 only, in parallel, and links the
shared library next to this file.  Every build recompiles.

--sanitize builds libconv_san.so instead: the host code (validation, output
extents, planning, the chunk and frame-window arithmetic, the launch
wrappers) with AddressSanitizer and UndefinedBehaviorSanitizer; device code
is built as usual.  Load it with LIBCONV_LIBRARY=<path> and clang's ASan
runtime preloaded (see sanitizer_runtime()).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libconv.so")
SAN_LIB_PATH = os.path.join(HERE, "libconv_san.so")
# host-only sanitizer flags: each -fsanitize= applies to the host pass only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SOURCES = ["api.cpp", "direct.hip", "igemm.hip", "layout.hip",
           # the implicit-GEMM tiles, one unit per group so that they build in parallel
           "igemm_inst_a.hip", "igemm_inst_b.hip", "igemm_inst_c.hip", "igemm_inst_d.hip",
           "igemm_inst_e.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Werror",
    "-Wno-unused-function",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def sanitizer_runtime() -> str:
    """clang's ASan runtime (which carries the UBSan handlers too), to preload
    into the Python process that loads libconv_san.so."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("clang ASan runtime not found next to hipcc")
    return hits[-1]


def _compile(src: str, obj: str, extra=()) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def _check_stubs(lib: str) -> None:
    """Fail when a kernel's host launch stub is missing from the library (the
    host pass can drop one silently; the library would then not load)."""
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return  # no nm: the load test catches it
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("kernel launch stubs missing from libconv.so:\n" + "\n".join(missing))


def build(verbose: bool = True, sanitize: bool = False) -> str:
    extra = SAN_FLAGS if sanitize else []
    out = SAN_LIB_PATH if sanitize else LIB_PATH
    with tempfile.TemporaryDirectory(prefix="libconv_build_") as tmp:
        objs = [os.path.join(tmp, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
            list(ex.map(lambda a: _compile(*a, extra), zip(SOURCES, objs)))
        out_tmp = out + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", out_tmp, *objs]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        _check_stubs(out_tmp)
        os.replace(out_tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
