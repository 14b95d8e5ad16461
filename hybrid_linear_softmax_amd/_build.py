"""Build libhybrid_attn.so in-tree with hipcc for gfx950.

Every source is compiled each time build() runs (object files under _build/,
one hipcc process per source in parallel), then linked into
hybrid_linear_softmax_amd/libhybrid_attn.so.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libhybrid_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ("api.cpp", "kv_state.hip", "apply.hip", "anchor.hip", "proj.hip", "linear_bwd.hip", "anchor_bwd.hip", "attnres.hip",
           "probe.hip", "noalloc.hip")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", *lang,
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def _check_no_undefined_kernels(lib: str) -> None:
    """A kernel whose host launch stub the compiler failed to emit shows up as
    an undefined symbol of the library's own namespace; refuse such a library
    (it would only fail later, when loaded)."""
    nm = shutil.which("nm") or shutil.which("llvm-nm")
    if nm is None:
        return
    res = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    missing = [line.split()[-1] for line in res.stdout.splitlines() if "_ZN2ha" in line]
    if missing:
        raise RuntimeError(f"{lib} has undefined symbols of its own code: {missing[:4]}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stderr}")
    _check_no_undefined_kernels(tmp)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (the C-ABI validation and every launcher's host code; device code is
# built as usual, with no sanitizer).  Each sanitizer flag reaches the host
# compilation only; the link is a plain host link with clang++.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized library needs (preloaded
    into the process that loads it)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang++"
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime not found")
    return path


def build_host_sanitized(out_dir: str) -> str:
    """Build libhybrid_attn.so with host-side ASan/UBSan into out_dir; returns
    the library path (load it with asan_runtime() preloaded)."""
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc(), *COMMON_FLAGS, *SANITIZE_HOST, "-I", INCLUDE, "-I", CSRC, "-c", *lang,
               os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(one, SOURCES))
    lib = os.path.join(out_dir, LIB_NAME)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    clang = os.path.join(rocm, "llvm", "bin", "clang++")
    cmd = [clang, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", *objs,
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{' '.join(cmd)}\n{res.stderr}")
    return lib


if __name__ == "__main__":
    build()
