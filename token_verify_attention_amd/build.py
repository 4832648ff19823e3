"""Build libspecverify.so (gfx950) in-tree with hipcc.

    python -m token_verify_attention_amd.build

Every HIP source under csrc/ is compiled for gfx950 only and linked into
token_verify_attention_amd/_lib/libspecverify.so.  No fast-math: fp32
division stays IEEE correctly rounded, which the INT8 codes depend on.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_lib")
LIB_NAME = "libspecverify.so"
OBJ_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of every kernel on purpose.  MFMA
# accumulators are kept in architectural VGPRs (the softmax rescales them with
# VALU ops, which cannot read AGPRs), instead of being copied between register
# files on every iteration.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def compile_flags():
    return COMMON_FLAGS + DEVICE_FLAGS


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that note.
    lines = [ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0 or (verbose and lines):
        print("\n".join(lines), file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}")


# Host-side AddressSanitizer build (the C ABI's argument checks and planning;
# the GPU code is built as usual).  Each sanitizer flag is marked host-only.
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-g"]


def asan_runtime():
    """The clang AddressSanitizer runtime next to hipcc's compiler, or None."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build(verbose=False, jobs=4, out_dir=None, obj_dir=None, asan=False):
    """Compile every HIP source and link the shared library.  Returns its path.
    asan=True builds the host code with AddressSanitizer (into out_dir)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    out_dir = out_dir or OUT_DIR
    obj_dir = obj_dir or OBJ_DIR
    os.makedirs(out_dir, exist_ok=True)
    os.makedirs(obj_dir, exist_ok=True)
    extra = ASAN_HOST_FLAGS if asan else []
    srcs = sources()
    objs = [os.path.join(obj_dir, os.path.basename(s) + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [HIPCC] + compile_flags() + extra + ["-c", s, "-o", o], verbose)
                for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = os.path.join(out_dir, LIB_NAME + ".tmp")
    link_extra = ["-Xarch_host", "-fsanitize=address", "-shared-libsan"] if asan else []
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + link_extra + objs,
         verbose)
    final = os.path.join(out_dir, LIB_NAME)
    shutil.move(tmp, final)
    return final


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
