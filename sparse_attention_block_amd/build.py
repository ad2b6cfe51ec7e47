"""Build liblosa.so (the HIP library) for gfx950 with hipcc, in-tree.

Flags: -O3; -ffp-contract=off so that every a*b+c in the index-deciding fp32
chains stays two roundings (the kernels call fmaf explicitly where a fused
multiply-add is intended); packed fp32 instructions are disabled; matrix-core
instructions take their accumulators in ordinary VGPRs (gfx950 allows it), so
that accumulators the vector ALU also touches (the online-softmax rescale) are
not copied to and from AGPRs around every MFMA.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "liblosa.so")
SELFTEST_LIB = os.path.join(HERE, "liblosa_selftest.so")
SOURCES = ["losa_api.hip", "page_meta.hip", "prepare.hip", "select.hip", "prefix.hip", "finish.hip"]
ARCH = os.environ.get("LOSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form=1",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{out}")
    return out


def build(out: str = LIB, jobs: int = 8, extra=()) -> str:
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        _run([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


def build_selftest(out: str = SELFTEST_LIB) -> str:
    """liblosa_selftest.so: GPU checks of builtin rounding and MFMA lane layouts."""
    tmp = out + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "selftest.hip")])
    os.replace(tmp, out)
    return out


def build_all() -> None:
    build()
    build_selftest()


if __name__ == "__main__":
    build_all()
    print(LIB, SELFTEST_LIB, file=sys.stderr)
