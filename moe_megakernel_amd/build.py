"""Builds the C-ABI library libmoe_mi355x.so in-tree with hipcc for gfx950.

    python -m moe_megakernel_amd.build
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _sched(strategy):
    return ["-mllvm", f"--amdgpu-sched-strategy={strategy}"]


# Translation units and their own flags.  The weight gradients take LLVM's max-ilp
# instruction scheduling (1-4% faster per launch on MI355X); for the token GEMMs no
# strategy measured faster than the default.
SOURCES = [
    ("moe_api.hip", []),                     # C ABI, routing and row kernels
    ("gemm_tok.hip", []),                    # token-dimension GEMMs
    ("gemm_wgrad.hip", _sched("max-ilp")),   # weight gradients
]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed-FP32 VALU ops stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]
_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, out: str = LIB, defines: tuple = ()) -> str:
    """Compile the library to `out`; `defines` are extra -D options (tile variants).
    The translation units compile in parallel, then link into one shared library."""
    from concurrent.futures import ThreadPoolExecutor
    tmp = out + ".tmp"
    objs = [f"{out}.{i}.o" for i in range(len(SOURCES))]
    dflags = [f"-D{d}" for d in defines]

    def compile_one(i):
        src, extra = SOURCES[i]
        _run([HIPCC, *FLAGS, *extra, *dflags, "-c", os.path.join(PKG, "csrc", src), "-o", objs[i]], verbose)

    try:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            list(ex.map(compile_one, range(len(SOURCES))))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    os.replace(tmp, out)
    return out


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_caller", "moe_c_caller.c")
C_CALLER = os.path.join(ROOT, "tests", "c_caller", "moe_c_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_caller(lib: str = LIB, out: str = C_CALLER) -> str:
    """The plain C test caller of the library (host code only, gcc): it links
    libmoe_mi355x.so and the HIP runtime, and finds both through its run path."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           C_CALLER_SRC, "-o", out + ".tmp",
           "-L", os.path.dirname(lib), "-lmoe_mi355x", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../moe_megakernel_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_caller())
