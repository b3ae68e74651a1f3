"""Build libdq.so (HIP kernels + C ABI) for gfx950, in-tree, with hipcc.

    python fp8_dynamic_quant_amd/build.py   (by path: importing the package needs the library)

Every call recompiles. Objects go to fp8_dynamic_quant_amd/_build/, the library to
fp8_dynamic_quant_amd/libdq.so (replaced atomically).
"""
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdq.so")
SOURCES = ["csrc/dq_api.cpp", "csrc/quantize.hip", "csrc/gemm_fp8.hip", "csrc/attention.hip",
           "csrc/gemm_mx.hip"]
ARCH = "gfx950"

# -O3, no fast-math and no denormal flushing (the quantizer relies on IEEE fp32 division with
# subnormals). Packed fp32 instructions are disabled for all device code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source additions. The GEMM's matrix operations must stay in the phase between the two
# workgroup barriers that bracket them (the other wave of the SIMD reads LDS meanwhile); they
# touch no memory, so machine sinking may move them past those barriers into the loop's last
# block, which serializes the ping-pong (seen with the block-scaled operands: all 16 sank).
EXTRA = {"csrc/gemm_fp8.hip": ["-mllvm", "-disable-machine-sink"]}


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError(f"hipcc not found ({cand})")
    return cand


def _quiet(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature flag; that note is harmless
    keep = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    return "\n".join(keep)


def build_library(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(HERE, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        out = _quiet(out)
        if out.strip() and (verbose or p.returncode):
            print(out, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    fd, tmp = tempfile.mkstemp(prefix="libdq.", suffix=".so.tmp", dir=HERE)
    os.close(fd)
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        os.unlink(tmp)
        print(_quiet(r.stdout), file=sys.stderr)
        raise RuntimeError("link of libdq.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
