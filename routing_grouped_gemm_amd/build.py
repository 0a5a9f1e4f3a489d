"""Build libmoe.so (the HIP library behind include/moe.h) for gfx950 in-tree.

    python -m routing_grouped_gemm_amd.build

Each csrc/*.hip file is compiled by hipcc in parallel, then linked into
routing_grouped_gemm_amd/libmoe.so.  Packed-fp32 instructions are disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops) for all device code.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# per-file flags.  gemm_bf16.hip: one lane fetches the persistent weight-gradient
# kernel's next tile position with a global atomic whose result is used only
# after the tile's main loop; the compiler's atomic optimizer would turn it into
# a wave-wide form that reads the result (and so waits for every outstanding
# memory operation, the previous tile's output stores included) right away.
EXTRA = {"gemm_bf16.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(verbose=True):
    """Compile every csrc/*.hip and link libmoe.so.  The previous library is
    removed first, so a failed build leaves no stale library behind."""
    os.makedirs(BUILD, exist_ok=True)
    if os.path.exists(LIB):
        os.remove(LIB)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for (obj, msgs) in results:
        if msgs.strip() and verbose:
            print(msgs, file=sys.stderr)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
