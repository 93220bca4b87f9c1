"""Build the gfx950 HIP library ``libpaged_kv.so`` in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libpaged_kv.so")
SOURCES = ["paged_attention_decode.hip", "paged_attention_prefill.hip", "paged_attention_prefill_f32.hip", "kv_cache_ops.hip",
           "prefix_cache.hip", "decode_plan.cpp", "capi.cpp", "decode_noalloc.hip"]
ARCH = os.environ.get("PAGED_KV_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-command-line-argument", "-fvisibility=hidden",
    # no packed fp32 instructions in generated device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in arch VGPRs: the prefill kernel's accumulators are also
    # rescaled by VALU code, and in AGPRs every loop iteration copied them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc, *FLAGS, "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
