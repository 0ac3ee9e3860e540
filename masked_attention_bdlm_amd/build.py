"""Build the C-ABI shared library libbdlm_attn.so for gfx950 with hipcc.

Usage: python -m masked_attention_bdlm_amd.build   (or build() from Python).
The library is written next to this file so that it ships with the tree.
"""
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbdlm_attn.so")
SOURCES = ["bdlm_api.hip", "bdlm_kernels.hip", "bdlm_calib.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, extra=None) -> str:
    out_tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    t0 = time.time()
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libbdlm_attn.so")
    os.replace(out_tmp, LIB)
    if verbose:
        msgs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if msgs:
            sys.stderr.write("\n".join(msgs) + "\n")
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
