"""Build libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["api.cpp", "plan.cpp", "prefill.hip", "prefill_w64.hip", "prefill_f32.hip", "gqa_decode.hip", "decode.hip",
           "merge.hip", "quantize.hip"]
# per-source compiler options: the GQA decode and fp32 prefill kernels keep their matrix-core
# accumulators in ordinary vector registers (they need few registers; see the headers of those
# sources)
VGPR_MFMA = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {"gqa_decode.hip": VGPR_MFMA, "prefill_f32.hip": VGPR_MFMA}
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libattn.so next to this file."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [cc, "-x", "hip", *HIPCC_FLAGS, *EXTRA_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj]))
    with ThreadPoolExecutor(len(jobs)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB + ".tmp"
    outs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs]]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
