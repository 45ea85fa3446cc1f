"""Build libkda.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m linear_attention_recurrence_11_amd.build

Compiles every source under csrc/ with hipcc for gfx950 into
linear_attention_recurrence_11_amd/libkda.so. Packed-fp32 VALU instructions
are disabled for the device code.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.cpp", "kda_chunk.hip", "kda_decode.hip", "kda_spec.hip", "kda_scan.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose=False, extra_flags=()):
    """Compile libkda.so; always recompiles. Returns the library path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I" + INCLUDE, "-I" + CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # keep matrix-core accumulators in VGPRs: the state pass feeds them
           # to VALU work every chunk, and AGPR residency costs a move each way
           "-mllvm", "-amdgpu-mfma-vgpr-form",
           "-Wno-unused-command-line-argument"]
    cmd += list(extra_flags)
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
