"""Build the gfx950 shared library ``libroutedattn.so`` from csrc/*.hip with hipcc (in-tree).

Run ``python -m content_routed_sparse_amd.build``; the repository's ``__graft_entry__.build()``
calls :func:`build` too.  Host code compiles on any machine with ROCm; no GPU is needed.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libroutedattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
    # no packed-fp32 instructions (v_pk_*_f32) anywhere.  The driver cannot route -Xclang
    # pairs to the device compile alone, so the host compile sees the feature too and prints
    # HOST_FEATURE_NOTE once per source (it ignores the feature); build() drops that line.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-command-line-argument",
]


HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-I", os.path.join(HERE, "..", "include")] + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    rest = [ln for ln in proc.stdout.splitlines() if ln.strip() != HOST_FEATURE_NOTE]
    if rest:
        print("\n".join(rest), file=sys.stderr, flush=True)
    if proc.returncode != 0:
        raise subprocess.CalledProcessError(proc.returncode, cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
