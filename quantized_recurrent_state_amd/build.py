"""Build libleapq.so (gfx950) in-tree with hipcc, and the measurement probes
beside it (libleapq_probe.so: the append's memory traffic without its
arithmetic, a plain streaming read, matrix/VALU co-execution; the same
source built with AGPR accumulators as libleapq_probe_agpr.so).

Flags that matter for the numbers:
  -ffp-contract=off   no fused multiply-add except the explicit ones
  -amdgpu-mfma-vgpr-form  matrix-instruction accumulators in ordinary VGPRs
                      (no AGPR copies of the fold's state tile)
  packed-fp32-ops off the kernels are written for unpacked fp32 VALU
  (no fast-math, no denormal flush; '/' and sqrtf stay correctly rounded,
   which is hipcc's default for HIP)
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libleapq.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("leapq_append.hip", "leapq_fold.hip", "leapq_dense.hip", "leapq_abi.cpp")]
PROBE_LIB = os.path.join(PKG, "libleapq_probe.so")
PROBE_LIB_AGPR = os.path.join(PKG, "libleapq_probe_agpr.so")
PROBE_SOURCE = os.path.join(CSRC, "probe_pattern.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libleapq")


def build(out=LIB, extra=(), verbose=False, probe=True):
    """Compile every HIP source (one hipcc process each, in parallel) and
    link them into `out`, and (probe) the probe library; returns `out`."""
    tmp, ptmp, ptmp2 = out + ".tmp", PROBE_LIB + ".tmp", PROBE_LIB_AGPR + ".tmp"
    with tempfile.TemporaryDirectory(prefix="leapq_build_") as d:
        objs = [os.path.join(d, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[HIPCC, *FLAGS, *extra, "-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
        if probe:
            cmds.append([HIPCC, *FLAGS, "-shared", PROBE_SOURCE, "-o", ptmp])
            # the one -mllvm option of FLAGS is the accumulator form
            agpr_flags = [f for f in FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
            cmds.append([HIPCC, *agpr_flags, "-shared", PROBE_SOURCE, "-o", ptmp2])
        with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    if probe:
        os.replace(ptmp, PROBE_LIB)
        os.replace(ptmp2, PROBE_LIB_AGPR)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
