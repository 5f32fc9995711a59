"""Build libnq.so (HIP, gfx950) in place next to this file.

Usage: python -m e8_lattice_vector_amd.build   (or build() from Python)
"""

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnq.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every rounding in the decision path is spelled out; no contraction
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the quantize kernel reads
    # every product back into vector arithmetic, so AGPR copies would cost
    # one extra instruction per value
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # per-kernel register / scratch report, checked below
    "-Rpass-analysis=kernel-resource-usage",
]


def spilling_kernels(remarks: str):
    """Kernels whose resource report shows scratch (register spills): every
    kernel here is sized to keep its state in registers."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, f) for f in ("nq_api.cpp", "nq_kernels.hip", "nq_exact.hip", "nq_noalloc.hip")]
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libnq.so")
    spills = spilling_kernels(r.stderr)
    if spills:
        os.remove(tmp)
        raise RuntimeError(f"kernels spill to scratch: {spills[:5]} ({len(spills)} in all)")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
