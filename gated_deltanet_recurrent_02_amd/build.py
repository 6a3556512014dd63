"""Build libgdn.so in-tree with hipcc for gfx950.

    python -m gated_deltanet_recurrent_02_amd.build        # or __graft_entry__.build()

The library is the hand-written HIP kernels plus the C-ABI layer; it links only the HIP
runtime. A second, separate library, libgdn_probe.so, holds the benchmark's in-place stream
probe (a calibration kernel with the decode kernels' memory access pattern and no arithmetic);
the GDN library does not contain or load it. Packed-fp32 instruction selection is switched off (-packed-fp32-ops), and matrix-core
results are kept in ordinary VGPRs (-amdgpu-mfma-vgpr-form) so that the vector code of the
prefill kernel reads them without accumulator-register copies; kernels without matrix-core
instructions compile to the same code either way.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgdn.so")
SOURCES = [os.path.join(CSRC, "gdn_kernels.hip"), os.path.join(CSRC, "gdn_prefill.hip"),
           os.path.join(CSRC, "gdn_lowrank.hip"), os.path.join(CSRC, "gdn_api.cpp")]
PROBE_SOURCE = os.path.join(CSRC, "gdn_stream_probe.hip")
PROBE_LIBRARY = os.path.join(PKG, "libgdn_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(output: str = LIBRARY, extra_flags: list[str] | None = None, verbose: bool = False,
          probe_output: str | None = PROBE_LIBRARY) -> str:
    """Compile the kernels and the C ABI into one shared library; returns its path. Each source
    compiles to an object of its own, all at once, and one hipcc call links them. The stream
    probe library is built alongside (skipped when probe_output is None)."""
    objdir = os.path.join(os.path.dirname(os.path.abspath(output)), "_build")
    os.makedirs(objdir, exist_ok=True)
    cflags = [f for f in HIPFLAGS if f != "-shared"]
    objs, procs = [], []
    sources = SOURCES + ([PROBE_SOURCE] if probe_output else [])
    for src in sources:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *cflags, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", "-c", "-o", obj, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append((cmd, subprocess.Popen(cmd)))
    failed = [cmd for cmd, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    links = [(output, objs[:len(SOURCES)])]
    if probe_output:
        links.append((probe_output, objs[len(SOURCES):]))
    for out, lib_objs in links:
        tmp = out + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
