"""Build libspecverify.so in place with hipcc for gfx950.

    python speculative_decoding_verification_gemm_amd/build.py [-v] [--diagnostics]

Run it as a script (the package's own import needs the built library).

Compiles every source under csrc/ into one shared library next to this file.
``--diagnostics`` builds libspecverify_diag.so instead, with SPECV_DIAGNOSTICS
defined: the chain kernel then records per-workgroup barrier timestamps into
the device buffer named by SPECV_CHAIN_TRACE, SPECV_STREAM_WGS_PER_CU
overrides the streaming grid, and tile-parameter macros may be overridden
with -D flags in SPECV_EXTRA_FLAGS. The binding never loads that library.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
DIAG_LIB = os.path.join(HERE, "libspecverify_diag.so")
SOURCES = ["api.cpp", "gemm_stream.hip", "gemm_skinny.hip", "gemm_mfma.hip", "sampler.hip",
           "attention.hip", "probe.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose=False, diagnostics=False):
    """Compile every source and link the shared library; returns its path."""
    lib = DIAG_LIB if diagnostics else LIB
    flags = list(COMMON)
    if diagnostics:
        flags += ["-DSPECV_DIAGNOSTICS"] + os.environ.get("SPECV_EXTRA_FLAGS", "").split()
    with tempfile.TemporaryDirectory(prefix="specverify_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmds.append([HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        # one hipcc per source, run side by side
        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for cmd in cmds:
                if verbose:
                    print(" ".join(cmd), flush=True)
            for f in [pool.submit(subprocess.run, c, check=True) for c in cmds]:
                f.result()
        tmp_lib = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, diagnostics="--diagnostics" in sys.argv))
