"""Build libtq2.so (HIP, gfx950) in the package directory with hipcc.

Usage: ``python -m gemv_tq2_g128_amd.build`` or ``build()`` from Python.
"""

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
LIB_NAME = "libtq2.so"
SOURCES = ["tq2_api.hip", "tq2_reformat.hip", "tq2_gemv.hip", "tq2_gemm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Code object v5: loadable by the HIP runtime PyTorch ships as well.
    "-mcode-object-version=5",
    "-shared",
    # No packed-FP32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc_path():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


PROBE_LIB_NAME = "libtq2_probe.so"
PROBE_SOURCES = ["tq2_probe.hip"]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libtq2.so`` (and the benchmark's
    reference kernels into ``libtq2_probe.so``); returns the library path."""
    _compile(PROBE_SOURCES, PROBE_LIB_NAME, verbose)
    return _compile(SOURCES, LIB_NAME, verbose)


def _compile(sources, lib_name, verbose):
    out = os.path.join(PKG_DIR, lib_name)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc_path(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only target feature; drop that noise.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, msg))
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
