"""Build libtsd_attn.so (gfx950) in-tree with hipcc.

Usage: python -m tiled_scaled_dot_amd.build   (always recompiles)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libtsd_attn.so")
# (source, object name, extra defines): the kernel file is compiled once per
# unit (plain + merge, extended, per-block scaled) so the units build in
# parallel.
SOURCES = [
    ("attn_api.hip", "attn_api.o", []),
    ("attn_kernels.hip", "attn_kernels_plain.o", ["-DTSD_UNIT=0"]),
    ("attn_kernels.hip", "attn_kernels_ext.o", ["-DTSD_UNIT=1"]),
    ("attn_kernels.hip", "attn_kernels_scaled.o", ["-DTSD_UNIT=2"]),
]
ARCH = "gfx950"

# Packed-f32 VALU instructions are disabled for all device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-fvisibility=hidden",   # only the TSD_API entry points are exported
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(output: str = LIBRARY, extra_flags=None, verbose: bool = False) -> str:
    """Compile every HIP source into one shared library (always rebuilds)."""
    objs = []
    # one object folder per output, so that several builds may run at once
    tmpdir = os.path.join(PKG, "_build", os.path.splitext(os.path.basename(output))[0])
    os.makedirs(tmpdir, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])
    procs = []
    for src, obj_name, defines in SOURCES:
        obj = os.path.join(tmpdir, obj_name)
        cmd = [hipcc(), *flags, *defines, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT),
                      obj_name))
        objs.append(obj)
    failed = []
    for proc, src in procs:
        out, _ = proc.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; harmless.
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln
                 and "not a recognized feature" not in ln and ln.strip()
                 and not ln.startswith("1 warning generated")]
        if lines and (verbose or proc.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if proc.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = output + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
