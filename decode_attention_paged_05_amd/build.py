"""Build ``libpad.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python decode_attention_paged_05_amd/build.py [-v]`` (run as a file:
importing the package loads the library, which may not exist yet).  Always
recompiles.  The shared library lands next to this file, where the Python
binding loads it.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpad.so"
ARCH = "gfx950"

# Packed fp32 instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain (ROCm) is required to build libpad.so")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that note is expected
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


DEVICE_SOURCES = ["pad_kernels.hip", "pad_prefill.hip"] + [f"pad_attn_{dt}_{lay}_{form}.hip" for dt in ("bf16", "f32")
                                                             for lay in ("rows", "tiled") for form in ("split", "one_pass")]
# Per-source device flags.  The attention kernels accumulate in ordinary vector
# registers rather than accumulation registers: their lazy softmax rescale
# multiplies the accumulators on the vector ALU.  In the accumulation-register
# form the compiler copied the prefill accumulators across on every key step,
# and moved the decode P.V accumulators between the two register files (about
# 60 moves per 16-token block of phase 1, half its vector instructions);
# without them phase 1 measured about 0.5 us faster on the 100K-token step
# and every decode kernel needs fewer registers.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCE_FLAGS = {src: VGPR_FORM for src in DEVICE_SOURCES if src.startswith(("pad_prefill", "pad_attn_"))}
HOST_SOURCES = ["pad_api.cpp"]


def source_hash() -> str:
    """Hash of every file under csrc/ and include/ (names and contents, in name
    order): the build id the library reports through
    paged_attention_decode_build_id()."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(os.path.relpath(path, ROOT).encode())
                with open(path, "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, extra_flags=(), out: str = None) -> str:
    cc = hipcc()
    build_id = [f'-DPAD_SOURCE_HASH="{source_hash()}"']
    out = out or os.path.join(PKG, LIB_NAME)
    with tempfile.TemporaryDirectory(prefix="pad_build_") as tmp:
        jobs, objs = [], []
        for src in DEVICE_SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            jobs.append([cc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []),
                         *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        for src in HOST_SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            jobs.append([cc, *COMMON, *build_id, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp_out = out + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out], verbose)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
