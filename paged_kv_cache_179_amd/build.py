"""Build the HIP library ``libpaged_attention.so`` in-tree for gfx950.

Each source under ``csrc/`` is compiled by hipcc into ``_build/`` (in
parallel), then linked into the package directory.  Run as a module
(``python -m paged_kv_cache_179_amd.build``) or call ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
REPO = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIB = PKG / "libpaged_attention.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU ops are kept out of generated code on this target.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{REPO / 'include'}",
    f"-I{CSRC}",
]
# Per-source extras.  The MFMA kernels rescale their accumulators with
# vector ALU ops inside the loop; keeping MFMA results in ordinary VGPRs (not
# AGPRs) avoids a copy of every accumulator in and out on each pass.
EXTRA_FLAGS = {
    "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def sources():
    return sorted(list(CSRC.glob("*.hip")) + list(CSRC.glob("*.cpp")))


def _compile(src: Path, verbose: bool) -> Path:
    obj = BUILD / (src.name + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src.name, []), "-c", str(src), "-o", str(obj)]
    if src.suffix == ".cpp":
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> Path:
    """Compile every HIP source and link the shared library; returns its path."""
    BUILD.mkdir(exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
