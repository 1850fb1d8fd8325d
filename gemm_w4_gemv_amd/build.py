"""Compile the HIP sources under ``csrc/`` into ``libw4.so`` (gfx950 only).

Each ``.hip`` file is compiled to an object under ``_build/`` in parallel,
then linked into ``gemm_w4_gemv_amd/libw4.so``, next to this file.  No GPU is
needed: hipcc cross-compiles for gfx950.

    python gemm_w4_gemv_amd/build.py            # build
    python gemm_w4_gemv_amd/build.py --asm      # also write device assembly (.s)

(Run it as a script, or through ``__graft_entry__.build()``: importing the
package first would load the library this builds.)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libw4.so"
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and pathlib.Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def flags(extra=()) -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        f"-I{ROOT / 'include'}", f"-I{CSRC}",
        # no packed-FP32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in ordinary VGPRs: the prefill GEMM's 128 accumulator
        # registers otherwise bounce between AGPRs and VGPRs inside its K loop
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-command-line-argument",
        *extra,
    ]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the device-only feature above; that note is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    return res.returncode, "\n".join(lines)


def build(verbose: bool = False, asm: bool = False, defines=(), lib: pathlib.Path = LIB,
          build_dir: pathlib.Path = BUILD) -> pathlib.Path:
    """Compile and link; ``defines`` (NAME or NAME=VALUE) go to every source."""
    build_dir.mkdir(parents=True, exist_ok=True)
    lib.parent.mkdir(parents=True, exist_ok=True)
    cc = hipcc()
    extra = [f"-D{d}" for d in defines]
    sources = sorted(CSRC.glob("*.hip"))
    jobs = []
    for src in sources:
        obj = build_dir / (src.stem + ".o")
        jobs.append(([cc, *flags(extra), "-c", str(src), "-o", str(obj)], obj))
        if asm:
            jobs.append(([cc, *flags(extra), "--cuda-device-only", "-S", str(src),
                          "-o", str(build_dir / (src.stem + ".s"))], None))
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(lambda j: (_run(j[0]), j[0]), jobs))
    for (rc, out), cmd in results:
        if out and (verbose or rc):
            print(out, file=sys.stderr)
        if rc:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}")
    objs = [str(o) for _, o in jobs if o is not None]
    tmp = lib.with_suffix(".so.tmp")
    rc, out = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *objs])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    path = build(verbose=True, asm="--asm" in sys.argv)
    print(path)
