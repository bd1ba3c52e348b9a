"""Build libgmi.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: python -m grouped_mixed_input_amd.build   (or call build())."""
from __future__ import annotations

import concurrent.futures as cf
import os
import pathlib
import shutil
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libgmi.so"
OBJDIR = PKG / "_build"
SOURCES = ["gmi_api.hip", "kernels_gemm.hip", "kernels_conv.hip", "kernels_w4a16.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = pathlib.Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else (shutil.which("hipcc") or "hipcc")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def _compile(src: pathlib.Path, obj: pathlib.Path) -> None:
    cmd = [hipcc(), *flags(), "-c", str(src), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{err}")
    if err.strip():
        print(err)


def build(jobs: int | None = None) -> pathlib.Path:
    OBJDIR.mkdir(exist_ok=True)
    objs = [OBJDIR / (s.replace(".hip", ".o")) for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(CSRC / so[0], so[1]), zip(SOURCES, objs)))
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
