"""Build the HIP library (gfx950) in-tree: lvlm_kv_cache_amd/_build/libaircache.so."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "aircache.hip")
DEPS = [SRC, os.path.join(HERE, "csrc", "device_common.h"), os.path.join(ROOT, "include", "aircache.h")]
OUT = os.path.join(HERE, "_build", "libaircache.so")
ARCH = os.environ.get("AIRCACHE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the AirCache library)")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            # packed FP32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the library; force=False skips the build when it is up to date."""
    if not force and os.path.exists(OUT) and all(os.path.getmtime(OUT) >= os.path.getmtime(d) for d in DEPS):
        return OUT
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [hipcc(), *flags(), SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
