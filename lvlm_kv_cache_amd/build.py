"""Build the HIP libraries (gfx950) in-tree under lvlm_kv_cache_amd/_build/:
libaircache.so (the compression pass) and libhbmprobe.so (the plain streaming
kernels the benchmark measures its bandwidth ceilings with)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SRC = os.path.join(CSRC, "aircache.hip")
PROBE_SRC = os.path.join(CSRC, "hbm_probe.hip")
OUT = os.path.join(HERE, "_build", "libaircache.so")
PROBE_OUT = os.path.join(HERE, "_build", "libhbmprobe.so")
ARCH = os.environ.get("AIRCACHE_OFFLOAD_ARCH", "gfx950")


def deps() -> list[str]:
    """Every source the pass library is built from: aircache.hip, every header
    under csrc/ and the public header."""
    return [SRC] + sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")) + \
        [os.path.join(ROOT, "include", "aircache.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the AirCache library)")


def flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
            # packed FP32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, out: str, srcs: list[str], force: bool, verbose: bool) -> str:
    if not force and os.path.exists(out) and all(os.path.getmtime(out) >= os.path.getmtime(d) for d in srcs):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *flags(), src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, out)
    return out


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile both libraries; force=False skips a build that is up to date.
    Returns the path of the pass library."""
    _compile(PROBE_SRC, PROBE_OUT, [PROBE_SRC], force, verbose)
    return _compile(SRC, OUT, deps(), force, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
