"""Host-side sanitizer runs (CPU only): the oracle's C code built with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc), driven through every
entry point on small seeded inputs in a child Python process with the
sanitizer runtime preloaded. Any out-of-bounds access, use after free or
undefined behaviour aborts the child with a report, and the test fails with
that report. The HIP library is built a second time with AddressSanitizer on
its host code only (device code unoptimised, for build time; no kernel runs
without a GPU) and tests/test_abi.py, whose calls all return before any
launch, runs against it in a child with clang's sanitizer runtime preloaded."""
from __future__ import annotations

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "aircache_oracle.c")
OUT = os.path.join(ROOT, "oracle", "_build", "liboracle_san.so")

DRIVER = textwrap.dedent('''
    import numpy as np
    import oracle
    import workloads as wl

    for shape in (dict(L=2, B=2, Hq=6, Hkv=2, D=16, Nv=23, Nt=7, dtype="bf16", ratio=0.3),
                  dict(L=3, B=1, Hq=2, Hkv=1, D=8, Nv=5, Nt=1, ratio=1.0),
                  dict(L=1, B=3, Hq=4, Hkv=4, D=32, Nv=40, Nt=12, ratio=0.0)):
        w = wl.custom(**shape)
        inp = wl.make_inputs(w, 7)
        out = oracle.run(inp)
        oracle.run(inp, threads=2, compact=False)
        for b in range(w.B):
            el, pbar = oracle.elite_select(w, inp.q[0], inp.k[0], b)
            oracle.cross_score(w, inp.q[0], inp.k[0], b, el)
            oracle.cross_score_groups(w, inp.q[0], inp.k[0], b, el)
            qa = wl.prefill_queries(inp, 0)
            oracle.prefill_attention(w, qa, inp.k[0], inp.v[0], b, 0, None)
            oracle.visual_window(w, qa, inp.k[0], b, min(w.Nv, 3), groups=True)
            n = int(out["budget"][0, b]) + w.Nt
            off = int(out["out_off"][0, b])
            seg = out["k_out"][0][off:off + w.Hkv * n * w.D]
            oracle.decode_attention_segment(w, seg, seg, n, inp.q[0, b, :, 0, :])
            oracle.quantize_i8(seg, w.dtype)
        for mode in range(5):
            oracle.budget(np.linspace(0.5, 1.5, w.L), np.linspace(-1, 2, w.L), w.ratio, w.Nv, mode)
        oracle.topk(np.random.default_rng(0).random(w.Nv), w.Nv // 2)
    print("sanitized oracle ok")
''')


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.fixture(scope="module")
def san_lib():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-o", OUT, SRC, "-lm"])
    return asan


def test_oracle_under_address_and_undefined_sanitizers(san_lib):
    env = dict(os.environ, LD_PRELOAD=san_lib, AIRCACHE_ORACLE_LIB=OUT,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    p = subprocess.run([sys.executable, "-c", DRIVER], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert p.returncode == 0 and "sanitized oracle ok" in p.stdout, p.stdout[-3000:] + p.stderr[-6000:]


LIB_OUT = os.path.join(ROOT, "lvlm_kv_cache_amd", "_build", "libaircache_hostsan.so")
CLANG_RT = "/opt/rocm/lib/llvm/lib/clang"

ABI_DRIVER = textwrap.dedent('''
    import os, sys
    import pytest
    from lvlm_kv_cache_amd import _lib
    _lib.LIB_PATH = os.environ["AIRCACHE_ABI_TEST_LIB"]
    rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"])
    assert _lib._lib is not None and _lib._lib._name == _lib.LIB_PATH, "the sanitized library was not the one loaded"
    sys.exit(rc)
''')


def _clang_asan_runtime():
    if not os.path.isdir(CLANG_RT):
        return None
    for v in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_library_host_code_under_address_sanitizer():
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from lvlm_kv_cache_amd import build as b
    deps = b.deps()
    if not os.path.exists(LIB_OUT) or any(os.path.getmtime(d) > os.path.getmtime(LIB_OUT) for d in deps):
        os.makedirs(os.path.dirname(LIB_OUT), exist_ok=True)
        tmp = LIB_OUT + f".tmp{os.getpid()}"
        subprocess.check_call([b.hipcc(), "-g", "-std=c++17", f"--offload-arch={b.ARCH}", "-fPIC", "-shared",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-Xarch_host", "-O1", "-Xarch_device", "-O0",
                               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                               "-I", os.path.join(ROOT, "include"), "-I", b.CSRC, b.SRC, "-o", tmp],
                              stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        os.replace(tmp, LIB_OUT)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               AIRCACHE_ABI_TEST_LIB=LIB_OUT, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    p = subprocess.run([sys.executable, "-c", ABI_DRIVER], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-6000:]
