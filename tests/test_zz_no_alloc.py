"""aircache_run_noalloc (the pass on the library's static scratch, for callers
that cannot allocate) against aircache_run with a caller workspace, through
the C ABI: two calls in a row, the second with a smaller input (a different
descriptor, so the scratch is zeroed again), then the first shape once more.

The pass is deterministic, so every plan output and the compacted caches
must be bit-identical to aircache_run's on the same inputs; each result is
also checked against the CPU oracle by the parity rules."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import compare, make_aircache, reference, to_torch

pytestmark = pytest.mark.gpu

FIELDS = ("n_elite", "iv", "s_t", "s_k", "budget_x", "budget", "out_off", "status")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lvlm_kv_cache_amd import _lib
    _lib.load()  # raises if the HIP library is missing
    torch.cuda.set_device(0)


def host(plan, ko, vo, w):
    out = {f: getattr(plan, f).cpu().numpy() for f in FIELDS + ("elite_idx", "kept_idx")}
    store = np.float32 if w.dtype == wl.F32 else np.uint16
    def conv(t, n):
        a = t[:n].cpu()
        if w.dtype == wl.BF16:
            a = a.view(torch.int16)
        return a.numpy().view(store)
    out["k_out"] = [conv(ko[l], int(out["out_off"][l, w.B])) for l in range(w.L)]
    out["v_out"] = [conv(vo[l], int(out["out_off"][l, w.B])) for l in range(w.L)]
    return out


def run_both(w, seed):
    from lvlm_kv_cache_amd import _lib
    inp = wl.make_inputs(w, seed)
    q, k, v = to_torch(inp)
    ac = make_aircache(w)
    assert ac.ws_bytes <= _lib.NOALLOC_SCRATCH_BYTES
    # the existing entry point, with a caller workspace
    p1 = ac.alloc_plan()
    k1, v1 = ac.alloc_compacted()
    ac.run(q, k, v, p1, k1, v1)
    # the scratch entry point on the same inputs, into fresh outputs
    p2 = ac.alloc_plan()
    k2, v2 = ac.alloc_compacted()
    st = torch.cuda.current_stream().cuda_stream
    rc = _lib.run_noalloc(ac.desc, [t.data_ptr() for t in q], [t.data_ptr() for t in k], [t.data_ptr() for t in v],
                          p2.buf(), [t.data_ptr() for t in k2], [t.data_ptr() for t in v2], st)
    _lib.check(rc)
    torch.cuda.synchronize()
    a, b = host(p1, k1, v1, w), host(p2, k2, v2, w)
    for f in FIELDS:
        assert np.array_equal(a[f], b[f]), f
    for l in range(w.L):
        for bb in range(w.B):
            n = a["n_elite"][l, bb]
            assert np.array_equal(a["elite_idx"][l, bb, :n], b["elite_idx"][l, bb, :n])
            r = a["budget"][l, bb]
            assert np.array_equal(a["kept_idx"][l, bb, :r], b["kept_idx"][l, bb, :r])
        assert np.array_equal(a["k_out"][l], b["k_out"][l])
        assert np.array_equal(a["v_out"][l], b["v_out"][l])
    compare(inp, b, reference(inp, b))


def test_noalloc_matches_run_then_smaller_input():
    big = wl.custom(L=4, B=2, Hq=14, Hkv=2, D=128, Nv=900, Nt=40, dtype="bf16", ratio=0.2)
    small = wl.custom(L=2, B=1, Hq=4, Hkv=4, D=64, Nv=130, Nt=12, dtype="f32", ratio=0.3)
    print("[noalloc] first call, 4x2 layers/samples", flush=True)
    run_both(big, 5)
    print("[noalloc] second call, smaller input", flush=True)
    run_both(small, 6)
    print("[noalloc] the first shape again", flush=True)
    run_both(big, 7)


def test_noalloc_rejects_oversized_descriptor():
    from lvlm_kv_cache_amd import _lib
    w = wl.CONFIGS[5]
    ac_desc = __import__("lvlm_kv_cache_amd").make_desc(w.L, w.B, w.Hq, w.Hkv, w.D, w.Nv, w.Nt, w.dtype, path="tiled")
    assert _lib.workspace_size(ac_desc) > _lib.NOALLOC_SCRATCH_BYTES
    L = w.L
    null = [0] * L
    rc = _lib.run_noalloc(ac_desc, null, null, null, _lib.PlanBuf(), null, null, 0)
    assert rc == _lib.AIRCACHE_EINVAL
