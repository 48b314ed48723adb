"""Per-KV-head selection (the group-wise top-K of the edge-device survey
page, section 10.1 on GQA/MQA) and int8 per-head quantisation of the kept
cache (the UniCache blog, section 6.3), on the GPU, against the oracle.

Per-KV-head selection follows the rules of tests/parity.py (I_v^g within
1e-3 relative of the oracle's float64 value, kept sets exact for the GPU's
own scores, compacted rows bit-exact). The int8 codes and scales are bit-exact
against the oracle run on the GPU's own compacted segments: both sides decide
each code in float32 with correctly rounded divisions.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import compare, make_aircache, reference, run_gpu, to_torch

pytestmark = pytest.mark.gpu

SHAPES = [
    dict(Nv=120, Nt=20, Hq=8, Hkv=2, D=64, dtype="bf16", L=2, B=2),      # small path
    dict(Nv=700, Nt=40, Hq=12, Hkv=4, D=128, dtype="bf16", L=3, B=2),
    dict(Nv=257, Nt=33, Hq=4, Hkv=4, D=128, dtype="f32", L=2),
    dict(Nv=300, Nt=40, Hq=7, Hkv=1, D=128, dtype="bf16", B=2, L=2),      # one KV head: the shared choice
    dict(Nv=1000, Nt=24, Hq=14, Hkv=2, D=64, dtype="bf16", L=2, B=1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("path", ["auto", "auto-run", "tiled-run"])
def test_per_kv_head_selection(shape, path):
    w = wl.custom(ratio=0.25, **shape)
    print(f"[f4] per-KV-head {shape} path {path}", flush=True)
    inp = wl.make_inputs(w, 31)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"), select="per_kv_head")
    compare(inp, g, reference(inp, g, per_head=True))
    if w.Hkv == 1:
        # one KV head: its score is the shared score, bit for bit, so the
        # selection is the shared one
        assert np.array_equal(g["iv_head"][:, :, 0], g["iv"])


def test_per_kv_head_selection_workload_3():
    """Workload 3 at full size (the tiled path), elite cap 64."""
    print("[f4] per-KV-head workload 3", flush=True)
    inp = wl.make_inputs(3, 3)
    g = run_gpu(inp, max_elite=64, run=True, select="per_kv_head")
    rep = compare(inp, g, reference(inp, g, per_head=True))
    # the KV heads choose differently: the method's shared set is not every head's
    kb = g["budget"]
    same = all(np.array_equal(g["kept_idx"][l, 0, 0, :kb[l, 0]], g["kept_idx"][l, 0, h, :kb[l, 0]])
               for l in range(inp.w.L) for h in range(1, inp.w.Hkv))
    assert not same
    print(f"[f4] {rep}", flush=True)


def _quant_case(w, seed, select="shared", zero_v_layer=None):
    inp = wl.make_inputs(w, seed)
    ac = make_aircache(w, select=select)
    q, k, v = to_torch(inp)
    if zero_v_layer is not None:
        v[zero_v_layer].zero_()
    plan = ac.alloc_plan()
    ko, vo = ac.alloc_compacted()
    ac.run(q, k, v, plan, ko, vo)
    kq, vq, ks, vs = ac.quantize_i8(plan, ko, vo)
    torch.cuda.synchronize()
    assert int(plan.status.item()) == 0
    budget = plan.budget.cpu().numpy()
    out_off = plan.out_off.cpu().numpy()
    ks, vs = ks.cpu().numpy(), vs.cpu().numpy()
    store = np.float32 if w.dtype == wl.F32 else np.uint16
    for l in range(w.L):
        n_l = int(out_off[l, w.B])
        for name, src, codes, sc in (("K", ko, kq, ks), ("V", vo, vq, vs)):
            a = src[l][:n_l].cpu()
            if w.dtype == wl.BF16:
                a = a.view(torch.int16)
            vals = a.numpy().view(store)
            cod = codes[l][:n_l].cpu().numpy()
            for b in range(w.B):
                n = int(budget[l, b]) + w.Nt
                for g in range(w.Hkv):
                    o = int(out_off[l, b]) + g * n * w.D
                    c_ref, s_ref = oracle.quantize_i8(vals[o:o + n * w.D], w.dtype)
                    assert np.float32(sc[l, b, g]) == np.float32(s_ref), f"{name} scale ({l},{b},{g})"
                    assert np.array_equal(cod[o:o + n * w.D], c_ref), f"{name} codes ({l},{b},{g}) differ"
    return ks, vs


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_quantize_i8_workloads(cid):
    w = wl.CONFIGS[cid]
    print(f"[f4] quantise workload {cid}", flush=True)
    _quant_case(w, wl.parity_seeds(cid)[0])


@pytest.mark.parametrize("shape", SHAPES[:3], ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("ratio", [0.0, 0.3])
def test_quantize_i8_edge(shape, ratio):
    """Text rows only (budget 0), per-KV-head kept rows, and an all-zero V
    layer (scale 0, every code 0)."""
    w = wl.custom(ratio=ratio, **shape)
    print(f"[f4] quantise {shape} ratio {ratio}", flush=True)
    ks, vs = _quant_case(w, 32, select="per_kv_head", zero_v_layer=0)
    assert (vs[0] == 0).all() and (ks > 0).all()


def test_bound_quantize_matches_plain_call():
    w = wl.custom(Nv=300, Nt=40, Hq=8, Hkv=2, D=128, dtype="bf16", L=2, B=2, ratio=0.2)
    inp = wl.make_inputs(w, 5)
    ac = make_aircache(w)
    q, k, v = to_torch(inp)
    plan = ac.alloc_plan()
    ko, vo = ac.alloc_compacted()
    ac.run(q, k, v, plan, ko, vo)
    a = ac.quantize_i8(plan, ko, vo)
    kq = [torch.full_like(t, 99) for t in a[0]]
    vq = [torch.full_like(t, 99) for t in a[1]]
    ks, vs = torch.full_like(a[2], -1.0), torch.full_like(a[3], -1.0)
    bq = ac.bind_quantize(plan, ko, vo, kq, vq, ks, vs)
    bq()
    bq()  # twice: nothing carries over between calls
    torch.cuda.synchronize()
    n = plan.out_off[:, -1].cpu().tolist()
    for l in range(w.L):
        assert torch.equal(a[0][l][:n[l]], kq[l][:n[l]]) and torch.equal(a[1][l][:n[l]], vq[l][:n[l]])
    assert torch.equal(a[2], ks) and torch.equal(a[3], vs)
