"""Decode attention over the compacted cache (aircache_decode) against the
oracle's decode_attention, on the GPU's own compacted output.

The comparison is conditional on the GPU's plan (budgets, offsets) and
compacted rows, which the pass's own parity tests check bit for bit; here the
GPU's float32 decode is held to the oracle's float64 one per element:
|gpu - ref| <= 2e-4 |ref| + 2e-4 max|ref row|. float32 sums over up to
N_v + N_t rows of weights in [0, 1] against float64 keep a relative error of
a few 1e-6 on these inputs; the bound leaves room for the worst-case growth
of a long sum (n 2^-24 with n up to ~7000 rows).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import make_aircache, to_torch

pytestmark = pytest.mark.gpu

RTOL = 2e-4


def _decode_case(w, seed, max_elite=0, layers=None, int8=False):
    """int8: decode over the int8 cache of quantize_i8 (aircache_decode_i8),
    against the oracle's int8 decode fed the GPU's codes and scales (the
    quantisation itself is checked bit for bit in tests/test_f4_gpu.py)."""
    inp = wl.make_inputs(w, seed)
    ac = make_aircache(w, max_elite=max_elite)
    q, k, v = to_torch(inp)
    plan = ac.alloc_plan()
    ko, vo = ac.alloc_compacted()
    ac.run(q, k, v, plan, ko, vo)
    rng = np.random.default_rng(1000 + seed)
    qd32 = [(rng.standard_normal((w.B, w.Hq, w.D)) / np.sqrt(w.D) * 4.0).astype(np.float32) for _ in range(w.L)]
    if w.dtype == wl.BF16:
        qd_host = [wl.f32_to_bf16_bits(a) for a in qd32]
        qd = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in qd_host]
    else:
        qd_host = qd32
        qd = [torch.from_numpy(a).cuda() for a in qd32]
    print(f"[decode] {w.name} seed {seed} L={w.L} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} Nv={w.Nv} Nt={w.Nt}",
          flush=True)
    if int8:
        kq, vq, ks, vs = ac.quantize_i8(plan, ko, vo)
        o = ac.decode_i8(qd, plan, kq, vq, ks, vs)
        ks_h, vs_h = ks.cpu().numpy(), vs.cpu().numpy()
    else:
        o = ac.decode(qd, plan, ko, vo)
    torch.cuda.synchronize()
    assert int(plan.status.item()) == 0
    budget = plan.budget.cpu().numpy()
    out_off = plan.out_off.cpu().numpy()
    store = np.float32 if w.dtype == wl.F32 else np.uint16

    def host(t, n):
        a = t[:n].cpu()
        if w.dtype == wl.BF16:
            a = a.view(torch.int16)
        return a.numpy().view(store)

    layers = range(w.L) if layers is None else layers

    def check(l):
        n = int(out_off[l, w.B])
        if int8:
            kc, vc = kq[l][:n].cpu().numpy(), vq[l][:n].cpu().numpy()
            ref = np.zeros((w.B, w.Hq, w.D))
            for b in range(w.B):
                rows = int(budget[l, b]) + w.Nt
                off, size = int(out_off[l, b]), w.Hkv * rows * w.D
                ref[b] = oracle.decode_attention_i8_segment(w, kc[off:off + size], vc[off:off + size], ks_h[l, b],
                                                            vs_h[l, b], rows, qd_host[l][b])
        else:
            ref = oracle.decode_attention(w, host(ko[l], n), host(vo[l], n), out_off[l], budget[l], qd_host[l])
        got = o[l].cpu().numpy().astype(np.float64)
        scale = np.abs(ref).max(axis=-1, keepdims=True)
        err = np.abs(got - ref)
        bad = err > RTOL * np.abs(ref) + RTOL * scale
        assert not bad.any(), (f"layer {l}: {int(bad.sum())} elements off, max err "
                               f"{float((err / np.maximum(scale, 1e-30)).max()):.3g} of the row scale")
        return float((err / np.maximum(scale, 1e-30)).max())

    with ThreadPoolExecutor(8) as ex:
        worst = max(ex.map(check, layers))
    print(f"[decode] worst error {worst:.3g} of the row scale", flush=True)


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_decode_workload(cid):
    _decode_case(wl.CONFIGS[cid], wl.parity_seeds(cid)[0])


@pytest.mark.parametrize("cid", [4, 5])
def test_decode_workload_large(cid):
    """The default elite cap (N_t), full size; every layer checked."""
    _decode_case(wl.CONFIGS[cid], wl.parity_seeds(cid)[0])


EDGE = [
    dict(Nv=17, Nt=3, Hq=1, Hkv=1, D=64, dtype="f32"),
    dict(Nv=300, Nt=40, Hq=7, Hkv=1, D=128, dtype="bf16", B=3, L=3),
    dict(Nv=257, Nt=33, Hq=4, Hkv=4, D=128, dtype="f32", L=2),
    dict(Nv=129, Nt=17, Hq=32, Hkv=1, D=128, dtype="bf16", L=2),   # G = 32
    dict(Nv=700, Nt=80, Hq=14, Hkv=7, D=64, dtype="bf16", L=2, B=2),
    dict(Nv=333, Nt=24, Hq=8, Hkv=2, D=64, dtype="f32", L=3, B=5),
    # the matrix-core weights x V (bfloat16, 4 <= G <= 32): head_dim 64, a
    # second group of 16 heads only partly used
    dict(Nv=500, Nt=60, Hq=16, Hkv=2, D=64, dtype="bf16", L=2, B=2),
    dict(Nv=600, Nt=30, Hq=20, Hkv=1, D=128, dtype="bf16", L=2),
    dict(Nv=520, Nt=20, Hq=24, Hkv=1, D=64, dtype="bf16", L=2),
    # enough (layer, sample, KV head) units that at ratio 1.0 the per-wave
    # kernel takes two splits per unit (with the combine): head_dim 64 and
    # 128, one and two groups of 16 heads
    dict(Nv=500, Nt=20, Hq=32, Hkv=4, D=64, dtype="bf16", L=8, B=8),
    dict(Nv=500, Nt=20, Hq=80, Hkv=4, D=64, dtype="bf16", L=8, B=8),
    dict(Nv=500, Nt=20, Hq=40, Hkv=2, D=128, dtype="bf16", L=8, B=16),
    # bfloat16 with G > 32: the vector-unit weights x V
    dict(Nv=100, Nt=20, Hq=40, Hkv=1, D=64, dtype="bf16", L=2),
]


@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("ratio", [0.0, 0.2, 1.0])
def test_decode_edge_shapes(shape, ratio):
    """Budgets of 0 (text rows only), partial and every visual row."""
    _decode_case(wl.custom(ratio=ratio, **shape), 4)


@pytest.mark.parametrize("cid", [1, 3, 5])
def test_decode_int8_workload(cid):
    """Decode over the int8 cache, full size, every layer."""
    _decode_case(wl.CONFIGS[cid], wl.parity_seeds(cid)[0], int8=True)


@pytest.mark.parametrize("shape", EDGE[:4], ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("ratio", [0.0, 0.3])
def test_decode_int8_edge_shapes(shape, ratio):
    _decode_case(wl.custom(ratio=ratio, **shape), 5, int8=True)


def test_decode_out_of_range_plan_gives_nan_not_a_fault():
    """A plan whose budget or offset lies outside the buffers (not one this
    library wrote) makes the kernels' own range checks give NaN rows."""
    w = wl.custom(Nv=64, Nt=16, Hq=4, Hkv=2, D=64, dtype="bf16", L=2, B=2, ratio=0.25)
    inp = wl.make_inputs(w, 3)
    ac = make_aircache(w)
    q, k, v = to_torch(inp)
    plan = ac.alloc_plan()
    ko, vo = ac.alloc_compacted()
    ac.run(q, k, v, plan, ko, vo)
    torch.cuda.synchronize()
    plan.budget[0, 1] = w.Nv + 5          # budget out of range
    plan.out_off[1, 0] = 1 << 40           # offset past the buffer
    plan.out_off[1, 1] = (1 << 63) - 64    # near the top of int64: offset + size would wrap
    qd = [torch.randn(w.B, w.Hq, w.D, device="cuda").to(torch.bfloat16) for _ in range(w.L)]
    o = ac.decode(qd, plan, ko, vo)
    torch.cuda.synchronize()
    assert torch.isnan(o[0][1]).all() and torch.isnan(o[1][0]).all() and torch.isnan(o[1][1]).all()
    assert torch.isfinite(o[0][0]).all()
    # the int8 cache, its quantisation and the compaction skip the same segments
    kq, vq, ks, vs = ac.quantize_i8(plan, ko, vo)
    o8 = ac.decode_i8(qd, plan, kq, vq, ks, vs)
    ac.compress(plan, k, v, ko, vo)
    torch.cuda.synchronize()
    assert torch.isnan(o8[1][1]).all() and torch.isfinite(o8[0][0]).all()


def test_bound_decode_matches_plain_call():
    w = wl.custom(Nv=300, Nt=40, Hq=8, Hkv=2, D=128, dtype="bf16", L=2, B=2, ratio=0.2)
    inp = wl.make_inputs(w, 5)
    ac = make_aircache(w)
    q, k, v = to_torch(inp)
    plan = ac.alloc_plan()
    ko, vo = ac.alloc_compacted()
    ac.run(q, k, v, plan, ko, vo)
    qd = [torch.randn(w.B, w.Hq, w.D, device="cuda").to(torch.bfloat16) for _ in range(w.L)]
    a = ac.decode(qd, plan, ko, vo)
    o = [torch.full((w.B, w.Hq, w.D), float("nan"), device="cuda") for _ in range(w.L)]
    bd = ac.bind_decode(qd, plan, ko, vo, o)
    b = bd()
    b = bd()  # twice: the workspace needs no zeroing between calls
    torch.cuda.synchronize()
    for l in range(w.L):
        assert torch.equal(a[l], b[l])
    # the int8 cache: the bound call equals the plain aircache_decode_i8 call
    kq, vq, ks, vs = ac.quantize_i8(plan, ko, vo)
    a8 = ac.decode_i8(qd, plan, kq, vq, ks, vs)
    o8 = [torch.full((w.B, w.Hq, w.D), float("nan"), device="cuda") for _ in range(w.L)]
    bd8 = ac.bind_decode(qd, plan, kq, vq, o8, scales=(ks, vs))
    bd8()
    b8 = bd8()
    torch.cuda.synchronize()
    for l in range(w.L):
        assert torch.equal(a8[l], b8[l])
