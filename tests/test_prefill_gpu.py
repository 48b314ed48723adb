"""Prefill attention with the pass's scores fused in (aircache_prefill_layer,
aircache_prefill_attention) against the oracle.

Attention output: the bound of parity.check_prefill_o, derived from the
kernel's arithmetic (bfloat16 probabilities and output, float32 sums).

Plan outputs (elite sets, I_v, statistics, budgets, kept sets) and the
compacted cache follow the rules of tests/parity.py, against the oracle's pass
on the same text queries (the text rows of the prefill queries).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity import check_prefill_o as _check_o, compare, make_aircache, reference, run_gpu_prefill as _run_prefill

pytestmark = pytest.mark.gpu


SMALL = [
    # (name, shape): ragged key and query tiles, several text tiles, GQA groups, head_dim 64
    ("ragged_gqa", dict(L=2, B=2, Hq=4, Hkv=2, D=128, Nv=100, Nt=40)),
    ("two_text_tiles_g7", dict(L=2, B=1, Hq=7, Hkv=1, D=128, Nv=200, Nt=150, alpha=0.5)),
    ("aligned_mha", dict(L=3, B=1, Hq=4, Hkv=4, D=128, Nv=128, Nt=128)),
    ("d64", dict(L=2, B=2, Hq=8, Hkv=2, D=64, Nv=333, Nt=77)),
    ("short_text", dict(L=2, B=1, Hq=2, Hkv=1, D=128, Nv=70, Nt=1)),
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[n for n, _ in SMALL])
@pytest.mark.parametrize("seed", [1, 2])
def test_prefill_small_shapes(name, shape, seed):
    w = wl.custom(dtype="bf16", ratio=0.3, **shape)
    inp = wl.make_inputs(w, seed)
    ac = make_aircache(w)
    qa, o, gpu = _run_prefill(w, inp, ac)
    S = w.Nv + w.Nt
    for l in range(w.L):
        _check_o(w, inp, qa[l], o[l], l, {b: [(0, S)] for b in range(w.B)})
    ref = reference(inp, gpu)
    compare(inp, gpu, ref)


@pytest.mark.parametrize("variant", [dict(obs_window=16), dict(select="per_kv_head"), dict(budget_mode=4),
                                     dict(max_elite=8, alpha=0.0)])
def test_prefill_variants(variant):
    """The window ablation, one selection per KV head, the pyramid budget and
    an elite cap (alpha 0 makes every text token elite: the cap is exceeded
    and flagged, as on the other paths)."""
    w = wl.custom(L=3, B=2, Hq=6, Hkv=2, D=128, Nv=190, Nt=48, dtype="bf16", ratio=0.25)
    inp = wl.make_inputs(w, 5)
    alpha = variant.get("alpha")
    ac = make_aircache(w, alpha=alpha, max_elite=variant.get("max_elite", 0),
                       budget_mode=variant.get("budget_mode", 0), obs_window=variant.get("obs_window", 0),
                       select=variant.get("select", "shared"))
    qa, o, gpu = _run_prefill(w, inp, ac)
    if "max_elite" in variant:
        assert np.all(gpu["status"] & 1), "elite overflow not flagged"
        return
    assert np.all(gpu["status"] == 0)
    ref = reference(inp, gpu, alpha=alpha, budget_mode=variant.get("budget_mode", 0),
                    obs_window=variant.get("obs_window", 0), per_head="select" in variant)
    compare(inp, gpu, ref)


def test_prefill_plain_attention_matches_the_scored_call():
    """aircache_prefill_attention writes the same o, bit for bit, as the
    scoring call (the same attention arithmetic)."""
    w = wl.custom(L=2, B=2, Hq=4, Hkv=2, D=128, Nv=150, Nt=60, dtype="bf16")
    inp = wl.make_inputs(w, 3)
    ac = make_aircache(w)
    _, o1, _ = _run_prefill(w, inp, ac)
    _, o2, _ = _run_prefill(w, inp, ac, with_plan=False)
    for l in range(w.L):
        assert np.array_equal(o1[l], o2[l])


def test_prefill_rerun_is_bit_identical():
    w = wl.custom(L=2, B=1, Hq=7, Hkv=1, D=128, Nv=260, Nt=90, dtype="bf16", ratio=0.2)
    inp = wl.make_inputs(w, 4)
    ac = make_aircache(w)
    _, o1, g1 = _run_prefill(w, inp, ac)
    _, o2, g2 = _run_prefill(w, inp, ac)
    for l in range(w.L):
        assert np.array_equal(o1[l], o2[l])
    for f in ("iv", "s_t", "s_k", "budget", "out_off"):
        assert np.array_equal(g1[f], g2[f]), f
    for l in range(w.L):
        for b in range(w.B):
            n = int(g1["budget"][l, b])  # entries past the budget are not written
            assert np.array_equal(g1["kept_idx"][l, b, :n], g2["kept_idx"][l, b, :n])
    for l in range(w.L):
        assert np.array_equal(g1["k_out"][l], g2["k_out"][l])


@pytest.mark.parametrize("D", [128, 64])
def test_prefill_large_grid_two_blocks_per_wave(D):
    """A grid of at least one 128-row workgroup per CU takes 128 query rows per
    workgroup (two 16-row blocks per wave; smaller grids, as the other small
    cases here, take 64), at both head dimensions: o on sampled rows and every
    plan output against the oracle."""
    w = wl.custom(L=2, B=4, Hq=32, Hkv=8, D=D, Nv=1000, Nt=70, dtype="bf16", ratio=0.15)
    inp = wl.make_inputs(w, 6)
    ac = make_aircache(w)
    qa, o, gpu = _run_prefill(w, inp, ac)
    rng = np.random.default_rng(6)
    for l in range(w.L):
        _check_o(w, inp, qa[l], o[l], l, {b: _rows_sample(w, rng) for b in range(w.B)})
    compare(inp, gpu, reference(inp, gpu))
    _, o2, _ = _run_prefill(w, inp, ac, with_plan=False)
    for l in range(w.L):
        assert np.array_equal(o[l], o2[l])


def _rows_sample(w, rng):
    """Rows of a full-size check: the first, the last visual, the first text
    and the last position, plus a few random ones, in runs of 2."""
    S = w.Nv + w.Nt
    starts = {0, w.Nv - 2, w.Nv, S - 2} | set(int(x) for x in rng.integers(0, S - 2, size=4))
    return [(s, 2) for s in sorted(starts)]


@pytest.mark.parametrize("cid", [3, 2])
def test_prefill_full_size(cid):
    """Workloads 3 (gqa_tiled_image_2880) and 2 (mha7b_single_image) at full
    size: every plan output and the compacted cache against the oracle, o on
    sampled rows of every query head of three layers."""
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, cid)
    ac = make_aircache(w, max_elite=64)
    qa, o, gpu = _run_prefill(w, inp, ac)
    assert np.all(gpu["status"] == 0)
    rng = np.random.default_rng(cid)
    for l in (0, w.L // 2, w.L - 1):
        _check_o(w, inp, qa[l], o[l], l, {b: _rows_sample(w, rng) for b in range(w.B)})
    ref = reference(inp, gpu)
    compare(inp, gpu, ref)


@pytest.mark.parametrize("cid", [4, 5])
def test_prefill_full_size_large(cid):
    """Workloads 4 (gqa_video_32x196) and 5 (gqa_multi_image_3x1024) at full
    size, elite cap 64: every plan output and the compacted cache against the
    oracle, o on sampled rows of every query head of three layers (only those
    layers' queries and outputs are kept on the host)."""
    w = wl.CONFIGS[cid]
    inp = wl.make_inputs(w, cid)
    ac = make_aircache(w, max_elite=64)
    layers = (0, w.L // 2, w.L - 1)
    qa, o, gpu = _run_prefill(w, inp, ac, keep_layers=layers)
    assert np.all(gpu["status"] == 0)
    rng = np.random.default_rng(cid)
    for l in layers:
        _check_o(w, inp, qa[l], o[l], l, {b: _rows_sample(w, rng) for b in (0, w.B - 1)})
    compare(inp, gpu, reference(inp, gpu))
