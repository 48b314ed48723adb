"""The window ablation's visual window (obs_window = -k: the last k visual
tokens as the observation rows, normalised over the visual keys only) on the
GPU against the oracle's visual_window and the rest of the pass, with the
comparison rules of tests/parity.py. The query tables hold every position's
queries (the visual rows drawn by workloads.visual_queries)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as wl
from parity import compare, reference, run_gpu, to_torch

pytestmark = pytest.mark.gpu


def _case(w, seed, kwin, select="shared", run=False, ratio=None):
    inp = wl.make_inputs(w, seed)
    qa = [wl.prefill_queries(inp, l) for l in range(w.L)]
    _, k, v = to_torch(inp)
    if w.dtype == wl.BF16:
        q = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in qa]
    else:
        q = [torch.from_numpy(a).cuda() for a in qa]
    g = run_gpu(inp, tensors=(q, k, v), obs_window=-kwin, select=select, run=run, ratio=ratio)
    assert g["status"][0] == 0
    ref = reference(inp, g, ratio=ratio, obs_window=-kwin, per_head=select == "per_kv_head", q_all=qa)
    compare(inp, g, ref, ratio=ratio)
    # every row normalises over the visual keys: I_v sums to one
    np.testing.assert_allclose(g["iv"].sum(axis=-1), 1.0, rtol=1e-4)
    return g


SHAPES = [
    ("ragged_gqa_bf16", dict(L=2, B=2, Hq=6, Hkv=2, D=128, Nv=333, Nt=40, dtype="bf16", ratio=0.2), 32),
    ("mha_f32", dict(L=3, B=1, Hq=4, Hkv=4, D=64, Nv=130, Nt=20, dtype="f32", ratio=0.3), 16),
    ("window_of_one", dict(L=2, B=1, Hq=2, Hkv=1, D=64, Nv=50, Nt=8, dtype="f32", ratio=0.25), 1),
    ("window_is_all_text_long", dict(L=2, B=1, Hq=7, Hkv=1, D=128, Nv=100, Nt=100, dtype="bf16", ratio=0.2), 100),
]


@pytest.mark.parametrize("name,shape,kwin", SHAPES, ids=[s[0] for s in SHAPES])
def test_visual_window_small(name, shape, kwin):
    _case(wl.custom(**shape), 3, kwin)


def test_visual_window_one_call_and_per_kv_head():
    w = wl.custom(L=2, B=2, Hq=6, Hkv=2, D=128, Nv=300, Nt=48, dtype="bf16", ratio=0.2)
    _case(w, 4, 32, run=True)
    _case(w, 5, 32, select="per_kv_head")


@pytest.mark.parametrize("cid", [3, 2])
def test_visual_window_full_size(cid):
    """Workloads 3 and 2 at full size with the ablation's window of 32."""
    _case(wl.CONFIGS[cid], cid, 32)
