"""GPU-vs-oracle comparison helpers for the parity tests.

Comparison rules (per layer l and sample b):
  elite set   equal, except tokens whose head-mean score lies within 1e-5
              (relative to the row maximum) of the alpha threshold; when the
              sets differ only in such tokens, steps 2-6 of the oracle are fed
              the GPU's set (conditional check);
  I_v, s_t    |gpu - ref| <= 1e-3 |ref| (float32 accumulation vs double);
  s_k         |gpu - ref| <= 1e-3 max(|ref|, 1);
  budgets     oracle step 4 fed the GPU's s_t / s_k reproduces the GPU's
              pre-floor value and budget exactly; against the oracle's own
              statistics the budget may differ only where an integer lies
              between the two pre-floor values;
  kept sets   oracle step 5 fed the GPU's I_v and budget reproduces the GPU's
              indices exactly; against the oracle's own I_v the sets may differ
              only in tokens within 1e-5 (relative) of the cut-off score;
  compacted   bit-exact against oracle step 6 fed the GPU's kept indices.
With one selection per KV head, I_v^g follows the I_v rule and the kept sets
and compacted rows the same rules per KV head.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import workloads as wl
from lvlm_kv_cache_amd import AirCache

THREADS = 8


def to_torch(inp: wl.Inputs, device="cuda"):
    """Per-layer device tensors with the generator's exact bytes."""
    def conv(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if inp.w.dtype == wl.BF16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)
    L = inp.w.L
    return ([conv(inp.q[l]) for l in range(L)], [conv(inp.k[l]) for l in range(L)],
            [conv(inp.v[l]) for l in range(L)])


def torch_dtype(w):
    return torch.float32 if w.dtype == wl.F32 else torch.bfloat16


def make_aircache(w, alpha=None, ratio=None, max_elite=0, path="auto", budget_mode=0, obs_window=0,
                  select="shared"):
    return AirCache(w.L, w.B, w.Hq, w.Hkv, w.D, w.Nv, w.Nt, dtype=torch_dtype(w),
                    alpha=w.alpha if alpha is None else alpha,
                    ratio=w.ratio if ratio is None else ratio, max_elite=max_elite, path=path,
                    budget_mode=budget_mode, obs_window=obs_window, select=select)


def run_gpu(inp: wl.Inputs, alpha=None, ratio=None, max_elite=0, tensors=None, compress=True, path="auto", ac=None,
            run=False, budget_mode=0, obs_window=0, select="shared"):
    """Plan (and compress) on the GPU; ac: an AirCache to reuse (its workspace
    carries state from earlier calls); run: one aircache_run call instead of
    aircache_plan then aircache_compress."""
    w = inp.w
    if ac is None:
        ac = make_aircache(w, alpha, ratio, max_elite, path, budget_mode, obs_window, select)
    q, k, v = tensors if tensors is not None else to_torch(inp)
    out = {}
    if run:
        plan = ac.alloc_plan()
        ko, vo = ac.alloc_compacted()
        ac.run(q, k, v, plan, ko, vo)
        compress = True
    else:
        plan = ac.plan(q, k)
    if compress and not run:
        ko, vo = ac.alloc_compacted()
        ac.compress(plan, k, v, ko, vo)
    torch.cuda.synchronize()
    for f in ("elite_idx", "n_elite", "iv", "s_t", "s_k", "budget_x", "budget", "out_off", "kept_idx", "status"):
        out[f] = getattr(plan, f).cpu().numpy()
    if plan.iv_head is not None:
        out["iv_head"] = plan.iv_head.cpu().numpy()
    if compress:
        store = np.float32 if w.dtype == wl.F32 else np.uint16
        def host(t, n):
            a = t[:n].cpu()
            if w.dtype == wl.BF16:
                a = a.view(torch.int16)
            return a.numpy().view(store)
        out["k_out"] = [host(ko[l], int(out["out_off"][l, w.B])) for l in range(w.L)]
        out["v_out"] = [host(vo[l], int(out["out_off"][l, w.B])) for l in range(w.L)]
    return out


def reference(inp: wl.Inputs, gpu: dict, alpha=None, ratio=None, budget_mode=0, obs_window=0, per_head=False,
              q_all=None):
    """Oracle values for every (l, b), conditional on the GPU's elite sets where
    they differ only in threshold-ambiguous tokens. obs_window = -k: the
    visual window over every position's queries q_all[l] [B][H_q][S][D]."""
    w = inp.w
    alpha = w.alpha if alpha is None else alpha
    ratio = w.ratio if ratio is None else ratio
    L, B = w.L, w.B
    ref = dict(iv=np.zeros((L, B, w.Nv)), s_t=np.zeros((L, B)), s_k=np.zeros((L, B)),
               elite_diff=np.zeros((L, B), bool), n_elite=np.zeros((L, B), int))
    if per_head:
        ref["iv_head"] = np.zeros((L, B, w.Hkv, w.Nv))

    def one(lb):
        l, b = lb
        gel = gpu["elite_idx"][l, b, :gpu["n_elite"][l, b]]
        if obs_window < 0:
            # the visual window: its positions, and I_v over the visual keys only
            kw = -obs_window
            assert np.array_equal(gel, np.arange(w.Nv - kw, w.Nv)), f"(l={l}, b={b}) visual window differs"
            ref["n_elite"][l, b] = kw
            if per_head:
                iv, ref["iv_head"][l, b] = oracle.visual_window(w, q_all[l], inp.k[l], b, kw, groups=True)
            else:
                iv = oracle.visual_window(w, q_all[l], inp.k[l], b, kw)
            ref["iv"][l, b] = iv
            ref["s_t"][l, b], ref["s_k"][l, b] = oracle.layer_stats(iv)
            return
        if obs_window > 0:
            # a contiguous window: one exact answer
            el = oracle.window_select(w.Nt, obs_window)
            assert np.array_equal(el, gel), f"(l={l}, b={b}) window differs"
        else:
            el, pbar = oracle.elite_select(w, inp.q[l], inp.k[l], b, alpha=alpha)
        use = el
        if not np.array_equal(el, gel):
            diff = set(el.tolist()) ^ set(gel.tolist())
            pmax = pbar.max()
            for j in diff:
                assert abs(pbar[j] - alpha * pmax) <= 1e-5 * pmax, (
                    f"(l={l}, b={b}) elite token {j} differs but is not threshold-ambiguous: "
                    f"pbar={pbar[j]!r}, threshold={alpha * pmax!r}")
            use = gel
            ref["elite_diff"][l, b] = True
        ref["n_elite"][l, b] = len(el)
        iv = oracle.cross_score(w, inp.q[l], inp.k[l], b, use)
        ref["iv"][l, b] = iv
        if per_head:
            ref["iv_head"][l, b] = oracle.cross_score_groups(w, inp.q[l], inp.k[l], b, use)
        ref["s_t"][l, b], ref["s_k"][l, b] = oracle.layer_stats(iv)

    pairs = [(l, b) for l in range(L) for b in range(B)]
    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(one, pairs))
    ref["x"] = np.zeros((L, B))
    ref["budget"] = np.zeros((L, B), np.int32)
    for b in range(B):
        ref["x"][:, b], ref["budget"][:, b] = oracle.budget(ref["s_t"][:, b], ref["s_k"][:, b], ratio, w.Nv,
                                                            budget_mode)
    ref["budget_mode"] = budget_mode
    return ref


def compare(inp: wl.Inputs, gpu: dict, ref: dict, ratio=None, check_compacted=True) -> dict:
    """Assert every rule of the module docstring; return a small report."""
    w = inp.w
    ratio = w.ratio if ratio is None else ratio
    L, B = w.L, w.B
    rep = dict(elite_ambiguous=int(ref["elite_diff"].sum()), budget_ambiguous=0, kept_ambiguous=0)
    assert gpu["status"][0] == 0, f"device status {gpu['status'][0]}"
    # I_v, s_t, s_k against the oracle
    iv_g, iv_r = gpu["iv"].astype(np.float64), ref["iv"]
    err = np.abs(iv_g - iv_r)
    bad = err > 1e-3 * np.abs(iv_r)
    assert not bad.any(), f"I_v mismatch at {np.argwhere(bad)[:5].tolist()}, max rel {np.max(err / np.maximum(np.abs(iv_r), 1e-300)):.3g}"
    rep["iv_max_rel"] = float(np.max(err / np.maximum(np.abs(iv_r), 1e-300)))
    assert np.all(np.abs(gpu["s_t"] - ref["s_t"]) <= 1e-3 * np.abs(ref["s_t"])), "s_t mismatch"
    assert np.all(np.abs(gpu["s_k"] - ref["s_k"]) <= 1e-3 * np.maximum(np.abs(ref["s_k"]), 1.0)), (
        f"s_k mismatch: gpu {gpu['s_k'].ravel()[:6]} ref {ref['s_k'].ravel()[:6]}")
    # statistics of the GPU's own I_v (double on both sides, different order)
    for l in range(L):
        for b in range(B):
            st, sk = oracle.layer_stats(iv_g[l, b])
            assert abs(st - gpu["s_t"][l, b]) <= 1e-9 * abs(st)
            assert abs(sk - gpu["s_k"][l, b]) <= 1e-7 * max(1.0, abs(sk))
    # budgets: conditional (exact) and end to end
    for b in range(B):
        x, r = oracle.budget(gpu["s_t"][:, b], gpu["s_k"][:, b], ratio, w.Nv, ref.get("budget_mode", 0))
        assert np.array_equal(x, gpu["budget_x"][:, b]), f"budget_x differs for sample {b}"
        assert np.array_equal(r, gpu["budget"][:, b]), f"budget differs for sample {b}: {r} vs {gpu['budget'][:, b]}"
    for l in range(L):
        for b in range(B):
            if gpu["budget"][l, b] != ref["budget"][l, b]:
                xo, xg = ref["x"][l, b], gpu["budget_x"][l, b]
                lo, hi = min(xo, xg), max(xo, xg)
                assert math.floor(hi) > math.floor(lo) and hi - lo <= 1e-3 * max(1.0, abs(xo)), (
                    f"budget ({l},{b}) {gpu['budget'][l, b]} vs {ref['budget'][l, b]} (x {xg} vs {xo})")
                rep["budget_ambiguous"] += 1
    # kept sets: conditional (exact) and end to end; per KV head against I_v^g
    per_head = gpu["kept_idx"].ndim == 4
    if per_head:
        hg, hr = gpu["iv_head"].astype(np.float64), ref["iv_head"]
        err = np.abs(hg - hr)
        bad = err > 1e-3 * np.abs(hr)
        assert not bad.any(), f"I_v per KV head mismatch at {np.argwhere(bad)[:5].tolist()}"
        rep["iv_head_max_rel"] = float(np.max(err / np.maximum(np.abs(hr), 1e-300)))
    sels = [(l, b, g) for l in range(L) for b in range(B) for g in range(w.Hkv if per_head else 1)]
    for l, b, g in sels:
        kb = int(gpu["budget"][l, b])
        kg = gpu["kept_idx"][l, b, g, :kb] if per_head else gpu["kept_idx"][l, b, :kb]
        own = hg[l, b, g] if per_head else iv_g[l, b]
        rsc = hr[l, b, g] if per_head else iv_r[l, b]
        kc = oracle.topk(own, kb)
        assert np.array_equal(kg, kc), f"kept set ({l},{b},{g}) differs from top-k of the GPU's own scores"
        if kb == ref["budget"][l, b] and kb > 0:
            ko = oracle.topk(rsc, kb)
            if not np.array_equal(ko, kg):
                cut = np.sort(rsc)[::-1][kb - 1]
                for j in set(ko.tolist()) ^ set(kg.tolist()):
                    assert abs(rsc[j] - cut) <= 1e-5 * cut, f"kept ({l},{b},{g}) token {j} not near the cut-off"
                rep["kept_ambiguous"] += 1
    # compacted cache: offsets and bytes
    if check_compacted:
        for l in range(L):
            off = 0
            for b in range(B):
                assert gpu["out_off"][l, b] == off
                kb = int(gpu["budget"][l, b])
                n = w.Hkv * (kb + w.Nt) * w.D
                for name, src in (("k_out", inp.k), ("v_out", inp.v)):
                    seg = gpu[name][l][off:off + n]
                    if per_head:
                        exp = oracle.gather_groups(w, src[l], b, gpu["kept_idx"][l, b, :, :kb]).ravel()
                    else:
                        exp = oracle.gather(w, src[l], b, gpu["kept_idx"][l, b, :kb]).ravel()
                    assert np.array_equal(seg.view(np.uint8), exp.view(np.uint8)), f"{name} ({l},{b}) not bit-exact"
                off += n
            assert gpu["out_off"][l, B] == off
    return rep


# ---- prefill attention with the scores fused in ------------------------------

def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _o_bound(w, vh, ref):
    """Allowed |gpu - ref| per element of the prefill attention's output ref
    [Hq][rows][D] (vh: the KV head's values [Hkv][S][D] as float64):
        2^-8 (max_i |v_id| + |ref_d|) + 1e-5 max_i |v_id|.
    Logits and sums are float32; the probabilities p_i are rounded to
    bfloat16 (8-bit significand: relative error <= 2^-8 each) before the
    product with V, so the numerator is off by at most 2^-8 sum_i p_i |v_id|
    <= 2^-8 max_i |v_id| of the normalised row; the output is rounded to
    bfloat16 (<= 2^-8 |o_d|); float32 accumulation over at most a few
    thousand terms stays within 1e-5 of the value scale."""
    G = w.Hq // w.Hkv
    vmax = np.abs(vh).max(axis=1)  # [Hkv][D]
    vm = np.repeat(vmax, G, axis=0)[:, None, :]
    return 2.0 ** -8 * (vm + np.abs(ref)) + 1e-5 * vm


def check_prefill_o(w, inp, qa, o, l, rows_by_b):
    """o of layer l against the oracle at the given rows of every query head."""
    worst = 0.0
    for b, rows in rows_by_b.items():
        vh = wl.bf16_bits_to_f32(inp.v[l][b]).astype(np.float64)
        for r0, n in rows:
            ref = oracle.prefill_attention(w, qa, inp.k[l], inp.v[l], b, r0, n)
            got = wl.bf16_bits_to_f32(o[b, :, r0:r0 + n, :]).astype(np.float64)
            bound = _o_bound(w, vh, ref)
            err = np.abs(got - ref)
            bad = np.argwhere(err > bound)
            assert bad.size == 0, (f"layer {l} sample {b} rows {r0}+{n}: {len(bad)} elements off, first "
                                   f"{tuple(bad[0])} gpu {got[tuple(bad[0])]} ref {ref[tuple(bad[0])]}")
            worst = max(worst, float((err / bound).max()))
    return worst


def run_gpu_prefill(w, inp, ac, with_plan=True, keep_layers=None):
    """Every layer through aircache_prefill_layer (or the plain attention),
    then aircache_compress; returns (queries per layer, o per layer on the
    host, gpu dict). keep_layers: only those layers' queries and outputs come
    back to the host (the others are None), for sizes whose every-position
    queries do not fit the host comfortably."""
    L = w.L
    keep = set(range(L)) if keep_layers is None else set(keep_layers)
    qa, q = [], []
    for l in range(L):
        a = wl.prefill_queries(inp, l)
        q.append(_dev(a))
        qa.append(a if l in keep else None)
        del a
    _, k, v = to_torch(inp)
    o = [torch.empty_like(t) for t in q]
    out = {}
    if with_plan:
        plan = ac.alloc_plan()
        for l in range(L):
            ac.prefill_layer(l, q[l], k[l], v[l], o[l], plan)
        ko, vo = ac.alloc_compacted()
        ac.compress(plan, k, v, ko, vo)
        torch.cuda.synchronize()
        for f in ("elite_idx", "n_elite", "iv", "s_t", "s_k", "budget_x", "budget", "out_off", "kept_idx",
                  "status"):
            out[f] = getattr(plan, f).cpu().numpy()
        if plan.iv_head is not None:
            out["iv_head"] = plan.iv_head.cpu().numpy()
        out["k_out"] = [_host(ko[l][:int(out["out_off"][l, w.B])]) for l in range(L)]
        out["v_out"] = [_host(vo[l][:int(out["out_off"][l, w.B])]) for l in range(L)]
    else:
        for l in range(L):
            ac.prefill_attention(q[l], k[l], v[l], o[l])
        torch.cuda.synchronize()
    return qa, [_host(t) if l in keep else None for l, t in enumerate(o)], out
