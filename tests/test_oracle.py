"""Pins of the CPU oracle against facts fixed by the AirCache page and by
mathematics (no GPU). Each check would fail on a plausible slip in the oracle:
a dropped term, a wrong sign or index, a transposed operand, a wrong
normaliser or a wrong tie rule.

The page prints no worked numeric example of the method, so the pins are
invariants, closed forms, library routines on special cases and brute force on
tiny inputs.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import workloads as wl


def tiny(seed=0, **kw):
    w = wl.custom(**kw)
    return w, wl.make_inputs(w, seed)


# ---------------------------------------------------------------- step 1 ----

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("shape", [dict(Hq=1, Hkv=1, Nt=5), dict(Hq=4, Hkv=2, Nt=9),
                                   dict(Hq=6, Hkv=1, Nt=3, dtype="bf16"),
                                   dict(Hq=7, Hkv=7, Nt=1)])
def test_elite_rows_sum_to_one_and_argmax_is_elite(seed, shape):
    w, inp = tiny(seed, Nv=11, D=16, **shape)
    el, pbar = oracle.elite_select(w, inp.q[0], inp.k[0], 0)
    # every per-head softmax row sums to 1, so does their mean
    assert abs(pbar.sum() - 1.0) < 1e-12
    assert (pbar > 0).all()
    assert int(np.argmax(pbar)) in set(el.tolist())
    assert list(el) == sorted(el) and len(set(el.tolist())) == len(el)
    # the set is exactly the threshold set
    thr = 0.9 * pbar.max()
    assert set(el.tolist()) == set(np.nonzero(pbar >= thr)[0].tolist())


def test_elite_alpha_extremes():
    w, inp = tiny(3, Nv=8, Nt=12, Hq=3, Hkv=3, D=32)
    el0, _ = oracle.elite_select(w, inp.q[0], inp.k[0], 0, alpha=0.0)
    assert list(el0) == list(range(12))           # alpha = 0: every text token
    el1, pbar = oracle.elite_select(w, inp.q[0], inp.k[0], 0, alpha=1.0)
    assert list(el1) == [int(np.argmax(pbar))]     # alpha = 1: the maximum only


def test_elite_uniform_when_queries_are_zero():
    w = wl.custom(Nv=10, Nt=7, Hq=4, Hkv=2, D=16)
    inp = wl.make_inputs(w, 5, zero_q=True)
    el, pbar = oracle.elite_select(w, inp.q[0], inp.k[0], 0)
    assert np.allclose(pbar, 1.0 / 7, rtol=0, atol=1e-15)
    assert list(el) == list(range(7))


def test_elite_matches_library_softmax_single_head():
    # one head: pbar is exactly the softmax row of the last text query
    w, inp = tiny(9, Nv=5, Nt=13, Hq=1, Hkv=1, D=24)
    q = inp.q[0, 0, 0].astype(np.float64)
    k = inp.k[0, 0, 0].astype(np.float64)
    z = k[w.Nv:] @ q[-1] / math.sqrt(w.D)
    ref = scipy.special.softmax(z)
    _, pbar = oracle.elite_select(w, inp.q[0], inp.k[0], 0)
    assert np.allclose(pbar, ref, rtol=1e-13, atol=0)


def test_elite_gqa_head_mapping():
    # 4 query heads on 2 KV heads: heads 0,1 read KV head 0 and heads 2,3 read
    # KV head 1. Checked against per-head library softmax with that mapping.
    w, inp = tiny(4, Nv=6, Nt=10, Hq=4, Hkv=2, D=16)
    rows = []
    for h in range(4):
        q = inp.q[0, 0, h, -1].astype(np.float64)
        k = inp.k[0, 0, h // 2, w.Nv:].astype(np.float64)
        rows.append(scipy.special.softmax(k @ q / 4.0))
    _, pbar = oracle.elite_select(w, inp.q[0], inp.k[0], 0)
    assert np.allclose(pbar, np.mean(rows, axis=0), rtol=1e-13, atol=0)
    # a transposed mapping (h % Hkv) gives a different answer on this input
    rows_bad = [scipy.special.softmax(inp.k[0, 0, h % 2, w.Nv:].astype(np.float64)
                                      @ inp.q[0, 0, h, -1].astype(np.float64) / 4.0)
                for h in range(4)]
    assert not np.allclose(pbar, np.mean(rows_bad, axis=0), rtol=1e-6, atol=0)


def test_elite_uses_last_text_query_only():
    w, inp = tiny(8, Nv=6, Nt=6, Hq=2, Hkv=1, D=16)
    _, p0 = oracle.elite_select(w, inp.q[0], inp.k[0], 0)
    q2 = inp.q.copy()
    q2[0, 0, :, :-1] = 0.0   # change every text query but the last
    _, p1 = oracle.elite_select(w, q2[0], inp.k[0], 0)
    assert np.array_equal(p0, p1)
    k2 = inp.k.copy()
    k2[0, 0, :, :w.Nv] += 1.0   # visual keys do not enter step 1
    _, p2 = oracle.elite_select(w, inp.q[0], k2[0], 0)
    assert np.array_equal(p0, p2)


# ---------------------------------------------------------------- step 2 ----

def library_iv(w, inp, b, elite):
    """I_v from numpy matrix products and scipy's softmax."""
    G = w.Hq // w.Hkv
    acc = np.zeros(w.Nv)
    for h in range(w.Hq):
        K = inp.as_f32("k")[0, b, h // G].astype(np.float64)
        cols = np.concatenate([K[:w.Nv], K[w.Nv + np.asarray(elite, int)]])
        Qe = inp.as_f32("q")[0, b, h][np.asarray(elite, int)].astype(np.float64)
        P = scipy.special.softmax(Qe @ cols.T / math.sqrt(w.D), axis=1)
        acc += P[:, :w.Nv].sum(0)
    return acc / (w.Hq * len(elite))


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", [dict(Hq=1, Hkv=1), dict(Hq=6, Hkv=2), dict(Hq=3, Hkv=3, dtype="bf16")])
def test_cross_score_matches_library_softmax(seed, shape):
    w, inp = tiny(seed, Nv=17, Nt=9, D=32, B=2, **shape)
    for b in range(2):
        el, _ = oracle.elite_select(w, inp.q[0], inp.k[0], b, alpha=0.5)
        iv = oracle.cross_score(w, inp.q[0], inp.k[0], b, el)
        assert np.allclose(iv, library_iv(w, inp, b, el), rtol=1e-12, atol=0)
        # s_t < 1 because the elite text keys also take probability mass
        assert 0.0 < iv.sum() < 1.0


def test_cross_score_single_row_closed_form():
    # D = 1, one head, query 1: logits are the key values themselves.
    # Keys ln(c_i) give probabilities c_i / sum(c) exactly (up to rounding).
    c_vis = np.array([1, 2, 3, 4, 6], np.float64)
    c_txt = np.array([5, 7], np.float64)     # text key 1 is the elite one
    w = wl.custom(Nv=5, Nt=2, Hq=1, Hkv=1, D=1)
    q = np.ones((1, 1, 1, 2, 1), np.float32)
    k = np.log(np.concatenate([c_vis, c_txt])).astype(np.float32).reshape(1, 1, 1, 7, 1)
    # make the softmax exact in float32 inputs by using what the keys round to
    cv = np.exp(k.ravel()[:5].astype(np.float64))
    ct = np.exp(k.ravel()[6].astype(np.float64))
    iv = oracle.cross_score(w, q[0], k[0], 0, [1])
    assert np.allclose(iv, cv / (cv.sum() + ct), rtol=1e-14, atol=0)
    assert np.allclose(iv, c_vis / 23.0, rtol=1e-6, atol=0)


def test_cross_score_uniform_when_queries_are_zero():
    w = wl.custom(Nv=12, Nt=5, Hq=4, Hkv=2, D=16)
    inp = wl.make_inputs(w, 1, zero_q=True)
    el, _ = oracle.elite_select(w, inp.q[0], inp.k[0], 0)
    assert len(el) == 5
    iv = oracle.cross_score(w, inp.q[0], inp.k[0], 0, el)
    assert np.allclose(iv, 1.0 / (12 + 5), rtol=1e-14, atol=0)
    s_t, s_k = oracle.layer_stats(iv)
    assert abs(s_t - 12 / 17) < 1e-14 and s_k == 0.0


def test_cross_score_only_elite_text_columns_in_denominator():
    # adding a huge non-elite text key must not change I_v
    w, inp = tiny(2, Nv=9, Nt=6, Hq=2, Hkv=1, D=8)
    el = np.array([0, 3], np.int32)
    iv0 = oracle.cross_score(w, inp.q[0], inp.k[0], 0, el)
    k2 = inp.k.copy()
    k2[0, 0, 0, w.Nv + 5] *= 50.0
    iv1 = oracle.cross_score(w, inp.q[0], k2[0], 0, el)
    assert np.array_equal(iv0, iv1)
    # and the non-elite queries do not enter either
    q2 = inp.q.copy()
    q2[0, 0, :, [1, 2, 4, 5]] = 7.0
    iv2 = oracle.cross_score(w, q2[0], inp.k[0], 0, el)
    assert np.array_equal(iv0, iv2)


# ---------------------------------------------- step 2, per KV head (f4) ----

def library_iv_groups(w, inp, b, elite):
    """I_v per KV head from numpy matrix products and scipy's softmax: the
    rows of the G query heads that share KV head g, averaged."""
    G = w.Hq // w.Hkv
    out = np.zeros((w.Hkv, w.Nv))
    for g in range(w.Hkv):
        K = inp.as_f32("k")[0, b, g].astype(np.float64)
        cols = np.concatenate([K[:w.Nv], K[w.Nv + np.asarray(elite, int)]])
        for h in range(g * G, (g + 1) * G):
            Qe = inp.as_f32("q")[0, b, h][np.asarray(elite, int)].astype(np.float64)
            P = scipy.special.softmax(Qe @ cols.T / math.sqrt(w.D), axis=1)
            out[g] += P[:, :w.Nv].sum(0)
    return out / (G * len(elite))


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", [dict(Hq=6, Hkv=2), dict(Hq=4, Hkv=4, dtype="bf16"), dict(Hq=8, Hkv=2)])
def test_cross_score_groups_matches_library_softmax(seed, shape):
    w, inp = tiny(seed, Nv=15, Nt=7, D=32, B=2, **shape)
    for b in range(2):
        el, _ = oracle.elite_select(w, inp.q[0], inp.k[0], b, alpha=0.5)
        ivg = oracle.cross_score_groups(w, inp.q[0], inp.k[0], b, el)
        assert np.allclose(ivg, library_iv_groups(w, inp, b, el), rtol=1e-12, atol=0)
        # the heads' scores differ (the selection is per head for a reason)
        assert not np.allclose(ivg[0], ivg[1])


def test_cross_score_groups_one_kv_head_is_the_shared_score():
    w, inp = tiny(3, Nv=20, Nt=6, D=16, Hq=5, Hkv=1)
    el, _ = oracle.elite_select(w, inp.q[0], inp.k[0], 0, alpha=0.3)
    ivg = oracle.cross_score_groups(w, inp.q[0], inp.k[0], 0, el)
    assert np.array_equal(ivg[0], oracle.cross_score(w, inp.q[0], inp.k[0], 0, el))


def test_cross_score_groups_average_to_the_shared_score():
    # equal head groups: the mean over KV heads of I_v^g is I_v
    w, inp = tiny(4, Nv=11, Nt=5, D=16, Hq=6, Hkv=3, B=1)
    el = np.array([1, 4], np.int32)
    ivg = oracle.cross_score_groups(w, inp.q[0], inp.k[0], 0, el)
    iv = oracle.cross_score(w, inp.q[0], inp.k[0], 0, el)
    assert np.allclose(ivg.mean(0), iv, rtol=1e-13, atol=0)


def test_cross_score_groups_uniform_when_queries_are_zero():
    w = wl.custom(Nv=10, Nt=4, Hq=4, Hkv=2, D=16)
    inp = wl.make_inputs(w, 1, zero_q=True)
    ivg = oracle.cross_score_groups(w, inp.q[0], inp.k[0], 0, np.arange(4, dtype=np.int32))
    assert np.allclose(ivg, 1.0 / 14, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- step 3 ----

@pytest.mark.parametrize("n", [3, 4, 64, 576, 2880])
def test_skew_one_hot_is_sqrt_n(n):
    x = np.zeros(n)
    x[n // 3] = 1.0
    s_t, s_k = oracle.layer_stats(x)
    assert s_t == 1.0
    assert abs(s_k - math.sqrt(n)) <= 1e-12 * math.sqrt(n)


@pytest.mark.parametrize("n,m", [(10, 1), (10, 3), (50, 5), (64, 8), (7, 6)])
def test_skew_two_point_closed_form(n, m):
    # m ones and n-m zeros: fraction p = m/n,
    # s_k = sqrt(n(n-1))/(n-2) * (1-2p)/sqrt(p(1-p))
    x = np.zeros(n)
    x[:m] = 1.0
    p = m / n
    ref = math.sqrt(n * (n - 1)) / (n - 2) * (1 - 2 * p) / math.sqrt(p * (1 - p))
    _, s_k = oracle.layer_stats(x)
    assert abs(s_k - ref) <= 1e-12 * max(1.0, abs(ref))


def test_skew_symmetric_affine_negation_and_scipy():
    rng = np.random.default_rng(0)
    sym = np.concatenate([rng.random(20), -rng.random(20)])
    sym = np.concatenate([sym, -sym])
    assert abs(oracle.layer_stats(sym)[1]) < 1e-12
    for _ in range(20):
        n = int(rng.integers(3, 300))
        x = rng.exponential(size=n) ** 2
        _, s = oracle.layer_stats(x)
        assert abs(s - scipy.stats.skew(x, bias=False)) <= 1e-10 * max(1, abs(s))
        _, s2 = oracle.layer_stats(3.5 * x + 2.0)
        assert abs(s2 - s) <= 1e-10 * max(1, abs(s))
        _, s3 = oracle.layer_stats(-x)
        assert abs(s3 + s) <= 1e-10 * max(1, abs(s))
        assert abs(oracle.layer_stats(x)[0] - x.sum()) <= 1e-12 * x.sum()


def test_skew_constant_is_zero():
    assert oracle.layer_stats(np.full(9, 0.25)) == (2.25, 0.0)


# ---------------------------------------------------------------- step 4 ----

# Hand-derived two-layer cases (r = ratio * N_v):
#  a) s_t=[.25,.75] -> s't=[.5,1.5]; s_k=[1,3] -> s'k=[.5,1.5]; r=8 -> x=[4,12]
#  b) s_t=[.5,.5] -> [1,1]; s_k=[-1,1] shift by -1 -> u=[0,2] -> [0,2];
#     r=8 -> x=[.5*1*8, .5*3*8]=[4,12]
#  c) s_k=[-2,-2] -> u=[0,0], sum 0 -> s'k=[1,1]; s_t=[.5,.5]; r=8 -> [8,8]
#  d) N_v=10, ratio .9 -> r=9; s_t=[.25,.75] -> [.5,1.5]; s_k=[0,0] -> [1,1];
#     x=[.5*1.5*9, .5*2.5*9]=[6.75,11.25] -> floor [6,11] -> clamp [6,10]
#  e) s_k=[2,6] (no shift) -> [.5,1.5]; s_t=[.5,.5]; N_v=64, ratio .25 -> r=16;
#     x=[.5*1.5*16, .5*2.5*16]=[12,20]
BUDGET_CASES = [
    ([0.25, 0.75], [1.0, 3.0], 0.125, 64, [4.0, 12.0], [4, 12]),
    ([0.5, 0.5], [-1.0, 1.0], 0.125, 64, [4.0, 12.0], [4, 12]),
    ([0.5, 0.5], [-2.0, -2.0], 0.125, 64, [8.0, 8.0], [8, 8]),
    ([0.25, 0.75], [0.0, 0.0], 0.9, 10, [6.75, 11.25], [6, 10]),
    ([0.5, 0.5], [2.0, 6.0], 0.25, 64, [12.0, 20.0], [12, 20]),
]


@pytest.mark.parametrize("case", BUDGET_CASES)
def test_budget_hand_cases(case):
    st, sk, ratio, nv, x_ref, r_ref = case
    x, r = oracle.budget(st, sk, ratio, nv)
    assert np.allclose(x, x_ref, rtol=0, atol=1e-12)
    assert list(r) == r_ref


@pytest.mark.parametrize("L", [1, 2, 4, 8])
@pytest.mark.parametrize("ratio,nv", [(0.25, 64), (0.1, 576), (0.1, 2880)])
def test_budget_identical_layers(L, ratio, nv):
    # dyadic statistics keep every sum exact: each layer gets floor(r)
    x, r = oracle.budget([0.75] * L, [1.5] * L, ratio, nv)
    assert list(r) == [math.floor(ratio * nv)] * L
    x, r = oracle.budget([0.75] * L, [-0.5] * L, ratio, nv)   # shifted to 0
    assert list(r) == [math.floor(ratio * nv)] * L


def test_budget_mean_is_r_and_single_layer():
    rng = np.random.default_rng(1)
    for _ in range(50):
        L = int(rng.integers(1, 40))
        st = rng.uniform(0.5, 1.0, L)
        sk = rng.normal(1.0, 2.0, L)
        ratio, nv = float(rng.uniform(0.01, 0.3)), int(rng.integers(3, 7000))
        x, r = oracle.budget(st, sk, ratio, nv)
        assert abs(x.sum() - L * ratio * nv) <= 1e-9 * L * ratio * nv
        assert ((r >= 0) & (r <= nv)).all()
        assert np.array_equal(r, np.clip(np.floor(x), 0, nv).astype(int))
    x, r = oracle.budget([0.3], [-4.0], 0.1, 576)
    assert abs(x[0] - 57.6) < 1e-12 and r[0] == 57


# Allocation variants of the page's ablation ("Layer-wise KV Cache Budget
# Allocation", the allocation table), read as the r_hat equation with one
# term (or none): 1 uniform, 2 strength only, 3 skewness only.
#  a) uniform: every layer floor(ratio * N_v), whatever the statistics
#  b) strength only, s_t=[1,3] (L=2): s't=[0.5,1.5], r=0.125*64=8 -> x=[4,12]
#  c) skewness only, s_k=[-1,1]: m=-1, u=[0,2], s'k=[0,2], r=8 -> x=[0,16]
#  d) skewness only with sum(u)=0 (s_k all equal): s'k=1 -> x=r
@pytest.mark.parametrize("L", [1, 3, 28])
def test_budget_uniform_variant(L):
    rng = np.random.default_rng(L)
    st, sk = rng.uniform(0.1, 2.0, L), rng.normal(0.0, 3.0, L)
    x, r = oracle.budget(st, sk, 0.1, 2880, mode=1)
    assert np.all(x == 0.1 * 2880) and list(r) == [288] * L


def test_budget_single_term_variants():
    x, r = oracle.budget([1.0, 3.0], [5.0, -7.0], 0.125, 64, mode=2)
    assert np.allclose(x, [4.0, 12.0], rtol=0, atol=1e-12) and list(r) == [4, 12]
    x, r = oracle.budget([9.0, 0.1], [-1.0, 1.0], 0.125, 64, mode=3)
    assert np.allclose(x, [0.0, 16.0], rtol=0, atol=1e-12) and list(r) == [0, 16]
    x, r = oracle.budget([9.0, 0.1, 4.0], [-2.5, -2.5, -2.5], 0.125, 64, mode=3)
    assert np.all(x == 8.0) and list(r) == [8, 8, 8]


def test_budget_rule_is_mean_of_single_terms():
    """The page's x is the mean of the strength-only and skewness-only x, up to
    rounding; the budgets of the single-term variants also sum to L * r."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        L = int(rng.integers(1, 40))
        st, sk = rng.uniform(0.5, 1.0, L), rng.normal(1.0, 2.0, L)
        ratio, nv = float(rng.uniform(0.01, 0.3)), int(rng.integers(3, 7000))
        x0, _ = oracle.budget(st, sk, ratio, nv)
        x2, r2 = oracle.budget(st, sk, ratio, nv, mode=2)
        x3, r3 = oracle.budget(st, sk, ratio, nv, mode=3)
        assert np.allclose(x0, 0.5 * (x2 + x3), rtol=1e-12, atol=1e-9)
        for x in (x2, x3):
            assert abs(x.sum() - L * ratio * nv) <= 1e-9 * L * ratio * nv
        for x, r in ((x2, r2), (x3, r3)):
            assert np.array_equal(r, np.clip(np.floor(x), 0, nv).astype(int))


# e) pyramid (mode 4, the table's PyramidKV allocation read as a linear
#    pyramid with the method's mean): L=3, r=0.125*64=8 -> x = 8*2*(3-l)/4 =
#    [12, 8, 4]; L=1 -> x = r; whatever the statistics; sum L*r; falling with depth
def test_budget_pyramid_variant():
    x, r = oracle.budget([1.0, 3.0, 0.5], [5.0, -7.0, 0.0], 0.125, 64, mode=4)
    assert np.allclose(x, [12.0, 8.0, 4.0], rtol=0, atol=1e-12) and list(r) == [12, 8, 4]
    x, r = oracle.budget([2.0], [1.0], 0.1, 2880, mode=4)
    assert np.allclose(x, [288.0], rtol=0, atol=1e-12) and list(r) == [288]
    rng = np.random.default_rng(9)
    for _ in range(20):
        L = int(rng.integers(2, 40))
        ratio, nv = float(rng.uniform(0.01, 0.3)), int(rng.integers(3, 7000))
        a, ra = oracle.budget(rng.uniform(0.5, 1.0, L), rng.normal(1.0, 2.0, L), ratio, nv, mode=4)
        b, rb = oracle.budget(rng.uniform(0.5, 1.0, L), rng.normal(1.0, 2.0, L), ratio, nv, mode=4)
        assert np.array_equal(a, b) and np.array_equal(ra, rb)      # statistics play no part
        assert abs(a.sum() - L * ratio * nv) <= 1e-9 * L * ratio * nv
        assert np.all(np.diff(a) < 0)                                 # deeper layers get less
        r = ratio * nv
        assert np.allclose(a[[0, -1]], [2 * L * r / (L + 1), 2 * r / (L + 1)], rtol=1e-12)


def test_window_select():
    # the window ablation's contiguous windows: the last k text tokens
    assert list(oracle.window_select(128, 16)) == list(range(112, 128))
    assert list(oracle.window_select(128, 32)) == list(range(96, 128))
    assert list(oracle.window_select(40, 128)) == list(range(40))   # all text tokens
    assert list(oracle.window_select(7, 1)) == [6]


# ---------------------------------------------------------------- step 5 ----

def check_topk(scores, k, kept):
    """The unique answer: k indices, ascending, every kept score >= every
    dropped score, and among equal scores at the cut the lower indices win."""
    kept = list(kept)
    assert len(kept) == k and kept == sorted(kept) and len(set(kept)) == k
    drop = [i for i in range(len(scores)) if i not in set(kept)]
    if kept and drop:
        kmin = min(scores[i] for i in kept)
        dmax = max(scores[i] for i in drop)
        assert kmin >= dmax
        if kmin == dmax:
            assert max(i for i in kept if scores[i] == kmin) < min(i for i in drop if scores[i] == dmax)


@pytest.mark.parametrize("seed", range(30))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    s = rng.integers(0, 4, n).astype(np.float64) * 0.125   # many ties
    for k in range(0, n + 1):
        kept = oracle.topk(s, k)
        check_topk(s, k, kept)
        ref = np.sort(np.lexsort((np.arange(n), -s))[:k])   # numpy's sort
        assert np.array_equal(kept, ref)


def test_topk_extremes():
    s = np.array([0.3, 0.1, 0.2])
    assert oracle.topk(s, 0).size == 0
    assert list(oracle.topk(s, 3)) == [0, 1, 2]
    assert list(oracle.topk(s, 1)) == [0]
    assert list(oracle.topk(np.zeros(5), 2)) == [0, 1]


# ---------------------------------------------------------------- step 6 ----

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_identity_when_everything_is_kept(dtype):
    # L = 1 gives s't = s'k = 1, so ratio 1 keeps every visual token and the
    # compacted cache is the input byte for byte
    w = wl.custom(Nv=9, Nt=4, Hq=4, Hkv=2, D=16, B=3, dtype=dtype, ratio=1.0)
    inp = wl.make_inputs(w, 7)
    out = oracle.run(inp)
    assert (out["budget"] == 9).all()
    assert np.array_equal(out["k_out"][0], inp.k[0].ravel())
    assert np.array_equal(out["v_out"][0], inp.v[0].ravel())


def test_gather_layout_and_text_rows():
    w = wl.custom(Nv=12, Nt=3, Hq=2, Hkv=2, D=8, B=2, L=2, ratio=0.3)
    inp = wl.make_inputs(w, 11)
    out = oracle.run(inp)
    for l in range(2):
        for b in range(2):
            r = int(out["budget"][l, b])
            o = int(out["out_off"][l, b])
            seg = out["k_out"][l][o:o + 2 * (r + 3) * 8].reshape(2, r + 3, 8)
            kept = out["kept"][l, b, :r]
            for g in range(2):
                assert np.array_equal(seg[g, :r], inp.k[l, b, g, kept])
                assert np.array_equal(seg[g, r:], inp.k[l, b, g, 12:])
        assert out["out_off"][l, 2] == sum(2 * (int(out["budget"][l, b]) + 3) * 8 for b in range(2))


def test_gather_groups_layout_per_head():
    w = wl.custom(Nv=10, Nt=3, Hq=4, Hkv=2, D=8, B=2)
    inp = wl.make_inputs(w, 12)
    kept = np.array([[1, 4, 9], [0, 2, 3]], np.int32)
    for b in range(2):
        seg = oracle.gather_groups(w, inp.k[0], b, kept)
        for g in range(2):
            assert np.array_equal(seg[g, :3], inp.k[0, b, g, kept[g]])
            assert np.array_equal(seg[g, 3:], inp.k[0, b, g, 10:])
    # one list for every head: the shared gather
    same = np.array([[2, 5], [2, 5]], np.int32)
    assert np.array_equal(oracle.gather_groups(w, inp.v[0], 1, same), oracle.gather(w, inp.v[0], 1, same[0]))
    # no visual row kept: the text rows only
    assert np.array_equal(oracle.gather_groups(w, inp.k[0], 0, np.zeros((2, 0), np.int32)), inp.k[0, 0, :, 10:])


# -------------------------------------------- int8 quantisation (f4) ----

def test_quantize_exact_multiples_of_the_scale():
    # max |x| = 127 / 8, so s = 1/8 exactly and x = k / 8 has code k
    k = np.arange(-127, 128, dtype=np.float64)
    x = (k / 8.0).astype(np.float32)
    codes, s = oracle.quantize_i8(x, "f32")
    assert s == 0.125
    assert np.array_equal(codes.astype(np.int64), k.astype(np.int64))


def test_quantize_ties_round_half_to_even():
    x = np.array([127, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, -1.5, 126.5], np.float64) / 8.0
    codes, s = oracle.quantize_i8(x.astype(np.float32), "f32")
    assert s == 0.125
    assert codes.tolist() == [127, 2, 4, -2, 0, 0, 2, -2, 126]


def test_quantize_all_zero_head():
    codes, s = oracle.quantize_i8(np.zeros(40, np.float32), "f32")
    assert s == 0.0 and not codes.any()


@pytest.mark.parametrize("seed", range(5))
def test_quantize_error_bound_and_extremes(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(3000) * rng.uniform(0.1, 10)).astype(np.float32)
    codes, s = oracle.quantize_i8(x, "f32")
    i = int(np.argmax(np.abs(x)))
    assert abs(int(codes[i])) == 127 and np.sign(codes[i]) == np.sign(x[i])
    assert np.isclose(s, np.abs(x).max() / 127, rtol=1e-7)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(codes.astype(np.float64) * s - x.astype(np.float64))
    assert err.max() <= s * (0.5 + 1e-5)


def test_quantize_bf16_is_its_float32_value():
    rng = np.random.default_rng(9)
    bits = wl.f32_to_bf16_bits(rng.standard_normal(500).astype(np.float32))
    as_f32 = (bits.astype(np.uint32) << 16).view(np.float32)
    c16, s16 = oracle.quantize_i8(bits, "bf16")
    c32, s32 = oracle.quantize_i8(as_f32, "f32")
    assert s16 == s32 and np.array_equal(c16, c32)


# ------------------------------------------------------------ end to end ----

def test_run_threads_equals_single_call():
    w = wl.custom(Nv=40, Nt=8, Hq=4, Hkv=2, D=32, B=2, L=3, dtype="bf16", ratio=0.2)
    inp = wl.make_inputs(w, 3)
    a = oracle.run(inp)
    b = oracle.run(inp, threads=4)
    for key in ["n_elite", "iv", "s_t", "s_k", "x", "budget", "out_off", "kept"]:
        assert np.array_equal(a[key], b[key]), key
    for l in range(3):
        assert np.array_equal(a["k_out"][l], b["k_out"][l])
        assert np.array_equal(a["v_out"][l], b["v_out"][l])


def test_config1_end_to_end_properties():
    inp = wl.make_inputs(1, 1)
    o = oracle.run(inp)
    w = inp.w
    assert (o["n_elite"] >= 1).all()
    assert np.all((o["s_t"] > 0) & (o["s_t"] < 1))
    assert abs(o["x"].sum() - w.L * w.ratio * w.Nv) < 1e-9
    assert (o["budget"] <= w.Nv).all()


def test_config2_generator_reading_elite_is_all_text():
    # the mean-query planting of the 7B-like workload aims at the mean of all
    # text queries; under its N(0,1)/sqrt(D) base the elite window is all text
    w = wl.CONFIGS[2]
    small = wl.Workload(**{**w.__dict__, "L": 2, "cid": 0})
    inp = wl.make_inputs(small, 2)
    o = oracle.run(inp, compact=False, threads=4)
    assert (o["n_elite"] == w.Nt).all()


# ------------------------------------------------- decode attention (f2) ----
# The consumer of the compacted cache: o_h = softmax(q_h K_g^T / sqrt(D)) V_g
# (the KV-cache primer page, section 2.1, the o_t equation).

def _seg(w, rng, n, scale=1.0):
    k = (rng.standard_normal((w.Hkv, n, w.D)) * scale).astype(np.float32)
    v = rng.standard_normal((w.Hkv, n, w.D)).astype(np.float32)
    q = rng.standard_normal((w.Hq, w.D)).astype(np.float32)
    if w.dtype == "bf16":
        k, v, q = wl.f32_to_bf16_bits(k), wl.f32_to_bf16_bits(v), wl.f32_to_bf16_bits(q)
    return k, v, q


def _f64(w, a):
    return (a if w.dtype == "f32" else wl.bf16_bits_to_f32(a)).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_single_row_returns_its_value(dtype):
    w = wl.custom(Nv=8, Nt=2, Hq=6, Hkv=2, D=16, dtype=dtype)
    k, v, q = _seg(w, np.random.default_rng(1), 1)
    o = oracle.decode_attention_segment(w, k, v, 1, q)
    for h in range(w.Hq):
        assert np.array_equal(o[h], _f64(w, v)[h // 3, 0])


@pytest.mark.parametrize("n", [2, 7, 40])
def test_decode_uniform_keys_give_the_mean_value(n):
    w = wl.custom(Nv=8, Nt=2, Hq=4, Hkv=2, D=32)
    k, v, q = _seg(w, np.random.default_rng(n), n)
    k[:] = k[:, :1]  # every row of a head's keys equal: uniform weights
    o = oracle.decode_attention_segment(w, k, v, n, q)
    for h in range(w.Hq):
        np.testing.assert_allclose(o[h], _f64(w, v)[h // 2].mean(axis=0), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("shape", [dict(Hq=1, Hkv=1), dict(Hq=6, Hkv=2), dict(Hq=4, Hkv=4, dtype="bf16")])
def test_decode_matches_library_softmax(seed, shape):
    """Brute force with scipy's softmax, query head h on KV head h // G."""
    w = wl.custom(Nv=8, Nt=2, D=24, **shape)
    n = 5 + seed
    k, v, q = _seg(w, np.random.default_rng(10 + seed), n, scale=2.0)
    o = oracle.decode_attention_segment(w, k, v, n, q)
    K, V, Q = _f64(w, k), _f64(w, v), _f64(w, q)
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        p = scipy.special.softmax(K[h // G] @ Q[h] / math.sqrt(w.D))
        np.testing.assert_allclose(o[h], p @ V[h // G], rtol=1e-12, atol=1e-13)


def test_decode_is_invariant_to_row_order():
    w = wl.custom(Nv=8, Nt=2, Hq=4, Hkv=2, D=16)
    n = 9
    k, v, q = _seg(w, np.random.default_rng(3), n)
    perm = np.random.default_rng(4).permutation(n)
    a = oracle.decode_attention_segment(w, k, v, n, q)
    b = oracle.decode_attention_segment(w, np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm]), n, q)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_decode_dominant_key_selects_its_value():
    w = wl.custom(Nv=8, Nt=2, Hq=2, Hkv=1, D=16)
    rng = np.random.default_rng(5)
    n = 6
    k, v, q = _seg(w, rng, n, scale=0.01)
    k[0, 4] = 40.0 * q[0] / np.linalg.norm(q[0])  # a key along query 0
    o = oracle.decode_attention_segment(w, k, v, n, q)
    np.testing.assert_allclose(o[0], v[0, 4], atol=1e-6)


def test_decode_over_the_compacted_layer_uses_offsets_and_budgets():
    """Layer-level wrapper on the oracle's own compacted output: each sample's
    segment is found at out_off with budget + N_t rows per KV head."""
    w = wl.custom(Nv=12, Nt=3, Hq=4, Hkv=2, D=8, B=2, L=1, ratio=0.4)
    inp = wl.make_inputs(w, 2)
    out = oracle.run(inp)
    q = np.random.default_rng(6).standard_normal((w.B, w.Hq, w.D)).astype(np.float32)
    o = oracle.decode_attention(w, out["k_out"][0], out["v_out"][0], out["out_off"][0], out["budget"][0], q)
    for b in range(w.B):
        kept = out["kept"][0, b, :out["budget"][0, b]]
        rows = np.concatenate([kept, np.arange(w.Nv, w.Nv + w.Nt)])
        K = inp.k[0, b][:, rows].astype(np.float64)
        V = inp.v[0, b][:, rows].astype(np.float64)
        for h in range(w.Hq):
            p = scipy.special.softmax(K[h // 2] @ q[b, h].astype(np.float64) / math.sqrt(w.D))
            np.testing.assert_allclose(o[b, h], p @ V[h // 2], rtol=1e-12, atol=1e-13)


# ----------------------------------------- prefill attention (f3's attention) ----
# o_{h,t} = softmax(q_{h,t} K_g[0..t]^T / sqrt(D)) V_g[0..t] at every position t
# of the regrouped sequence (the KV-cache primer page, section 2.1, the o_t
# equation at each step of the prompt).

def _prefill_inputs(w, rng, kscale=1.0):
    S = w.Nv + w.Nt
    q = rng.standard_normal((w.B, w.Hq, S, w.D)).astype(np.float32)
    k = (rng.standard_normal((w.B, w.Hkv, S, w.D)) * kscale).astype(np.float32)
    v = rng.standard_normal((w.B, w.Hkv, S, w.D)).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v = wl.f32_to_bf16_bits(q), wl.f32_to_bf16_bits(k), wl.f32_to_bf16_bits(v)
    return q, k, v


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_first_position_returns_its_value(dtype):
    """Position 0 sees one key: its output is v_0 of its KV head, exactly."""
    w = wl.custom(Nv=5, Nt=3, Hq=6, Hkv=2, D=16, B=2, dtype=dtype)
    q, k, v = _prefill_inputs(w, np.random.default_rng(1))
    for b in range(w.B):
        o = oracle.prefill_attention(w, q[0:w.B], k, v, b, 0, 1)
        for h in range(w.Hq):
            assert np.array_equal(o[h, 0], _f64(w, v)[b, h // 3, 0])


def test_prefill_equal_keys_give_the_running_mean():
    """All keys of a head equal: uniform weights over 0..t, so o_t is the mean
    of v_0..v_t (a causal mask that leaked later keys would fail)."""
    w = wl.custom(Nv=6, Nt=4, Hq=4, Hkv=2, D=8)
    q, k, v = _prefill_inputs(w, np.random.default_rng(2))
    k[:] = k[:, :, :1]
    o = oracle.prefill_attention(w, q, k, v, 0)
    V = _f64(w, v)[0]
    for h in range(w.Hq):
        for t in range(w.Nv + w.Nt):
            np.testing.assert_allclose(o[h, t], V[h // 2, :t + 1].mean(axis=0), rtol=0, atol=1e-12)


def test_prefill_two_keys_closed_form():
    """Position 1 weighs v_1 by the logistic function of (q.k_1 - q.k_0)/sqrt(D)."""
    w = wl.custom(Nv=3, Nt=2, Hq=2, Hkv=1, D=8)
    q, k, v = _prefill_inputs(w, np.random.default_rng(3), kscale=2.0)
    o = oracle.prefill_attention(w, q, k, v, 0, 1, 1)
    Q, K, V = _f64(w, q)[0], _f64(w, k)[0, 0], _f64(w, v)[0, 0]
    for h in range(w.Hq):
        d = (Q[h, 1] @ K[1] - Q[h, 1] @ K[0]) / math.sqrt(w.D)
        p1 = 1.0 / (1.0 + math.exp(-d))
        np.testing.assert_allclose(o[h, 0], (1.0 - p1) * V[0] + p1 * V[1], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("shape", [dict(Hq=1, Hkv=1), dict(Hq=6, Hkv=2), dict(Hq=4, Hkv=4, dtype="bf16")])
def test_prefill_matches_library_softmax(seed, shape):
    """Brute force: scipy's softmax over the masked score matrix, query head h
    on KV head h // G, rows from a middle offset."""
    w = wl.custom(Nv=7, Nt=5, D=16, B=2, **shape)
    q, k, v = _prefill_inputs(w, np.random.default_rng(20 + seed), kscale=1.5)
    b, row0 = seed % 2, 3
    o = oracle.prefill_attention(w, q, k, v, b, row0, w.Nv + w.Nt - row0)
    Q, K, V = _f64(w, q)[b], _f64(w, k)[b], _f64(w, v)[b]
    G, S = w.Hq // w.Hkv, w.Nv + w.Nt
    mask = np.tril(np.ones((S, S), bool))
    for h in range(w.Hq):
        z = np.where(mask, Q[h] @ K[h // G].T / math.sqrt(w.D), -np.inf)
        ref = scipy.special.softmax(z, axis=1) @ V[h // G]
        np.testing.assert_allclose(o[h], ref[row0:], rtol=1e-12, atol=1e-13)


def test_prefill_ignores_later_positions():
    """Causality: changing keys and values after position t leaves o_t alone."""
    w = wl.custom(Nv=6, Nt=4, Hq=2, Hkv=2, D=8)
    q, k, v = _prefill_inputs(w, np.random.default_rng(4))
    a = oracle.prefill_attention(w, q, k, v, 0)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 6:] *= -3.0
    v2[:, :, 6:] += 5.0
    b = oracle.prefill_attention(w, q, k2, v2, 0)
    np.testing.assert_array_equal(a[:, :6], b[:, :6])
    assert not np.allclose(a[:, 6:], b[:, 6:])


def test_prefill_dominant_key_selects_its_value():
    w = wl.custom(Nv=4, Nt=4, Hq=2, Hkv=1, D=16)
    q, k, v = _prefill_inputs(w, np.random.default_rng(5), kscale=0.01)
    t = 6
    k[0, 0, 2] = 40.0 * q[0, 0, t] / np.linalg.norm(q[0, 0, t])  # a key along head 0's query t
    o = oracle.prefill_attention(w, q, k, v, 0, t, 1)
    np.testing.assert_allclose(o[0, 0], v[0, 0, 2], atol=1e-6)


# ------------------------------------------- visual observation window (f1) ----
# The window ablation's visual window: the last k visual tokens as the
# observation rows, each normalised over the N_v visual keys.

def _vw_inputs(w, seed):
    inp = wl.make_inputs(w, seed)
    return inp, wl.prefill_queries(inp, 0)


def test_visual_window_rows_sum_to_one_so_strength_is_one():
    """Every row's probabilities over the visual keys sum to 1, so I_v sums to
    1 whatever the inputs (s_t = 1 on every layer)."""
    w = wl.custom(Nv=40, Nt=8, Hq=6, Hkv=2, D=16, B=2)
    inp, qa = _vw_inputs(w, 1)
    for b in range(w.B):
        iv = oracle.visual_window(w, qa, inp.k[0], b, 5)
        assert abs(iv.sum() - 1.0) < 1e-12
        s_t, _ = oracle.layer_stats(iv)
        assert abs(s_t - 1.0) < 1e-12


def test_visual_window_zero_queries_uniform():
    w = wl.custom(Nv=30, Nt=4, Hq=2, Hkv=1, D=8)
    inp, qa = _vw_inputs(w, 2)
    qa[:] = 0
    iv = oracle.visual_window(w, qa, inp.k[0], 0, 7)
    np.testing.assert_allclose(iv, np.full(w.Nv, 1.0 / w.Nv), rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("shape", [dict(Hq=1, Hkv=1), dict(Hq=6, Hkv=2), dict(Hq=4, Hkv=4, dtype="bf16")])
def test_visual_window_matches_library_softmax(seed, shape):
    """Brute force: scipy's softmax over the visual keys for the last k visual
    queries, query head h on KV head h // G, no mask."""
    w = wl.custom(Nv=23, Nt=5, D=16, B=2, **shape)
    inp, qa = _vw_inputs(w, 30 + seed)
    b, kwin = seed % 2, 4 + seed
    iv, ivg = oracle.visual_window(w, qa, inp.k[0], b, kwin, groups=True)
    Q = (qa if w.dtype == "f32" else wl.bf16_bits_to_f32(qa)).astype(np.float64)[b]
    K = inp.as_f32("k").astype(np.float64)[0, b]
    G = w.Hq // w.Hkv
    ref = np.zeros(w.Nv)
    refg = np.zeros((w.Hkv, w.Nv))
    for h in range(w.Hq):
        P = scipy.special.softmax(Q[h, w.Nv - kwin:w.Nv] @ K[h // G, :w.Nv].T / math.sqrt(w.D), axis=1)
        ref += P.sum(0)
        refg[h // G] += P.sum(0)
    np.testing.assert_allclose(iv, ref / (w.Hq * kwin), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ivg, refg / (G * kwin), rtol=1e-12, atol=1e-15)


def test_visual_window_ignores_text_positions():
    """Only visual queries and visual keys enter: text rows of q, and text keys,
    may change freely."""
    w = wl.custom(Nv=20, Nt=6, Hq=2, Hkv=1, D=8)
    inp, qa = _vw_inputs(w, 4)
    a = oracle.visual_window(w, qa, inp.k[0], 0, 3)
    qa2, k2 = qa.copy(), inp.k[0].copy()
    qa2[:, :, w.Nv:] *= 5.0
    k2[:, :, w.Nv:] += 1.0
    b = oracle.visual_window(w, qa2, k2, 0, 3)
    np.testing.assert_array_equal(a, b)


# ----------------------------------------------- decode over the int8 cache ----
# The decode attention with every cached value read as code * scale.

def _i8seg(w, rng, n):
    kq = rng.integers(-127, 128, size=(w.Hkv, n, w.D)).astype(np.int8)
    vq = rng.integers(-127, 128, size=(w.Hkv, n, w.D)).astype(np.int8)
    q = rng.standard_normal((w.Hq, w.D)).astype(np.float32)
    if w.dtype == "bf16":
        q = wl.f32_to_bf16_bits(q)
    return kq, vq, q


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_i8_equals_decode_on_exactly_dequantised_values(dtype):
    """With power-of-two scales code * scale is exact in float32, so the int8
    decode equals the float decode of that segment (pinned above) bit for bit."""
    w = wl.custom(Nv=8, Nt=2, Hq=6, Hkv=2, D=16, dtype=dtype)
    rng = np.random.default_rng(40)
    n = 9
    kq, vq, q = _i8seg(w, rng, n)
    ks = np.array([2.0 ** -6, 2.0 ** -8], np.float32)
    vs = np.array([2.0 ** -5, 2.0 ** -7], np.float32)
    o8 = oracle.decode_attention_i8_segment(w, kq, vq, ks, vs, n, q)
    kf = (kq.astype(np.float32) * ks[:, None, None]).astype(np.float32)
    vf = (vq.astype(np.float32) * vs[:, None, None]).astype(np.float32)
    if dtype == "bf16":  # codes times 2^-k are exact in bfloat16 too (8-bit significand holds |code| <= 127)
        kf, vf = wl.f32_to_bf16_bits(kf), wl.f32_to_bf16_bits(vf)
    np.testing.assert_array_equal(o8, oracle.decode_attention_segment(w, kf, vf, n, q))


def test_decode_i8_single_row_and_value_scale():
    w = wl.custom(Nv=8, Nt=2, Hq=2, Hkv=1, D=8)
    rng = np.random.default_rng(41)
    kq, vq, q = _i8seg(w, rng, 1)
    ks, vs = np.array([0.013], np.float32), np.array([0.021], np.float32)
    o = oracle.decode_attention_i8_segment(w, kq, vq, ks, vs, 1, q)
    for h in range(w.Hq):
        np.testing.assert_array_equal(o[h], vq[0, 0].astype(np.float64) * float(vs[0]))
    # o is linear in the V scale; zero V codes give zero
    kq, vq, q = _i8seg(w, rng, 5)
    a = oracle.decode_attention_i8_segment(w, kq, vq, ks, vs, 5, q)
    b = oracle.decode_attention_i8_segment(w, kq, vq, ks, 2 * vs, 5, q)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-14, atol=0)
    z = oracle.decode_attention_i8_segment(w, kq, np.zeros_like(vq), ks, vs, 5, q)
    assert not z.any()
