"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Full-size workloads 1-5 (every parity seed) in the launch configuration the
benchmark times, and 4-5 also with no elite cap (max_elite = 0, the library's
default), each scoring path on the workloads
it serves, plus small edge shapes: ragged tails, one and eight KV heads, MHA,
head_dim 64, float32 and bfloat16, a single text token, alpha and ratio at
their extremes, zero queries (every text token elite, several row passes),
several samples, a workspace reused across calls, and workload 3 with flat
attention (every text token elite).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import compare, reference, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lvlm_kv_cache_amd import _lib
    _lib.load()  # raises if the HIP library is missing
    torch.cuda.set_device(0)


CASES = [(c, s) for c in (1, 2, 3, 4, 5) for s in wl.parity_seeds(c)]


@pytest.mark.parametrize("cid,seed", CASES)
def test_workload(cid, seed):
    print(f"[parity] workload {cid} seed {seed}", flush=True)
    inp = wl.make_inputs(cid, seed)
    g = run_gpu(inp, max_elite=0 if cid <= 2 else 64)
    ref = reference(inp, g)
    rep = compare(inp, g, ref)
    print(f"[parity] workload {cid} seed {seed}: {rep}", flush=True)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_run(cid):
    """aircache_run (plan and compaction in one call, one launch on the chunked
    path) on the full-size workloads."""
    print(f"[parity] workload {cid} run", flush=True)
    inp = wl.make_inputs(cid, cid)
    g = run_gpu(inp, max_elite=0 if cid <= 2 else 64, run=True)
    compare(inp, g, reference(inp, g))


@pytest.mark.parametrize("cid", [4, 5])
def test_workload_run_no_elite_cap(cid):
    """aircache_run on workloads 4 and 5 at full size with max_elite = 0 (the
    elite cap is N_t, the library's default), whatever path that resolves to."""
    print(f"[parity] workload {cid} run, no elite cap", flush=True)
    inp = wl.make_inputs(cid, cid)
    g = run_gpu(inp, max_elite=0, run=True)
    compare(inp, g, reference(inp, g))


def test_workload_3_flat_attention_stress():
    """Workload 3 at full size with the N(0,1)/sqrt(D) base (the stress run
    behind bench.py --base-scale inv_sqrt_d): attention is flat, so every text
    token is elite (N_tk = 128, 56 row tiles per KV head, many row groups);
    no elite cap, one launch."""
    import dataclasses
    w = dataclasses.replace(wl.CONFIGS[3], base="inv_sqrt_d")
    print("[parity] workload 3 flat-attention stress", flush=True)
    inp = wl.make_inputs(w, 3)
    g = run_gpu(inp, max_elite=0, run=True)
    assert (g["n_elite"] == w.Nt).all()
    compare(inp, g, reference(inp, g))


@pytest.mark.parametrize("path,cid", [("tiled", 1), ("tiled", 2), ("tiled", 3), ("tiled", 5),
                                      ("rows", 1), ("rows", 3), ("rows", 5), ("chunked", 4), ("chunked", 1),
                                      ("chunked-run", 1)])
def test_workload_other_paths(path, cid):
    """The scoring paths auto does not pick, on the workloads they can serve."""
    print(f"[parity] workload {cid} path {path}", flush=True)
    inp = wl.make_inputs(cid, cid)
    g = run_gpu(inp, max_elite=0 if cid <= 2 else 64, path=path.split("-")[0], run=path.endswith("-run"))
    compare(inp, g, reference(inp, g))


EDGE = [
    dict(Nv=17, Nt=3, Hq=1, Hkv=1, D=64, dtype="f32"),
    dict(Nv=3, Nt=1, Hq=2, Hkv=1, D=64, dtype="bf16"),
    dict(Nv=300, Nt=40, Hq=7, Hkv=1, D=128, dtype="bf16", B=3, L=3),
    dict(Nv=257, Nt=33, Hq=4, Hkv=4, D=128, dtype="f32", L=2),
    dict(Nv=1000, Nt=20, Hq=14, Hkv=2, D=64, dtype="bf16", L=4, B=2),
    dict(Nv=129, Nt=17, Hq=32, Hkv=1, D=128, dtype="bf16", L=2),   # G = 32 > 16
    dict(Nv=4100, Nt=9, Hq=8, Hkv=2, D=128, dtype="bf16", L=2),
    dict(Nv=700, Nt=80, Hq=8, Hkv=8, D=128, dtype="bf16", L=3, B=2),   # eight KV heads
    dict(Nv=333, Nt=24, Hq=8, Hkv=2, D=64, dtype="f32", L=3, B=5),     # several samples
]


def _small_ok(w):
    from lvlm_kv_cache_amd import _lib, make_desc
    d = make_desc(w.L, w.B, w.Hq, w.Hkv, w.D, w.Nv, w.Nt, w.dtype, path="small")
    return _lib.resolved_path(d) == _lib.PATH_SMALL


@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("path", ["auto", "auto-run", "chunked-run", "small", "small-run", "tiled", "rows"])
def test_edge_shapes(shape, seed, path):
    if path == "rows" and shape["Nv"] > 3072:
        pytest.skip("the rows path serves N_v <= 3072")
    if path.startswith("small") and not _small_ok(wl.custom(ratio=0.2, **shape)):
        pytest.skip("the small path serves shapes whose keys and text queries fit its LDS")
    print(f"[parity] edge {shape} seed {seed} path {path}", flush=True)
    w = wl.custom(ratio=0.2, **shape)
    inp = wl.make_inputs(w, seed)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"))
    compare(inp, g, reference(inp, g))


SMALL_EDGE = [
    dict(Nv=40, Nt=8, Hq=2, Hkv=1, D=64, dtype="bf16", L=12, B=2),     # more layers than waves
    dict(Nv=200, Nt=90, Hq=2, Hkv=1, D=64, dtype="bf16", L=2, B=2),    # N_t over one 64-lane block
    dict(Nv=500, Nt=12, Hq=4, Hkv=1, D=64, dtype="bf16", L=1, B=3),    # N_v near the rank's limit, G = 4
    dict(Nv=150, Nt=10, Hq=2, Hkv=1, D=128, dtype="f32", L=1, B=2),
    dict(Nv=65, Nt=33, Hq=6, Hkv=3, D=128, dtype="bf16", L=1, B=2),    # ragged N_v, three KV heads
    dict(Nv=3, Nt=1, Hq=1, Hkv=1, D=64, dtype="f32", L=5, B=4),
]


@pytest.mark.parametrize("shape", SMALL_EDGE, ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("path", ["small", "small-run", "auto-run"])
def test_small_shapes(shape, path):
    """Shapes of the one-workgroup path: layers shared by waves, N_t over a
    lane block, N_v up to the direct rank's limit, several samples."""
    w = wl.custom(ratio=0.3, **shape)
    assert _small_ok(w)
    print(f"[parity] small {shape} path {path}", flush=True)
    inp = wl.make_inputs(w, 21)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"))
    compare(inp, g, reference(inp, g))


@pytest.mark.parametrize("mode", [1, 2, 3, 4])
def test_small_budget_variants(mode):
    w = wl.custom(Nv=90, Nt=20, Hq=4, Hkv=2, D=64, dtype="bf16", L=3, B=2, ratio=0.25)
    assert _small_ok(w)
    inp = wl.make_inputs(w, 22)
    g = run_gpu(inp, path="small", run=True, budget_mode=mode)
    compare(inp, g, reference(inp, g, budget_mode=mode))


@pytest.mark.parametrize("window", [4, 20])
def test_small_observation_windows(window):
    w = wl.custom(Nv=90, Nt=20, Hq=4, Hkv=2, D=64, dtype="bf16", L=3, B=2, ratio=0.25)
    inp = wl.make_inputs(w, 23)
    g = run_gpu(inp, path="small", run=True, obs_window=window)
    assert (g["n_elite"] == window).all()
    compare(inp, g, reference(inp, g, obs_window=window))


def test_small_all_text_elite_and_overflow():
    """Zero queries: every text token elite (N_t = 70, over one lane block);
    then an elite cap below N_t flags the overflow."""
    w = wl.custom(Nv=120, Nt=70, Hq=2, Hkv=1, D=64, dtype="bf16", L=3, B=2, ratio=0.2)
    assert _small_ok(w)
    inp = wl.make_inputs(w, 24, zero_q=True)
    g = run_gpu(inp, path="small", run=True)
    assert (g["n_elite"] == 70).all()
    compare(inp, g, reference(inp, g))
    g = run_gpu(inp, path="small", max_elite=16, compress=False)
    assert g["status"][0] == 1


@pytest.mark.parametrize("path", ["auto", "auto-run", "tiled", "rows"])
def test_all_text_elite_many_rows(path):
    """Zero queries make every text token elite: G * N_tk = 280 rows per KV head,
    several row passes of the chunked path, elite text columns spanning chunks."""
    w = wl.custom(Nv=500, Nt=40, Hq=14, Hkv=2, D=128, dtype="bf16", L=2, B=2, ratio=0.3)
    inp = wl.make_inputs(w, 6, zero_q=True)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"))
    assert (g["n_elite"] == 40).all()
    compare(inp, g, reference(inp, g))


@pytest.mark.parametrize("path", ["rows", "tiled", "auto-run"])
def test_more_than_128_elite_tokens(path):
    """Zero queries with N_t = 200 make all 200 text tokens elite: the rows
    path then has more elite text tiles than waves (16 x 8 = 128 tokens); the
    one-launch pass takes seven MHA KV heads one per head group, 200 elite
    rows in three row passes and 200 elite text columns in its last chunks."""
    w = wl.custom(Nv=300, Nt=200, Hq=7, Hkv=7, D=128, dtype="bf16", L=2, B=1, ratio=0.2)
    print(f"[parity] 200 elite tokens, path {path}", flush=True)
    inp = wl.make_inputs(w, 12, zero_q=True)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"))
    assert (g["n_elite"] == 200).all()
    compare(inp, g, reference(inp, g))


def test_workspace_reused_across_calls():
    """One workspace, three calls with different inputs: each result matches the
    oracle (records of earlier calls must never be taken for current ones)."""
    from parity import make_aircache
    w = wl.custom(Nv=900, Nt=30, Hq=8, Hkv=4, D=128, dtype="bf16", L=3, B=2, ratio=0.2)
    ac = make_aircache(w)
    for seed, run in ((21, False), (22, True), (21, True), (23, False)):
        inp = wl.make_inputs(w, seed)
        g = run_gpu(inp, ac=ac, run=run)
        compare(inp, g, reference(inp, g))


def test_bound_pass_matches_plain_calls():
    """AirCache.bind (marshalling done once) gives bit-identical results to
    the per-call plan / compress, over repeated calls."""
    from parity import make_aircache, to_torch
    w = wl.custom(Nv=900, Nt=30, Hq=8, Hkv=4, D=128, dtype="bf16", L=3, B=2, ratio=0.2)
    inp = wl.make_inputs(w, 31)
    q, k, v = to_torch(inp)
    ac = make_aircache(w)
    plain = run_gpu(inp, ac=ac, tensors=(q, k, v))
    plan = ac.alloc_plan()
    ko, vo = ac.alloc_compacted()
    bp = ac.bind(q, k, v, plan, ko, vo)
    for _ in range(3):
        bp()
        torch.cuda.synchronize()
        for f in ("elite_idx", "n_elite", "iv", "s_t", "s_k", "budget_x", "budget", "out_off", "kept_idx", "status"):
            a, b = getattr(plan, f).cpu().numpy(), plain[f]
            if f == "elite_idx":
                a = np.concatenate([a[l, bb, :plain["n_elite"][l, bb]] for l in range(w.L) for bb in range(w.B)])
                b = np.concatenate([b[l, bb, :plain["n_elite"][l, bb]] for l in range(w.L) for bb in range(w.B)])
            if f == "kept_idx":
                a = np.concatenate([a[l, bb, :plain["budget"][l, bb]] for l in range(w.L) for bb in range(w.B)])
                b = np.concatenate([b[l, bb, :plain["budget"][l, bb]] for l in range(w.L) for bb in range(w.B)])
            assert np.array_equal(a, b), f
        for l in range(w.L):
            n = int(plain["out_off"][l, w.B])
            assert torch.equal(ko[l][:n].cpu(), torch.from_numpy(plain["k_out"][l].view(np.int16)).view(ko[l].dtype))
            assert torch.equal(vo[l][:n].cpu(), torch.from_numpy(plain["v_out"][l].view(np.int16)).view(vo[l].dtype))


def _random_shapes(n, seed=2024):
    """Seeded small shapes over the knobs the launch configuration depends on:
    layers x samples (how many elite-set parts and merges, and on which
    workgroups), KV heads and group size, ragged N_v and N_t, dtype, alpha and
    ratio."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 3, 7]))
        out.append(dict(L=int(rng.integers(1, 9)), B=int(rng.integers(1, 4)), Hkv=hkv, Hq=hkv * G,
                        D=int(rng.choice([64, 128])), Nv=int(rng.integers(3, 1500)), Nt=int(rng.integers(1, 150)),
                        dtype=str(rng.choice(["bf16", "f32"])), alpha=float(rng.choice([0.5, 0.9, 1.0])),
                        ratio=float(rng.choice([0.05, 0.2, 0.5]))))
    return out


@pytest.mark.parametrize("shape", _random_shapes(20), ids=lambda s: "x".join(f"{k}{v}" for k, v in s.items()))
@pytest.mark.parametrize("path", ["auto-run", "chunked-run", "rows"])
def test_random_shapes(shape, path):
    """Seeded random small shapes on the automatic path (small or one-launch),
    the one-launch pass and the rows path."""
    if path == "rows" and shape["Nv"] > 3072:
        pytest.skip("the rows path serves N_v <= 3072")
    print(f"[parity] random {shape} path {path}", flush=True)
    kw = dict(shape)
    alpha, ratio = kw.pop("alpha"), kw.pop("ratio")
    w = wl.custom(alpha=alpha, ratio=ratio, **kw)
    inp = wl.make_inputs(w, 11)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"))
    compare(inp, g, reference(inp, g, alpha=alpha, ratio=ratio), ratio=ratio)


_BUDGET_MODES = {"uniform": 1, "strength": 2, "skewness": 3, "pyramid": 4}


@pytest.mark.parametrize("mode", list(_BUDGET_MODES))
@pytest.mark.parametrize("path", ["auto-run", "rows", "tiled"])
def test_budget_variants(mode, path):
    """The allocation ablation's variants (uniform, strength only, skewness
    only) on every scoring path."""
    print(f"[parity] budget {mode} path {path}", flush=True)
    w = wl.custom(Nv=700, Nt=40, Hq=12, Hkv=4, D=128, dtype="bf16", L=6, B=2, ratio=0.2)
    inp = wl.make_inputs(w, 9)
    m = _BUDGET_MODES[mode]
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"), budget_mode=m)
    compare(inp, g, reference(inp, g, budget_mode=m))
    if mode == "uniform":
        assert (g["budget"] == int(0.2 * 700)).all()


@pytest.mark.parametrize("mode", list(_BUDGET_MODES))
def test_workload_3_budget_variants(mode):
    print(f"[parity] workload 3 budget {mode}", flush=True)
    inp = wl.make_inputs(3, 3)
    m = _BUDGET_MODES[mode]
    g = run_gpu(inp, max_elite=64, run=True, budget_mode=m)
    compare(inp, g, reference(inp, g, budget_mode=m))


@pytest.mark.parametrize("window", [16, 32, 40])
@pytest.mark.parametrize("path", ["auto-run", "rows", "tiled"])
def test_observation_windows(window, path):
    """The window ablation's contiguous windows (the last 16 or 32 text
    tokens, or all 40) in place of the elite window, on every scoring path."""
    print(f"[parity] window {window} path {path}", flush=True)
    w = wl.custom(Nv=700, Nt=40, Hq=12, Hkv=4, D=128, dtype="bf16", L=6, B=2, ratio=0.2)
    inp = wl.make_inputs(w, 10)
    g = run_gpu(inp, path=path.split("-")[0], run=path.endswith("-run"), obs_window=window)
    assert (g["n_elite"] == min(window, w.Nt)).all()
    compare(inp, g, reference(inp, g, obs_window=window))


def test_workload_3_window_16():
    print("[parity] workload 3 window 16", flush=True)
    inp = wl.make_inputs(3, 3)
    g = run_gpu(inp, max_elite=64, run=True, obs_window=16)
    compare(inp, g, reference(inp, g, obs_window=16))


@pytest.mark.parametrize("alpha,ratio", [(0.0, 0.1), (1.0, 0.1), (0.9, 0.0), (0.9, 1.0), (0.5, 0.5)])
def test_alpha_ratio_extremes(alpha, ratio):
    w = wl.custom(Nv=200, Nt=24, Hq=6, Hkv=2, D=128, dtype="bf16", L=3, B=2)
    inp = wl.make_inputs(w, 3)
    g = run_gpu(inp, alpha=alpha, ratio=ratio)
    compare(inp, g, reference(inp, g, alpha=alpha, ratio=ratio), ratio=ratio)
    if ratio == 0.0:
        assert (g["budget"] == 0).all()


def test_zero_queries_uniform():
    w = wl.custom(Nv=96, Nt=12, Hq=4, Hkv=2, D=64, dtype="bf16", L=2)
    inp = wl.make_inputs(w, 4, zero_q=True)
    g = run_gpu(inp)
    assert (g["n_elite"] == 12).all()
    assert np.all(g["iv"] == g["iv"][..., :1])
    assert (g["s_k"] == 0).all()
    compare(inp, g, reference(inp, g))


def test_identity_when_everything_is_kept():
    w = wl.custom(Nv=50, Nt=6, Hq=4, Hkv=2, D=128, dtype="bf16", L=1, B=2, ratio=1.0)
    inp = wl.make_inputs(w, 8)
    g = run_gpu(inp)
    assert (g["budget"] == 50).all()
    assert np.array_equal(g["k_out"][0], inp.k[0].ravel())
    assert np.array_equal(g["v_out"][0], inp.v[0].ravel())


def test_elite_overflow_is_flagged():
    w = wl.custom(Nv=64, Nt=8, Hq=2, Hkv=2, D=64, dtype="f32", L=1)
    inp = wl.make_inputs(w, 2, zero_q=True)   # uniform: all 8 text tokens are elite
    g = run_gpu(inp, max_elite=4, compress=False)
    assert g["status"][0] == 1


def test_deterministic_rerun():
    inp = wl.make_inputs(3, 3)
    from parity import to_torch
    t = to_torch(inp)
    a = run_gpu(inp, max_elite=64, tensors=t)
    b = run_gpu(inp, max_elite=64, tensors=t)
    for key in a:
        if isinstance(a[key], list):
            assert all(np.array_equal(x, y) for x, y in zip(a[key], b[key])), key
        else:
            assert np.array_equal(a[key], b[key]), key


def test_deterministic_rerun_one_launch():
    """aircache_run (the one launch the benchmark times) twice on workload 3
    with one workspace: bit-identical plans and compacted caches."""
    from parity import make_aircache, to_torch
    inp = wl.make_inputs(3, 3)
    t = to_torch(inp)
    ac = make_aircache(inp.w, max_elite=64)
    a = run_gpu(inp, tensors=t, ac=ac, run=True)
    b = run_gpu(inp, tensors=t, ac=ac, run=True)
    for key in a:
        if isinstance(a[key], list):
            assert all(np.array_equal(x, y) for x, y in zip(a[key], b[key])), key
        elif key in ("elite_idx", "kept_idx"):
            n = a["n_elite"] if key == "elite_idx" else a["budget"]
            for l in range(inp.w.L):
                for bb in range(inp.w.B):
                    assert np.array_equal(a[key][l, bb, :n[l, bb]], b[key][l, bb, :n[l, bb]]), key
        else:
            assert np.array_equal(a[key], b[key]), key


def _set_word(ac, index, value):
    """Set 32-bit word `index` of the pass's workspace (the one-launch path
    keeps its call count at word 0 and its condition flags at word 2)."""
    import struct
    ac.workspace[4 * index:4 * index + 4] = torch.tensor(np.frombuffer(struct.pack("<I", value & 0xFFFFFFFF),
                                                                       np.uint8).copy(), device=ac.workspace.device)


@pytest.mark.parametrize("start", [(1 << 21) - 1, 0xFFFFFFFF])
def test_epoch_wrap(start):
    """Call counts at the edges of the record tags: a call whose epoch is a
    multiple of 2^21 first zeroes every record and waits for the whole grid;
    the count wrapping past 2^32 skips epoch 0 (the tag of a zeroed record).
    Both that call and the next match the oracle."""
    from parity import make_aircache
    w = wl.custom(L=3, B=2, Hq=8, Hkv=2, D=128, Nv=500, Nt=30, dtype="bf16", ratio=0.2)
    ac = make_aircache(w)
    assert ac.scoring_path == "chunked"
    if start != 0xFFFFFFFF:
        inp = wl.make_inputs(w, 60)
        compare(inp, g := run_gpu(inp, ac=ac, run=True), reference(inp, g))
    torch.cuda.synchronize()
    _set_word(ac, 0, start)
    for seed in (61, 62):
        print(f"[parity] epoch wrap from {start:#x}, seed {seed}", flush=True)
        inp = wl.make_inputs(w, seed)
        g = run_gpu(inp, ac=ac, run=True)
        compare(inp, g, reference(inp, g))


def test_forced_timeout_is_flagged_then_cleared():
    """The bounded waits of the one-launch pass, forced from the host: with the
    workspace's flags word set to AIRCACHE_DEV_TIMEOUT before a call, every wait
    gives up after its first 256 polls; the kernel still ends, reports the bit
    in the status word and clears the flags, and the next call is exact."""
    from parity import make_aircache
    w = wl.custom(L=3, B=2, Hq=8, Hkv=2, D=128, Nv=500, Nt=30, dtype="bf16", ratio=0.2)
    ac = make_aircache(w)
    assert ac.scoring_path == "chunked"
    inp = wl.make_inputs(w, 70)
    g = run_gpu(inp, ac=ac, run=True)
    compare(inp, g, reference(inp, g))
    torch.cuda.synchronize()
    _set_word(ac, 2, 2)  # AIRCACHE_DEV_TIMEOUT
    print("[parity] forced timeout", flush=True)
    g = run_gpu(wl.make_inputs(w, 71), ac=ac, run=True)
    assert g["status"][0] & 2
    inp = wl.make_inputs(w, 72)
    g = run_gpu(inp, ac=ac, run=True)
    compare(inp, g, reference(inp, g))
