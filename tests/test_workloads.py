"""The seeded input generator: determinism, shapes and the bf16 rounding."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, 3.0e38], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.f32_to_bf16_bits(x), ref)
    back = wl.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_determinism_and_shapes():
    w = wl.custom(L=2, B=2, Hq=4, Hkv=2, D=16, Nv=20, Nt=5, dtype="bf16")
    a = wl.make_inputs(w, 4)
    b = wl.make_inputs(w, 4)
    c = wl.make_inputs(w, 5)
    assert a.q.shape == (2, 2, 4, 5, 16) and a.k.shape == (2, 2, 2, 25, 16)
    assert a.q.dtype == np.uint16
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.k, c.k)


def test_planted_keys_point_at_a_text_query():
    w = wl.CONFIGS[1]
    inp = wl.make_inputs(w, 1)
    for l in range(w.L):
        pos = inp.planted[0][l]
        assert len(pos) == 8
        kp = inp.k[l, 0, :, pos, :]                 # [Hkv][8][D]
        assert np.allclose(np.linalg.norm(kp, axis=-1), 3.0, rtol=1e-5)


def test_video_keys_are_correlated_across_frames():
    w = wl.Workload(**{**wl.CONFIGS[4].__dict__, "L": 1, "B": 1, "Hq": 7, "Hkv": 1, "cid": 0})
    inp = wl.make_inputs(w, 3)
    kv = wl.bf16_bits_to_f32(inp.k[0, 0, 0, :w.Nv]).reshape(32, 196, w.D)
    clean = np.ones(w.Nv, bool)
    clean[inp.planted[0][0]] = False                # planted keys are replaced
    clean = clean.reshape(32, 196)
    both = clean[1:] & clean[:-1]
    a, b = kv[1:][both].ravel(), kv[:-1][both].ravel()
    corr = np.corrcoef(a, b)[0, 1]
    assert 0.87 < corr < 0.93                       # AR(1) coefficient 0.9


def test_config_table():
    assert [wl.CONFIGS[i].Nv for i in range(1, 6)] == [64, 576, 2880, 6272, 3072]
    assert [wl.CONFIGS[i].ratio for i in range(1, 6)] == [0.25, 0.10, 0.10, 0.01, 0.10]
    assert wl.CONFIGS[1].dtype == "f32" and all(wl.CONFIGS[i].dtype == "bf16" for i in range(2, 6))
