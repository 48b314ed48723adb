"""Seeded synthetic inputs for the AirCache compression pass.

This module only draws inputs. It holds none of the method's arithmetic (no
softmax, no elite selection, no scoring, no budgets): both the HIP path and the
CPU oracle consume what it produces, and neither is imported here.

Shapes follow the per-layer cache layout of the multimodal KV-compression
pages: each layer's cache is [batch][heads][seq][head_dim], with the sequence
regrouped as visual tokens first and text tokens after them (AirCache notes,
"Elite Observation Window", the regrouping X = Concat(X_v, X_t)).

Per layer l the generator produces
  q_txt[l] : [B][H_q][N_t][D]         text queries (post-RoPE, as stored)
  k[l]     : [B][H_kv][N_v + N_t][D]  keys, visual rows first
  v[l]     : [B][H_kv][N_v + N_t][D]  values, same layout
as float32 (the tiny config) or bfloat16 bit patterns (uint16, round to
nearest even from float32 draws).

Draw order is fixed: for each sample b, for each layer l: Q_txt, K, V, then the
salience draws of that (l, b). The five workloads are described in CONFIGS.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    L: int
    B: int
    Hq: int
    Hkv: int
    D: int
    Nv: int
    Nt: int
    dtype: str
    ratio: float
    alpha: float = 0.9
    # generator knobs
    base: str = "unit"            # "unit": N(0,1); "inv_sqrt_d": N(0,1)/sqrt(D)
    salience: str = "direction"   # "direction" | "mean_query"
    sal_frac: float = 0.125       # fraction of visual keys planted per layer
    sal_frac_range: tuple | None = None   # per-sample U[lo, hi] fraction
    frames: int = 0               # >0: AR(1) over frames for visual K
    ar_rho: float = 0.9
    ar_sigma: float = 0.44

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def S(self) -> int:
        return self.Nv + self.Nt

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def describe(self) -> dict:
        return {"workload": self.name, "layers": self.L, "batch": self.B,
                "q_heads": self.Hq, "kv_heads": self.Hkv, "head_dim": self.D,
                "n_vis": self.Nv, "n_txt": self.Nt, "dtype": self.dtype,
                "ratio": self.ratio, "alpha": self.alpha}


CONFIGS: dict[int, Workload] = {
    1: Workload(1, "tiny_mha_fp32", L=2, B=1, Hq=2, Hkv=2, D=64, Nv=64, Nt=16,
                dtype=F32, ratio=0.25, sal_frac=8 / 64),
    2: Workload(2, "mha7b_single_image", L=32, B=1, Hq=32, Hkv=32, D=128,
                Nv=576, Nt=64, dtype=BF16, ratio=0.10, base="inv_sqrt_d",
                salience="mean_query", sal_frac=0.10),
    3: Workload(3, "gqa_tiled_image_2880", L=28, B=1, Hq=28, Hkv=4, D=128,
                Nv=2880, Nt=128, dtype=BF16, ratio=0.10),
    4: Workload(4, "gqa_video_32x196", L=28, B=4, Hq=28, Hkv=4, D=128,
                Nv=32 * 196, Nt=256, dtype=BF16, ratio=0.01, frames=32),
    5: Workload(5, "gqa_multi_image_3x1024", L=28, B=8, Hq=28, Hkv=4, D=128,
                Nv=3 * 1024, Nt=1024, dtype=BF16, ratio=0.10,
                sal_frac_range=(0.05, 0.20)),
}


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit sizes (tests of ragged and edge shapes)."""
    base = dict(cid=0, name=name, L=1, B=1, Hq=1, Hkv=1, D=64, Nv=16, Nt=4,
                dtype=F32, ratio=0.25)
    base.update(kw)
    return Workload(**base)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt((x.astype(np.float64) ** 2).sum(-1, keepdims=True))
    n[n == 0] = 1.0
    return (x / n).astype(np.float32)


@dataclasses.dataclass
class Inputs:
    w: Workload
    seed: int
    q: np.ndarray   # [L][B][Hq][Nt][D]  float32 or uint16 (bf16 bits)
    k: np.ndarray   # [L][B][Hkv][S][D]
    v: np.ndarray   # [L][B][Hkv][S][D]
    planted: list   # planted[b][l] = visual indices that got salience

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return a if self.w.dtype == F32 else bf16_bits_to_f32(a)


def make_inputs(w: Workload | int, seed: int, *, zero_q: bool = False) -> Inputs:
    """Draw one seeded batch of inputs for workload ``w``.

    zero_q=True replaces every text query by zeros after drawing (a degenerate
    case: all attention rows become uniform).
    """
    if isinstance(w, int):
        w = CONFIGS[w]
    rng = np.random.Generator(np.random.PCG64(seed))
    store = np.float32 if w.dtype == F32 else np.uint16
    q = np.empty((w.L, w.B, w.Hq, w.Nt, w.D), dtype=store)
    k = np.empty((w.L, w.B, w.Hkv, w.S, w.D), dtype=store)
    v = np.empty((w.L, w.B, w.Hkv, w.S, w.D), dtype=store)
    scale = 1.0 if w.base == "unit" else 1.0 / math.sqrt(w.D)
    G = w.G
    planted = []
    for b in range(w.B):
        frac = w.sal_frac
        if w.sal_frac_range is not None:
            frac = float(rng.uniform(*w.sal_frac_range))
        n_sal = int(round(frac * w.Nv))
        pl_b = []
        for l in range(w.L):
            ql = rng.standard_normal((w.Hq, w.Nt, w.D), dtype=np.float32)
            kl = rng.standard_normal((w.Hkv, w.S, w.D), dtype=np.float32)
            vl = rng.standard_normal((w.Hkv, w.S, w.D), dtype=np.float32)
            if scale != 1.0:
                ql *= scale
                kl *= scale
                vl *= scale
            if w.frames:
                # visual keys: frames x spatial positions, AR(1) along frames
                P = w.Nv // w.frames
                kv = kl[:, :w.Nv, :].reshape(w.Hkv, w.frames, P, w.D)
                for f in range(1, w.frames):
                    kv[:, f] = w.ar_rho * kv[:, f - 1] + w.ar_sigma * kv[:, f]
                kl[:, :w.Nv, :] = kv.reshape(w.Hkv, w.Nv, w.D)
            pos = np.sort(rng.choice(w.Nv, size=n_sal, replace=False)) if n_sal else np.zeros(0, np.int64)
            if w.salience == "direction":
                # key set to 3x the unit direction of a random text query of
                # the first query head served by that KV head
                js = rng.integers(0, w.Nt, size=n_sal)
                for g in range(w.Hkv):
                    qd = _unit_rows(ql[g * G, js, :])
                    kl[g, pos, :] = 3.0 * qd
            elif w.salience == "mean_query":
                # component toward the mean text query of the KV head's query
                # heads; per-layer scale s_l, per-key weight u_i
                s_l = float(rng.uniform(0.5, 4.0))
                u = rng.uniform(0.0, 1.0, size=n_sal).astype(np.float64)
                for g in range(w.Hkv):
                    qbar = ql[g * G:(g + 1) * G].astype(np.float64).reshape(-1, w.D).mean(0)
                    nrm2 = float((qbar ** 2).sum())
                    add = (s_l * u[:, None] * math.sqrt(w.D) / nrm2) * qbar[None, :]
                    kl[g, pos, :] = (kl[g, pos, :].astype(np.float64) + add).astype(np.float32)
            else:
                raise ValueError(w.salience)
            if zero_q:
                ql[...] = 0.0
            if w.dtype == F32:
                q[l, b], k[l, b], v[l, b] = ql, kl, vl
            else:
                q[l, b] = f32_to_bf16_bits(ql)
                k[l, b] = f32_to_bf16_bits(kl)
                v[l, b] = f32_to_bf16_bits(vl)
            pl_b.append(pos)
        planted.append(pl_b)
    return Inputs(w=w, seed=seed, q=q, k=k, v=v, planted=planted)


def visual_queries(w: Workload, seed: int, layer: int) -> np.ndarray:
    """The queries of the visual positions of one layer, [B][Hq][Nv][D], for
    the prefill attention (whose query rows are every position's): drawn like
    the text queries (N(0, 1), times 1/sqrt(D) on the scaled base), from a
    generator of their own keyed by (seed, layer), so that the text queries of
    make_inputs are unchanged. Float32 or bfloat16 bits."""
    rng = np.random.Generator(np.random.PCG64([seed, 7919, layer]))
    x = rng.standard_normal((w.B, w.Hq, w.Nv, w.D), dtype=np.float32)
    if w.base != "unit":
        x *= 1.0 / math.sqrt(w.D)
    return x if w.dtype == F32 else f32_to_bf16_bits(x)


def prefill_queries(inp: Inputs, layer: int) -> np.ndarray:
    """Every position's query of one layer, [B][Hq][Nv + Nt][D]: the visual
    rows of visual_queries, then the text queries of make_inputs."""
    return np.ascontiguousarray(np.concatenate([visual_queries(inp.w, inp.seed, layer), inp.q[layer]], axis=2))


def parity_seeds(cid: int) -> list[int]:
    return [cid, 100 + cid, 200 + cid]
