"""ctypes wrapper of the AirCache CPU oracle (aircache_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product library never imports this
package. The oracle is plain single-threaded C in double precision; see the
header comment of aircache_oracle.c for the page sections each step follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aircache_oracle.c")
_SO = os.path.join(_HERE, "_build", "liboracle.so")
_CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into oracle/_build/liboracle.so."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        os.makedirs(os.path.dirname(_SO), exist_ok=True)
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Desc(C.Structure):
    _fields_ = [("L", C.c_int), ("B", C.c_int), ("Hq", C.c_int), ("Hkv", C.c_int),
                ("D", C.c_int), ("Nv", C.c_int), ("Nt", C.c_int), ("dtype", C.c_int),
                ("alpha", C.c_double), ("ratio", C.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        # AIRCACHE_ORACLE_LIB: another build of the same source (the
        # sanitizer build of tests/test_host_sanitizers.py)
        l = C.CDLL(os.environ.get("AIRCACHE_ORACLE_LIB") or build())
        P = C.c_void_p
        l.orc_elite_select.argtypes = [C.POINTER(Desc), P, P, C.c_int, P, P]
        l.orc_elite_select.restype = C.c_int
        l.orc_cross_score.argtypes = [C.POINTER(Desc), P, P, C.c_int, P, C.c_int, P]
        l.orc_cross_score.restype = None
        l.orc_layer_stats.argtypes = [P, C.c_int, P, P]
        l.orc_layer_stats.restype = None
        l.orc_budget.argtypes = [P, P, C.c_int, C.c_double, C.c_int, C.c_int, P, P]
        l.orc_budget.restype = None
        l.orc_topk.argtypes = [P, C.c_int, C.c_int, P]
        l.orc_topk.restype = None
        l.orc_gather.argtypes = [C.POINTER(Desc), P, C.c_int, P, C.c_int, P]
        l.orc_gather.restype = None
        l.orc_cross_score_groups.argtypes = [C.POINTER(Desc), P, P, C.c_int, P, C.c_int, P]
        l.orc_cross_score_groups.restype = None
        l.orc_gather_groups.argtypes = [C.POINTER(Desc), P, C.c_int, P, C.c_int, C.c_int, P]
        l.orc_gather_groups.restype = None
        l.orc_quantize_i8.argtypes = [P, C.c_int, C.c_size_t, P, P]
        l.orc_quantize_i8.restype = None
        l.orc_decode_attention.argtypes = [C.POINTER(Desc), P, P, C.c_int, P, P]
        l.orc_decode_attention.restype = None
        l.orc_prefill_attention.argtypes = [C.POINTER(Desc), P, P, P, C.c_int, C.c_int, C.c_int, P]
        l.orc_prefill_attention.restype = None
        l.orc_decode_attention_i8.argtypes = [C.POINTER(Desc), P, P, P, P, C.c_int, P, P]
        l.orc_decode_attention_i8.restype = None
        l.orc_visual_window.argtypes = [C.POINTER(Desc), P, P, C.c_int, C.c_int, P, P]
        l.orc_visual_window.restype = None
        l.orc_run.argtypes = [C.POINTER(Desc)] + [P] * 15
        l.orc_run.restype = C.c_int
        _lib = l
    return _lib


def desc_of(w, alpha=None, ratio=None) -> Desc:
    return Desc(w.L, w.B, w.Hq, w.Hkv, w.D, w.Nv, w.Nt, 0 if w.dtype == "f32" else 1,
                float(w.alpha if alpha is None else alpha),
                float(w.ratio if ratio is None else ratio))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _check_inputs(w, q, k):
    store = np.float32 if w.dtype == "f32" else np.uint16
    assert q.dtype == store and k.dtype == store
    assert q.shape[-3:] == (w.Hq, w.Nt, w.D), q.shape
    assert k.shape[-3:] == (w.Hkv, w.Nv + w.Nt, w.D), k.shape


# ---- single steps (one layer, one sample) -----------------------------------

def elite_select(w, q_l: np.ndarray, k_l: np.ndarray, b: int, alpha=None):
    """Step 1 on layer arrays q_l [B][Hq][Nt][D], k_l [B][Hkv][S][D].
    Returns (elite indices ascending, pbar[N_t])."""
    _check_inputs(w, q_l, k_l)
    d = desc_of(w, alpha=alpha)
    pbar = np.zeros(w.Nt, np.float64)
    el = np.zeros(w.Nt, np.int32)
    n = lib().orc_elite_select(C.byref(d), _ptr(q_l), _ptr(k_l), b, _ptr(pbar), _ptr(el))
    return el[:n].copy(), pbar


def window_select(Nt: int, k: int) -> np.ndarray:
    """Step 1 with a contiguous observation window instead of the elite one
    (the window ablation of "Elite Observation Window": the last 16 or 32 text
    tokens, or all of them): the last min(k, N_t) text tokens, ascending."""
    k = min(int(k), int(Nt))
    return np.arange(Nt - k, Nt, dtype=np.int32)


def cross_score(w, q_l, k_l, b: int, elite) -> np.ndarray:
    """Step 2: I_v[N_v] (float64) for the given elite set."""
    _check_inputs(w, q_l, k_l)
    d = desc_of(w)
    el = np.ascontiguousarray(elite, dtype=np.int32)
    iv = np.zeros(w.Nv, np.float64)
    lib().orc_cross_score(C.byref(d), _ptr(q_l), _ptr(k_l), b, _ptr(el), len(el), _ptr(iv))
    return iv


def cross_score_groups(w, q_l, k_l, b: int, elite) -> np.ndarray:
    """Step 2 per KV head (group-wise selection): I_v^g as [H_kv][N_v] float64."""
    _check_inputs(w, q_l, k_l)
    d = desc_of(w)
    el = np.ascontiguousarray(elite, dtype=np.int32)
    iv = np.zeros((w.Hkv, w.Nv), np.float64)
    lib().orc_cross_score_groups(C.byref(d), _ptr(q_l), _ptr(k_l), b, _ptr(el), len(el), _ptr(iv))
    return iv


def layer_stats(iv) -> tuple[float, float]:
    """Step 3: (s_t, s_k) of one I_v vector."""
    a = np.ascontiguousarray(iv, dtype=np.float64)
    st, sk = C.c_double(), C.c_double()
    lib().orc_layer_stats(_ptr(a), len(a), C.addressof(st), C.addressof(sk))
    return st.value, sk.value


def budget(s_t, s_k, ratio: float, Nv: int, mode: int = 0):
    """Step 4 for one sample: (x[L], budget[L]). mode: 0 the page's rule
    (strength and skewness), 1 uniform, 2 strength only, 3 skewness only (the
    allocation ablation's variants, see orc_budget)."""
    st = np.ascontiguousarray(s_t, dtype=np.float64)
    sk = np.ascontiguousarray(s_k, dtype=np.float64)
    L = len(st)
    x = np.zeros(L, np.float64)
    r = np.zeros(L, np.int32)
    lib().orc_budget(_ptr(st), _ptr(sk), L, float(ratio), int(Nv), int(mode), _ptr(x), _ptr(r))
    return x, r


def topk(iv, k: int) -> np.ndarray:
    """Step 5: indices of the k largest scores (ties to lower index), ascending."""
    a = np.ascontiguousarray(iv, dtype=np.float64)
    out = np.zeros(max(len(a), 1), np.int32)
    lib().orc_topk(_ptr(a), len(a), int(k), _ptr(out))
    return out[:k].copy()


def gather(w, src_l: np.ndarray, b: int, kept) -> np.ndarray:
    """Step 6 for one sample of one layer: [H_kv][k + N_t][D] array."""
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    d = desc_of(w)
    out = np.zeros((w.Hkv, len(kept) + w.Nt, w.D), dtype=src_l.dtype)
    lib().orc_gather(C.byref(d), _ptr(src_l), b, _ptr(kept), len(kept), _ptr(out))
    return out


def gather_groups(w, src_l: np.ndarray, b: int, kept_g) -> np.ndarray:
    """Step 6 with per-KV-head kept lists kept_g [H_kv][k]: [H_kv][k + N_t][D]."""
    kept_g = np.ascontiguousarray(kept_g, dtype=np.int32).reshape(w.Hkv, -1)
    k = kept_g.shape[1]
    d = desc_of(w)
    out = np.zeros((w.Hkv, k + w.Nt, w.D), dtype=src_l.dtype)
    lib().orc_gather_groups(C.byref(d), _ptr(src_l), b, _ptr(kept_g), max(k, 0), k, _ptr(out))
    return out


def quantize_i8(seg, dtype: str):
    """int8 quantisation of one head's kept cache: (codes int8[n], scale).
    seg holds float32 values (dtype "f32") or bfloat16 bit patterns ("bf16")."""
    a = np.ascontiguousarray(seg)
    codes = np.zeros(max(a.size, 1), np.int8)
    sc = C.c_float()
    lib().orc_quantize_i8(_ptr(a), 0 if dtype == "f32" else 1, a.size, _ptr(codes), C.addressof(sc))
    return codes[:a.size].reshape(a.shape), sc.value


def decode_attention_segment(w, k_seg, v_seg, n: int, q) -> np.ndarray:
    """Decode attention over one (layer, sample) segment [H_kv][n][D] of the
    compacted cache for the new queries q [H_q][D]: o [H_q][D] (float64)."""
    store = np.float32 if w.dtype == "f32" else np.uint16
    k_seg = np.ascontiguousarray(k_seg, dtype=store).ravel()
    v_seg = np.ascontiguousarray(v_seg, dtype=store).ravel()
    q = np.ascontiguousarray(q, dtype=store)
    assert k_seg.size == v_seg.size == w.Hkv * n * w.D and q.shape == (w.Hq, w.D)
    o = np.zeros((w.Hq, w.D), np.float64)
    lib().orc_decode_attention(C.byref(desc_of(w)), _ptr(k_seg), _ptr(v_seg), int(n), _ptr(q), _ptr(o))
    return o


def decode_attention_i8_segment(w, kq_seg, vq_seg, k_scale, v_scale, n: int, q) -> np.ndarray:
    """Decode attention over one (layer, sample) segment [H_kv][n][D] of the
    int8 cache (value = code * the KV head's scale): o [H_q][D] (float64)."""
    store = np.float32 if w.dtype == "f32" else np.uint16
    kq_seg = np.ascontiguousarray(kq_seg, dtype=np.int8).ravel()
    vq_seg = np.ascontiguousarray(vq_seg, dtype=np.int8).ravel()
    ks = np.ascontiguousarray(k_scale, dtype=np.float32).ravel()
    vs = np.ascontiguousarray(v_scale, dtype=np.float32).ravel()
    q = np.ascontiguousarray(q, dtype=store)
    assert kq_seg.size == vq_seg.size == w.Hkv * n * w.D and ks.size == vs.size == w.Hkv
    assert q.shape == (w.Hq, w.D)
    o = np.zeros((w.Hq, w.D), np.float64)
    lib().orc_decode_attention_i8(C.byref(desc_of(w)), _ptr(kq_seg), _ptr(vq_seg), _ptr(ks), _ptr(vs), int(n),
                                  _ptr(q), _ptr(o))
    return o


def decode_attention(w, k_out_l, v_out_l, out_off_l, budget_l, q_l) -> np.ndarray:
    """Decode attention over layer l's compacted cache (k_out_l / v_out_l flat,
    out_off_l [B+1], budget_l [B]) for the new queries q_l [B][H_q][D]:
    o [B][H_q][D] (float64)."""
    o = np.zeros((w.B, w.Hq, w.D), np.float64)
    for b in range(w.B):
        n = int(budget_l[b]) + w.Nt
        off = int(out_off_l[b])
        size = w.Hkv * n * w.D
        o[b] = decode_attention_segment(w, k_out_l[off:off + size], v_out_l[off:off + size], n, q_l[b])
    return o


def visual_window(w, q_all_l, k_l, b: int, kwin: int, groups: bool = False):
    """I_v of the window ablation's visual window (the last kwin visual
    tokens as the observation rows, softmax over the N_v visual keys):
    q_all_l [B][H_q][S][D] (every position's query), k_l [B][H_kv][S][D].
    Returns iv [N_v], or (iv, iv per KV head [H_kv][N_v]) with groups."""
    store = np.float32 if w.dtype == "f32" else np.uint16
    q_all_l = np.ascontiguousarray(q_all_l, dtype=store)
    k_l = np.ascontiguousarray(k_l, dtype=store)
    assert q_all_l.shape[-3:] == (w.Hq, w.Nv + w.Nt, w.D) and 1 <= kwin <= w.Nv
    iv = np.zeros(w.Nv, np.float64)
    ivg = np.zeros((w.Hkv, w.Nv), np.float64) if groups else None
    lib().orc_visual_window(C.byref(desc_of(w)), _ptr(q_all_l), _ptr(k_l), int(b), int(kwin), _ptr(iv),
                            _ptr(ivg) if groups else None)
    return (iv, ivg) if groups else iv


def prefill_attention(w, q_all_l, k_l, v_l, b: int, row0: int = 0, nrows=None) -> np.ndarray:
    """Causal prefill attention of one layer and sample: q_all_l [B][H_q][S][D]
    (every position's query), k_l / v_l [B][H_kv][S][D]; rows row0 ..
    row0 + nrows - 1 of every query head: o [H_q][nrows][D] (float64)."""
    store = np.float32 if w.dtype == "f32" else np.uint16
    S = w.Nv + w.Nt
    if nrows is None:
        nrows = S - row0
    assert 0 <= row0 and row0 + nrows <= S
    q_all_l = np.ascontiguousarray(q_all_l, dtype=store)
    k_l = np.ascontiguousarray(k_l, dtype=store)
    v_l = np.ascontiguousarray(v_l, dtype=store)
    assert q_all_l.shape[-3:] == (w.Hq, S, w.D), q_all_l.shape
    assert k_l.shape[-3:] == (w.Hkv, S, w.D) and v_l.shape == k_l.shape
    o = np.zeros((w.Hq, nrows, w.D), np.float64)
    lib().orc_prefill_attention(C.byref(desc_of(w)), _ptr(q_all_l), _ptr(k_l), _ptr(v_l), int(b), int(row0),
                                int(nrows), _ptr(o))
    return o


# ---- the whole pass ---------------------------------------------------------

def run(inp, alpha=None, ratio=None, compact=True, threads: int = 1) -> dict:
    """Run the pass on workloads.Inputs. threads > 1 runs independent
    (layer, sample) step calls concurrently (each call is still the plain
    single-threaded C code); threads = 1 is a single call of orc_run."""
    w = inp.w
    L, B = w.L, w.B
    d = desc_of(w, alpha=alpha, ratio=ratio)
    elite = np.zeros((L, B, w.Nt), np.int32)
    n_elite = np.zeros((L, B), np.int32)
    pbar = np.zeros((L, B, w.Nt), np.float64)
    iv = np.zeros((L, B, w.Nv), np.float64)
    s_t = np.zeros((L, B), np.float64)
    s_k = np.zeros((L, B), np.float64)
    x = np.zeros((L, B), np.float64)
    bud = np.zeros((L, B), np.int32)
    off = np.zeros((L, B + 1), np.int64)
    kept = np.zeros((L, B, w.Nv), np.int32)
    out = dict(elite=elite, n_elite=n_elite, pbar=pbar, iv=iv, s_t=s_t, s_k=s_k, x=x,
               budget=bud, out_off=off, kept=kept)
    if threads <= 1:
        qp = (C.c_void_p * L)(*[_ptr(inp.q[l]) for l in range(L)])
        kp = (C.c_void_p * L)(*[_ptr(inp.k[l]) for l in range(L)])
        vp = (C.c_void_p * L)(*[_ptr(inp.v[l]) for l in range(L)])
        cap = w.B * w.Hkv * (w.Nv + w.Nt) * w.D
        if compact:
            kout = [np.zeros(cap, inp.k.dtype) for _ in range(L)]
            vout = [np.zeros(cap, inp.v.dtype) for _ in range(L)]
            kop = (C.c_void_p * L)(*[_ptr(a) for a in kout])
            vop = (C.c_void_p * L)(*[_ptr(a) for a in vout])
        else:
            kop = vop = None
        rc = lib().orc_run(C.byref(d), qp, kp, vp, _ptr(elite), _ptr(n_elite), _ptr(pbar),
                           _ptr(iv), _ptr(s_t), _ptr(s_k), _ptr(x), _ptr(bud), _ptr(off),
                           _ptr(kept), kop, vop)
        if rc != 0:
            raise ValueError("oracle rejected the descriptor")
        if compact:
            out["k_out"] = [kout[l][:off[l, B]] for l in range(L)]
            out["v_out"] = [vout[l][:off[l, B]] for l in range(L)]
        return out

    def score(lb):
        l, b = lb
        el, pb = elite_select(w, inp.q[l], inp.k[l], b, alpha=d.alpha)
        elite[l, b, :len(el)] = el
        n_elite[l, b] = len(el)
        pbar[l, b] = pb
        iv[l, b] = cross_score(w, inp.q[l], inp.k[l], b, el)
        s_t[l, b], s_k[l, b] = layer_stats(iv[l, b])

    pairs = [(l, b) for l in range(L) for b in range(B)]
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(score, pairs))
    for b in range(B):
        x[:, b], bud[:, b] = budget(s_t[:, b], s_k[:, b], d.ratio, w.Nv)

    def select(lb):
        l, b = lb
        kept[l, b, :bud[l, b]] = topk(iv[l, b], int(bud[l, b]))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(select, pairs))
    for l in range(L):
        acc = 0
        for b in range(B):
            off[l, b] = acc
            acc += w.Hkv * (int(bud[l, b]) + w.Nt) * w.D
        off[l, B] = acc
    if compact:
        out["k_out"], out["v_out"] = [], []
        for l in range(L):
            out["k_out"].append(np.concatenate(
                [gather(w, inp.k[l], b, kept[l, b, :bud[l, b]]).ravel() for b in range(B)]))
            out["v_out"].append(np.concatenate(
                [gather(w, inp.v[l], b, kept[l, b, :bud[l, b]]).ravel() for b in range(B)]))
    return out
