"""PyTorch-facing wrapper of the AirCache C ABI (argument marshalling only).

PyTorch provides device memory and the stream; every step of the pass runs in
the HIP kernels of libaircache.so. Shapes, dtypes, devices and contiguity are
checked here, because the C ABI only sees raw pointers.
"""
from __future__ import annotations

import dataclasses

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.AIRCACHE_F32, torch.bfloat16: _lib.AIRCACHE_BF16}


_PATHS = {"auto": _lib.PATH_AUTO, "tiled": _lib.PATH_TILED, "rows": _lib.PATH_ROWS, "chunked": _lib.PATH_CHUNKED,
          "small": _lib.PATH_SMALL}
# layer budget rules: the method's, then its allocation ablation's variants
_BUDGETS = {"aircache": 0, "uniform": 1, "strength": 2, "skewness": 3, "pyramid": 4}
# visual-token selection: one per (layer, sample), the method's, or one per KV head
_SELECT = {"shared": _lib.SELECT_SHARED, "per_kv_head": _lib.SELECT_PER_KV_HEAD}


def make_desc(n_layers, batch, n_q_heads, n_kv_heads, head_dim, n_vis, n_txt, dtype,
              alpha=0.9, ratio=0.1, max_elite=0, path="auto", budget_mode=0, obs_window=0,
              select="shared") -> _lib.Desc:
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPES[dtype]
    elif isinstance(dtype, str):
        dtype = {"f32": _lib.AIRCACHE_F32, "bf16": _lib.AIRCACHE_BF16}[dtype]
    return _lib.Desc(n_layers, batch, n_q_heads, n_kv_heads, head_dim, n_vis, n_txt, dtype,
                     float(alpha), float(ratio), int(max_elite), _PATHS[path] if isinstance(path, str) else int(path),
                     _BUDGETS[budget_mode] if isinstance(budget_mode, str) else int(budget_mode), int(obs_window),
                     _SELECT[select] if isinstance(select, str) else int(select))


@dataclasses.dataclass
class PlanOutputs:
    elite_idx: torch.Tensor  # int32 [L, B, N_t]
    n_elite: torch.Tensor    # int32 [L, B]
    iv: torch.Tensor         # float32 [L, B, N_v]
    s_t: torch.Tensor        # float64 [L, B]
    s_k: torch.Tensor        # float64 [L, B]
    budget_x: torch.Tensor   # float64 [L, B]
    budget: torch.Tensor     # int32 [L, B]
    out_off: torch.Tensor    # int64 [L, B + 1]
    kept_idx: torch.Tensor   # int32 [L, B, N_v], or [L, B, H_kv, N_v] with one selection per KV head
    status: torch.Tensor     # int32 [1]
    iv_head: torch.Tensor | None = None  # float32 [L, B, H_kv, N_v] with one selection per KV head

    @classmethod
    def empty(cls, L, B, Nv, Nt, device, per_kv_head: int = 0) -> "PlanOutputs":
        """per_kv_head: H_kv for one selection per KV head, else 0."""
        i32 = dict(dtype=torch.int32, device=device)
        f64 = dict(dtype=torch.float64, device=device)
        sel = (per_kv_head,) if per_kv_head else ()
        return cls(elite_idx=torch.empty(L, B, Nt, **i32), n_elite=torch.empty(L, B, **i32),
                   iv=torch.empty(L, B, Nv, dtype=torch.float32, device=device),
                   s_t=torch.empty(L, B, **f64), s_k=torch.empty(L, B, **f64),
                   budget_x=torch.empty(L, B, **f64), budget=torch.empty(L, B, **i32),
                   out_off=torch.empty(L, B + 1, dtype=torch.int64, device=device),
                   kept_idx=torch.empty(L, B, *sel, Nv, **i32), status=torch.zeros(1, **i32),
                   iv_head=torch.empty(L, B, per_kv_head, Nv, dtype=torch.float32, device=device)
                   if per_kv_head else None)

    def buf(self) -> _lib.PlanBuf:
        ptr = lambda t: 0 if t is None else t.data_ptr()
        return _lib.PlanBuf(*[ptr(getattr(self, f.name)) for f in dataclasses.fields(self)])


class AirCache:
    """One compression pass configuration with its workspace.

    plan(q_txt, k) scores, budgets and selects; compress(...) writes the
    compacted per-layer K/V; run(...) does both (one launch where the chunked
    path serves the shape). All run on the current stream of the device and
    return without synchronising.

    alpha: the elite threshold; ratio: r / N_v; max_elite: workspace cap on
    elite tokens (0: N_t); path: "auto", "small", "chunked", "rows" or "tiled";
    budget_mode: "aircache" (the method's layer allocation) or one of its
    allocation ablation's variants, "uniform", "strength", "skewness",
    "pyramid";
    obs_window: 0 for the elite observation window, k > 0 for the last k
    text tokens instead (the window ablation's contiguous windows), -k for
    the last k visual tokens (its visual window; q_txt then holds every
    position's queries, [B][H_q][N_v + N_t][D] per layer);
    select: "shared" (one selection per layer and sample, the method's) or
    "per_kv_head" (each KV head its own top-r_hat, the group-wise top-K).
    """

    def __init__(self, n_layers, batch, n_q_heads, n_kv_heads, head_dim, n_vis, n_txt,
                 dtype=torch.bfloat16, alpha=0.9, ratio=0.1, max_elite=0, device="cuda", path="auto",
                 budget_mode="aircache", obs_window=0, select="shared"):
        self.shape = dict(L=n_layers, B=batch, Hq=n_q_heads, Hkv=n_kv_heads, D=head_dim,
                          Nv=n_vis, Nt=n_txt)
        self.dtype = dtype
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.desc = make_desc(n_layers, batch, n_q_heads, n_kv_heads, head_dim, n_vis, n_txt,
                              dtype, alpha, ratio, max_elite, path, budget_mode, obs_window, select)
        self.per_kv_head = self.desc.select_mode == _lib.SELECT_PER_KV_HEAD
        ws = _lib.workspace_size(self.desc)
        if ws == 0:
            _lib.check(_lib.AIRCACHE_EINVAL)
        self.ws_bytes = ws
        # zero-filled once; the library keeps it valid from call to call
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=self.device)

    @property
    def q_rows(self) -> int:
        """Rows per query head of the query tables: N_t (text queries), or
        N_v + N_t (every position's) with a visual observation window."""
        s = self.shape
        return s["Nv"] + s["Nt"] if self.desc.obs_window < 0 else s["Nt"]

    @property
    def scoring_path(self) -> str:
        """"tiled", "rows", "chunked" or "small": the scoring path the plan call takes."""
        return {_lib.PATH_TILED: "tiled", _lib.PATH_ROWS: "rows",
                _lib.PATH_CHUNKED: "chunked", _lib.PATH_SMALL: "small"}[_lib.resolved_path(self.desc)]

    @property
    def run_launches(self) -> int:
        """Kernel launches of run(): 1 when the chunked path compacts inside
        its launch."""
        return _lib.run_launches(self.desc)

    # -- validation ------------------------------------------------------
    def _check_layers(self, ts, shape, name):
        s = self.shape
        if len(ts) != s["L"]:
            raise ValueError(f"{name}: {len(ts)} layers given, {s['L']} expected")
        for l, t in enumerate(ts):
            if t.device != self.device or t.dtype != self.dtype:
                raise ValueError(f"{name}[{l}]: {t.dtype} on {t.device}, expected {self.dtype} on {self.device}")
            if tuple(t.shape) != shape:
                raise ValueError(f"{name}[{l}]: shape {tuple(t.shape)}, expected {shape}")
            if not t.is_contiguous():
                raise ValueError(f"{name}[{l}] is not contiguous")

    def _check_outputs(self, k_out, v_out):
        s = self.shape
        cap = _lib.max_compacted_elems(self.desc)
        for name, outs in (("k_out", k_out), ("v_out", v_out)):
            if len(outs) != s["L"]:
                raise ValueError(f"{name}: {len(outs)} layers given")
            for l, t in enumerate(outs):
                if t.device != self.device or t.dtype != self.dtype or not t.is_contiguous() or t.numel() < cap:
                    raise ValueError(f"{name}[{l}] must be a contiguous {self.dtype} tensor on "
                                     f"{self.device} with at least {cap} elements")

    def _stream(self, stream):
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)

    # -- calls -------------------------------------------------------------
    def alloc_plan(self) -> PlanOutputs:
        s = self.shape
        return PlanOutputs.empty(s["L"], s["B"], s["Nv"], s["Nt"], self.device,
                                 s["Hkv"] if self.per_kv_head else 0)

    def plan(self, q_txt, k, out: PlanOutputs | None = None, stream=None, events=None) -> PlanOutputs:
        """events: optional list of 5 torch.cuda.Event (timing=True) recorded
        around the plan's 4 kernels."""
        s = self.shape
        self._check_layers(q_txt, (s["B"], s["Hq"], self.q_rows, s["D"]), "q_txt")
        self._check_layers(k, (s["B"], s["Hkv"], s["Nv"] + s["Nt"], s["D"]), "k")
        out = out or self.alloc_plan()
        _lib.check(_lib.plan(self.desc, [t.data_ptr() for t in q_txt], [t.data_ptr() for t in k],
                             out.buf(), self.workspace.data_ptr(), self.ws_bytes, self._stream(stream),
                             events=None if events is None else [e.cuda_event for e in events]))
        return out

    def run(self, q_txt, k, v, plan: PlanOutputs, k_out, v_out, stream=None, events=None) -> PlanOutputs:
        """plan + compress in one call (one launch where the chunked path
        serves the shape); events: optional list of 2 torch.cuda.Event
        recorded around the whole pass."""
        s = self.shape
        self._check_layers(q_txt, (s["B"], s["Hq"], self.q_rows, s["D"]), "q_txt")
        shp = (s["B"], s["Hkv"], s["Nv"] + s["Nt"], s["D"])
        self._check_layers(k, shp, "k")
        self._check_layers(v, shp, "v")
        self._check_outputs(k_out, v_out)
        _lib.check(_lib.run(self.desc, [t.data_ptr() for t in q_txt], [t.data_ptr() for t in k],
                            [t.data_ptr() for t in v], plan.buf(), [t.data_ptr() for t in k_out],
                            [t.data_ptr() for t in v_out], self.workspace.data_ptr(), self.ws_bytes,
                            self._stream(stream),
                            events=None if events is None else [e.cuda_event for e in events]))
        return plan

    def bind(self, q_txt, k, v, plan: PlanOutputs, k_out, v_out, stream=None) -> "BoundPass":
        """A BoundPass running plan + compress on these tensors with the
        argument checks and marshalling done once, here."""
        return BoundPass(self, q_txt, k, v, plan, k_out, v_out, stream)

    def alloc_compacted(self):
        """Worst-case (every visual row kept) per-layer output buffers for K and V."""
        n = _lib.max_compacted_elems(self.desc)
        L = self.shape["L"]
        mk = lambda: [torch.empty(n, dtype=self.dtype, device=self.device) for _ in range(L)]
        return mk(), mk()

    def decode(self, q_dec, plan: PlanOutputs, k_out, v_out, o=None, stream=None):
        """Decode attention over the compacted cache (aircache_decode): for
        every layer, q_dec[l] [B][H_q][D] (the pass's dtype) against the rows
        that run / compress wrote for plan; returns o, per layer [B][H_q][D]
        float32 (allocated when not given). The decode workspace is kept on
        the object."""
        s = self.shape
        self._check_layers(q_dec, (s["B"], s["Hq"], s["D"]), "q_dec")
        self._check_outputs(k_out, v_out)
        if o is None:
            o = [torch.empty(s["B"], s["Hq"], s["D"], dtype=torch.float32, device=self.device)
                 for _ in range(s["L"])]
        for l, t in enumerate(o):
            if t.device != self.device or t.dtype != torch.float32 or not t.is_contiguous() or \
                    tuple(t.shape) != (s["B"], s["Hq"], s["D"]):
                raise ValueError(f"o[{l}] must be a contiguous float32 [B, H_q, D] tensor on {self.device}")
        need = _lib.decode_workspace_size(self.desc)
        if getattr(self, "dec_workspace", None) is None or self.dec_workspace.numel() < need:
            self.dec_workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        _lib.check(_lib.decode(self.desc, [t.data_ptr() for t in q_dec], plan.buf(),
                               [t.data_ptr() for t in k_out], [t.data_ptr() for t in v_out],
                               [t.data_ptr() for t in o], self.dec_workspace.data_ptr(), need,
                               self._stream(stream)))
        return o

    def decode_i8(self, q_dec, plan: PlanOutputs, kq, vq, k_scale, v_scale, o=None, stream=None):
        """Decode attention over the int8 cache of quantize_i8()
        (aircache_decode_i8): as decode(), every cached value read as code *
        scale. kq, vq: per layer int8 tensors of at least out_off[l][B]
        elements; k_scale, v_scale: float32 [L][B][H_kv]."""
        s = self.shape
        self._check_layers(q_dec, (s["B"], s["Hq"], s["D"]), "q_dec")
        cap = _lib.max_compacted_elems(self.desc)
        for name, ts in (("kq", kq), ("vq", vq)):
            if len(ts) != s["L"]:
                raise ValueError(f"{name}: {len(ts)} layers given")
            for l, t in enumerate(ts):
                if t.device != self.device or t.dtype != torch.int8 or not t.is_contiguous() or t.numel() < cap:
                    raise ValueError(f"{name}[{l}] must be a contiguous int8 tensor on {self.device} "
                                     f"with at least {cap} elements")
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t.device != self.device or t.dtype != torch.float32 or not t.is_contiguous() or \
                    tuple(t.shape) != (s["L"], s["B"], s["Hkv"]):
                raise ValueError(f"{name} must be a contiguous float32 [L, B, H_kv] tensor on {self.device}")
        if o is None:
            o = [torch.empty(s["B"], s["Hq"], s["D"], dtype=torch.float32, device=self.device)
                 for _ in range(s["L"])]
        need = _lib.decode_workspace_size(self.desc)
        if getattr(self, "dec_workspace", None) is None or self.dec_workspace.numel() < need:
            self.dec_workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        _lib.check(_lib.decode_i8(self.desc, [t.data_ptr() for t in q_dec], plan.buf(),
                                  [t.data_ptr() for t in kq], [t.data_ptr() for t in vq], k_scale.data_ptr(),
                                  v_scale.data_ptr(), [t.data_ptr() for t in o], self.dec_workspace.data_ptr(),
                                  need, self._stream(stream)))
        return o

    def quantize_i8(self, plan: PlanOutputs, k_out, v_out, kq=None, vq=None, k_scale=None, v_scale=None,
                    stream=None):
        """int8 codes of the compacted cache with one float32 scale per
        (layer, sample, KV head) for K and for V (aircache_quantize_i8).
        Returns (kq, vq, k_scale, v_scale); kq / vq per layer int8 with the
        compacted layout, scales [L, B, H_kv]; allocated when not given."""
        s = self.shape
        self._check_outputs(k_out, v_out)
        cap = _lib.max_compacted_elems(self.desc)
        if kq is None:
            kq = [torch.empty(cap, dtype=torch.int8, device=self.device) for _ in range(s["L"])]
        if vq is None:
            vq = [torch.empty(cap, dtype=torch.int8, device=self.device) for _ in range(s["L"])]
        for name, ts in (("kq", kq), ("vq", vq)):
            if len(ts) != s["L"] or any(t.dtype != torch.int8 or t.device != self.device or not t.is_contiguous()
                                        or t.numel() < cap for t in ts):
                raise ValueError(f"{name}: {s['L']} contiguous int8 tensors on {self.device} of at least "
                                 f"{cap} elements expected")
        if k_scale is None:
            k_scale = torch.empty(s["L"], s["B"], s["Hkv"], dtype=torch.float32, device=self.device)
        if v_scale is None:
            v_scale = torch.empty(s["L"], s["B"], s["Hkv"], dtype=torch.float32, device=self.device)
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t.dtype != torch.float32 or t.device != self.device or not t.is_contiguous() or \
                    t.numel() != s["L"] * s["B"] * s["Hkv"]:
                raise ValueError(f"{name} must be a contiguous float32 [L, B, H_kv] tensor on {self.device}")
        _lib.check(_lib.quantize_i8(self.desc, plan.buf(), [t.data_ptr() for t in k_out],
                                    [t.data_ptr() for t in v_out], [t.data_ptr() for t in kq],
                                    [t.data_ptr() for t in vq], k_scale.data_ptr(), v_scale.data_ptr(),
                                    self._stream(stream)))
        return kq, vq, k_scale, v_scale

    def bind_quantize(self, plan: PlanOutputs, k_out, v_out, kq, vq, k_scale, v_scale,
                      stream=None) -> "BoundQuantize":
        """A BoundQuantize running quantize_i8() on these tensors with the
        checks and marshalling done once, here."""
        return BoundQuantize(self, plan, k_out, v_out, kq, vq, k_scale, v_scale, stream)

    def bind_decode(self, q_dec, plan: PlanOutputs, k_out, v_out, o, stream=None, scales=None) -> "BoundDecode":
        """A BoundDecode running decode() on these tensors with the checks and
        marshalling done once, here; with scales = (k_scale, v_scale), k_out
        and v_out are the int8 codes and it runs decode_i8()."""
        return BoundDecode(self, q_dec, plan, k_out, v_out, o, stream, scales)

    # -- prefill attention with the scores fused in (aircache_prefill_layer) --
    def _check_prefill(self, q, k, v, o):
        s = self.shape
        S = s["Nv"] + s["Nt"]
        for name, t, shp in (("q", q, (s["B"], s["Hq"], S, s["D"])), ("k", k, (s["B"], s["Hkv"], S, s["D"])),
                             ("v", v, (s["B"], s["Hkv"], S, s["D"])), ("o", o, (s["B"], s["Hq"], S, s["D"]))):
            if t.device != self.device or t.dtype != self.dtype or not t.is_contiguous() or tuple(t.shape) != shp:
                raise ValueError(f"{name} must be a contiguous {self.dtype} tensor of shape {shp} on {self.device}")

    @property
    def prefill_workspace(self) -> torch.Tensor:
        """The scoring workspace of the prefill calls (one layer's scoring
        terms and the pass's counters), allocated on first use."""
        if getattr(self, "_pf_ws", None) is None:
            n = _lib.prefill_workspace_size(self.desc)
            if n == 0:
                _lib.check(_lib.AIRCACHE_EINVAL)
            self._pf_ws = torch.zeros(n, dtype=torch.uint8, device=self.device)
        return self._pf_ws

    def prefill_layer(self, layer: int, q, k, v, o, plan: PlanOutputs, stream=None):
        """Causal prefill attention of one layer (aircache_prefill_layer):
        o = softmax(q K^T / sqrt(D), causal) V with q, o [B][H_q][N_v+N_t][D]
        and k, v [B][H_kv][N_v+N_t][D] (bfloat16), writing that layer's elite
        set, I_v and statistics into plan; the call for the last layer also
        budgets and selects every layer. Call for layers 0..L-1 in order on
        one stream, then compress()."""
        self._check_prefill(q, k, v, o)
        ws = self.prefill_workspace
        _lib.check(_lib.prefill_layer(self.desc, layer, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      plan.buf(), ws.data_ptr(), ws.numel(), self._stream(stream)))
        return o

    def prefill_attention(self, q, k, v, o=None, stream=None):
        """The same attention of one layer without the scores
        (aircache_prefill_attention)."""
        o = torch.empty_like(q) if o is None else o
        self._check_prefill(q, k, v, o)
        _lib.check(_lib.prefill_attention(self.desc, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          self._stream(stream)))
        return o

    def bind_prefill(self, q, k, v, o, plan: PlanOutputs | None, stream=None) -> "BoundPrefill":
        """A BoundPrefill running every layer's prefill attention (with the
        scores when plan is given) over these per-layer tensor lists, checked
        and marshalled once, here."""
        return BoundPrefill(self, q, k, v, o, plan, stream)

    def compress(self, plan: PlanOutputs, k, v, k_out, v_out, stream=None, events=None) -> None:
        s = self.shape
        shp = (s["B"], s["Hkv"], s["Nv"] + s["Nt"], s["D"])
        self._check_layers(k, shp, "k")
        self._check_layers(v, shp, "v")
        self._check_outputs(k_out, v_out)
        _lib.check(_lib.compress(self.desc, plan.buf(), [t.data_ptr() for t in k],
                                 [t.data_ptr() for t in v], [t.data_ptr() for t in k_out],
                                 [t.data_ptr() for t in v_out], self._stream(stream),
                                 events=None if events is None else [e.cuda_event for e in events]))


class BoundPass:
    """plan + compress over fixed tensors, validated once.

    Built by AirCache.bind: the pointer arrays and the plan buffer struct are
    marshalled when it is built, so each call only crosses into the library
    (the per-call checks and array building of AirCache.plan / .compress cost
    tens of microseconds of host time, comparable with the pass itself). The
    tensors must stay alive and keep their storage while it is used.
    """

    def __init__(self, ac: "AirCache", q_txt, k, v, plan: PlanOutputs, k_out, v_out, stream=None):
        s = ac.shape
        ac._check_layers(q_txt, (s["B"], s["Hq"], ac.q_rows, s["D"]), "q_txt")
        shp = (s["B"], s["Hkv"], s["Nv"] + s["Nt"], s["D"])
        ac._check_layers(k, shp, "k")
        ac._check_layers(v, shp, "v")
        ac._check_outputs(k_out, v_out)
        self.plan_out = plan
        self._keep = (ac, q_txt, k, v, plan, k_out, v_out)
        self._lib = _lib.load()
        self._desc = _lib.C.byref(ac.desc)
        self._buf = plan.buf()
        self._pbuf = _lib.C.byref(self._buf)
        self._q = _lib.ptr_array([t.data_ptr() for t in q_txt])
        self._k = _lib.ptr_array([t.data_ptr() for t in k])
        self._v = _lib.ptr_array([t.data_ptr() for t in v])
        self._ko = _lib.ptr_array([t.data_ptr() for t in k_out])
        self._vo = _lib.ptr_array([t.data_ptr() for t in v_out])
        self._ws = _lib.C.c_void_p(ac.workspace.data_ptr())
        self._ws_bytes = ac.ws_bytes
        self._st = _lib.C.c_void_p(ac._stream(stream))

    def with_status(self, ptr: int) -> "BoundPass":
        """A copy of this bound pass whose calls write their device status word
        to ptr (an int32 in device memory) instead of the plan's: a caller
        that makes many calls can then read every call's status afterwards."""
        import copy
        other = copy.copy(self)
        buf = _lib.PlanBuf.from_buffer_copy(self._buf)
        buf.status = ptr
        other._buf = buf
        other._pbuf = _lib.C.byref(buf)
        return other

    def plan(self, events=None) -> PlanOutputs:
        if events is None:
            rc = self._lib.aircache_plan(self._desc, self._q, self._k, self._pbuf, self._ws, self._ws_bytes,
                                         self._st)
        else:
            ev = [e.cuda_event for e in events]
            rc = self._lib.aircache_plan_profiled(self._desc, self._q, self._k, self._pbuf, self._ws,
                                                  self._ws_bytes, self._st, _lib.ptr_array(ev), len(ev))
        if rc:
            _lib.check(rc)
        return self.plan_out

    def compress(self, events=None) -> None:
        if events is None:
            rc = self._lib.aircache_compress(self._desc, self._pbuf, self._k, self._v, self._ko, self._vo,
                                             self._st)
        else:
            ev = [e.cuda_event for e in events]
            rc = self._lib.aircache_compress_profiled(self._desc, self._pbuf, self._k, self._v, self._ko,
                                                      self._vo, self._st, _lib.ptr_array(ev), len(ev))
        if rc:
            _lib.check(rc)

    def run(self, events=None) -> PlanOutputs:
        """plan + compress in one library call (aircache_run)."""
        if events is None:
            rc = self._lib.aircache_run(self._desc, self._q, self._k, self._v, self._pbuf, self._ko, self._vo,
                                        self._ws, self._ws_bytes, self._st)
        else:
            ev = [e.cuda_event for e in events]
            rc = self._lib.aircache_run_profiled(self._desc, self._q, self._k, self._v, self._pbuf, self._ko,
                                                 self._vo, self._ws, self._ws_bytes, self._st, _lib.ptr_array(ev),
                                                 len(ev))
        if rc:
            _lib.check(rc)
        return self.plan_out

    def __call__(self) -> PlanOutputs:
        return self.run()


class BoundQuantize:
    """AirCache.quantize_i8 over fixed tensors, validated and marshalled once
    (as BoundPass does for the pass). The tensors must stay alive while it is
    used."""

    def __init__(self, ac: "AirCache", plan: PlanOutputs, k_out, v_out, kq, vq, k_scale, v_scale, stream=None):
        ac.quantize_i8(plan, k_out, v_out, kq, vq, k_scale, v_scale, stream=stream)  # the checks, once
        self.out = (kq, vq, k_scale, v_scale)
        self._keep = (ac, plan, k_out, v_out, kq, vq, k_scale, v_scale)
        self._lib = _lib.load()
        self._desc = _lib.C.byref(ac.desc)
        self._buf = plan.buf()
        self._pbuf = _lib.C.byref(self._buf)
        self._ko = _lib.ptr_array([t.data_ptr() for t in k_out])
        self._vo = _lib.ptr_array([t.data_ptr() for t in v_out])
        self._kq = _lib.ptr_array([t.data_ptr() for t in kq])
        self._vq = _lib.ptr_array([t.data_ptr() for t in vq])
        self._ks = _lib.C.c_void_p(k_scale.data_ptr())
        self._vs = _lib.C.c_void_p(v_scale.data_ptr())
        self._st = _lib.C.c_void_p(ac._stream(stream))

    def __call__(self):
        rc = self._lib.aircache_quantize_i8(self._desc, self._pbuf, self._ko, self._vo, self._kq, self._vq,
                                            self._ks, self._vs, self._st)
        if rc:
            _lib.check(rc)
        return self.out


class BoundDecode:
    """AirCache.decode over fixed tensors, validated and marshalled once (as
    BoundPass does for the pass). The tensors must stay alive while it is used."""

    def __init__(self, ac: "AirCache", q_dec, plan: PlanOutputs, k_out, v_out, o, stream=None, scales=None):
        s = ac.shape
        self._i8 = scales is not None
        if self._i8:
            ac.decode_i8(q_dec, plan, k_out, v_out, scales[0], scales[1], o=o, stream=stream)  # the checks, once
            self._ks = _lib.C.c_void_p(scales[0].data_ptr())
            self._vs = _lib.C.c_void_p(scales[1].data_ptr())
        else:
            ac._check_layers(q_dec, (s["B"], s["Hq"], s["D"]), "q_dec")
            ac._check_outputs(k_out, v_out)
        for l, t in enumerate(o):
            if t.device != ac.device or t.dtype != torch.float32 or not t.is_contiguous() or \
                    tuple(t.shape) != (s["B"], s["Hq"], s["D"]):
                raise ValueError(f"o[{l}] must be a contiguous float32 [B, H_q, D] tensor on {ac.device}")
        need = _lib.decode_workspace_size(ac.desc)
        self.workspace = torch.empty(need, dtype=torch.uint8, device=ac.device)
        self.out = o
        self._keep = (ac, q_dec, plan, k_out, v_out, o, scales)
        self._lib = _lib.load()
        self._desc = _lib.C.byref(ac.desc)
        self._buf = plan.buf()
        self._pbuf = _lib.C.byref(self._buf)
        self._q = _lib.ptr_array([t.data_ptr() for t in q_dec])
        self._ko = _lib.ptr_array([t.data_ptr() for t in k_out])
        self._vo = _lib.ptr_array([t.data_ptr() for t in v_out])
        self._o = _lib.ptr_array([t.data_ptr() for t in o])
        self._ws = _lib.C.c_void_p(self.workspace.data_ptr())
        self._ws_bytes = need
        self._st = _lib.C.c_void_p(ac._stream(stream))

    def __call__(self):
        if self._i8:
            rc = self._lib.aircache_decode_i8(self._desc, self._q, self._pbuf, self._ko, self._vo, self._ks, self._vs,
                                              self._o, self._ws, self._ws_bytes, self._st)
        else:
            rc = self._lib.aircache_decode(self._desc, self._q, self._pbuf, self._ko, self._vo, self._o, self._ws,
                                           self._ws_bytes, self._st)
        if rc:
            _lib.check(rc)
        return self.out


class BoundPrefill:
    """The prefill calls of every layer over fixed per-layer tensors,
    validated and marshalled once (as BoundPass does for the pass): with a
    plan, aircache_prefill_layer for layers 0..L-1 (the plan is complete after
    the last); without, aircache_prefill_attention per layer. The tensors must
    stay alive while it is used."""

    def __init__(self, ac: "AirCache", q, k, v, o, plan: PlanOutputs | None, stream=None):
        L = ac.shape["L"]
        for name, ts in (("q", q), ("k", k), ("v", v), ("o", o)):
            if len(ts) != L:
                raise ValueError(f"{name}: {len(ts)} layers given, {L} expected")
        for l in range(L):
            ac._check_prefill(q[l], k[l], v[l], o[l])
        self.out = o
        self._keep = (ac, q, k, v, o, plan)
        self._lib = _lib.load()
        self._desc = _lib.C.byref(ac.desc)
        V = _lib.C.c_void_p
        self._args = [(V(q[l].data_ptr()), V(k[l].data_ptr()), V(v[l].data_ptr()), V(o[l].data_ptr()))
                      for l in range(L)]
        self._st = V(ac._stream(stream))
        self._score = plan is not None
        if self._score:
            self._buf = plan.buf()
            self._pbuf = _lib.C.byref(self._buf)
            ws = ac.prefill_workspace
            self._ws, self._ws_bytes = V(ws.data_ptr()), ws.numel()

    def __call__(self):
        f = self._lib.aircache_prefill_layer if self._score else self._lib.aircache_prefill_attention
        for l, (q, k, v, o) in enumerate(self._args):
            if self._score:
                rc = f(self._desc, l, q, k, v, o, self._pbuf, self._ws, self._ws_bytes, self._st)
            else:
                rc = f(self._desc, q, k, v, o, self._st)
            if rc:
                _lib.check(rc)
        return self.out
