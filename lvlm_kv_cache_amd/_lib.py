"""ctypes binding of libaircache.so (include/aircache.h).

Argument marshalling only: every step of the pass runs in the HIP library.
PyTorch supplies device memory and the current stream. There is no fallback:
if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_build", "libaircache.so")

AIRCACHE_OK, AIRCACHE_EINVAL, AIRCACHE_EWORKSPACE, AIRCACHE_EHIP = 0, 1, 2, 3
AIRCACHE_F32, AIRCACHE_BF16 = 0, 1
AIRCACHE_DEV_ELITE_OVERFLOW, AIRCACHE_DEV_TIMEOUT = 1, 2
PATH_AUTO, PATH_TILED, PATH_ROWS, PATH_CHUNKED, PATH_SMALL = 0, 1, 2, 3, 4
SELECT_SHARED, SELECT_PER_KV_HEAD = 0, 1
MAX_LAYERS = 128

EXPORTS = ["aircache_abi_version", "aircache_workspace_size", "aircache_max_compacted_elems",
           "aircache_resolved_path", "aircache_run_launches",
           "aircache_plan", "aircache_compress", "aircache_run", "aircache_plan_profiled",
           "aircache_compress_profiled", "aircache_run_profiled", "aircache_run_noalloc", "aircache_strerror",
           "aircache_last_error", "aircache_decode_workspace_size", "aircache_decode", "aircache_quantize_i8",
           "aircache_prefill_workspace_size", "aircache_prefill_layer", "aircache_prefill_attention",
           "aircache_decode_i8"]
NOALLOC_SCRATCH_BYTES = 128 << 20  # AIRCACHE_NOALLOC_SCRATCH_BYTES
PLAN_KERNELS = ["elite_select", "cross_score", "finalize", "topk_select"]
COMPRESS_KERNELS = ["kv_gather"]
RUN_KERNELS = ["aircache_pass"]


class Desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("batch", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("n_vis", C.c_int32),
                ("n_txt", C.c_int32), ("dtype", C.c_int32), ("alpha", C.c_double),
                ("ratio", C.c_double), ("max_elite", C.c_int32), ("path", C.c_int32),
                ("budget_mode", C.c_int32), ("obs_window", C.c_int32), ("select_mode", C.c_int32)]


class PlanBuf(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("elite_idx", "n_elite", "iv", "s_t", "s_k", "budget_x",
                                          "budget", "out_off", "kept_idx", "status", "iv_head")]


class AirCacheError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"aircache status {status}: {message}")
        self.status = status


_lib = None


def load() -> C.CDLL:
    """Load the in-tree HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with lvlm_kv_cache_amd.build.build()")
        lib = C.CDLL(LIB_PATH)
        P = C.c_void_p
        lib.aircache_abi_version.restype = C.c_int
        lib.aircache_abi_version.argtypes = []
        lib.aircache_workspace_size.restype = C.c_size_t
        lib.aircache_workspace_size.argtypes = [C.POINTER(Desc)]
        lib.aircache_max_compacted_elems.restype = C.c_int64
        lib.aircache_max_compacted_elems.argtypes = [C.POINTER(Desc)]
        lib.aircache_resolved_path.restype = C.c_int32
        lib.aircache_resolved_path.argtypes = [C.POINTER(Desc)]
        lib.aircache_run_launches.restype = C.c_int32
        lib.aircache_run_launches.argtypes = [C.POINTER(Desc)]
        lib.aircache_plan.restype = C.c_int
        lib.aircache_plan.argtypes = [C.POINTER(Desc), P, P, C.POINTER(PlanBuf), P, C.c_size_t, P]
        lib.aircache_compress.restype = C.c_int
        lib.aircache_compress.argtypes = [C.POINTER(Desc), C.POINTER(PlanBuf), P, P, P, P, P]
        lib.aircache_plan_profiled.restype = C.c_int
        lib.aircache_plan_profiled.argtypes = [C.POINTER(Desc), P, P, C.POINTER(PlanBuf), P, C.c_size_t, P,
                                               P, C.c_int]
        lib.aircache_compress_profiled.restype = C.c_int
        lib.aircache_compress_profiled.argtypes = [C.POINTER(Desc), C.POINTER(PlanBuf), P, P, P, P, P, P, C.c_int]
        lib.aircache_run.restype = C.c_int
        lib.aircache_run.argtypes = [C.POINTER(Desc), P, P, P, C.POINTER(PlanBuf), P, P, P, C.c_size_t, P]
        lib.aircache_run_profiled.restype = C.c_int
        lib.aircache_run_profiled.argtypes = [C.POINTER(Desc), P, P, P, C.POINTER(PlanBuf), P, P, P, C.c_size_t, P,
                                              P, C.c_int]
        lib.aircache_run_noalloc.restype = C.c_int
        lib.aircache_run_noalloc.argtypes = [C.POINTER(Desc), P, P, P, C.POINTER(PlanBuf), P, P, P]
        lib.aircache_decode_workspace_size.restype = C.c_size_t
        lib.aircache_decode_workspace_size.argtypes = [C.POINTER(Desc)]
        lib.aircache_decode.restype = C.c_int
        lib.aircache_decode.argtypes = [C.POINTER(Desc), P, C.POINTER(PlanBuf), P, P, P, P, C.c_size_t, P]
        lib.aircache_decode_i8.restype = C.c_int
        lib.aircache_decode_i8.argtypes = [C.POINTER(Desc), P, C.POINTER(PlanBuf), P, P, P, P, P, P, C.c_size_t, P]
        lib.aircache_quantize_i8.restype = C.c_int
        lib.aircache_quantize_i8.argtypes = [C.POINTER(Desc), C.POINTER(PlanBuf), P, P, P, P, P, P, P]
        lib.aircache_prefill_workspace_size.restype = C.c_size_t
        lib.aircache_prefill_workspace_size.argtypes = [C.POINTER(Desc)]
        lib.aircache_prefill_layer.restype = C.c_int
        lib.aircache_prefill_layer.argtypes = [C.POINTER(Desc), C.c_int32, P, P, P, P, C.POINTER(PlanBuf), P,
                                               C.c_size_t, P]
        lib.aircache_prefill_attention.restype = C.c_int
        lib.aircache_prefill_attention.argtypes = [C.POINTER(Desc), P, P, P, P, P]
        lib.aircache_strerror.restype = C.c_char_p
        lib.aircache_strerror.argtypes = [C.c_int]
        lib.aircache_last_error.restype = C.c_char_p
        lib.aircache_last_error.argtypes = []
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != AIRCACHE_OK:
        lib = load()
        raise AirCacheError(status, f"{lib.aircache_strerror(status).decode()}: "
                                    f"{lib.aircache_last_error().decode()}")


def ptr_array(ptrs) -> C.Array:
    return (C.c_void_p * len(ptrs))(*[C.c_void_p(int(p)) for p in ptrs])


def workspace_size(desc: Desc) -> int:
    return int(load().aircache_workspace_size(C.byref(desc)))


def max_compacted_elems(desc: Desc) -> int:
    return int(load().aircache_max_compacted_elems(C.byref(desc)))


def resolved_path(desc: Desc) -> int:
    return int(load().aircache_resolved_path(C.byref(desc)))


def run_launches(desc: Desc) -> int:
    return int(load().aircache_run_launches(C.byref(desc)))


def plan(desc: Desc, q_ptrs, k_ptrs, buf: PlanBuf, ws_ptr: int, ws_bytes: int, stream: int,
         events=None) -> int:
    q = ptr_array(q_ptrs) if q_ptrs is not None else None
    k = ptr_array(k_ptrs) if k_ptrs is not None else None
    if events is None:
        return load().aircache_plan(C.byref(desc), q, k, C.byref(buf), C.c_void_p(ws_ptr), ws_bytes,
                                    C.c_void_p(stream))
    return load().aircache_plan_profiled(C.byref(desc), q, k, C.byref(buf), C.c_void_p(ws_ptr), ws_bytes,
                                         C.c_void_p(stream), ptr_array(events), len(events))


def run(desc: Desc, q_ptrs, k_ptrs, v_ptrs, buf: PlanBuf, ko_ptrs, vo_ptrs, ws_ptr: int, ws_bytes: int,
        stream: int, events=None) -> int:
    q, k, v, ko, vo = [ptr_array(p) if p is not None else None for p in (q_ptrs, k_ptrs, v_ptrs, ko_ptrs, vo_ptrs)]
    if events is None:
        return load().aircache_run(C.byref(desc), q, k, v, C.byref(buf), ko, vo, C.c_void_p(ws_ptr), ws_bytes,
                                   C.c_void_p(stream))
    return load().aircache_run_profiled(C.byref(desc), q, k, v, C.byref(buf), ko, vo, C.c_void_p(ws_ptr), ws_bytes,
                                        C.c_void_p(stream), ptr_array(events), len(events))


def run_noalloc(desc: Desc, q_ptrs, k_ptrs, v_ptrs, buf: PlanBuf, ko_ptrs, vo_ptrs, stream: int) -> int:
    """aircache_run_noalloc: the whole pass on the library's static scratch."""
    q, k, v, ko, vo = [ptr_array(p) if p is not None else None for p in (q_ptrs, k_ptrs, v_ptrs, ko_ptrs, vo_ptrs)]
    return load().aircache_run_noalloc(C.byref(desc), q, k, v, C.byref(buf), ko, vo, C.c_void_p(stream))


def compress(desc: Desc, buf: PlanBuf, k_ptrs, v_ptrs, ko_ptrs, vo_ptrs, stream: int, events=None) -> int:
    arrs = [ptr_array(p) if p is not None else None for p in (k_ptrs, v_ptrs, ko_ptrs, vo_ptrs)]
    if events is None:
        return load().aircache_compress(C.byref(desc), C.byref(buf), *arrs, C.c_void_p(stream))
    return load().aircache_compress_profiled(C.byref(desc), C.byref(buf), *arrs, C.c_void_p(stream),
                                             ptr_array(events), len(events))


def decode_workspace_size(desc: Desc) -> int:
    return int(load().aircache_decode_workspace_size(C.byref(desc)))


def decode(desc: Desc, q_ptrs, buf: PlanBuf, ko_ptrs, vo_ptrs, o_ptrs, ws_ptr: int, ws_bytes: int,
           stream: int) -> int:
    """aircache_decode: decode attention over the compacted cache."""
    q, ko, vo, o = [ptr_array(p) if p is not None else None for p in (q_ptrs, ko_ptrs, vo_ptrs, o_ptrs)]
    return load().aircache_decode(C.byref(desc), q, C.byref(buf), ko, vo, o, C.c_void_p(ws_ptr), ws_bytes,
                                  C.c_void_p(stream))


def decode_i8(desc: Desc, q_ptrs, buf: PlanBuf, kq_ptrs, vq_ptrs, k_scale: int, v_scale: int, o_ptrs,
              ws_ptr: int, ws_bytes: int, stream: int) -> int:
    """aircache_decode_i8: decode attention over the int8 cache."""
    q, kq, vq, o = [ptr_array(p) if p is not None else None for p in (q_ptrs, kq_ptrs, vq_ptrs, o_ptrs)]
    return load().aircache_decode_i8(C.byref(desc), q, C.byref(buf), kq, vq, C.c_void_p(k_scale),
                                     C.c_void_p(v_scale), o, C.c_void_p(ws_ptr), ws_bytes, C.c_void_p(stream))


def quantize_i8(desc: Desc, buf: PlanBuf, ko_ptrs, vo_ptrs, kq_ptrs, vq_ptrs, k_scale: int, v_scale: int,
                stream: int) -> int:
    ko, vo, kq, vq = [ptr_array(p) for p in (ko_ptrs, vo_ptrs, kq_ptrs, vq_ptrs)]
    return load().aircache_quantize_i8(C.byref(desc), C.byref(buf), ko, vo, kq, vq, C.c_void_p(k_scale),
                                       C.c_void_p(v_scale), C.c_void_p(stream))


def prefill_workspace_size(desc: Desc) -> int:
    return int(load().aircache_prefill_workspace_size(C.byref(desc)))


def prefill_layer(desc: Desc, layer: int, q: int, k: int, v: int, o: int, buf: PlanBuf, ws_ptr: int,
                  ws_bytes: int, stream: int) -> int:
    """aircache_prefill_layer: one layer's prefill attention with its scores."""
    return load().aircache_prefill_layer(C.byref(desc), int(layer), C.c_void_p(q), C.c_void_p(k), C.c_void_p(v),
                                         C.c_void_p(o), C.byref(buf), C.c_void_p(ws_ptr), ws_bytes,
                                         C.c_void_p(stream))


def prefill_attention(desc: Desc, q: int, k: int, v: int, o: int, stream: int) -> int:
    """aircache_prefill_attention: one layer's prefill attention alone."""
    return load().aircache_prefill_attention(C.byref(desc), C.c_void_p(q), C.c_void_p(k), C.c_void_p(v),
                                             C.c_void_p(o), C.c_void_p(stream))
