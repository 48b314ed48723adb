"""The C ABI library: it loads, exports every function include/aircache.h
declares, and rejects invalid arguments on the host before touching the GPU
(no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

from lvlm_kv_cache_amd import _lib, make_desc
from lvlm_kv_cache_amd.build import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    # AIRCACHE_ABI_TEST_LIB: another build of the same library (the host
    # sanitizer build of tests/test_host_sanitizers.py)
    other = os.environ.get("AIRCACHE_ABI_TEST_LIB")
    if other:
        _lib.LIB_PATH = other
    elif not os.path.exists(_lib.LIB_PATH):
        build(force=False)
    return _lib.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "aircache.h")).read()
    return sorted(set(re.findall(r"^[a-z_0-9 ]+[ *](aircache_[a-z_0-9]+)\(", text, re.M)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 7, names
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.aircache_abi_version() == 4


def test_struct_layouts():
    # eight int32, two doubles, five int32 (padded to the doubles' alignment)
    assert C.sizeof(_lib.Desc) == 8 * 4 + 2 * 8 + 5 * 4 + 4
    assert _lib.Desc.budget_mode.offset == 8 * 4 + 2 * 8 + 2 * 4
    assert _lib.Desc.obs_window.offset == 8 * 4 + 2 * 8 + 3 * 4
    assert _lib.Desc.select_mode.offset == 8 * 4 + 2 * 8 + 4 * 4
    assert C.sizeof(_lib.PlanBuf) == 11 * 8
    assert _lib.PlanBuf.iv_head.offset == 10 * 8


def desc(**kw):
    base = dict(n_layers=28, batch=1, n_q_heads=28, n_kv_heads=4, head_dim=128, n_vis=2880,
                n_txt=128, dtype="bf16", alpha=0.9, ratio=0.1, max_elite=0, path=0, budget_mode=0, obs_window=0,
                select=0)
    base.update(kw)
    return make_desc(*[base[k] for k in ("n_layers", "batch", "n_q_heads", "n_kv_heads", "head_dim",
                                         "n_vis", "n_txt", "dtype", "alpha", "ratio", "max_elite", "path",
                                         "budget_mode", "obs_window", "select")])


def test_workspace_size(lib):
    assert _lib.workspace_size(desc()) > 0
    # the tiled path spills exponentials for up to max_elite elite rows
    assert _lib.workspace_size(desc(max_elite=8, path=1)) < _lib.workspace_size(desc(path=1))
    assert _lib.workspace_size(desc(path=2)) < _lib.workspace_size(desc(path=1))
    assert _lib.max_compacted_elems(desc()) == 1 * 4 * 3008 * 128


def test_resolved_path(lib):
    # chunked (one launch) whenever the shape fits it: any number of KV heads
    # (head groups of up to eight), N_t <= 1024, n_layers * batch <= 2048 and
    # the consumer statistics within its LDS; else rows while N_v fits 8 waves
    # x 16 keys x 24 tiles (3072 keys); else tiled
    assert _lib.resolved_path(desc()) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(n_vis=6272, n_txt=256)) == _lib.PATH_CHUNKED
    for hkv in (1, 2, 3, 7, 8, 32):
        assert _lib.resolved_path(desc(n_q_heads=8 * hkv, n_kv_heads=hkv)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(n_q_heads=32, n_kv_heads=32)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(n_txt=1100)) == _lib.PATH_ROWS            # N_t beyond the elite parts
    assert _lib.resolved_path(desc(dtype="f32", n_vis=8192)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(n_layers=128, batch=16)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(batch=64, n_txt=1024)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(n_layers=128, n_txt=1024)) == _lib.PATH_ROWS   # statistics of 128 layers x 31 chunks
    assert _lib.resolved_path(desc(n_layers=128, batch=17)) == _lib.PATH_ROWS    # more pairs than the schedule holds
    assert _lib.resolved_path(desc(n_layers=128, batch=17, n_vis=3073)) == _lib.PATH_TILED
    assert _lib.resolved_path(desc(path=1)) == _lib.PATH_TILED
    assert _lib.resolved_path(desc(path=2)) == _lib.PATH_ROWS
    assert _lib.resolved_path(desc(path=2, n_vis=17)) == _lib.PATH_ROWS
    assert _lib.resolved_path(desc(path=3, n_vis=17)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(path=3, n_kv_heads=7)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(path=3, n_txt=1100)) == -1
    assert _lib.resolved_path(desc(path=2, n_vis=3073)) == -1
    # tiny shapes: one workgroup for the whole pass
    tiny = dict(n_layers=2, n_q_heads=2, n_kv_heads=2, head_dim=64, n_vis=64, n_txt=16, dtype="f32")
    assert _lib.resolved_path(desc(**tiny)) == _lib.PATH_SMALL
    assert _lib.resolved_path(desc(path=3, **tiny)) == _lib.PATH_CHUNKED
    assert _lib.resolved_path(desc(path=4, **tiny)) == _lib.PATH_SMALL
    assert _lib.run_launches(desc(**tiny)) == 1
    assert 0 < _lib.workspace_size(desc(**tiny)) <= 256
    assert _lib.resolved_path(desc(path=4)) == -1           # workload 3 is far beyond 256 KB of keys


def test_chunked_workspace_sizes(lib):
    """The one-launch path's records are sized for the most chunks a pair can
    have, which grows with the elite cap (more elite rows, narrower chunks);
    row normaliser slots are reused pass after pass, so the default
    max_elite = 0 (cap N_t) keeps the five workloads on the one-launch path
    with workspaces under 128 MiB."""
    for kw in (dict(), dict(n_vis=6272, n_txt=256, batch=4), dict(n_vis=3072, n_txt=1024, batch=8),
               dict(n_layers=32, n_q_heads=32, n_kv_heads=32, n_vis=576, n_txt=64)):
        a = _lib.workspace_size(desc(max_elite=0, **kw))
        assert _lib.workspace_size(desc(max_elite=8, **kw)) <= a < 128 << 20
        assert _lib.resolved_path(desc(max_elite=0, **kw)) == _lib.PATH_CHUNKED


def test_run_launches(lib):
    # one launch where the chunked path also compacts (5 * n_layers pointers
    # fit its table), else the plan call's kernels and kv_gather_kernel
    assert _lib.run_launches(desc()) == 1
    assert _lib.run_launches(desc(n_layers=51)) == 1
    assert _lib.run_launches(desc(n_layers=52)) == 2
    assert _lib.run_launches(desc(path=2)) == 4
    assert _lib.run_launches(desc(path=1)) == 5
    assert _lib.run_launches(desc(n_layers=0)) == -1


@pytest.mark.parametrize("bad", [dict(n_layers=0), dict(n_layers=129), dict(batch=0), dict(n_kv_heads=5),
                                 dict(head_dim=96), dict(n_vis=2), dict(n_vis=9000), dict(n_txt=0),
                                 dict(dtype="x"), dict(alpha=1.5), dict(alpha=float("nan")),
                                 dict(ratio=-0.1), dict(max_elite=129), dict(n_txt=4000), dict(path=4),
                                 dict(path=2, n_vis=4000), dict(budget_mode=5), dict(budget_mode=-1),
                                 dict(obs_window=-129), dict(obs_window=-8, path=3), dict(obs_window=-8, path=4),
                                 dict(obs_window=-8, n_vis=5), dict(select=2), dict(select=-1), dict(select=1, path=2),
                                 dict(select=1, path=3)])
def test_invalid_descriptor(lib, bad):
    if bad.get("dtype") == "x":
        d = desc()
        d.dtype = 7
    else:
        d = desc(**bad)
    assert _lib.workspace_size(d) == 0
    assert lib.aircache_last_error().decode()
    assert _lib.resolved_path(d) == -1
    rc = _lib.plan(d, [1] * max(d.n_layers, 1), [1] * max(d.n_layers, 1), _lib.PlanBuf(), 16, 1 << 40, 0)
    assert rc == _lib.AIRCACHE_EINVAL


def fake_buf():
    return _lib.PlanBuf(*([4096] * 10))


def test_plan_argument_errors(lib):
    d = desc(n_layers=2)
    ws = _lib.workspace_size(d)
    ok = [4096, 8192]
    assert _lib.plan(d, ok, ok, _lib.PlanBuf(), 4096, ws, 0) == _lib.AIRCACHE_EINVAL       # NULL outputs
    assert _lib.plan(d, ok, ok, fake_buf(), 0, ws, 0) == _lib.AIRCACHE_EWORKSPACE         # no workspace
    assert _lib.plan(d, ok, ok, fake_buf(), 4096, ws - 1, 0) == _lib.AIRCACHE_EWORKSPACE  # too small
    assert _lib.plan(d, ok, ok, fake_buf(), 4100, ws, 0) == _lib.AIRCACHE_EINVAL          # misaligned
    assert _lib.plan(d, None, ok, fake_buf(), 4096, ws, 0) == _lib.AIRCACHE_EINVAL
    assert _lib.plan(d, [4096, 0], ok, fake_buf(), 4096, ws, 0) == _lib.AIRCACHE_EINVAL   # NULL layer
    assert _lib.plan(d, ok, [4096, 8200], fake_buf(), 4096, ws, 0) == _lib.AIRCACHE_EINVAL
    assert "not 16-byte aligned" in lib.aircache_last_error().decode()


def test_compress_argument_errors(lib):
    d = desc(n_layers=1, batch=1, n_vis=64, n_txt=16)
    k, v = [1 << 20], [2 << 20]
    layer = 4 * 80 * 128 * 2
    assert _lib.compress(d, fake_buf(), k, v, None, [3 << 20], 0) == _lib.AIRCACHE_EINVAL
    # an output that overlaps an input is rejected
    assert _lib.compress(d, fake_buf(), k, v, [(1 << 20) + layer // 2], [3 << 20], 0) == _lib.AIRCACHE_EINVAL
    assert "overlap" in lib.aircache_last_error().decode()
    assert _lib.compress(d, _lib.PlanBuf(), k, v, [3 << 20], [4 << 20], 0) == _lib.AIRCACHE_EINVAL


def test_strerror(lib):
    assert lib.aircache_strerror(0) == b"ok"
    assert lib.aircache_strerror(2) == b"workspace too small"


def test_noalloc_argument_errors(lib):
    """aircache_run_noalloc rejects, on the host and before anything touches
    the scratch, a descriptor whose workspace exceeds the static scratch and
    the argument errors aircache_run rejects."""
    big = desc(path=1, n_layers=28, batch=8, n_vis=3072, n_txt=1024)  # tiled: gigabytes of workspace
    assert _lib.workspace_size(big) > _lib.NOALLOC_SCRATCH_BYTES
    ptrs = [4096] * 28
    rc = _lib.run_noalloc(big, ptrs, ptrs, ptrs, fake_buf(), ptrs, ptrs, 0)
    assert rc == _lib.AIRCACHE_EINVAL
    assert "scratch" in lib.aircache_last_error().decode()
    d = desc(n_layers=2, n_vis=64, n_txt=16)
    assert _lib.workspace_size(d) <= _lib.NOALLOC_SCRATCH_BYTES
    ok = [1 << 20, 2 << 20]
    assert _lib.run_noalloc(d, ok, ok, ok, _lib.PlanBuf(), [3 << 20, 4 << 20], [5 << 20, 6 << 20], 0) == \
        _lib.AIRCACHE_EINVAL                                                              # NULL plan outputs
    assert _lib.run_noalloc(d, None, ok, ok, fake_buf(), [3 << 20, 4 << 20], [5 << 20, 6 << 20], 0) == \
        _lib.AIRCACHE_EINVAL                                                              # no queries
    assert _lib.run_noalloc(d, ok, ok, ok, fake_buf(), [(1 << 20) + 64, 4 << 20], [5 << 20, 6 << 20], 0) == \
        _lib.AIRCACHE_EINVAL                                                              # output overlaps input
    d.n_layers = 0
    assert _lib.run_noalloc(d, ok, ok, ok, fake_buf(), ok, ok, 0) == _lib.AIRCACHE_EINVAL


def test_decode_workspace_and_argument_errors(lib):
    """aircache_decode's host-side checks (nothing reaches the device)."""
    d = desc()
    assert _lib.decode_workspace_size(d) > 0
    assert _lib.decode_workspace_size(desc(n_layers=0)) == 0
    buf = _lib.PlanBuf()
    fake = [16 * (i + 1) for i in range(28)]
    # no plan buffers
    assert _lib.decode(d, fake, buf, fake, fake, fake, 16, 1 << 30, 0) == _lib.AIRCACHE_EINVAL
    # too many query heads per KV head for one workgroup's LDS
    big = desc(n_q_heads=66, n_kv_heads=2)
    buf.budget = 16
    buf.out_off = 32
    assert _lib.decode(big, fake, buf, fake, fake, fake, 16, 1 << 30, 0) == _lib.AIRCACHE_EINVAL
    # workspace too small
    assert _lib.decode(d, fake, buf, fake, fake, fake, 16, 8, 0) == _lib.AIRCACHE_EWORKSPACE
    # a NULL layer pointer
    assert _lib.decode(d, fake[:-1] + [0], buf, fake, fake, fake, 16, 1 << 30, 0) == _lib.AIRCACHE_EINVAL


def test_per_kv_head_selection_paths(lib):
    """One selection per KV head runs on the tiled and small paths only."""
    assert _lib.resolved_path(desc(select=1)) == _lib.PATH_TILED
    assert _lib.resolved_path(desc(select=0)) == _lib.PATH_CHUNKED
    tiny = dict(n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, n_vis=64, n_txt=16)
    assert _lib.resolved_path(desc(select=1, **tiny)) == _lib.PATH_SMALL
    assert _lib.resolved_path(desc(select=1, path=1, **tiny)) == _lib.PATH_TILED
    # the plan call needs iv_head then
    d = desc(select=1, **tiny)
    ws = _lib.workspace_size(d)
    ok = [4096, 8192]
    assert _lib.plan(d, ok, ok, fake_buf(), 4096, ws, 0) == _lib.AIRCACHE_EINVAL
    assert "iv_head" in lib.aircache_last_error().decode()


def test_quantize_argument_errors(lib):
    d = desc(n_layers=2)
    p = [1 << 20, 2 << 20]
    assert _lib.quantize_i8(d, _lib.PlanBuf(), p, p, p, p, 4096, 8192, 0) == _lib.AIRCACHE_EINVAL   # no plan
    assert _lib.quantize_i8(d, fake_buf(), p, p, p, p, 0, 8192, 0) == _lib.AIRCACHE_EINVAL        # no scale
    assert _lib.quantize_i8(d, fake_buf(), p, p, [1 << 20, 0], p, 4096, 8192, 0) == _lib.AIRCACHE_EINVAL
    assert _lib.quantize_i8(d, fake_buf(), p, [(2 << 20) + 8, 4096], p, p, 4096, 8192, 0) == _lib.AIRCACHE_EINVAL
    d.n_layers = 0
    assert _lib.quantize_i8(d, fake_buf(), p, p, p, p, 4096, 8192, 0) == _lib.AIRCACHE_EINVAL


def test_prefill_workspace_size(lib):
    """Two slots of one layer's scoring terms plus the pass's counters: grows
    with the elite cap, independent of the layer count beyond the counters;
    float32 descriptors have no prefill path (size 0)."""
    small = _lib.prefill_workspace_size(desc(max_elite=16))
    big = _lib.prefill_workspace_size(desc(max_elite=64))
    assert 0 < small < big
    assert _lib.prefill_workspace_size(desc(dtype="f32")) == 0
    d1, d28 = _lib.prefill_workspace_size(desc(n_layers=1)), _lib.prefill_workspace_size(desc(n_layers=28))
    assert d28 - d1 < 8 << 20  # counters and elite parts only


def test_prefill_argument_errors(lib):
    d = desc(n_layers=2, n_vis=300, n_txt=40)
    ws_need = _lib.prefill_workspace_size(d)
    q = k = v = 1 << 20
    o = 1 << 40
    buf = fake_buf()
    assert _lib.prefill_layer(d, 2, q, k, v, o, buf, 4096, ws_need, 0) == _lib.AIRCACHE_EINVAL      # layer range
    assert _lib.prefill_layer(d, -1, q, k, v, o, buf, 4096, ws_need, 0) == _lib.AIRCACHE_EINVAL
    assert _lib.prefill_layer(d, 0, q, k, v, o, buf, 4096, ws_need - 1, 0) == _lib.AIRCACHE_EWORKSPACE
    assert _lib.prefill_layer(d, 0, q, k, v, o, _lib.PlanBuf(), 4096, ws_need, 0) == _lib.AIRCACHE_EINVAL
    assert _lib.prefill_layer(d, 0, 0, k, v, o, buf, 4096, ws_need, 0) == _lib.AIRCACHE_EINVAL       # NULL q
    assert _lib.prefill_layer(d, 0, q + 8, k, v, o, buf, 4096, ws_need, 0) == _lib.AIRCACHE_EINVAL   # alignment
    assert _lib.prefill_layer(d, 0, q, k, v, q, buf, 4096, ws_need, 0) == _lib.AIRCACHE_EINVAL       # o overlaps q
    assert _lib.prefill_attention(d, q, k, v, q + 4096, 0) == _lib.AIRCACHE_EINVAL                   # overlap
    f = desc(n_layers=2, dtype="f32")
    assert _lib.prefill_attention(f, q, k, v, o, 0) == _lib.AIRCACHE_EINVAL                          # bf16 only
    assert "bfloat16" in lib.aircache_last_error().decode()


def test_visual_window_descriptor(lib):
    """A visual window (obs_window = -k) resolves to the tiled path, sizes its
    rows for the window, and is refused by the prefill entry points."""
    d = desc(obs_window=-32)
    assert _lib.resolved_path(d) == _lib.PATH_TILED
    assert _lib.workspace_size(d) > 0
    assert _lib.resolved_path(desc(obs_window=-32, path=1)) == _lib.PATH_TILED
    assert _lib.resolved_path(desc(obs_window=-32, select=1)) == _lib.PATH_TILED
    assert _lib.prefill_workspace_size(d) == 0
