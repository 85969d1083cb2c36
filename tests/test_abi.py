"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

from query_adaptive_sparse_amd import native as N
from query_adaptive_sparse_amd.decoder import make_config
from synth import configs

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def test_header_symbols_exported():
    src = "".join(open(os.path.join(INCLUDE, f)).read() for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h"))
    declared = sorted(set(re.findall(r"\b(sparse_(?:decode|prefill|gist_prefill)_\w+)\s*\(", src)))
    assert declared, "no declarations found"
    lib = ctypes.CDLL(N.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in the header but not exported"
    assert sorted(N.EXPORTS) == declared


def _params(name="c3s", **kw):
    p = configs.library_params(configs.get(name))
    p.update(kw)
    return p


def _init(**kw):
    cfg, hm = make_config(**kw)
    return N.sparse_decode_init(cfg)


@pytest.mark.parametrize("name", sorted(configs.ALL))
def test_init_every_workload(name):
    h, n = _init(**_params(name))
    assert n > 0 and n % 256 == 0
    lv = N.sparse_decode_num_levels(h)
    assert lv == (2 if configs.get(name).mode == "hier" else 1)
    N.sparse_decode_destroy(h)


BAD = [
    (dict(batch=0), N.SD_EINVAL, "batch"),
    (dict(kv_batch=3), N.SD_EINVAL, "kv_batch"),
    (dict(n_kv_heads=5), N.SD_EINVAL, "multiple"),
    (dict(n_q_heads=136, n_kv_heads=8), N.SD_EUNSUPPORTED, "query rows per KV group"),
    (dict(head_dim=96), N.SD_EUNSUPPORTED, "head_dim"),
    (dict(n_ctx=16384 + 7), N.SD_EINVAL, "divide"),
    (dict(chunk_size=48, n_ctx=48 * 100), N.SD_EUNSUPPORTED, "power of two"),
    (dict(top_p=0.0), N.SD_EINVAL, "top_p"),
    (dict(top_p=1.5), N.SD_EINVAL, "top_p"),
    (dict(select_scale=0.0), N.SD_EINVAL, "select_scale"),
    (dict(softmax_scale=-1.0), N.SD_EINVAL, "softmax_scale"),
    (dict(mode="topk", top_k=0), N.SD_EINVAL, "top_k"),
    (dict(attend_blocks=-1), N.SD_EINVAL, "attend_blocks"),
    (dict(keep_first=-1), N.SD_EINVAL, "keep_first"),
    (dict(head_mode=[0, 1, 0, 0, 0, 0, 0, 2]), N.SD_EINVAL, "head_mode"),
    (dict(head_mode=[0, 1, 0, 0, 0, 0, 0, 0]), N.SD_EINVAL, "chunk_size must be 1"),
]


@pytest.mark.parametrize("kw,status,msg", BAD, ids=[b[2] + str(i) for i, b in enumerate(BAD)])
def test_init_rejects(kw, status, msg):
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params(**kw))
    assert e.value.status == status
    assert msg in str(e.value)


def test_init_rejects_proxy_and_hier_shapes():
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c5s", route_dim=8))
    assert e.value.status == N.SD_EUNSUPPORTED
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c4s", seg_size=48))
    assert e.value.status == N.SD_EINVAL
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c5s", attend_summary=True))
    assert e.value.status == N.SD_EINVAL


COVERAGE_BAD = [
    (dict(tau=-0.1), N.SD_EINVAL, "tau"),
    (dict(tau=1.0), N.SD_EINVAL, "tau"),
    (dict(tau=float("nan")), N.SD_EINVAL, "tau"),
    (dict(select_scale=0.0), N.SD_EINVAL, "select_scale"),
    (dict(n_ctx=4096 * 16, chunk_size=16), N.SD_EUNSUPPORTED, "chunks per row"),
]


@pytest.mark.parametrize("kw,status,msg", COVERAGE_BAD, ids=[b[2] + str(i) for i, b in enumerate(COVERAGE_BAD)])
def test_init_rejects_coverage(kw, status, msg):
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c3s_coverage", **kw))
    assert e.value.status == status
    assert msg in str(e.value)


def test_init_coverage_needs_summary_route():
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c5s", mode="coverage", tau=0.1))
    assert e.value.status == N.SD_EUNSUPPORTED


MULTI_BAD = [
    (dict(n_queries=-1), N.SD_EINVAL, "n_queries"),
    (dict(n_queries=5), N.SD_EUNSUPPORTED, "query rows per KV group"),
]


@pytest.mark.parametrize("kw,status,msg", MULTI_BAD, ids=[b[2] + str(i) for i, b in enumerate(MULTI_BAD)])
def test_init_rejects_multi_query(kw, status, msg):
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c3s", **kw))
    assert e.value.status == status
    assert msg in str(e.value)


def test_init_multi_query_limits():
    # 16 rows per group on summary routing; proxy routing stops at 8
    h, n1 = _init(**_params("c3s", n_queries=4))
    N.sparse_decode_destroy(h)
    h, n0 = _init(**_params("c3s"))
    N.sparse_decode_destroy(h)
    assert n1 > n0  # four query rows per head: per-row scores and bitmaps grow
    h, _ = _init(**_params("c5s", n_queries=2))
    N.sparse_decode_destroy(h)
    with pytest.raises(N.SparseDecodeError) as e:
        _init(**_params("c5s", n_queries=3))
    assert e.value.status == N.SD_EUNSUPPORTED and "proxy" in str(e.value)


def test_init_null_arguments():
    L = N.lib()
    h = ctypes.c_void_p()
    n = ctypes.c_size_t()
    assert L.sparse_decode_init(None, ctypes.byref(h), ctypes.byref(n)) == N.SD_EINVAL
    assert b"NULL" in L.sparse_decode_last_error()


def test_calls_reject_before_enqueue():
    """Every compute call validates on the host; these all fail without touching a GPU."""
    h, nbytes = _init(**_params())
    L = N.lib()
    t = N.sd_tensors()
    # NULL handle
    assert L.sparse_decode_select(None, 0, 256, None) == N.SD_EINVAL
    # bad level
    assert L.sparse_decode_select(h, 1, 256, None) == N.SD_EINVAL
    assert L.sparse_decode_score_chunks(h, ctypes.byref(t), -1, 256, None) == N.SD_EINVAL
    # workspace NULL / misaligned
    assert L.sparse_decode_select(h, 0, None, None) == N.SD_EWORKSPACE
    assert L.sparse_decode_attend(h, ctypes.byref(t), 0x1008, None) == N.SD_EWORKSPACE
    assert L.sparse_decode_combine(h, 0x1001, 0x2000, 0x3000, None) == N.SD_EWORKSPACE
    # tensors missing
    assert L.sparse_decode_score_chunks(h, None, 0, 256, None) == N.SD_EINVAL
    assert L.sparse_decode_score_chunks(h, ctypes.byref(t), 0, 256, None) == N.SD_EINVAL
    assert b"q must be" in L.sparse_decode_last_error()
    t.q, t.q_sb, t.q_sh = 0x10000, 32 * 128, 128
    assert L.sparse_decode_score_chunks(h, ctypes.byref(t), 0, 256, None) == N.SD_EINVAL
    assert b"kg" in L.sparse_decode_last_error()
    assert L.sparse_decode_attend(h, ctypes.byref(t), 256, None) == N.SD_EINVAL
    t.q_sh = 100  # rows not 16-byte aligned
    assert L.sparse_decode_attend(h, ctypes.byref(t), 256, None) == N.SD_EINVAL
    # outputs
    assert L.sparse_decode_combine(h, 256, None, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_combine(h, 256, 0x2004, 0x3000, None) == N.SD_EINVAL
    v = N.sd_selection_view()
    assert L.sparse_decode_selection_view(h, 256, ctypes.byref(v)) == N.SD_OK
    assert v.list - 256 > 0 and v.len0 == configs.get("c3s").n_chunks
    N.sparse_decode_destroy(h)


def test_step_static_rejects_before_enqueue():
    """The no-allocation step checks everything on the host first: a handle whose workspace is
    larger than the static scratch, a NULL handle, tensors or outputs are rejected without touching
    a GPU."""
    L = N.lib()
    t = N.sd_tensors()
    h, nbytes = _init(**_params("c5_rtpurbo_1m"))
    assert nbytes > 16 << 20
    assert L.sparse_decode_step_static(h, ctypes.byref(t), 0x2000, 0x3000, None) == N.SD_EUNSUPPORTED
    assert b"static scratch" in L.sparse_decode_last_error()
    N.sparse_decode_destroy(h)
    h, nbytes = _init(**_params("c3s"))
    assert nbytes <= 16 << 20
    assert L.sparse_decode_step_static(None, ctypes.byref(t), 0x2000, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_step_static(h, None, 0x2000, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_step_static(h, ctypes.byref(t), 0x2000, 0x3000, None) == N.SD_EINVAL
    assert b"q must be" in L.sparse_decode_last_error()
    t.q, t.q_sb, t.q_sh = 0x10000, 32 * 128, 128
    t.kg, t.vg, t.g_st = 0x20000, 0x30000, 128
    t.k, t.v, t.kv_st = 0x40000, 0x50000, 128
    assert L.sparse_decode_step_static(h, ctypes.byref(t), None, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_step_static(h, ctypes.byref(t), 0x2004, 0x3000, None) == N.SD_EINVAL
    assert b"out" in L.sparse_decode_last_error()
    N.sparse_decode_destroy(h)


def test_workspace_grows_with_batch():
    _, a = _init(**_params("c3s", batch=1, kv_batch=1))
    _, b = _init(**_params("c3s", batch=2, kv_batch=2))
    assert b > a


def test_attend_blocks_default_and_override():
    """One persistent attention workgroup per CU by default; an explicit count is kept."""
    cases = [(dict(), 256), (dict(attend_blocks=7), 7), (dict(dtype="f32", head_dim=64), 256),
             (dict(attend_blocks=4096), 4096)]
    for kw, want in cases:
        h, _ = _init(**_params("c3s", **kw))
        assert N.sparse_decode_attend_blocks(h) == want, kw
        N.sparse_decode_destroy(h)
    assert N.sparse_decode_attend_blocks(None) == 0


# ---- Token-Sparse prefill entry points
def _prefill_cfg(**kw):
    w = configs.get("p1s")
    base = dict(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                seq_len=w.seq_len, window=w.window, tau=w.tau, softmax_scale=w.softmax_scale, kv_dtype=N.SD_BF16)
    base.update(kw)
    cfg = N.sp_config()
    for k, v in base.items():
        setattr(cfg, k, v)
    return cfg


@pytest.mark.parametrize("name", sorted(configs.PREFILL))
def test_prefill_init_every_workload(name):
    w = configs.get(name)
    h, n = N.sparse_prefill_init(_prefill_cfg(batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                                              seq_len=w.seq_len, window=w.window, tau=w.tau))
    # the fp64 proxy scores dominate: B Hq L W x 8 bytes
    assert n >= w.batch * w.n_q_heads * w.seq_len * w.window * 8 and n % 256 == 0
    N.sparse_prefill_destroy(h)


PREFILL_BAD = [
    (dict(batch=0), N.SD_EINVAL, "batch"),
    (dict(n_kv_heads=5), N.SD_EINVAL, "multiple"),
    (dict(head_dim=64), N.SD_EUNSUPPORTED, "head_dim"),
    (dict(kv_dtype=N.SD_F32), N.SD_EUNSUPPORTED, "kv_dtype"),
    (dict(window=0), N.SD_EINVAL, "window"),
    (dict(window=65), N.SD_EUNSUPPORTED, "window"),
    (dict(seq_len=16, window=32), N.SD_EINVAL, "seq_len"),
    (dict(tau=1.0), N.SD_EINVAL, "tau"),
    (dict(tau=-0.5), N.SD_EINVAL, "tau"),
    (dict(softmax_scale=0.0), N.SD_EINVAL, "softmax_scale"),
]


@pytest.mark.parametrize("kw,status,msg", PREFILL_BAD, ids=[b[2] + str(i) for i, b in enumerate(PREFILL_BAD)])
def test_prefill_init_rejects(kw, status, msg):
    with pytest.raises(N.SparseDecodeError) as e:
        N.sparse_prefill_init(_prefill_cfg(**kw))
    assert e.value.status == status
    assert msg in str(e.value)


def test_prefill_calls_reject_before_enqueue():
    h, _ = N.sparse_prefill_init(_prefill_cfg())
    L = N.lib()
    t = N.sp_tensors()
    assert L.sparse_prefill_select(None, ctypes.byref(t), 256, None) == N.SD_EINVAL
    assert L.sparse_prefill_select(h, ctypes.byref(t), None, None) == N.SD_EWORKSPACE
    assert L.sparse_prefill_select(h, ctypes.byref(t), 0x1001, None) == N.SD_EWORKSPACE
    assert L.sparse_prefill_select(h, ctypes.byref(t), 256, None) == N.SD_EINVAL   # null tensors
    t.q, t.k, t.v = 0x1000, 0x2000, 0x3000
    t.q_st, t.kv_st = 100, 128                                                    # q rows not 16-byte aligned
    assert L.sparse_prefill_select(h, ctypes.byref(t), 256, None) == N.SD_EINVAL
    t.q_st = 128
    assert L.sparse_prefill_attend(h, ctypes.byref(t), 256, None, None) == N.SD_EINVAL  # null out
    v = N.sp_view()
    assert L.sparse_prefill_view(h, 256, ctypes.byref(v)) == N.SD_OK
    assert v.words == (configs.get("p1s").seq_len + 31) // 32
    N.sparse_prefill_destroy(h)


def _gist_cfg(**kw):
    w = configs.get("p2s")
    c = N.gp_config()
    c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    c.n_tokens, c.chunk_size, c.kv_dtype, c.softmax_scale = w.n_tokens, w.chunk_size, N.SD_BF16, w.softmax_scale
    for k, v in kw.items():
        setattr(c, k, v)
    return c


GIST_BAD = [
    (dict(batch=0), N.SD_EINVAL, "batch"),
    (dict(n_kv_heads=5), N.SD_EINVAL, "multiple"),
    (dict(head_dim=64), N.SD_EUNSUPPORTED, "head_dim"),
    (dict(kv_dtype=N.SD_F32), N.SD_EUNSUPPORTED, "kv_dtype"),
    (dict(chunk_size=0), N.SD_EINVAL, "chunk_size"),
    (dict(n_tokens=0), N.SD_EINVAL, "n_tokens"),
    (dict(n_tokens=1 << 31), N.SD_EINVAL, "n_tokens"),
    (dict(n_tokens=2050), N.SD_EINVAL, "multiple of chunk_size"),
    (dict(softmax_scale=float("inf")), N.SD_EINVAL, "softmax_scale"),
]


@pytest.mark.parametrize("kw,status,msg", GIST_BAD, ids=[b[2] + str(i) for i, b in enumerate(GIST_BAD)])
def test_gist_init_rejects(kw, status, msg):
    with pytest.raises(N.SparseDecodeError) as e:
        N.sparse_gist_prefill_init(_gist_cfg(**kw))
    assert e.value.status == status
    assert msg in str(e.value)


def test_gist_attend_rejects_before_enqueue():
    h, nbytes = N.sparse_gist_prefill_init(_gist_cfg())
    w = configs.get("p2s")
    # the fp16 value copy (gists, then raw rows, per sequence and KV head) dominates the workspace
    assert nbytes >= w.batch * w.n_kv_heads * (w.n_tokens + w.n_tokens // w.chunk_size) * w.head_dim * 2
    L = N.lib()
    t = N.gp_tensors()
    ws = 0x100000
    assert L.sparse_gist_prefill_attend(None, ctypes.byref(t), ws, 0x1000, 0x2000, None) == N.SD_EINVAL
    assert L.sparse_gist_prefill_attend(h, ctypes.byref(t), None, 0x1000, 0x2000, None) == N.SD_EWORKSPACE
    assert L.sparse_gist_prefill_attend(h, ctypes.byref(t), ws + 16, 0x1000, 0x2000, None) == N.SD_EWORKSPACE
    assert L.sparse_gist_prefill_attend(h, None, ws, 0x1000, 0x2000, None) == N.SD_EINVAL
    assert L.sparse_gist_prefill_attend(h, ctypes.byref(t), ws, 0x1000, 0x2000, None) == N.SD_EINVAL  # null tensors
    t.q, t.k, t.v, t.qg, t.kg, t.vg = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000
    t.q_st = t.kv_st = t.qg_st = t.kvg_st = 128
    t.kvg_st = 100                                                      # gist rows not 16-byte aligned
    assert L.sparse_gist_prefill_attend(h, ctypes.byref(t), ws, 0x1000, 0x2000, None) == N.SD_EINVAL
    t.kvg_st = 128
    assert L.sparse_gist_prefill_attend(h, ctypes.byref(t), ws, None, 0x2000, None) == N.SD_EINVAL  # null out
    assert L.sparse_gist_prefill_attend(h, ctypes.byref(t), ws, 0x1000, 0x2008, None) == N.SD_EINVAL  # misaligned
    N.sparse_gist_prefill_destroy(h)


def test_step_rejects_before_enqueue():
    """The whole-step call checks its handle, workspace, tensors and outputs on the host before it
    enqueues anything."""
    L = N.lib()
    t = N.sd_tensors()
    h, _ = _init(**_params("c3s"))
    assert L.sparse_decode_step(None, ctypes.byref(t), 256, 0x2000, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_step(h, ctypes.byref(t), None, 0x2000, 0x3000, None) == N.SD_EWORKSPACE
    assert L.sparse_decode_step(h, ctypes.byref(t), 0x104, 0x2000, 0x3000, None) == N.SD_EWORKSPACE
    assert L.sparse_decode_step(h, None, 256, 0x2000, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_step(h, ctypes.byref(t), 256, 0x2000, 0x3000, None) == N.SD_EINVAL
    assert b"q must be" in L.sparse_decode_last_error()
    t.q, t.q_sb, t.q_sh = 0x10000, 32 * 128, 128
    t.kg, t.vg, t.g_st = 0x20000, 0x30000, 128
    t.k, t.v, t.kv_st = 0x40000, 0x50000, 128
    assert L.sparse_decode_step(h, ctypes.byref(t), 256, None, 0x3000, None) == N.SD_EINVAL
    assert L.sparse_decode_step(h, ctypes.byref(t), 256, 0x2004, 0x3000, None) == N.SD_EINVAL
    assert b"step: out" in L.sparse_decode_last_error()
    N.sparse_decode_destroy(h)
