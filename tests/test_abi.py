"""The C ABI on a machine without a GPU: the library loads, exports every entry
point declared in include/sia.h, validates arguments on the host before any
launch, and the host-side zigzag assignment matches the pages' worked example."""
import ctypes
import json
import os
import re

import pytest

import indexer_top_sparse_02_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "sia.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[a-z_ ]*?(?:int|size_t|char \*|void)\s*\*?\s*([a-z_0-9]+)\s*\(", src, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    decl = _declared()
    assert len(decl) >= 12
    for name in decl:
        assert hasattr(lib, name), name
    assert set(decl) == set(L.EXPORTS)


def test_version():
    assert L.version() == 100


def _fake(n=64):
    # host buffers stand in for device pointers: validation must reject the call
    # before anything dereferences them or touches the GPU
    return (ctypes.c_int32 * n)()


def _descs(**kw):
    buf = _fake()
    addr = ctypes.addressof(buf)
    pt = L.PageTable(addr, addr, kw.get("batch", 1), kw.get("max_pages", 4), kw.get("page_size", 64))
    c = L.PagedCache(addr, addr if kw.get("fp8", True) else None, kw.get("num_pages", 4),
                     kw.get("dim", 128), 1 if kw.get("fp8", True) else 0)
    q = L.Queries(kw.get("num_q", 1), addr, addr, kw.get("group", 1), kw.get("max_visible", 100))
    return buf, pt, c, q, addr


def _topk(pt, c, q, addr, heads=64, topk=16, out=True, ws=None, ws_bytes=1 << 20):
    return L.lib().sparse_indexer_topk(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), addr, addr,
                                       heads, topk, addr if out else None, None, -1,
                                       addr if ws is None else ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=32), L.SIA_ERR_UNSUPPORTED),
    (dict(dim=96), L.SIA_ERR_UNSUPPORTED),
    (dict(batch=0), L.SIA_ERR_INVALID_ARG),
    (dict(max_pages=0), L.SIA_ERR_INVALID_ARG),
    (dict(num_q=-1), L.SIA_ERR_INVALID_ARG),
    (dict(group=0), L.SIA_ERR_INVALID_ARG),
    (dict(max_visible=1000), L.SIA_ERR_INVALID_ARG),      # > max_pages * 64
    (dict(num_pages=0), L.SIA_ERR_INVALID_ARG),
])
def test_indexer_rejects_bad_descriptors(kw, code):
    buf, pt, c, q, addr = _descs(**kw)
    assert _topk(pt, c, q, addr) == code
    assert L.last_error()


def test_indexer_rejects_bad_scalars_and_pointers():
    buf, pt, c, q, addr = _descs()
    assert _topk(pt, c, q, addr, heads=65) == L.SIA_ERR_UNSUPPORTED
    assert _topk(pt, c, q, addr, heads=0) == L.SIA_ERR_UNSUPPORTED
    assert _topk(pt, c, q, addr, topk=0) == L.SIA_ERR_UNSUPPORTED
    assert _topk(pt, c, q, addr, out=False) == L.SIA_ERR_INVALID_ARG
    c.scale = None                                          # fp8 without scales
    assert _topk(pt, c, q, addr) == L.SIA_ERR_INVALID_ARG
    lib = L.lib()
    assert lib.sparse_indexer_topk(None, ctypes.byref(c), ctypes.byref(q), addr, addr, 64, 16, addr,
                                   None, -1, addr, 1 << 20, None) == L.SIA_ERR_INVALID_ARG


def test_indexer_rejects_small_or_missing_workspace():
    buf, pt, c, q, addr = _descs()
    need = L.lib().sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), 64, 16)
    assert need >= 256
    assert _topk(pt, c, q, addr, ws_bytes=need - 1) == L.SIA_ERR_WORKSPACE
    rc = L.lib().sparse_indexer_topk(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), addr, addr,
                                     64, 16, addr, None, -1, None, need, None)
    assert rc == L.SIA_ERR_WORKSPACE


def test_workspace_size_grows_with_context():
    lib = L.lib()
    buf, pt, c, q, addr = _descs(max_pages=2048, max_visible=131072, num_q=128, group=2, batch=64)
    big = lib.sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), 64, 2048)
    # room for a candidate key and position and a dense key per visible position of
    # every query (the worst case keeps every position), plus per-part histograms
    assert big >= 128 * 131072 * 4
    q.max_visible = 4000
    small = lib.sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), 64, 2048)
    assert 128 * 4000 * 4 <= small < big
    assert lib.sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), 64, 0) == 0


def test_attention_rejects_bad_arguments():
    lib = L.lib()
    buf, pt, _, q, addr = _descs()
    kv = L.PagedCache(addr, None, 4, 576, 0)

    def call(heads=128, d_v=512, topk=64, kvd=kv, scale=0.05, ws_bytes=1 << 30):
        return lib.sparse_mla_attention(ctypes.byref(pt), ctypes.byref(kvd), ctypes.byref(q), addr, heads,
                                        d_v, addr, topk, scale, addr, None, addr, ws_bytes, None)
    assert call(heads=24) == L.SIA_ERR_UNSUPPORTED
    assert call(d_v=256) == L.SIA_ERR_UNSUPPORTED
    assert call(topk=0) == L.SIA_ERR_INVALID_ARG
    assert call(kvd=L.PagedCache(addr, None, 4, 512, 0)) == L.SIA_ERR_UNSUPPORTED
    # fp8 latent rows carry their scales: a separate scale pool is refused; MXFP8
    # is an index-cache format only
    assert call(kvd=L.PagedCache(addr, addr, 4, 576, 1)) == L.SIA_ERR_INVALID_ARG
    assert call(kvd=L.PagedCache(addr, None, 4, 576, 2)) == L.SIA_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == L.SIA_ERR_INVALID_ARG
    assert call(ws_bytes=10) == L.SIA_ERR_WORKSPACE
    assert lib.sia_mla_workspace_size(ctypes.byref(q), 128, 512, 2048) >= 256


def test_topk_from_scores_rejects_bad_arguments():
    lib = L.lib()
    a = ctypes.addressof(_fake())
    assert lib.sparse_topk_from_scores(a, 10, a, 1, 20, 4, a, None, a, 1 << 20, None) == L.SIA_ERR_INVALID_ARG
    assert lib.sparse_topk_from_scores(a, 10, a, 1, 5, 0, a, None, a, 1 << 20, None) == L.SIA_ERR_UNSUPPORTED
    assert lib.sparse_topk_from_scores(None, 10, a, 1, 5, 4, a, None, a, 1 << 20, None) == L.SIA_ERR_INVALID_ARG


def test_zigzag_matches_pages_example():
    with open(os.path.join(ROOT, "tests", "golden", "zigzag_8.json")) as f:
        g = json.load(f)
    assert L.zigzag_assign(g["shards"]) == g["cards"]


@pytest.mark.parametrize("S", [1, 2, 5, 8, 9, 64, 255])
def test_zigzag_covers_every_shard_once_with_balanced_linear_cost(S):
    pairs = L.zigzag_assign(S)
    flat = [s for p in pairs for s in p]
    assert sorted(flat) == list(range(S))
    assert len(pairs) == (S + 1) // 2
    # with cost linear in the shard index, every full pair costs the same
    full = [sum(p) for p in pairs if len(p) == 2]
    assert len(set(full)) <= 1


def test_noalloc_attention_rejects_calls_beyond_its_scratch():
    """sparse_mla_attention_noalloc checks its scratch need on the host: a call
    whose row-slice partials exceed SIA_MLA_NOALLOC_MAX_BYTES (64 queries x 4
    slices of 8192 rows x 128 heads) is refused with SIA_ERR_WORKSPACE before
    anything is launched; bad shapes are refused like the workspace form's."""
    buf, pt, c, q, addr = _descs(num_q=64)
    kv = L.PagedCache(addr, None, 4, 576, 0)
    f = L.lib().sparse_mla_attention_noalloc
    rc = f(ctypes.byref(pt), ctypes.byref(kv), ctypes.byref(q), addr, 128, 512, addr, 8192,
           ctypes.c_float(0.04), addr, None, None)
    assert rc == L.SIA_ERR_WORKSPACE
    assert "no-allocation" in L.last_error()
    need = L.lib().sia_mla_workspace_size(ctypes.byref(q), 128, 512, 8192)
    assert need > L.MLA_NOALLOC_MAX_BYTES
    rc = f(ctypes.byref(pt), ctypes.byref(kv), ctypes.byref(q), addr, 24, 512, addr, 256,
           ctypes.c_float(0.04), addr, None, None)
    assert rc == L.SIA_ERR_UNSUPPORTED
    rc = f(ctypes.byref(pt), ctypes.byref(kv), ctypes.byref(q), addr, 128, 512, addr, 256,
           ctypes.c_float(float("nan")), addr, None, None)
    assert rc == L.SIA_ERR_INVALID_ARG
    assert L.MLA_NOALLOC_MAX_BYTES == _header_noalloc_max()


def _header_noalloc_max():
    src = open(os.path.join(ROOT, "include", "sia.h")).read()
    m = re.search(r"#define SIA_MLA_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    return int(m.group(1)) << int(m.group(2))
