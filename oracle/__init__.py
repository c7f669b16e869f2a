"""ORACLE -- test infrastructure only.

ctypes front end of ``sia_oracle.c``, the plain double-precision CPU definition
of the indexer -> Top-K -> sparse MLA attention path. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package; the
HIP library and its Python binding never do.

Parity unpinned: nothing here is checked against a trained model's indexer
weights or real Top-K structure (no weights or data exist for that); every
other function is pinned by ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sia_oracle.c")
_LIB = os.path.join(_HERE, "libsia_oracle.so")

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3fn_value.restype = ctypes.c_double
        L.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        L.oracle_decode_bf16.argtypes = [_vp, _f64p, ctypes.c_int64]
        L.oracle_decode_e4m3fn.argtypes = [_vp, _f64p, ctypes.c_int64]
        L.oracle_indexer_scores.argtypes = [
            ctypes.c_int32, _i32p, _i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
            ctypes.c_int64, _vp, ctypes.c_int32, _f32p, ctypes.c_int32, _vp, _f32p,
            ctypes.c_int32, _f64p, ctypes.c_int64, _i32p]
        L.oracle_topk.argtypes = [ctypes.c_int32, _f64p, ctypes.c_int64, _i32p, ctypes.c_int32,
                                  _i32p, _f64p]
        L.oracle_sparse_mla.argtypes = [
            ctypes.c_int32, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int64, _vp,
            ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32, _i32p, ctypes.c_int32,
            ctypes.c_double, _f64p, _f64p]
        L.oracle_quantize_mxfp8.argtypes = [_vp, ctypes.c_int64, _vp, _vp]
        L.oracle_indexer_scores_mx.argtypes = [
            ctypes.c_int32, _i32p, _i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
            ctypes.c_int64, _vp, _vp, ctypes.c_int32, _vp, _vp, _f32p, ctypes.c_int32, _f64p,
            ctypes.c_int64, _i32p]
        L.oracle_sparse_mla_fp8.argtypes = [
            ctypes.c_int32, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int64, _vp, _vp,
            ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_double, _f64p, _f64p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Use n OpenMP threads from now on; returns the previous count."""
    return int(lib().oracle_set_num_threads(int(n)))


def _np(t, dtype=None):
    """Host, contiguous numpy view of a tensor/array (bf16 -> uint16 bits,
    float8 -> uint8 codes)."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
            a = t.numpy().view(np.uint16)
        elif t.dtype == torch.float8_e4m3fn:
            a = t.view(torch.uint8).numpy()
        else:
            a = t.numpy()
    else:
        a = np.ascontiguousarray(t)
    if dtype is not None:
        a = a.astype(dtype, copy=False)
    return np.ascontiguousarray(a)


def _p(a, ct):
    return a.ctypes.data_as(ct)


def bf16_values(bits) -> np.ndarray:
    b = _np(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    rc = lib().oracle_decode_bf16(_p(b, _vp), _p(out, _f64p), b.size)
    assert rc == 0
    return out


def e4m3fn_values(codes) -> np.ndarray:
    c = _np(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    rc = lib().oracle_decode_e4m3fn(_p(c, _vp), _p(out, _f64p), c.size)
    assert rc == 0
    return out


def indexer_scores(q_seq, q_pos, seq_lens, page_table, idx_k, idx_scale, q_idx, w, ld=None):
    """Scores [Q, ld] (double; -inf where not visible) and row lengths [Q]."""
    q_seq, q_pos = _np(q_seq, np.int32), _np(q_pos, np.int32)
    seq_lens, table = _np(seq_lens, np.int32), _np(page_table, np.int32)
    k = _np(idx_k)
    fp8 = k.dtype == np.uint8
    scale = _np(idx_scale, np.float32) if fp8 else None
    q = _np(q_idx, np.uint16)
    wv = _np(w, np.float32)
    Q, H, D = q.shape
    if ld is None:
        ld = max(1, int(min(q_pos.max(initial=0) + 1, seq_lens.max(initial=0))))
    scores = np.empty((Q, ld), dtype=np.float64)
    row_len = np.empty(Q, dtype=np.int32)
    rc = lib().oracle_indexer_scores(
        Q, _p(q_seq, _i32p), _p(q_pos, _i32p), len(seq_lens), _p(seq_lens, _i32p),
        _p(table, _i32p), table.shape[1], k.shape[0], _p(k, _vp), 1 if fp8 else 0,
        _p(scale, _f32p) if fp8 else None, D, _p(q, _vp), _p(wv, _f32p), H,
        _p(scores, _f64p), ld, _p(row_len, _i32p))
    if rc != 0:
        raise ValueError(f"oracle_indexer_scores failed ({rc})")
    return scores, row_len


def topk(scores, row_len, K):
    """Top-K positions per row (ascending, -1 padded) and their scores."""
    s = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    rl = _np(row_len, np.int32)
    Q, ld = s.shape
    idx = np.empty((Q, K), dtype=np.int32)
    sc = np.empty((Q, K), dtype=np.float64)
    rc = lib().oracle_topk(Q, _p(s, _f64p), ld, _p(rl, _i32p), K, _p(idx, _i32p), _p(sc, _f64p))
    if rc != 0:
        raise ValueError(f"oracle_topk failed ({rc})")
    return idx, sc


def sparse_mla(q_seq, seq_count, page_table, kv, q_attn, idx, sm_scale, d_v=512):
    """Attention output [Q, H, d_v] and lse [Q, H], both double."""
    q_seq = _np(q_seq, np.int32)
    table = _np(page_table, np.int32)
    kvb = _np(kv, np.uint16)
    q = _np(q_attn, np.uint16)
    ix = _np(idx, np.int32)
    Q, H, Dk = q.shape
    out = np.empty((Q, H, d_v), dtype=np.float64)
    lse = np.empty((Q, H), dtype=np.float64)
    rc = lib().oracle_sparse_mla(
        Q, _p(q_seq, _i32p), int(seq_count), _p(table, _i32p), table.shape[1], kvb.shape[0],
        _p(kvb, _vp), Dk, d_v, _p(q, _vp), H, _p(ix, _i32p), ix.shape[1], float(sm_scale),
        _p(out, _f64p), _p(lse, _f64p))
    if rc != 0:
        raise ValueError(f"oracle_sparse_mla failed ({rc})")
    return out, lse


def quantize_mxfp8(x):
    """MXFP8 codes [..., D] and E8M0 scale bytes [..., D/32] of bf16 values x
    (last dimension a multiple of 32)."""
    xb = _np(x, np.uint16)
    D = xb.shape[-1]
    assert D % 32 == 0
    codes = np.empty(xb.shape, dtype=np.uint8)
    scales = np.empty(xb.shape[:-1] + (D // 32,), dtype=np.uint8)
    rc = lib().oracle_quantize_mxfp8(_p(xb, _vp), xb.size // 32, _p(codes, _vp), _p(scales, _vp))
    assert rc == 0
    return codes, scales


def indexer_scores_mx(q_seq, q_pos, seq_lens, page_table, k_codes, k_scales, q_codes, q_scales, w,
                      ld=None):
    """MXFP8-path scores [Q, ld] (double; -inf where not visible) and row lengths."""
    q_seq, q_pos = _np(q_seq, np.int32), _np(q_pos, np.int32)
    seq_lens, table = _np(seq_lens, np.int32), _np(page_table, np.int32)
    kc, ks = _np(k_codes, np.uint8), _np(k_scales, np.uint8)
    qc, qs = _np(q_codes, np.uint8), _np(q_scales, np.uint8)
    wv = _np(w, np.float32)
    Q, H, D = qc.shape
    if ld is None:
        ld = max(1, int(min(q_pos.max(initial=0) + 1, seq_lens.max(initial=0))))
    scores = np.empty((Q, ld), dtype=np.float64)
    row_len = np.empty(Q, dtype=np.int32)
    rc = lib().oracle_indexer_scores_mx(
        Q, _p(q_seq, _i32p), _p(q_pos, _i32p), len(seq_lens), _p(seq_lens, _i32p), _p(table, _i32p),
        table.shape[1], kc.shape[0], _p(kc, _vp), _p(ks, _vp), D, _p(qc, _vp), _p(qs, _vp),
        _p(wv, _f32p), H, _p(scores, _f64p), ld, _p(row_len, _i32p))
    if rc != 0:
        raise ValueError(f"oracle_indexer_scores_mx failed ({rc})")
    return scores, row_len


def sparse_mla_fp8(q_seq, seq_count, page_table, kv8, q_attn, idx, sm_scale):
    """Sparse attention over an FP8 latent cache of 656-byte rows ([pages, 64,
    656] uint8: 512 e4m3 codes, four fp32 block scales, 64 bf16 rope values).
    Returns (out [Q, H, 512], lse [Q, H]) in double."""
    qs, table = _np(q_seq, np.int32), _np(page_table, np.int32)
    kv = _np(kv8, np.uint8)
    assert kv.shape[-1] == 656
    q = _np(q_attn, np.uint16)
    ix = _np(idx, np.int32)
    Q, H, D = q.shape
    K = ix.shape[1] if ix.ndim == 2 else 0
    out = np.zeros((Q, H, 512), dtype=np.float64)
    lse = np.full((Q, H), -np.inf, dtype=np.float64)
    if Q == 0 or K == 0:
        return out, lse
    rc = lib().oracle_sparse_mla_fp8(Q, _p(qs, _i32p), int(seq_count), _p(table, _i32p), table.shape[1],
                                     kv.shape[0], _p(kv, _vp), _p(q, _vp), H, _p(ix, _i32p), K,
                                     float(sm_scale), _p(out, _f64p), _p(lse, _f64p))
    if rc not in (0, -2):
        raise ValueError(f"oracle_sparse_mla_fp8 failed ({rc})")
    return out, lse


def indexer_prepare(xq, xh, wq, wk, k_gamma, k_beta, ww, eps):
    """The indexer's inputs from the projections' inputs, in double precision
    (all bf16 operands are exact in double):
        q = xq Wq^T                         [M, heads * dim]
        k = LayerNorm(xh Wk^T) * gamma + beta   (mean and biased variance over dim)
        w = xh Ww^T                         [M, heads]
    ("Rapid Adaptation ...", section 4.3: query projection, key normalization,
    head-weight projection.) The matrix products are numpy's."""
    def f64(t):
        return t.double().cpu().numpy() if hasattr(t, "double") else np.asarray(t, dtype=np.float64)
    q = f64(xq) @ f64(wq).T
    kp = f64(xh) @ f64(wk).T
    mean = kp.mean(axis=1, keepdims=True)
    var = ((kp - mean) ** 2).mean(axis=1, keepdims=True)
    k = (kp - mean) / np.sqrt(var + float(eps)) * f64(k_gamma) + f64(k_beta)
    w = f64(xh) @ f64(ww).T
    return q, k, w


@dataclass
class Reference:
    scores: np.ndarray
    row_len: np.ndarray
    idx: np.ndarray
    top_scores: np.ndarray
    out: np.ndarray
    lse: np.ndarray


def run(wl, attention: bool = True) -> Reference:
    """The whole path on a ``workloads.Workload`` (any device; copied to host)."""
    s = wl.spec
    scores, row_len = indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                     wl.idx_scale, wl.q_idx, wl.w)
    idx, top = topk(scores, row_len, s.topk)
    out = lse = None
    if attention:
        out, lse = sparse_mla(wl.q_seq, wl.seq_lens.numel(), wl.page_table, wl.kv, wl.q_attn,
                              idx, s.sm_scale)
    return Reference(scores, row_len, idx, top, out, lse)
