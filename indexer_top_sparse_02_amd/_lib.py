"""ctypes binding of libsia.so (include/sia.h) for torch tensors.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. Tensors must be contiguous and on the GPU; work is enqueued on the
current torch stream unless ``stream`` is given. The library must be built
(``python -m indexer_top_sparse_02_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsia.so")

SIA_OK = 0
SIA_ERR_INVALID_ARG = -1
SIA_ERR_UNSUPPORTED = -2
SIA_ERR_WORKSPACE = -3
SIA_ERR_HIP = -4
SIA_BF16 = 0
SIA_FP8_E4M3FN = 1
SIA_MXFP8_E4M3 = 2
SCHED_AUTO, SCHED_NAIVE, SCHED_HEAVY_FIRST, SCHED_ZIGZAG = -1, 0, 1, 2
DEVSTATUS_BAD_SEQ, DEVSTATUS_BAD_PAGE, DEVSTATUS_ROW_TOO_LONG, DEVSTATUS_BAD_INDEX = 1, 2, 4, 8

EXPORTS = [
    "sia_indexer_workspace_size", "sparse_indexer_topk", "sparse_indexer_topk_traced",
    "sparse_indexer_topk_mxfp8", "sparse_indexer_scores_mxfp8", "sia_quantize_mxfp8",
    "sia_indexer_prepare_workspace_size", "sia_indexer_prepare",
    "sparse_indexer_scores",
    "sia_topk_workspace_size", "sparse_topk_from_scores", "sia_mla_workspace_size",
    "sparse_mla_attention", "sparse_mla_attention_noalloc", "sia_zigzag_assign",
    "sia_clear_device_status", "sia_read_device_status", "sia_last_error", "sia_version",
]


class SiaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"sia error {code}: {msg}")
        self.code = code


class PageTable(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


class PagedCache(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class IndexerWeights(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("k_gamma", ctypes.c_void_p),
                ("k_beta", ctypes.c_void_p), ("ww", ctypes.c_void_p), ("dq", ctypes.c_int32),
                ("dh", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("eps", ctypes.c_float)]


class Queries(ctypes.Structure):
    _fields_ = [("num_q", ctypes.c_int32), ("q_seq", ctypes.c_void_p), ("q_pos", ctypes.c_void_p),
                ("group", ctypes.c_int32), ("max_visible", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m indexer_top_sparse_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, c_i32, c_i64, c_sz, c_f = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_size_t, ctypes.c_float)
        pPT, pPC, pQ = ctypes.POINTER(PageTable), ctypes.POINTER(PagedCache), ctypes.POINTER(Queries)
        sig = {
            "sia_indexer_workspace_size": (c_sz, [pPT, pPC, pQ, c_i32, c_i32]),
            "sparse_indexer_topk": (ctypes.c_int, [pPT, pPC, pQ, P, P, c_i32, c_i32, P, P, c_i32, P,
                                                   c_sz, P]),
            "sparse_indexer_topk_traced": (ctypes.c_int, [pPT, pPC, pQ, P, P, c_i32, c_i32, P, P, c_i32,
                                                          P, c_sz, P, P, c_i32]),
            "sparse_indexer_scores": (ctypes.c_int, [pPT, pPC, pQ, P, P, c_i32, P, c_i64, P, c_sz, P]),
            "sparse_indexer_topk_mxfp8": (ctypes.c_int, [pPT, pPC, pQ, P, P, P, c_i32, c_i32, P, P, c_i32, P,
                                                         c_sz, P]),
            "sparse_indexer_scores_mxfp8": (ctypes.c_int, [pPT, pPC, pQ, P, P, P, c_i32, P, c_i64, P, c_sz,
                                                           P]),
            "sia_quantize_mxfp8": (ctypes.c_int, [P, c_i64, c_i32, P, P, P]),
            "sia_indexer_prepare_workspace_size": (c_sz, [ctypes.POINTER(IndexerWeights), c_i32]),
            "sia_indexer_prepare": (ctypes.c_int, [ctypes.POINTER(IndexerWeights), P, P, pPT, pPC, pQ, P, P, P,
                                                   P, P, P, c_sz, ctypes.POINTER(ctypes.c_void_p),
                                                   ctypes.POINTER(ctypes.c_void_p)]),
            "sia_topk_workspace_size": (c_sz, [c_i32, c_i32, c_i32]),
            "sparse_topk_from_scores": (ctypes.c_int, [P, c_i64, P, c_i32, c_i32, c_i32, P, P, P, c_sz,
                                                       P]),
            "sia_mla_workspace_size": (c_sz, [pQ, c_i32, c_i32, c_i32]),
            "sparse_mla_attention": (ctypes.c_int, [pPT, pPC, pQ, P, c_i32, c_i32, P, c_i32, c_f, P, P,
                                                    P, c_sz, P]),
            "sparse_mla_attention_noalloc": (ctypes.c_int, [pPT, pPC, pQ, P, c_i32, c_i32, P, c_i32, c_f,
                                                            P, P, P]),
            "sia_zigzag_assign": (ctypes.c_int, [c_i32, ctypes.POINTER(ctypes.c_int32)]),
            "sia_clear_device_status": (ctypes.c_int, [P, P]),
            "sia_read_device_status": (ctypes.c_int, [P, P, ctypes.POINTER(ctypes.c_uint32)]),
            "sia_last_error": (ctypes.c_char_p, []),
            "sia_version": (ctypes.c_int, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().sia_last_error().decode()


def _check(rc: int):
    if rc != SIA_OK:
        raise SiaError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def page_table_desc(page_table: torch.Tensor, seq_lens: torch.Tensor) -> PageTable:
    return PageTable(_ptr(page_table), _ptr(seq_lens), int(page_table.shape[0]),
                     int(page_table.shape[1]), 64)


def cache_desc(rows: torch.Tensor, scale: Optional[torch.Tensor] = None) -> PagedCache:
    """bf16 rows (no scale); e4m3 codes with fp32 per-token scales; or e4m3
    codes with uint8 E8M0 block scales (MXFP8)."""
    if rows.dtype == torch.bfloat16:
        dt = SIA_BF16
    elif rows.dtype in (torch.uint8, torch.float8_e4m3fn):
        dt = SIA_MXFP8_E4M3 if scale is not None and scale.dtype == torch.uint8 else SIA_FP8_E4M3FN
    else:
        raise ValueError(f"unsupported cache dtype {rows.dtype}")
    return PagedCache(_ptr(rows), _ptr(scale), int(rows.shape[0]), int(rows.shape[2]), dt)


KV8_ROW_BYTES = 656   # fp8 latent row: 512 e4m3 codes, 4 fp32 block scales, 64 bf16 rope values


def kv_desc(kv: torch.Tensor) -> PagedCache:
    """Latent cache descriptor: bf16 [pages, 64, 576], or fp8 rows as uint8
    [pages, 64, 656] (512 e4m3 codes, four fp32 scales per 128, 64 bf16 rope)."""
    if kv.dtype == torch.uint8 and int(kv.shape[2]) == KV8_ROW_BYTES:
        return PagedCache(_ptr(kv), None, int(kv.shape[0]), 576, SIA_FP8_E4M3FN)
    return cache_desc(kv)


def visible_max(q_seq, q_pos, seq_lens) -> int:
    """max_j min(t_j + 1, n_{b_j}) (synchronizes)."""
    if q_seq.numel() == 0:
        return 0
    n = seq_lens.long()[q_seq.long().clamp(0, seq_lens.numel() - 1)]
    return int(torch.minimum(q_pos.long() + 1, n).max().item())


def queries_desc(q_seq, q_pos, group: int, max_visible: int) -> Queries:
    return Queries(int(q_seq.numel()), _ptr(q_seq), _ptr(q_pos), int(group), int(max_visible))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-initialized workspace (the status word starts clear)."""
    return torch.zeros(max(256, int(nbytes)), dtype=torch.uint8, device=device)


def indexer_workspace_size(page_table, seq_lens, rows, scale, q_seq, q_pos, heads, topk, *,
                           group=1, max_visible=None) -> int:
    if max_visible is None:
        max_visible = visible_max(q_seq, q_pos, seq_lens)
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(rows, scale)
    q = queries_desc(q_seq, q_pos, group, max_visible)
    return int(lib().sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q),
                                                int(heads), int(topk)))


def sparse_indexer_topk(page_table, seq_lens, rows, scale, q_seq, q_pos, q_idx, w, topk, *,
                        group=1, max_visible=None, out_idx=None, out_score=None, want_score=False,
                        sched=SCHED_AUTO, workspace=None, stream=None):
    """Fused indexer + Top-K. Returns (idx int32 [Q, topk], score fp32 [Q, topk] or None)."""
    Q, H = int(q_idx.shape[0]), int(q_idx.shape[1])
    dev = q_idx.device
    if max_visible is None:
        max_visible = visible_max(q_seq, q_pos, seq_lens)
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(rows, scale)
    q = queries_desc(q_seq, q_pos, group, max_visible)
    need = lib().sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), H,
                                            int(topk))
    if need == 0:
        raise SiaError(SIA_ERR_INVALID_ARG, "invalid shapes for the indexer")
    if workspace is None:
        workspace = new_workspace(need, dev)
    if out_idx is None:
        out_idx = torch.empty((Q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_score:
        out_score = torch.empty((Q, topk), dtype=torch.float32, device=dev)
    _check(lib().sparse_indexer_topk(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), _ptr(q_idx),
                                     _ptr(w), H, int(topk), _ptr(out_idx), _ptr(out_score), int(sched),
                                     _ptr(workspace), workspace.numel(), _stream(stream)))
    return out_idx, out_score


def sparse_indexer_topk_traced(page_table, seq_lens, rows, scale, q_seq, q_pos, q_idx, w, topk,
                               trace, *, group=1, max_visible=None, out_idx=None, sched=SCHED_AUTO,
                               workspace=None, stream=None):
    """sparse_indexer_topk that also fills `trace` (int64 [n, 4] on the GPU) with
    one record per workgroup of the causal stream kernel: hardware ids
    (XCC_ID << 32 | HW_ID), start and end ticks of a 100 MHz clock, tiles run."""
    Q, H = int(q_idx.shape[0]), int(q_idx.shape[1])
    dev = q_idx.device
    if max_visible is None:
        max_visible = visible_max(q_seq, q_pos, seq_lens)
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(rows, scale)
    q = queries_desc(q_seq, q_pos, group, max_visible)
    need = lib().sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), H,
                                            int(topk))
    if workspace is None:
        workspace = new_workspace(need, dev)
    if out_idx is None:
        out_idx = torch.empty((Q, topk), dtype=torch.int32, device=dev)
    _check(lib().sparse_indexer_topk_traced(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), _ptr(q_idx),
                                            _ptr(w), H, int(topk), _ptr(out_idx), None, int(sched),
                                            _ptr(workspace), workspace.numel(), _stream(stream), _ptr(trace),
                                            int(trace.shape[0])))
    return out_idx


def sparse_indexer_topk_mxfp8(page_table, seq_lens, k_codes, k_scales, q_seq, q_pos, q_codes, q_scales, w,
                              topk, *, group=1, max_visible=None, out_idx=None, out_score=None,
                              want_score=False, sched=SCHED_AUTO, workspace=None, stream=None):
    """The MXFP8 index path: MXFP8 cache (e4m3 codes + E8M0 block scales) and
    MXFP8 query. Returns (idx int32 [Q, topk], score fp32 [Q, topk] or None)."""
    Q, H = int(q_codes.shape[0]), int(q_codes.shape[1])
    dev = q_codes.device
    if max_visible is None:
        max_visible = visible_max(q_seq, q_pos, seq_lens)
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(k_codes, k_scales)
    q = queries_desc(q_seq, q_pos, group, max_visible)
    need = lib().sia_indexer_workspace_size(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), H,
                                            int(topk))
    if need == 0:
        raise SiaError(SIA_ERR_INVALID_ARG, "invalid shapes for the MXFP8 indexer")
    if workspace is None:
        workspace = new_workspace(need, dev)
    if out_idx is None:
        out_idx = torch.empty((Q, topk), dtype=torch.int32, device=dev)
    if out_score is None and want_score:
        out_score = torch.empty((Q, topk), dtype=torch.float32, device=dev)
    _check(lib().sparse_indexer_topk_mxfp8(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), _ptr(q_codes),
                                           _ptr(q_scales), _ptr(w), H, int(topk), _ptr(out_idx),
                                           _ptr(out_score), int(sched), _ptr(workspace), workspace.numel(),
                                           _stream(stream)))
    return out_idx, out_score


def sparse_indexer_scores_mxfp8(page_table, seq_lens, k_codes, k_scales, q_seq, q_pos, q_codes, q_scales, w,
                                *, group=1, max_visible=None, ld=None, stream=None):
    """MXFP8-path scores without selection: fp32 [Q, ld], -inf where not visible."""
    Q, H = int(q_codes.shape[0]), int(q_codes.shape[1])
    if max_visible is None:
        max_visible = visible_max(q_seq, q_pos, seq_lens)
    if ld is None:
        ld = max(1, max_visible)
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(k_codes, k_scales)
    q = queries_desc(q_seq, q_pos, group, max_visible)
    workspace = new_workspace(256, q_codes.device)
    scores = torch.empty((Q, ld), dtype=torch.float32, device=q_codes.device)
    _check(lib().sparse_indexer_scores_mxfp8(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), _ptr(q_codes),
                                             _ptr(q_scales), _ptr(w), H, _ptr(scores), int(ld), _ptr(workspace),
                                             workspace.numel(), _stream(stream)))
    return scores


def quantize_mxfp8(x: torch.Tensor, codes=None, scales=None, stream=None):
    """MXFP8 codes (uint8, shape of x) and E8M0 scale bytes (last dim / 32) of
    the bf16 tensor x (last dimension a multiple of 32)."""
    if x.dtype != torch.bfloat16:
        raise ValueError("quantize_mxfp8 takes bf16")
    D = int(x.shape[-1])
    rows = x.numel() // D if D else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(tuple(x.shape[:-1]) + (D // 32,), dtype=torch.uint8, device=x.device)
    _check(lib().sia_quantize_mxfp8(_ptr(x), rows, D, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def indexer_prepare(xq, xh, wq, wk, k_gamma, k_beta, ww, page_table, seq_lens, k_codes, k_scales, q_seq, q_pos,
                    *, eps=1e-6, streams=None, events=None, q_bf16=None, k_bf16=None, workspace=None):
    """Three-stream indexer input preparation (MXFP8 path): returns (q_codes,
    q_scales, w) and writes the tokens' MXFP8 keys into (k_codes, k_scales) at
    (q_seq, q_pos). `streams`: three torch streams (default: the current stream
    three times, a serial chain); the result joins back into streams[0]."""
    M = int(xq.shape[0])
    dim = int(wk.shape[0])
    heads = int(ww.shape[0])
    dev = xq.device
    W = IndexerWeights(_ptr(wq), _ptr(wk), _ptr(k_gamma), _ptr(k_beta), _ptr(ww), int(xq.shape[1]),
                       int(xh.shape[1]), heads, dim, float(eps))
    need = lib().sia_indexer_prepare_workspace_size(ctypes.byref(W), M)
    if need == 0:
        raise SiaError(SIA_ERR_INVALID_ARG, "invalid shapes for the input preparation")
    if workspace is None:
        workspace = new_workspace(need, dev)
    if streams is None:
        streams = [torch.cuda.current_stream()] * 3
    if events is None:
        events = [torch.cuda.Event() for _ in range(3)]
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(k_codes, k_scales)
    q = queries_desc(q_seq, q_pos, 1, 0)
    q_codes = torch.empty((M, heads, dim), dtype=torch.uint8, device=dev)
    q_scales = torch.empty((M, heads, dim // 32), dtype=torch.uint8, device=dev)
    w = torch.empty((M, heads), dtype=torch.float32, device=dev)
    for e, st in zip(events, [streams[0], streams[1], streams[2]]):
        e.record(st)   # (makes sure every event exists before its handle is taken)
    sh = (ctypes.c_void_p * 3)(*[st.cuda_stream for st in streams])
    eh = (ctypes.c_void_p * 3)(*[e.cuda_event for e in events])
    _check(lib().sia_indexer_prepare(ctypes.byref(W), _ptr(xq), _ptr(xh), ctypes.byref(pt), ctypes.byref(c),
                                     ctypes.byref(q), _ptr(q_codes), _ptr(q_scales), _ptr(w), _ptr(q_bf16),
                                     _ptr(k_bf16), _ptr(workspace), workspace.numel(), sh, eh))
    return q_codes, q_scales, w


def sparse_indexer_scores(page_table, seq_lens, rows, scale, q_seq, q_pos, q_idx, w, *, group=1,
                          max_visible=None, ld=None, workspace=None, stream=None):
    """Indexer scores without selection: fp32 [Q, ld], -inf where not visible."""
    Q, H = int(q_idx.shape[0]), int(q_idx.shape[1])
    if max_visible is None:
        max_visible = visible_max(q_seq, q_pos, seq_lens)
    if ld is None:
        ld = max(1, max_visible)
    pt, c = page_table_desc(page_table, seq_lens), cache_desc(rows, scale)
    q = queries_desc(q_seq, q_pos, group, max_visible)
    if workspace is None:
        workspace = new_workspace(256, q_idx.device)
    scores = torch.empty((Q, ld), dtype=torch.float32, device=q_idx.device)
    _check(lib().sparse_indexer_scores(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(q), _ptr(q_idx),
                                       _ptr(w), H, _ptr(scores), int(ld), _ptr(workspace),
                                       workspace.numel(), _stream(stream)))
    return scores


def sparse_topk_from_scores(scores, row_len, topk, *, max_row_len=None, want_score=True,
                            stream=None):
    """Top-K of given fp32 score rows (row j: candidates 0..row_len[j]-1)."""
    Q, ld = int(scores.shape[0]), int(scores.shape[1])
    if max_row_len is None:
        max_row_len = int(row_len.max().item()) if Q else 0
    need = lib().sia_topk_workspace_size(Q, int(max_row_len), int(topk))
    if need == 0:
        raise SiaError(SIA_ERR_INVALID_ARG, "invalid shapes for top-k")
    ws = new_workspace(need, scores.device)
    idx = torch.empty((Q, topk), dtype=torch.int32, device=scores.device)
    sc = torch.empty((Q, topk), dtype=torch.float32, device=scores.device) if want_score else None
    _check(lib().sparse_topk_from_scores(_ptr(scores), ld, _ptr(row_len), Q, int(max_row_len),
                                         int(topk), _ptr(idx), _ptr(sc), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    return idx, sc


def mla_workspace_size(num_q, heads, topk, d_v=512) -> int:
    q = Queries(int(num_q), None, None, 1, 0)
    return int(lib().sia_mla_workspace_size(ctypes.byref(q), int(heads), int(d_v), int(topk)))


def sparse_mla_attention(page_table, seq_lens, kv, q_seq, q, idx, sm_scale, *, d_v=512, out=None,
                         lse=None, want_lse=False, workspace=None, stream=None):
    """Sparse MLA attention. Returns (out bf16 [Q, H, d_v], lse fp32 [Q, H] or None)."""
    Q, H = int(q.shape[0]), int(q.shape[1])
    topk = int(idx.shape[1])
    pt, c = page_table_desc(page_table, seq_lens), kv_desc(kv)
    qd = Queries(Q, _ptr(q_seq), None, 1, 0)
    need = lib().sia_mla_workspace_size(ctypes.byref(qd), H, int(d_v), topk)
    if need == 0:
        raise SiaError(SIA_ERR_UNSUPPORTED, f"attention shapes H={H} d_v={d_v} topk={topk}")
    if workspace is None:
        workspace = new_workspace(need, q.device)
    if out is None:
        out = torch.empty((Q, H, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Q, H), dtype=torch.float32, device=q.device)
    _check(lib().sparse_mla_attention(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(qd), _ptr(q), H,
                                      int(d_v), _ptr(idx), topk, float(sm_scale), _ptr(out), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def sparse_mla_attention_noalloc(page_table, seq_lens, kv, q_seq, q, idx, sm_scale, *, d_v=512,
                                 out=None, lse=None, want_lse=False, stream=None):
    """Sparse MLA attention with the library's static scratch instead of a
    workspace (no device allocation inside the library). Returns (out, lse)."""
    Q, H = int(q.shape[0]), int(q.shape[1])
    topk = int(idx.shape[1])
    pt, c = page_table_desc(page_table, seq_lens), kv_desc(kv)
    qd = Queries(Q, _ptr(q_seq), None, 1, 0)
    if out is None:
        out = torch.empty((Q, H, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Q, H), dtype=torch.float32, device=q.device)
    _check(lib().sparse_mla_attention_noalloc(ctypes.byref(pt), ctypes.byref(c), ctypes.byref(qd), _ptr(q),
                                              H, int(d_v), _ptr(idx), topk, float(sm_scale), _ptr(out),
                                              _ptr(lse), _stream(stream)))
    return out, lse


MLA_NOALLOC_MAX_BYTES = 64 << 20   # SIA_MLA_NOALLOC_MAX_BYTES of include/sia.h


def zigzag_assign(num_shards: int):
    """Shard pairs per worker: [[0, S-1], [1, S-2], ...] (host function)."""
    out = (ctypes.c_int32 * max(1, num_shards))()
    _check(lib().sia_zigzag_assign(int(num_shards), out))
    flat = list(out)[:num_shards]
    return [flat[i:i + 2] for i in range(0, num_shards, 2)]


def read_device_status(workspace: torch.Tensor, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().sia_read_device_status(_ptr(workspace), _stream(stream), ctypes.byref(v)))
    return int(v.value)


def version() -> int:
    return int(lib().sia_version())
