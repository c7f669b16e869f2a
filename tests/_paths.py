"""Shared helpers of the GPU tests: run the HIP path on a workload and compare it
with the oracle by the agreed rules."""
from __future__ import annotations

import contextlib
import os

import numpy as np
import torch

import indexer_top_sparse_02_amd as sia
import oracle
import workloads as W


def group_of(wl) -> int:
    return wl.num_q if wl.spec.prefill else wl.spec.q_per_seq


def score_tol(wl) -> float:
    # indexer scores: 1e-2 for a bf16 index cache, 3e-2 for fp8
    return 3e-2 if wl.spec.idx_fp8 else 1e-2


ATTN_TOL = 2e-2   # relative L2 error of each (query, head) output row

# Attention kernels of the bf16 latent cache, chosen by the library's plan
# through its environment: the row-split kernel (two waves per 16 heads, P
# exchanged through LDS) and the whole-tile kernel with 64 or 128 heads per
# workgroup (one wave per 16 heads over all rows of a tile), or with 64 heads
# and two waves per 16 heads, one per half of each 64-row tile, or with 128
# heads in four waves of 32.
ATTN_KERNELS = {
    "rowsplit": dict(SIA_ATTN_WAVE=0, SIA_ATTN_RH=1, SIA_ATTN_WIDE=0),
    "wave64": dict(SIA_ATTN_WAVE=1, SIA_ATTN_HB=64, SIA_ATTN_RH=1, SIA_ATTN_WIDE=0),
    "wave128": dict(SIA_ATTN_WAVE=1, SIA_ATTN_HB=128, SIA_ATTN_RH=1, SIA_ATTN_WIDE=0),
    "wave64x2": dict(SIA_ATTN_WAVE=1, SIA_ATTN_HB=64, SIA_ATTN_RH=2, SIA_ATTN_WIDE=0),
    "wide128": dict(SIA_ATTN_WAVE=1, SIA_ATTN_HB=128, SIA_ATTN_RH=1, SIA_ATTN_WIDE=1),
}


@contextlib.contextmanager
def env(**kv):
    old = {k: os.environ.get(k) for k in kv}
    try:
        for k, v in kv.items():
            os.environ[k] = str(v)
        yield
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def gpu_topk(wl, **kw):
    idx, sc = sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                      wl.q_pos, wl.q_idx, wl.w, wl.spec.topk, group=group_of(wl),
                                      want_score=True, **kw)
    torch.cuda.synchronize()
    return idx, sc


def gpu_scores(wl, ld=None):
    s = sia.sparse_indexer_scores(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                  wl.q_pos, wl.q_idx, wl.w, group=group_of(wl), ld=ld)
    torch.cuda.synchronize()
    return s


def gpu_attention(wl, idx, **kw):
    out, lse = sia.sparse_mla_attention(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn, idx,
                                        wl.spec.sm_scale, want_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


def check_scores(gpu: np.ndarray, ref: np.ndarray, row_len: np.ndarray, tol: float):
    """|g - r| <= tol + tol*|r| on visible positions; -inf elsewhere."""
    for j in range(ref.shape[0]):
        n = int(row_len[j])
        g, r = gpu[j, :n].astype(np.float64), ref[j, :n]
        bad = np.abs(g - r) > tol + tol * np.abs(r)
        assert not bad.any(), (j, np.flatnonzero(bad)[:5], g[bad][:5], r[bad][:5])
        assert np.all(np.isneginf(gpu[j, n:])), j


def check_band(gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_scores: np.ndarray, tol: float):
    """Sets computed end to end: equal sizes; every position in the symmetric
    difference scores (oracle) within tol of the oracle's K-th score."""
    worst = 0
    for j in range(ref_idx.shape[0]):
        g = set(int(x) for x in gpu_idx[j] if x >= 0)
        r = set(int(x) for x in ref_idx[j] if x >= 0)
        assert len(g) == len(r), (j, len(g), len(r))
        assert list(gpu_idx[j][:len(g)]) == sorted(g), j          # ascending, -1 padded
        assert np.all(gpu_idx[j][len(g):] == -1), j
        diff = g ^ r
        if not diff:
            continue
        vk = ref_scores[j, sorted(r, key=lambda s: (-ref_scores[j, s], s))[-1]]
        for s in diff:
            assert abs(ref_scores[j, s] - vk) <= tol + tol * abs(vk), (j, s, ref_scores[j, s], vk)
        worst = max(worst, len(diff))
    return worst


def check_attention(out_gpu: torch.Tensor, out_ref: np.ndarray, lse_gpu=None, lse_ref=None):
    o = out_gpu.float().cpu().numpy().astype(np.float64)
    num = np.linalg.norm(o - out_ref, axis=-1)
    den = np.linalg.norm(out_ref, axis=-1)
    empty = den == 0
    assert np.all(num[empty] == 0)
    rel = num[~empty] / den[~empty]
    assert rel.max(initial=0) <= ATTN_TOL, rel.max()
    if lse_gpu is not None:
        lg = lse_gpu.cpu().numpy().astype(np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.allclose(lg[fin], lse_ref[fin], rtol=1e-4, atol=1e-3)
    return float(rel.max(initial=0))


def oracle_topk_of(scores_gpu: torch.Tensor, row_len: np.ndarray, K: int):
    """The oracle's selection applied to the GPU's own fp32 scores."""
    s = scores_gpu.cpu().numpy().astype(np.float64)
    return oracle.topk(s, row_len, K)


def row_lengths(wl) -> np.ndarray:
    lens = wl.seq_lens.cpu().numpy()
    q_seq = wl.q_seq.cpu().numpy()
    return np.minimum(wl.q_pos.cpu().numpy() + 1, lens[q_seq]).astype(np.int32)
