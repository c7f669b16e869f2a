"""GPU edge cases through the C ABI: queries that do not pair up, device data
the host cannot check (out-of-range page ids, sequence ids and stage-2
indices, each flagged in the status word and never dereferenced), stage-2
index lists in any order with duplicates and interior padding, head counts
outside the five workloads, and decode rows whose scores rise or fall along
the row (every position kept, or the running floor climbing at once). Every
result is compared with the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import indexer_top_sparse_02_amd as sia
import oracle
import workloads as W
from _paths import (ATTN_KERNELS, check_attention, check_band, check_scores, env, gpu_attention, gpu_scores,
                    gpu_topk, oracle_topk_of, row_lengths, score_tol)

pytestmark = pytest.mark.gpu


def _indexer_ws(wl, group):
    s = wl.spec
    need = sia.indexer_workspace_size(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                      wl.q_pos, s.heads_idx, s.topk, group=group)
    return sia.new_workspace(need, "cuda")


def _topk(wl, group, ws):
    idx, sc = sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                      wl.q_pos, wl.q_idx, wl.w, wl.spec.topk, group=group,
                                      want_score=True, workspace=ws)
    torch.cuda.synchronize()
    return idx, sc


def _attention(wl, idx, ws=None):
    out, lse = sia.sparse_mla_attention(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn, idx,
                                        wl.spec.sm_scale, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


def _oracle_attention(wl, idx_np):
    c = wl.to("cpu")
    return oracle.sparse_mla(c.q_seq, c.seq_lens.numel(), c.page_table, c.kv, c.q_attn, idx_np,
                             wl.spec.sm_scale)


@pytest.mark.parametrize("nq", [1, 3, 5])
def test_odd_query_count_with_draft_pairs(nq):
    """group = 2 (draft-token pairs) with an odd number of queries: the last
    query has no partner. Selection is bit-exact against the oracle's on the
    GPU's own scores, the scores are within tolerance, and the first queries
    give the same bits as in the even call."""
    s = W.spec("spec_decode_128k", batch=3, ctx_lo=5037, ctx_hi=5037)
    full = W.make(s, device="cuda", poison=True)
    wl = full.queries(0, nq)
    print(f"odd pairs: {nq} queries", flush=True)
    idx, top = _topk(wl, 2, _indexer_ws(wl, 2))
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    ref, ref_sc = oracle_topk_of(sc, rl, s.topk)
    assert np.array_equal(idx.cpu().numpy(), ref)
    c = wl.to("cpu")
    r = oracle.run(c, attention=False)
    check_scores(sc.cpu().numpy(), r.scores, rl, score_tol(wl))
    even, _ = _topk(full, 2, _indexer_ws(full, 2))
    assert torch.equal(even[:nq], idx)


def test_bad_page_id_is_dropped_and_flagged():
    """A visible logical page whose physical id is out of range: the indexer
    never selects its positions (the scores hook leaves them at -inf) and sets
    BAD_PAGE; attention skips the rows on it and sets BAD_PAGE. Everything
    else matches the oracle, which is given the same selection without them."""
    s = W.spec("decode_b32", batch=2, ctx_lo=5000, ctx_hi=6000, topk=512, heads_attn=32)
    wl = W.make(s, device="cuda", poison=True)
    good_table = wl.page_table.clone()
    bad_lp = 7   # logical page 7 of sequence 1: positions 448..511
    wl.page_table[1, bad_lp] = wl.num_pages + 5
    ws = _indexer_ws(wl, 1)
    idx, top = _topk(wl, 1, ws)
    assert sia.read_device_status(ws) & sia.DEVSTATUS_BAD_PAGE
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    scn = sc.cpu().numpy()
    assert np.all(np.isneginf(scn[1, bad_lp * 64:(bad_lp + 1) * 64]))
    got = idx.cpu().numpy()
    assert not np.any((got[1] >= bad_lp * 64) & (got[1] < (bad_lp + 1) * 64))
    ref, _ = oracle_topk_of(sc, rl, s.topk)
    assert np.array_equal(got, ref)
    # attention: give it indices on the bad page too
    idx_att = idx.clone()
    idx_att[1, :8] = torch.arange(bad_lp * 64, bad_lp * 64 + 8, dtype=torch.int32, device="cuda")
    ws_a = sia.new_workspace(sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk), "cuda")
    out, lse = _attention(wl, idx_att, ws_a)
    assert sia.read_device_status(ws_a) & sia.DEVSTATUS_BAD_PAGE
    ia = idx_att.cpu().numpy().copy()
    ia[1][(ia[1] >= bad_lp * 64) & (ia[1] < (bad_lp + 1) * 64)] = -1
    wl_good = dataclasses.replace(wl, page_table=good_table)
    ref_out, ref_lse = _oracle_attention(wl_good, ia)
    check_attention(out, ref_out, lse, ref_lse)


def test_bad_query_sequence_is_flagged_and_selects_nothing():
    """A query naming a sequence outside [0, batch): its indexer row is all -1,
    its attention output is zero with lse -inf, BAD_SEQ is set in both
    workspaces, and the other queries are unaffected."""
    s = W.spec("decode_b32", batch=3, ctx_lo=3000, ctx_hi=4000, topk=256, heads_attn=16)
    wl = W.make(s, device="cuda")
    ref_idx, _ = _topk(wl, 1, _indexer_ws(wl, 1))
    ref_out, ref_lse = _attention(wl, ref_idx)
    wl.q_seq[1] = 9
    ws = _indexer_ws(wl, 1)
    idx, _ = _topk(wl, 1, ws)
    assert sia.read_device_status(ws) & sia.DEVSTATUS_BAD_SEQ
    assert torch.all(idx[1] == -1)
    assert torch.equal(idx[[0, 2]], ref_idx[[0, 2]])
    ws_a = sia.new_workspace(sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk), "cuda")
    out, lse = _attention(wl, ref_idx, ws_a)
    assert sia.read_device_status(ws_a) & sia.DEVSTATUS_BAD_SEQ
    assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))
    assert torch.equal(out[[0, 2]].view(torch.int16), ref_out[[0, 2]].view(torch.int16))


@pytest.mark.parametrize("kernel", list(ATTN_KERNELS))
def test_attention_index_past_sequence_is_skipped(kernel):
    """Stage-2 indices >= n_b are skipped and flag BAD_INDEX; the output equals
    the oracle's over the remaining entries."""
    s = W.spec("decode_b32", batch=2, ctx_lo=3000, ctx_hi=3500, topk=256, heads_attn=32)
    wl = W.make(s, device="cuda", poison=True)
    idx, _ = gpu_topk(wl)
    n = wl.seq_lens.cpu().numpy()
    bad = idx.clone()
    bad[0, 5] = int(n[0]) + 3
    bad[1, 100] = int(n[1]) + 1000
    print(f"attention past-sequence indices: kernel {kernel}", flush=True)
    with env(**ATTN_KERNELS[kernel]):
        ws_a = sia.new_workspace(sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk), "cuda")
        out, lse = _attention(wl, bad, ws_a)
    assert sia.read_device_status(ws_a) & sia.DEVSTATUS_BAD_INDEX
    ia = bad.cpu().numpy().copy()
    ia[0, 5] = -1
    ia[1, 100] = -1
    ref_out, ref_lse = _oracle_attention(wl, ia)
    check_attention(out, ref_out, lse, ref_lse)


@pytest.mark.parametrize("kernel", list(ATTN_KERNELS))
@pytest.mark.parametrize("heads_attn", [16, 64, 128])
def test_attention_unsorted_duplicate_and_interior_padding(heads_attn, kernel):
    """Stage-2 index lists in any order, with duplicates (a duplicate counts
    twice) and -1 entries in the middle, against the oracle on the same lists.
    Lists of 300 entries span several 32-row tiles and a ragged one."""
    s = W.spec("decode_b32", batch=3, ctx_lo=2000, ctx_hi=4000, topk=300, heads_attn=heads_attn)
    wl = W.make(s, device="cuda", poison=True)
    g = np.random.default_rng(11)
    n = wl.seq_lens.cpu().numpy()
    rows = []
    for j in range(wl.num_q):
        r = g.integers(0, int(n[j]), size=300).astype(np.int32)
        r[g.choice(300, 40, replace=False)] = -1          # interior padding
        r[10:20] = r[0]                                   # duplicates of one row
        r[200:230] = r[100:130]                           # a duplicated block
        rows.append(r)
    ia = np.stack(rows)
    print(f"attention index lists: heads {heads_attn} kernel {kernel}", flush=True)
    with env(**ATTN_KERNELS[kernel]):
        out, lse = _attention(wl, torch.from_numpy(ia).cuda())
    ref_out, ref_lse = _oracle_attention(wl, ia)
    check_attention(out, ref_out, lse, ref_lse)


@pytest.mark.parametrize("heads_idx,dim", [(5, 128), (1, 64), (40, 64)])
def test_indexer_head_counts_outside_the_workloads(heads_idx, dim):
    """Head counts that leave a 32-head block partly empty: scores within
    tolerance of the oracle and Top-K bit-exact on the GPU's scores."""
    s = W.spec("decode_b32", batch=3, ctx_lo=2500, ctx_hi=5000, topk=512, heads_idx=heads_idx,
               dim_idx=dim, idx_fp8=dim == 128, heads_attn=16)
    wl = W.make(s, device="cuda", poison=True, with_attn=False)
    print(f"indexer heads {heads_idx} dim {dim}", flush=True)
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    r = oracle.run(wl.to("cpu"), attention=False)
    check_scores(sc.cpu().numpy(), r.scores, rl, score_tol(wl))
    idx, _ = gpu_topk(wl)
    ref, _ = oracle_topk_of(sc, rl, s.topk)
    assert np.array_equal(idx.cpu().numpy(), ref)
    check_band(idx.cpu().numpy(), r.idx, r.scores, score_tol(wl))


def _monotone_rows(wl, direction):
    """Index rows whose first element rises (or falls) along each sequence in
    steps shared by five positions, one head (q = e_0, w = 1): every key ties
    with at least four others. direction 0 leaves the drawn rows alone."""
    if direction == 0:
        return
    s = wl.spec
    wl.q_idx.zero_()
    wl.q_idx[:, 0, 0] = 1.0
    wl.w.zero_()
    wl.w[:, 0] = 1.0
    flat = wl.idx_k.view(-1, s.dim_idx)
    for b in range(int(wl.seq_lens.numel())):
        n = int(wl.seq_lens[b])
        pos = torch.arange(n, device="cuda")
        step = pos // 5 if direction > 0 else (n - 1 - pos) // 5
        val = step.float() / 64.0 + 0.25
        phys = wl.page_table[b].long()[pos // 64] * 64 + pos % 64
        row = torch.zeros((n, s.dim_idx), device="cuda", dtype=torch.float32)
        row[:, 0] = val
        if s.idx_fp8:
            flat[phys] = row.to(torch.float8_e4m3fn).view(torch.uint8)
            wl.idx_scale.view(-1)[phys] = 1.0
        else:
            flat[phys] = row.to(torch.bfloat16)


@pytest.mark.parametrize("parts", [0, 2])
@pytest.mark.parametrize("direction", [1, -1, 0])
@pytest.mark.parametrize("group", [1, 2])
def test_decode_rows_exact_with_running_floor(direction, group, parts):
    """Decode rows whose scores rise along the row keep every position (each
    new key beats the running floor), filling the candidate lists; rows whose
    scores fall raise the floor at once; drawn rows (direction 0) raise it
    gradually. With two forced parts of 20000 positions the floor has room to
    rise. All are selected bit-exactly (the oracle's selection of the GPU's
    own scores), with the pair path (group 2) and the one-query path, and with
    a garbage workspace."""
    s = W.spec("spec_decode_128k", batch=2, ctx_lo=40000, ctx_hi=40000, topk=2048)
    wl = W.make(s, device="cuda", poison=True, with_attn=False)
    _monotone_rows(wl, direction)
    print(f"running floor: direction {direction} group {group} parts {parts}", flush=True)
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    kw = {"SIA_ROWS_PARTS": parts} if parts else {}
    with env(**kw):
        ws = _indexer_ws(wl, group)
        ws.fill_(0x5a)
        ws[:256].zero_()
        idx, top = _topk(wl, group, ws)
    ref, ref_sc = oracle_topk_of(sc, rl, s.topk)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref)
    g_top = top.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_top[got >= 0], ref_sc[got >= 0])
