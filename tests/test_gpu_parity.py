"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, at
sizes the oracle finishes in seconds that still span several tiles, chunks and
a ragged tail. Tolerances: indexer scores 1e-2 (bf16 cache) / 3e-2 (fp8 cache),
abs + rel; Top-K bit-exact on identical scores; end-to-end sets equal except
within the score tolerance of the K-th score; attention 2e-2 relative L2."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from _paths import (ATTN_KERNELS, check_attention, check_band, check_scores, env, gpu_attention, gpu_scores,
                    group_of, gpu_topk, oracle_topk_of, row_lengths, score_tol)

pytestmark = pytest.mark.gpu

CASES = {
    # the tiny decode workload at its full size
    "tiny_decode": dict(name="tiny_decode"),
    # fp8 index cache, 64x128 indexer heads, Top-2048, several context chunks
    "decode_fp8": dict(name="decode_b32", batch=4, ctx_lo=2500, ctx_hi=9000),
    # two draft tokens per sequence, ragged page tail
    "spec_decode": dict(name="spec_decode_128k", batch=3, ctx_lo=5037, ctx_hi=5037),
    # bf16 index cache, small K, 32 attention heads
    "decode_bf16": dict(name="decode_b32", batch=3, ctx_lo=700, ctx_hi=3000, idx_fp8=False,
                        topk=300, heads_attn=32),
    # causal prefill (streaming Top-K path), rows longer than the candidate buffer
    "prefill": dict(name="prefill_16k", ctx_lo=2600, ctx_hi=2600, topk=384),
}
PREFILL_SAMPLE = 40


def _spec(case):
    kw = dict(CASES[case])
    return W.spec(kw.pop("name"), **kw)


_cache = {}


def _run(case):
    """GPU results + oracle reference for one case (computed once)."""
    if case in _cache:
        return _cache[case]
    s = _spec(case)
    wl = W.make(s, device="cuda", poison=True)
    idx, top = gpu_topk(wl)
    scores = gpu_scores(wl)
    rl = row_lengths(wl)
    if s.prefill:
        rows = np.unique(np.linspace(0, wl.num_q - 1, PREFILL_SAMPLE).astype(int))
    else:
        rows = np.arange(wl.num_q)
    wl_cpu = wl.to("cpu")
    sub = [wl_cpu.queries(int(r), int(r) + 1) for r in rows]
    refs = [oracle.run(x, attention=False) for x in sub]
    ld = scores.shape[1]
    ref_scores = np.full((len(rows), ld), -np.inf)
    for i, r in enumerate(refs):
        ref_scores[i, :r.scores.shape[1]] = r.scores[0]
    ref_idx = np.concatenate([r.idx for r in refs])
    out = dict(wl=wl, wl_cpu=wl_cpu, idx=idx, top=top, scores=scores, rl=rl, rows=rows,
               ref_scores=ref_scores, ref_idx=ref_idx)
    _cache[case] = out
    return out


@pytest.mark.parametrize("case", list(CASES))
def test_scores_match_oracle(case):
    r = _run(case)
    g = r["scores"].cpu().numpy()[r["rows"]]
    check_scores(g, r["ref_scores"], r["rl"][r["rows"]], score_tol(r["wl"]))


@pytest.mark.parametrize("case", list(CASES))
def test_fused_topk_is_exact_selection_of_its_scores(case):
    """The fused pass computes the same scores as the scores hook, so its indices
    must equal the oracle's selection on those scores bit for bit."""
    r = _run(case)
    K = r["wl"].spec.topk
    ref, ref_sc = oracle_topk_of(r["scores"], r["rl"], K)
    got = r["idx"].cpu().numpy()
    assert np.array_equal(got, ref)
    top = r["top"].cpu().numpy().astype(np.float64)
    assert np.array_equal(top[got >= 0], ref_sc[got >= 0])
    assert np.all(np.isneginf(top[got < 0]))


@pytest.mark.parametrize("case", list(CASES))
def test_topk_from_scores_is_bit_exact(case):
    r = _run(case)
    import indexer_top_sparse_02_amd as sia
    K = r["wl"].spec.topk
    rl = torch.from_numpy(r["rl"]).cuda()
    idx, sc = sia.sparse_topk_from_scores(r["scores"], rl, K)
    torch.cuda.synchronize()
    ref, _ = oracle_topk_of(r["scores"], r["rl"], K)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("case", list(CASES))
def test_end_to_end_sets_within_band(case):
    r = _run(case)
    got = r["idx"].cpu().numpy()[r["rows"]]
    check_band(got, r["ref_idx"], r["ref_scores"], score_tol(r["wl"]))


@pytest.mark.parametrize("kernel", list(ATTN_KERNELS))
@pytest.mark.parametrize("case", list(CASES))
def test_attention_matches_oracle(case, kernel):
    r = _run(case)
    wl, rows = r["wl"], r["rows"]
    print(f"attention {case} kernel {kernel}", flush=True)
    with env(**ATTN_KERNELS[kernel]):
        out, lse = gpu_attention(wl, r["idx"])
    sub = wl.to("cpu").queries(0, wl.num_q)
    idx = r["idx"].cpu().numpy()[rows]
    ref_out, ref_lse = oracle.sparse_mla(sub.q_seq[rows], sub.seq_lens.numel(), sub.page_table, sub.kv,
                                         sub.q_attn[rows], idx, wl.spec.sm_scale)
    check_attention(out[torch.from_numpy(rows).cuda()], ref_out, lse[torch.from_numpy(rows).cuda()],
                    ref_lse)


# ------------------------------------------------------------------ invariants

def test_row_and_stream_paths_agree():
    s = W.spec("prefill_16k", ctx_lo=1800, ctx_hi=1800, topk=256)
    wl = W.make(s, device="cuda")
    with env(SIA_INDEXER_PATH=1):
        a, _ = gpu_topk(wl)
    with env(SIA_INDEXER_PATH=2):
        b, _ = gpu_topk(wl)
    assert torch.equal(a, b)


@pytest.mark.parametrize("parts", [0, 3, 7])
@pytest.mark.parametrize("fp8", [False, True])
def test_row_path_causal_rows_exact(parts, fp8):
    """Score + selection passes on causal rows: with the library's part choice
    and with forced part counts that leave late parts invisible to early
    queries (ragged parts, and parts whose waves have no tiles). The workspace
    starts as garbage, so a key, histogram or row length that is never written
    would show."""
    import indexer_top_sparse_02_amd as sia
    s = W.spec("prefill_16k", ctx_lo=1800, ctx_hi=1800, topk=256, idx_fp8=fp8)
    wl = W.make(s, device="cuda")
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    kw = dict(SIA_INDEXER_PATH=1)
    if parts:
        kw["SIA_ROWS_PARTS"] = parts
    with env(**kw):
        need = sia.indexer_workspace_size(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                          wl.q_pos, s.heads_idx, s.topk, group=group_of(wl))
        ws = sia.new_workspace(need, "cuda")
        ws.fill_(0x5a)
        ws[:256].zero_()   # the status word starts clear
        got, _ = gpu_topk(wl, workspace=ws)
    ref, _ = oracle_topk_of(sc, rl, s.topk)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("layout", ["causal", "scattered"])
@pytest.mark.parametrize("dim,fp8,heads", [(128, False, 64), (128, True, 64), (64, False, 32),
                                          (64, True, 32), (64, True, 64), (128, True, 32)])
def test_stream_path_exact_selection(dim, fp8, heads, layout):
    """The fused streaming Top-K (the four queries of a workgroup share one LDS
    ring of K tiles) against the oracle's selection on the GPU's own scores,
    bit for bit, for every index row shape it is built for (64 or 128 wide,
    bf16 or fp8; 32 or 64 heads). Rows are longer than the candidate buffer, so
    the in-buffer re-selection runs. "scattered" gives the four queries of a
    workgroup very different row lengths (a workgroup walks its longest row;
    shorter rows must ignore the tiles past their end)."""
    import dataclasses
    s = W.spec("prefill_16k", ctx_lo=2600, ctx_hi=2600, topk=256, idx_fp8=fp8, dim_idx=dim,
               heads_idx=heads, heads_attn=16)
    wl = W.make(s, device="cuda", poison=True)
    if layout == "scattered":
        g = torch.Generator().manual_seed(7)
        perm = torch.randperm(wl.num_q, generator=g).to(wl.q_pos.device)
        wl = dataclasses.replace(wl, q_pos=wl.q_pos[perm].contiguous())
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    # the scores themselves, on a few rows, against the oracle
    rows = [0, 3, 1001, wl.num_q - 1]
    cpu = wl.to("cpu")
    ref_rows = [oracle.run(cpu.queries(r, r + 1), attention=False).scores[0] for r in rows]
    ref_scores = np.full((len(rows), sc.shape[1]), -np.inf)
    for i, r in enumerate(ref_rows):
        ref_scores[i, :r.shape[0]] = r[:sc.shape[1]]
    check_scores(sc.cpu().numpy()[rows], ref_scores, rl[rows], score_tol(wl))
    with env(SIA_INDEXER_PATH=2):
        got, top = gpu_topk(wl)
    ref, ref_sc = oracle_topk_of(sc, rl, s.topk)
    g_idx = got.cpu().numpy()
    assert np.array_equal(g_idx, ref)
    g_top = top.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_top[g_idx >= 0], ref_sc[g_idx >= 0])


@pytest.mark.parametrize("fp8", [False, True])
def test_stream_reselection_on_rising_scores(fp8):
    """Scores that rise along the row (one head, q = e_0, the key's first element
    rising in steps shared by seven positions) make every position beat the
    running threshold of the streaming Top-K, so its candidate buffer fills and
    is re-selected again and again, mostly by the one-pass superset rule, with
    ties at every step. Indices and scores must be the oracle's selection of the
    GPU's own scores, bit for bit, and the scores are exactly the key values."""
    s = W.spec("prefill_16k", ctx_lo=6000, ctx_hi=6000, topk=256, idx_fp8=fp8, heads_attn=16)
    wl = W.make(s, device="cuda", poison=True, with_attn=False)
    n = 6000
    pos = torch.arange(n, device="cuda")
    val = (pos // 7).float() / 64.0 + 0.25
    phys = wl.page_table[0].long()[pos // 64] * 64 + pos % 64
    flat = wl.idx_k.view(-1, s.dim_idx)
    row = torch.zeros((n, s.dim_idx), device="cuda", dtype=torch.float32)
    row[:, 0] = val
    if fp8:
        flat[phys] = row.to(torch.float8_e4m3fn).view(torch.uint8)
        wl.idx_scale.view(-1)[phys] = 1.0
        key0 = row[:, 0].to(torch.float8_e4m3fn).float()
    else:
        flat[phys] = row.to(torch.bfloat16)
        key0 = row[:, 0].to(torch.bfloat16).float()
    wl.q_idx.zero_()
    wl.q_idx[:, 0, 0] = 1.0
    wl.w.zero_()
    wl.w[:, 0] = 1.0
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    last = sc[n - 1, :n].cpu()
    assert torch.equal(last, key0.cpu())
    with env(SIA_INDEXER_PATH=2):
        got, top = gpu_topk(wl)
    ref, ref_sc = oracle_topk_of(sc, rl, s.topk)
    g_idx = got.cpu().numpy()
    assert np.array_equal(g_idx, ref)
    g_top = top.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_top[g_idx >= 0], ref_sc[g_idx >= 0])


@pytest.mark.parametrize("fp8", [False, True])
def test_stream_group_reselection_with_mixed_rows(fp8):
    """The four queries of a stream workgroup re-select together when any of
    them might overflow its buffer. Here they differ (query j % 4: scores
    rising along the row, so that its buffer fills again and again and votes;
    falling, so that after its first re-selection it holds exactly K keys and
    skips the vote's re-selections; flat, the rising and falling parts summed,
    with ties everywhere; and random), so that re-selections run in buffers that
    are not full, with and without ties. Indices and scores must be the
    oracle's selection of the GPU's own scores, bit for bit."""
    s = W.spec("prefill_16k", ctx_lo=6000, ctx_hi=6000, topk=256, idx_fp8=fp8, heads_attn=16)
    wl = W.make(s, device="cuda", poison=True, with_attn=False)
    n = 6000
    pos = torch.arange(n, device="cuda")
    phys = wl.page_table[0].long()[pos // 64] * 64 + pos % 64
    flat = wl.idx_k.view(-1, s.dim_idx)
    # (the other elements keep their random values: they score the random query)
    row = flat[phys].view(torch.float8_e4m3fn).float() if fp8 else flat[phys].float()
    row[:, 0] = (pos // 7).float() / 64.0 + 0.25
    row[:, 1] = ((n - 1 - pos) // 7).float() / 64.0 + 0.25
    if fp8:
        flat[phys] = row.to(torch.float8_e4m3fn).view(torch.uint8)
        wl.idx_scale.view(-1)[phys] = 1.0
    else:
        flat[phys] = row.to(torch.bfloat16)
    pattern = torch.arange(wl.num_q, device="cuda") % 4
    q = wl.q_idx[:, 0, :].float()
    q[pattern < 3] = 0.0
    q[pattern == 0, 0] = 1.0
    q[pattern == 1, 1] = 1.0
    q[pattern == 2, 0] = 1.0
    q[pattern == 2, 1] = 1.0
    wl.q_idx.zero_()
    wl.q_idx[:, 0, :] = q.to(torch.bfloat16)
    wl.w.zero_()
    wl.w[:, 0] = 1.0
    sc = gpu_scores(wl)
    rl = row_lengths(wl)
    with env(SIA_INDEXER_PATH=2):
        got, top = gpu_topk(wl)
    ref, ref_sc = oracle_topk_of(sc, rl, s.topk)
    g_idx = got.cpu().numpy()
    assert np.array_equal(g_idx, ref)
    g_top = top.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_top[g_idx >= 0], ref_sc[g_idx >= 0])


@pytest.mark.parametrize("sched", [0, 1, 2])
def test_prefill_schedules_agree(sched):
    s = W.spec("prefill_16k", ctx_lo=1500, ctx_hi=1500, topk=128, idx_fp8=True)
    wl = W.make(s, device="cuda")
    ref, _ = gpu_topk(wl, sched=1)
    got, _ = gpu_topk(wl, sched=sched)
    assert torch.equal(ref, got)


@pytest.mark.parametrize("fp8", [False, True])
def test_chunked_prefill_equals_single_shot(fp8):
    """A causal prefill run as three chunks of queries (each chunk one indexer
    call and one attention call against the full caches, seeing positions 0..t)
    gives the same indices and the same attention output bits as one call over
    all queries: a query's result depends only on its own row."""
    s = W.spec("prefill_16k", ctx_lo=3000, ctx_hi=3000, topk=256, idx_fp8=fp8, heads_attn=32)
    wl = W.make(s, device="cuda", poison=True)
    import indexer_top_sparse_02_amd as sia
    idx_all, _ = sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                         wl.q_pos, wl.q_idx, wl.w, s.topk, group=wl.num_q)
    out_all, lse_all = gpu_attention(wl, idx_all)
    parts_idx, parts_out, parts_lse = [], [], []
    for a, b in ((0, 1024), (1024, 2048), (2048, wl.num_q)):
        c = wl.queries(a, b)
        i, _ = sia.sparse_indexer_topk(c.page_table, c.seq_lens, c.idx_k, c.idx_scale, c.q_seq, c.q_pos,
                                       c.q_idx, c.w, s.topk, group=b - a)
        o, l = gpu_attention(c, i)
        parts_idx.append(i)
        parts_out.append(o)
        parts_lse.append(l)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts_idx), idx_all)
    assert torch.equal(torch.cat(parts_out).view(torch.int16), out_all.view(torch.int16))
    assert torch.equal(torch.cat(parts_lse), lse_all)


@pytest.mark.parametrize("case", ["spec_decode", "decode_bf16", "prefill"])
def test_graph_replay_matches_eager(case):
    """The whole path (indexer + Top-K, then attention) captured in a HIP graph
    and replayed several times, with eager work and synchronizations between the
    replays: every replay reproduces the eager results bit for bit (the library
    enqueues only its own kernels, including its counter and fill resets)."""
    import indexer_top_sparse_02_amd as sia
    s = _spec(case)
    wl = W.make(s, device="cuda")
    group = group_of(wl)
    maxv = int(torch.minimum(wl.q_pos.long() + 1, wl.seq_lens.long()[wl.q_seq.long()]).max())
    ws_i = sia.new_workspace(sia.indexer_workspace_size(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale,
                                                        wl.q_seq, wl.q_pos, s.heads_idx, s.topk, group=group,
                                                        max_visible=maxv), "cuda")
    ws_a = sia.new_workspace(sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk), "cuda")
    idx = torch.empty((wl.num_q, s.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.num_q, s.heads_attn, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.num_q, s.heads_attn), dtype=torch.float32, device="cuda")

    def step():
        sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq, wl.q_pos,
                                wl.q_idx, wl.w, s.topk, group=group, max_visible=maxv, out_idx=idx,
                                workspace=ws_i)
        sia.sparse_mla_attention(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn, idx, s.sm_scale,
                                 out=out, lse=lse, workspace=ws_a)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        idx.fill_(-7)
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0])
        assert torch.equal(out.view(torch.int16), ref[1].view(torch.int16))
        assert torch.equal(lse, ref[2])


@pytest.mark.parametrize("case", ["decode_fp8", "spec_decode", "tiny_decode"])
def test_graph_replay_matches_oracle(case):
    """A decode step (indexer + Top-K, then attention) captured in one HIP graph
    and replayed three times, with eager work between the replays: every
    replay's indices are the oracle's selection of the GPU's scores, bit for
    bit, its sets meet the band rule against the oracle's own selection, and its
    attention output matches the oracle's on those indices."""
    import indexer_top_sparse_02_amd as sia
    r = _run(case)
    wl, s = r["wl"], r["wl"].spec
    group = group_of(wl)
    maxv = int(r["rl"].max())
    ws_i = sia.new_workspace(sia.indexer_workspace_size(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale,
                                                        wl.q_seq, wl.q_pos, s.heads_idx, s.topk, group=group,
                                                        max_visible=maxv), "cuda")
    ws_a = sia.new_workspace(sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk), "cuda")
    idx = torch.empty((wl.num_q, s.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.num_q, s.heads_attn, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.num_q, s.heads_attn), dtype=torch.float32, device="cuda")

    def step():
        sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq, wl.q_pos,
                                wl.q_idx, wl.w, s.topk, group=group, max_visible=maxv, out_idx=idx,
                                workspace=ws_i)
        sia.sparse_mla_attention(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn, idx, s.sm_scale,
                                 out=out, lse=lse, workspace=ws_a)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    ref_sel, _ = oracle_topk_of(r["scores"], r["rl"], s.topk)
    rows = r["rows"]
    sub = wl.to("cpu")
    for rep in range(3):
        idx.fill_(-7)
        out.zero_()
        lse.zero_()
        _ = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        assert np.array_equal(got, ref_sel), rep
        check_band(got[rows], r["ref_idx"], r["ref_scores"], score_tol(wl))
        ref_out, ref_lse = oracle.sparse_mla(sub.q_seq[rows], sub.seq_lens.numel(), sub.page_table, sub.kv,
                                             sub.q_attn[rows], got[rows], s.sm_scale)
        sel = torch.from_numpy(rows).cuda()
        check_attention(out[sel], ref_out, lse[sel], ref_lse)


def test_page_placement_does_not_change_results():
    s = W.spec("decode_b32", batch=3, ctx_lo=3000, ctx_hi=6000, topk=512, heads_attn=64)
    a = W.make(s, device="cuda", shuffle=False)
    b = W.make(s, device="cuda", shuffle=True)
    ta, tb = a.page_table.cpu().numpy(), b.page_table.cpu().numpy()
    for bb in range(ta.shape[0]):
        for p in range(ta.shape[1]):
            if ta[bb, p] >= 0:
                b.idx_k[tb[bb, p]] = a.idx_k[ta[bb, p]]
                b.idx_scale[tb[bb, p]] = a.idx_scale[ta[bb, p]]
                b.kv[tb[bb, p]] = a.kv[ta[bb, p]]
    b.q_idx.copy_(a.q_idx); b.w.copy_(a.w); b.q_attn.copy_(a.q_attn)
    ia, _ = gpu_topk(a)
    ib, _ = gpu_topk(b)
    assert torch.equal(ia, ib)
    oa, la = gpu_attention(a, ia)
    ob, lb = gpu_attention(b, ia)
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_repeated_runs_are_bit_identical():
    s = W.spec("spec_decode_128k", batch=2, ctx_lo=9000, ctx_hi=9000)
    wl = W.make(s, device="cuda")
    i0, s0 = gpu_topk(wl)
    o0, _ = gpu_attention(wl, i0)
    for _ in range(3):
        i1, s1 = gpu_topk(wl)
        o1, _ = gpu_attention(wl, i1)
        assert torch.equal(i0, i1) and torch.equal(s0, s1) and torch.equal(o0, o1)


def test_many_parts_match_oracle_selection():
    s = W.spec("decode_b32", batch=2, ctx_lo=40000, ctx_hi=41000, heads_idx=16, topk=2048)
    wl = W.make(s, device="cuda")
    with env(SIA_ROWS_PARTS=20):      # 20 per-part histograms per row
        idx, _ = gpu_topk(wl)
    sc = gpu_scores(wl)
    ref, _ = oracle_topk_of(sc, row_lengths(wl), s.topk)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_selection_beyond_lds_candidates_uses_global_keys():
    """Every score equal (zero queries): the threshold bin holds the whole row,
    more candidates than the selection keeps in LDS, so the threshold and the
    ordered compaction run over the key rows in global memory; ties go to the
    lowest positions."""
    s = W.spec("decode_b32", batch=2, ctx_lo=20000, ctx_hi=30000, topk=3000)
    wl = W.make(s, device="cuda")
    wl.q_idx.zero_()
    idx, top = gpu_topk(wl)
    assert torch.equal(idx, torch.arange(3000, dtype=torch.int32, device="cuda").expand(2, 3000))
    assert torch.all(top == 0)


# ------------------------------------------------------------------ edge cases

def test_short_rows_take_everything_and_pad():
    s = W.spec("decode_b32", batch=3, ctx_lo=1, ctx_hi=200, topk=256, heads_attn=16)
    wl = W.make(s, device="cuda", poison=True)
    idx, top = gpu_topk(wl)
    rl = row_lengths(wl)
    got = idx.cpu().numpy()
    for j in range(wl.num_q):
        assert got[j, :rl[j]].tolist() == list(range(rl[j]))
        assert np.all(got[j, rl[j]:] == -1)
    out, lse = gpu_attention(wl, idx)
    c = wl.to("cpu")
    ref_out, ref_lse = oracle.sparse_mla(c.q_seq, c.seq_lens.numel(), c.page_table, c.kv, c.q_attn,
                                         got, s.sm_scale)
    check_attention(out, ref_out, lse, ref_lse)


def test_zero_queries_select_lowest_positions():
    s = W.spec("decode_b32", batch=2, ctx_lo=5000, ctx_hi=7000, topk=1000)
    wl = W.make(s, device="cuda")
    wl.q_idx.zero_()
    idx, top = gpu_topk(wl)
    assert torch.equal(idx, torch.arange(1000, dtype=torch.int32, device="cuda").expand(2, 1000))
    assert torch.all(top == 0)


def test_no_queries_is_a_no_op():
    s = W.spec("decode_b32", batch=2, ctx_lo=500, ctx_hi=700, topk=64)
    wl = W.make(s, device="cuda").queries(0, 0)
    idx, _ = gpu_topk(wl)
    assert idx.shape == (0, 64)
    out, _ = gpu_attention(wl, idx)
    assert out.shape[0] == 0


@pytest.mark.parametrize("kernel", list(ATTN_KERNELS))
def test_topk_of_all_positions_is_dense_causal_attention(kernel):
    s = W.spec("prefill_16k", ctx_lo=700, ctx_hi=700, topk=1024, heads_attn=32)
    wl = W.make(s, device="cuda")
    idx, _ = gpu_topk(wl)
    got = idx.cpu().numpy()
    L = 700
    assert np.array_equal(got[:, :L] >= 0, np.tril(np.ones((L, L), bool)))
    with env(**ATTN_KERNELS[kernel]):
        out, _ = gpu_attention(wl, idx)
    # dense causal attention over the logical latent rows (fp32, CPU)
    t = wl.page_table.cpu()[0].long()
    pos = torch.arange(L)
    rows = wl.kv.cpu()[t[pos // 64], pos % 64].float()
    q = wl.q_attn.cpu().float().permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, rows[None].expand(32, L, 576).contiguous(), rows[None, :, :512].expand(32, L, 512).contiguous(),
        is_causal=True, scale=s.sm_scale)
    check_attention(out, o.permute(1, 0, 2).double().numpy())
