"""Pins of the CPU oracle against facts that do not come from the oracle itself:
library conversions, hand-worked examples, closed forms, library routines
(numpy matmul, numpy lexsort, torch scaled_dot_product_attention) on special
cases, and invariants. Runs without a GPU."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- element codecs

def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_values(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3fn_landmarks():
    v = oracle.e4m3fn_values(np.array([0x7E, 0x01, 0x08, 0x38, 0xB8, 0x40, 0x00, 0x80],
                                      dtype=np.uint8))
    assert list(v[:6]) == [448.0, 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 2.0]
    assert v[6] == 0.0 and v[7] == 0.0 and math.copysign(1.0, v[7]) == -1.0


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_values(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert list(oracle.bf16_values(np.array([0x3F80, 0xC000], dtype=np.uint16))) == [1.0, -2.0]


# ---------------------------------------------------------------- golden example

def _tiny_from_golden(g, cache, t):
    dim, H = g["dim"], g["heads"]
    n = len(g["k"])
    table = np.array([[1]], dtype=np.int32)           # the sequence lives on physical page 1
    if cache == "bf16":
        pool = torch.full((2, 64, dim), float("nan"), dtype=torch.bfloat16)
        pool[1, :n] = torch.tensor(g["k"], dtype=torch.bfloat16)
        scale = None
    else:
        pool = torch.full((2, 64, dim), 0x7F, dtype=torch.uint8)
        pool[1, :n] = torch.tensor(g["k"], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
        scale = torch.full((2, 64), float("nan"), dtype=torch.float32)
        scale[1, :n] = torch.tensor(g["sigma"], dtype=torch.float32)
    q = torch.tensor([g["q"]], dtype=torch.bfloat16)
    w = torch.tensor([g["w"]], dtype=torch.float32)
    return dict(q_seq=np.array([0], np.int32), q_pos=np.array([t], np.int32),
                seq_lens=np.array([n], np.int32), page_table=table, idx_k=pool, idx_scale=scale,
                q_idx=q, w=w)


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_golden_scores(cache):
    g = _gold("indexer_topk_tiny.json")
    sc, rl = oracle.indexer_scores(**_tiny_from_golden(g, cache, 3))
    assert rl.tolist() == [4]
    assert sc[0].tolist() == g[f"expected_scores_{cache}"]


def test_golden_topk():
    g = _gold("indexer_topk_tiny.json")
    for case in g["cases"]:
        sc, rl = oracle.indexer_scores(**_tiny_from_golden(g, case["cache"], case["t"]))
        idx, _ = oracle.topk(sc, rl, case["K"])
        assert idx[0].tolist() == case["idx"], case


def test_golden_attention():
    g = _gold("attention_tiny.json")
    rows = torch.tensor(g["rows"], dtype=torch.bfloat16)
    pool = torch.full((1, 64, 2), float("nan"), dtype=torch.bfloat16)
    pool[0, 5] = rows[0]
    pool[0, 9] = rows[1]
    q = torch.tensor([[g["q"]]], dtype=torch.bfloat16)
    out, lse = oracle.sparse_mla(np.array([0], np.int32), 1, np.array([[0]], np.int32), pool, q,
                                 np.array([[5, 9, -1]], np.int32), math.log(3.0), d_v=2)
    assert np.allclose(out[0, 0], g["expected_out"], rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-15


# ---------------------------------------------------------------- indexer scores

def _small(name="decode_b32", **kw):
    base = dict(batch=3, ctx_lo=150, ctx_hi=300, heads_idx=8, dim_idx=32, topk=40, heads_attn=4)
    base.update(kw)
    return W.make(W.spec(name, **base))


def _logical_rows(wl, b, n, pool):
    """Rows 0..n-1 of sequence b, read through the page table with numpy."""
    t = wl.page_table.numpy()[b]
    s = np.arange(n)
    return pool[t[s // 64], s % 64]


@pytest.mark.parametrize("fp8", [False, True])
def test_scores_one_hot_heads_reduce_to_relu_matmul(fp8):
    wl = _small(idx_fp8=fp8)
    H = wl.spec.heads_idx
    if fp8:
        kval = oracle.e4m3fn_values(wl.idx_k.numpy())
    else:
        kval = wl.idx_k.to(torch.float64).numpy()
    for h in [0, H - 1]:
        w = torch.zeros_like(wl.w)
        w[:, h] = 1.0
        sc, rl = oracle.indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                       wl.idx_scale, wl.q_idx, w)
        for j in range(wl.num_q):
            b = int(wl.q_seq[j])
            n = int(rl[j])
            assert n == min(int(wl.q_pos[j]) + 1, int(wl.seq_lens[b]))
            K = _logical_rows(wl, b, n, kval)                               # [n, d]
            qh = wl.q_idx[j, h].to(torch.float64).numpy()                  # [d]
            ref = np.maximum(K @ qh, 0.0)
            if fp8:
                ref = ref * _logical_rows(wl, b, n, wl.idx_scale.numpy().astype(np.float64))
            np.testing.assert_allclose(sc[j, :n], ref, rtol=1e-13, atol=1e-12)
            assert np.all(np.isneginf(sc[j, n:]))


def test_scores_linear_in_head_weights_and_odd_in_sign():
    wl = _small(idx_fp8=True)
    args = (wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k, wl.idx_scale, wl.q_idx)
    g = torch.Generator().manual_seed(5)
    w1 = torch.randn(wl.w.shape, generator=g)
    w2 = torch.randn(wl.w.shape, generator=g)
    s1, rl = oracle.indexer_scores(*args, w1)
    s2, _ = oracle.indexer_scores(*args, w2)
    s12, _ = oracle.indexer_scores(*args, w1 + w2)
    sn, _ = oracle.indexer_scores(*args, -w1)
    for j in range(wl.num_q):
        n = rl[j]
        # w1 + w2 is rounded to fp32 before the oracle sees it: compare loosely
        np.testing.assert_allclose(s12[j, :n], s1[j, :n] + s2[j, :n], rtol=1e-6, atol=1e-5)
        assert np.array_equal(sn[j, :n], -s1[j, :n])


def test_scores_scale_is_per_token_factor():
    wl = _small(idx_fp8=True)
    ones = torch.ones_like(wl.idx_scale)
    a, rl = oracle.indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                  wl.idx_scale, wl.q_idx, wl.w)
    b, _ = oracle.indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                 ones, wl.q_idx, wl.w)
    sig = wl.idx_scale.numpy().astype(np.float64)
    for j in range(wl.num_q):
        n = rl[j]
        bseq = int(wl.q_seq[j])
        np.testing.assert_allclose(a[j, :n], b[j, :n] * _logical_rows(wl, bseq, n, sig),
                                   rtol=1e-15, atol=0)


def test_scores_do_not_depend_on_page_placement():
    s = W.spec("decode_b32", batch=3, ctx_lo=150, ctx_hi=300, heads_idx=8, dim_idx=32)
    a = W.make(s, shuffle=False)
    b = W.make(s, shuffle=True)
    # same logical content placed on different physical pages
    ta, tb = a.page_table.numpy(), b.page_table.numpy()
    kb = b.idx_k.clone()
    sb = b.idx_scale.clone()
    for bb in range(ta.shape[0]):
        for p in range(ta.shape[1]):
            if ta[bb, p] >= 0:
                kb[tb[bb, p]] = a.idx_k[ta[bb, p]]
                sb[tb[bb, p]] = a.idx_scale[ta[bb, p]]
    ra, _ = oracle.indexer_scores(a.q_seq, a.q_pos, a.seq_lens, a.page_table, a.idx_k,
                                  a.idx_scale, a.q_idx, a.w)
    rb, _ = oracle.indexer_scores(b.q_seq, b.q_pos, b.seq_lens, b.page_table, kb, sb, a.q_idx,
                                  a.w)
    assert np.array_equal(ra, rb)


def test_scores_visibility_and_poison():
    wl = W.make(W.spec("decode_b32", batch=3, ctx_lo=100, ctx_hi=200, heads_idx=8, dim_idx=32,
                       q_per_seq=2), poison=True)
    sc, rl = oracle.indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                   wl.idx_scale, wl.q_idx, wl.w)
    for j in range(wl.num_q):
        t = int(wl.q_pos[j])
        n = int(wl.seq_lens[int(wl.q_seq[j])])
        assert rl[j] == min(t + 1, n)
        assert np.all(np.isfinite(sc[j, :rl[j]]))
        assert np.all(np.isneginf(sc[j, rl[j]:]))
    # the second draft token sees the first, the first does not see the second
    assert rl[1] == rl[0] + 1


# ---------------------------------------------------------------- Top-K

def _lexsort_topk(row, n, K):
    order = np.lexsort((np.arange(n), -row[:n]))          # score desc, then position asc
    sel = np.sort(order[:min(n, K)])
    out = np.full(K, -1, dtype=np.int64)
    out[:len(sel)] = sel
    return out


@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 511])
def test_topk_matches_lexsort_with_ties(n):
    rng = np.random.default_rng(n)
    Q = 6
    ld = 512
    sc = np.full((Q, ld), -np.inf)
    sc[:, :n] = np.round(rng.normal(size=(Q, n)) * 3) / 2      # heavy ties
    rl = np.full(Q, n, dtype=np.int32)
    for K in sorted({1, 7, max(1, n - 1), n, n + 5}):
        idx, top = oracle.topk(sc, rl, K)
        for j in range(Q):
            ref = _lexsort_topk(sc[j], n, K)
            assert np.array_equal(idx[j], ref), (n, K, j)
            m = min(n, K)
            assert np.array_equal(top[j, :m], sc[j, idx[j, :m]])


def test_topk_all_equal_scores_take_lowest_positions():
    sc = np.zeros((2, 300))
    idx, _ = oracle.topk(sc, np.array([300, 10], np.int32), 16)
    assert idx[0].tolist() == list(range(16))
    assert idx[1].tolist() == list(range(10)) + [-1] * 6


def test_topk_signed_zero_and_nan():
    row = np.array([np.nan, -0.0, 0.0, -1.0, np.nan, 2.0])
    idx, _ = oracle.topk(row[None, :], np.array([6], np.int32), 4)
    # 2.0 first, then the two zeros (equal: lower position first), then -1.0
    assert idx[0].tolist() == [1, 2, 3, 5]
    idx, _ = oracle.topk(row[None, :], np.array([6], np.int32), 6)
    assert idx[0].tolist() == [0, 1, 2, 3, 4, 5]


def test_topk_zero_query_selects_first_positions():
    wl = _small()
    q0 = torch.zeros_like(wl.q_idx)
    sc, rl = oracle.indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                   wl.idx_scale, q0, wl.w)
    idx, _ = oracle.topk(sc, rl, 40)
    for j in range(wl.num_q):
        assert idx[j].tolist() == list(range(40))


# ---------------------------------------------------------------- attention

def _attn_small(**kw):
    base = dict(batch=2, ctx_lo=100, ctx_hi=180, heads_idx=4, dim_idx=32, topk=24, heads_attn=3)
    base.update(kw)
    return W.make(W.spec("decode_b32", **base), poison=True)


def test_attention_single_row_is_that_row():
    wl = _attn_small()
    idx = np.full((wl.num_q, 24), -1, np.int32)
    idx[:, 0] = 7
    out, lse = oracle.sparse_mla(wl.q_seq, 2, wl.page_table, wl.kv, wl.q_attn, idx, 1 / 24)
    kv = wl.kv.to(torch.float64).numpy()
    for j in range(wl.num_q):
        row = _logical_rows(wl, int(wl.q_seq[j]), 8, kv)[7]
        for a in range(3):
            assert np.array_equal(out[j, a], row[:512])
            z = (wl.q_attn[j, a].to(torch.float64).numpy() @ row) / 24
            assert abs(lse[j, a] - z) <= 1e-12 * max(1.0, abs(z))


def test_attention_zero_query_is_mean_of_values():
    wl = _attn_small()
    q0 = torch.zeros_like(wl.q_attn)
    idx = np.stack([np.sort(np.random.default_rng(j).choice(90, 24, replace=False))
                    for j in range(wl.num_q)]).astype(np.int32)
    out, lse = oracle.sparse_mla(wl.q_seq, 2, wl.page_table, wl.kv, q0, idx, 1 / 24)
    kv = wl.kv.to(torch.float64).numpy()
    for j in range(wl.num_q):
        rows = _logical_rows(wl, int(wl.q_seq[j]), 100, kv)[idx[j]]
        np.testing.assert_allclose(out[j], np.broadcast_to(rows[:, :512].mean(0), (3, 512)),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[j], math.log(24), rtol=1e-14)


def test_attention_ignores_order_and_padding():
    wl = _attn_small()
    rng = np.random.default_rng(3)
    idx = np.full((wl.num_q, 24), -1, np.int32)
    for j in range(wl.num_q):
        idx[j, :17] = np.sort(rng.choice(99, 17, replace=False))
    perm = idx.copy()
    for j in range(wl.num_q):
        perm[j] = idx[j][rng.permutation(24)]
    a, la = oracle.sparse_mla(wl.q_seq, 2, wl.page_table, wl.kv, wl.q_attn, idx, 1 / 24)
    b, lb = oracle.sparse_mla(wl.q_seq, 2, wl.page_table, wl.kv, wl.q_attn, perm, 1 / 24)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-13)
    e, le = oracle.sparse_mla(wl.q_seq, 2, wl.page_table, wl.kv, wl.q_attn,
                              np.full_like(idx, -1), 1 / 24)
    assert np.all(e == 0) and np.all(np.isneginf(le))


def test_topk_of_all_positions_is_dense_causal_attention():
    """With K >= t+1 every position is selected, so the path is ordinary causal
    attention over the latent rows: compare with torch's SDPA in fp64."""
    s = W.spec("prefill_16k", ctx_lo=150, ctx_hi=150, heads_idx=4, dim_idx=32, topk=256,
               heads_attn=3)
    wl = W.make(s)
    ref = oracle.run(wl)
    L = 150
    assert np.array_equal(ref.idx[:, :L] >= 0, np.tril(np.ones((L, L), bool)))
    kv = _logical_rows(wl, 0, L, wl.kv.to(torch.float64).numpy())
    k = torch.from_numpy(kv)[None].expand(3, L, 576)
    v = torch.from_numpy(kv[:, :512])[None].expand(3, L, 512)
    q = wl.q_attn.to(torch.float64).permute(1, 0, 2)            # [H, L, 576]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                         scale=s.sm_scale)
    np.testing.assert_allclose(ref.out, o.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    z = torch.einsum("hld,md->hlm", q, torch.from_numpy(kv)) * s.sm_scale
    z = z.masked_fill(~torch.tril(torch.ones(L, L, dtype=torch.bool)), float("-inf"))
    np.testing.assert_allclose(ref.lse, torch.logsumexp(z, -1).T.numpy(), rtol=1e-12)


# ---------------------------------------------------------------- chunking

def test_chunked_prefill_equals_single_shot():
    s = W.spec("chunked_prefill_128k", ctx_lo=384, ctx_hi=384, chunk=128, heads_idx=4,
               dim_idx=32, topk=50, heads_attn=2)
    wl = W.make(s)
    full = oracle.run(wl, attention=True)
    for c in range(3):
        ch = W.chunk_queries(wl, c)
        r = oracle.run(ch, attention=True)
        sl = slice(c * 128, (c + 1) * 128)
        assert np.array_equal(r.idx, full.idx[sl])
        assert np.array_equal(r.out, full.out[sl])
