"""The MXFP8 index path on the GPU (through the C ABI) against the oracle:

* the quantizer bit for bit (codes and scale bytes) on spread-out, all-zero,
  exactly-at-maximum, tiny and halfway values;
* scores of the MXFP8 query against MXFP8 rows within 1e-2 (products of the
  dequantized values are exact in fp32; only the summation order differs);
* Top-K bit-exact against the oracle's selection of the GPU's own scores, and
  the boundary-band rule against the oracle's own selection, for the pair
  (draft tokens), one-query and streaming (prefill) kernels, and at the 128K
  speculative-decode size;
* the Top-K hit rate of the MXFP8 path (query and rows quantized by the
  library) against the bf16-query path on the same data, which the pages ask
  to check when the index path is quantized."""
import numpy as np
import pytest
import torch

import indexer_top_sparse_02_amd as sia
import oracle
import workloads as W
from _paths import check_band, check_scores, env

pytestmark = pytest.mark.gpu
MX_TOL = 1e-2


def test_quantizer_bit_exact():
    g = torch.Generator(device="cuda").manual_seed(17)
    x = torch.randn(512, 128, generator=g, device="cuda") * \
        torch.logspace(-20, 20, 512, base=2.0, device="cuda")[:, None]
    x[0] = 0.0
    x[1, :32] = 448.0 * 2.0 ** 3
    x[2, :32] = 1e-30
    x[3, :64] = -x[3, :64]
    e4 = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().cuda()
    x[4, 0] = 448.0
    x[4, 1:31] = (e4[8:38] + e4[9:39]) / 2.0        # halfway points (ties)
    xb = x.to(torch.bfloat16)
    codes, scales = sia.quantize_mxfp8(xb)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_mxfp8(xb.cpu())
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


CASES = {
    "pairs": (dict(name="spec_decode_128k", batch=3, ctx_lo=5037, ctx_hi=5037), 2),
    "rows": (dict(name="decode_b32", batch=4, ctx_lo=2500, ctx_hi=9000), 1),
    "stream": (dict(name="prefill_16k", ctx_lo=2600, ctx_hi=2600, topk=256, idx_fp8=True, heads_attn=16), 0),
}


def _mx_run(wl, mx, group, **kw):
    s = wl.spec
    idx, top = sia.sparse_indexer_topk_mxfp8(wl.page_table, wl.seq_lens, wl.idx_k, mx.k_scales, wl.q_seq,
                                             wl.q_pos, mx.q_codes, mx.q_scales, wl.w, s.topk, group=group,
                                             want_score=True, **kw)
    sc = sia.sparse_indexer_scores_mxfp8(wl.page_table, wl.seq_lens, wl.idx_k, mx.k_scales, wl.q_seq, wl.q_pos,
                                         mx.q_codes, mx.q_scales, wl.w, group=group)
    torch.cuda.synchronize()
    return idx, top, sc


@pytest.mark.parametrize("case", list(CASES))
def test_mx_path_matches_oracle(case):
    kw, group = CASES[case]
    kw = dict(kw)
    s = W.spec(kw.pop("name"), **kw)
    wl = W.make(s, device="cuda", poison=True, with_attn=False)
    mx = W.make_mx(wl, poison=True)
    group = group or wl.num_q
    print(f"mxfp8 {case}: {wl.num_q} queries, group {group}", flush=True)
    path = {"SIA_INDEXER_PATH": 2} if case == "stream" else {}
    with env(**path):
        idx, top, sc = _mx_run(wl, mx, group)
    rl = np.minimum(wl.q_pos.cpu().numpy() + 1, wl.seq_lens.cpu().numpy()[wl.q_seq.cpu().numpy()])
    rows = np.unique(np.linspace(0, wl.num_q - 1, min(wl.num_q, 40)).astype(int))
    c = wl.to("cpu")
    ref, ref_rl = oracle.indexer_scores_mx(c.q_seq[rows], c.q_pos[rows], c.seq_lens, c.page_table, c.idx_k,
                                           mx.k_scales.cpu(), mx.q_codes[rows].cpu(), mx.q_scales[rows].cpu(),
                                           c.w[rows], ld=sc.shape[1])
    g_sc = sc.cpu().numpy()
    check_scores(g_sc[rows], ref, rl[rows], MX_TOL)
    sel, sel_sc = oracle.topk(g_sc.astype(np.float64), rl.astype(np.int32), s.topk)
    got = idx.cpu().numpy()
    assert np.array_equal(got, sel)
    g_top = top.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_top[got >= 0], sel_sc[got >= 0])
    ref_idx, _ = oracle.topk(ref, ref_rl, s.topk)
    check_band(got[rows], ref_idx, ref, MX_TOL)


def test_mx_path_full_size_speculative_decode():
    """The 128K speculative-decode workload on the MXFP8 path: selection
    bit-exact on every row, scores and the band rule on three sequences."""
    s = W.spec("spec_decode_128k")
    wl = W.make(s, device="cuda", poison=True, with_attn=False)
    mx = W.make_mx(wl, poison=True)
    idx, top, sc = _mx_run(wl, mx, 2)
    rl = np.minimum(wl.q_pos.cpu().numpy() + 1, wl.seq_lens.cpu().numpy()[wl.q_seq.cpu().numpy()]).astype(np.int32)
    g_sc = sc.cpu().numpy()
    sel, _ = oracle.topk(g_sc.astype(np.float64), rl, s.topk)
    got = idx.cpu().numpy()
    assert np.array_equal(got, sel)
    c = wl.to("cpu")
    for seq in (0, 31, 63):
        rows = np.flatnonzero(c.q_seq.numpy() == seq)
        print(f"mxfp8 full size: sequence {seq}", flush=True)
        ref, ref_rl = oracle.indexer_scores_mx(c.q_seq[rows], c.q_pos[rows], c.seq_lens, c.page_table, c.idx_k,
                                               mx.k_scales.cpu(), mx.q_codes[rows].cpu(),
                                               mx.q_scales[rows].cpu(), c.w[rows], ld=g_sc.shape[1])
        check_scores(g_sc[rows], ref, rl[rows], MX_TOL)
        ref_idx, _ = oracle.topk(ref, ref_rl, s.topk)
        check_band(got[rows], ref_idx, ref, MX_TOL)


def mx_from_reference(wl):
    """The MXFP8 form of a bf16-query, fp8-with-token-scale workload, made by the
    library's quantizer: rows from the cache's values e4m3 * sigma (rounded to
    bf16), the query from its bf16 heads."""
    vals = wl.idx_k.view(torch.float8_e4m3fn).float() * wl.idx_scale[..., None]
    k_codes, k_scales = sia.quantize_mxfp8(vals.to(torch.bfloat16))
    q_codes, q_scales = sia.quantize_mxfp8(wl.q_idx)
    return k_codes, k_scales, q_codes, q_scales


def hit_rate(a, b):
    """Mean over queries of |A & B| / |B| (B: the reference selection)."""
    a, b = a.cpu().numpy(), b.cpu().numpy()
    r = []
    for x, y in zip(a, b):
        ys = set(y[y >= 0].tolist())
        if ys:
            r.append(len(set(x[x >= 0].tolist()) & ys) / len(ys))
    return float(np.mean(r))


@pytest.mark.parametrize("name,kw", [("spec_decode_128k", dict(batch=4, ctx_lo=40000, ctx_hi=40000)),
                                     ("decode_b32", dict(batch=8))])
def test_mx_hit_rate_against_bf16_query_path(name, kw):
    s = W.spec(name, **kw)
    wl = W.make(s, device="cuda", with_attn=False)
    ref, _ = sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq, wl.q_pos,
                                     wl.q_idx, wl.w, s.topk, group=s.q_per_seq)
    kc, ks, qc, qs = mx_from_reference(wl)
    got, _ = sia.sparse_indexer_topk_mxfp8(wl.page_table, wl.seq_lens, kc, ks, wl.q_seq, wl.q_pos, qc, qs, wl.w,
                                           s.topk, group=s.q_per_seq)
    torch.cuda.synchronize()
    h = hit_rate(got, ref)
    print(f"{name}: MXFP8 Top-{s.topk} hit rate against the bf16-query path {h:.4f}", flush=True)
    assert h >= 0.9
