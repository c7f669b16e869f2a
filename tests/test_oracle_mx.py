"""Pins of the oracle's MXFP8 index path (CPU only), each against something
other than the oracle itself:

* the quantizer against its definition: the scale exponent is the smallest in
  [-127, 127] that keeps the group's largest magnitude within 448 * 2^e, and
  every code is torch's round-to-nearest-even e4m3fn cast of x / 2^e;
* the MXFP8 scores against numpy: elements dequantized with torch's e4m3fn
  decoder times 2^(byte - 127) per 32-element block, paged rows gathered by
  explicit numpy indexing, then sum_h w_h max(0, q_h . k_s) by matmul;
* exact homogeneity: raising every key block scale by one doubles every score,
  raising one head's query scales scales that head's term;
* with every block scale 2^0 the MXFP8 scores equal the fp8 path's with
  per-token scale 1 on a bf16 query holding the same e4m3 values."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def test_quantizer_matches_its_definition():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(64, 128, generator=g) * torch.logspace(-8, 8, 64, base=2.0)[:, None]
    x[0] = 0.0                                   # all-zero groups
    x[1, :32] = 448.0 * 2.0 ** 3                 # largest magnitude exactly 448 * 2^3
    x[1, 32:64] = -448.0 * 2.0 ** -5
    x[2, :32] = 1e-30                            # tiny groups
    x[5, :32] = 448.0                            # e = 0 with negative values that round to -0
    x[5, 1:8] = -torch.tensor([1e-6, 5e-4, 9.7e-4, 2e-3, 0.0, 1.9e-3, 1e-30])
    x[6, 32:64] = -0.0
    xb = _bf16(x)
    codes, scales = oracle.quantize_mxfp8(xb)
    xv = xb.double().numpy().reshape(64, 4, 32)
    e = scales.astype(np.int64).reshape(64, 4) - 127
    m = np.abs(xv).max(axis=-1)
    assert np.all(e >= -127) and np.all(e <= 127)
    # smallest e with m <= 448 * 2^e
    assert np.all(m <= 448.0 * 2.0 ** e)
    assert np.all((e == -127) | (m > 448.0 * 2.0 ** (e - 1)))
    assert np.all(e[0] == -127) and np.all(codes[0] == 0)
    assert e[1, 0] == 3 and e[1, 1] == -5
    assert codes[1, 0] == 0x7E and codes[1, 32] == 0xFE          # +448 and -448
    assert codes[5, 1] == 0x80 and codes[6, 32] == 0x80          # -0 keeps its sign
    # codes: torch's RNE cast of x / 2^e
    scaled = torch.from_numpy(xv / 2.0 ** e[..., None]).float().reshape(64, 128)
    ref = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_quantizer_ties_go_to_even_codes():
    """x / 2^e exactly halfway between neighbouring e4m3 codes c and c + 1
    takes the even one of the two."""
    e4 = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    lo_codes = np.arange(8, 38)                       # normal neighbours (c, c + 1)
    mids = (e4[lo_codes] + e4[lo_codes + 1]) / 2.0
    x = np.zeros((1, 32))
    x[0, 0] = 448.0                                   # fixes e = 0
    x[0, 1:31] = mids
    assert np.array_equal(_bf16(x).double().numpy(), x)   # (the halfway points are exact in bf16)
    codes, scales = oracle.quantize_mxfp8(_bf16(x))
    assert scales[0, 0] == 127
    want = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1)
    assert np.array_equal(codes[0, 1:31], want)


def _mx_case(seed=3, batch=2, ctx=700, heads=5):
    s = W.spec("decode_b32", batch=batch, ctx_lo=ctx, ctx_hi=ctx + 150, heads_idx=heads, topk=64,
               heads_attn=16, seed=seed)
    wl = W.make(s, device="cpu", with_attn=False)
    mx = W.make_mx(wl, scale_lo=120, scale_hi=134)
    return s, wl, mx


def _numpy_mx_scores(wl, mx):
    kc = wl.idx_k.numpy().reshape(-1, wl.spec.dim_idx)
    ks = mx.k_scales.numpy().reshape(-1, wl.spec.dim_idx // 32).astype(np.int64)
    kv = _e4m3_values(kc) * np.repeat(2.0 ** (ks - 127), 32, axis=1)
    qc, qs = mx.q_codes.numpy(), mx.q_scales.numpy().astype(np.int64)
    qv = _e4m3_values(qc) * np.repeat(2.0 ** (qs - 127), 32, axis=2)
    w = wl.w.numpy().astype(np.float64)
    lens = wl.seq_lens.numpy()
    out = []
    for j in range(wl.num_q):
        b = int(wl.q_seq[j])
        n = min(int(wl.q_pos[j]) + 1, int(lens[b]))
        pos = np.arange(n)
        rows = wl.page_table.numpy()[b][pos // 64].astype(np.int64) * 64 + pos % 64
        a = qv[j] @ kv[rows].T                       # [H, n]
        out.append((w[j][:, None] * np.maximum(a, 0.0)).sum(axis=0))
    return out


def test_mx_scores_equal_numpy_on_dequantized_values():
    s, wl, mx = _mx_case()
    sc, rl = oracle.indexer_scores_mx(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k, mx.k_scales,
                                      mx.q_codes, mx.q_scales, wl.w)
    ref = _numpy_mx_scores(wl, mx)
    for j, r in enumerate(ref):
        assert rl[j] == len(r)
        assert np.allclose(sc[j, :len(r)], r, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(sc[j, len(r):]))


def test_mx_scores_are_homogeneous_in_the_block_scales():
    s, wl, mx = _mx_case(seed=9, heads=3)
    base, _ = oracle.indexer_scores_mx(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                       mx.k_scales, mx.q_codes, mx.q_scales, wl.w)
    up, _ = oracle.indexer_scores_mx(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                     mx.k_scales + 1, mx.q_codes, mx.q_scales, wl.w)
    fin = np.isfinite(base)
    assert np.array_equal(up[fin], 2.0 * base[fin])
    # one head's query scales up by one: only that head's term doubles
    w0 = wl.w.clone()
    w0[:, 1:] = 0.0
    h0, _ = oracle.indexer_scores_mx(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k, mx.k_scales,
                                     mx.q_codes, mx.q_scales, w0)
    qs = mx.q_scales.clone()
    qs[:, 0] += 1
    h0_up, _ = oracle.indexer_scores_mx(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                        mx.k_scales, mx.q_codes, qs, w0)
    assert np.array_equal(h0_up[fin], 2.0 * h0[fin])


def test_unit_scales_reduce_to_the_fp8_path():
    s, wl, mx = _mx_case(seed=4)
    ones_k = torch.full_like(mx.k_scales, 127)
    ones_q = torch.full_like(mx.q_scales, 127)
    a, _ = oracle.indexer_scores_mx(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k, ones_k,
                                    mx.q_codes, ones_q, wl.w)
    # the same e4m3 query values as bf16 (exact), an fp8 cache with scale 1
    q_bf16 = torch.from_numpy(_e4m3_values(mx.q_codes.numpy())).float().to(torch.bfloat16)
    b, _ = oracle.indexer_scores(wl.q_seq, wl.q_pos, wl.seq_lens, wl.page_table, wl.idx_k,
                                 torch.ones_like(wl.idx_scale), q_bf16, wl.w)
    assert np.array_equal(np.isfinite(a), np.isfinite(b))
    fin = np.isfinite(a)
    assert np.array_equal(a[fin], b[fin])
