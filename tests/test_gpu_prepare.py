"""Three-stream indexer input preparation on the GPU against the oracle:

* the bf16 query and key (before quantization) within bf16 rounding of the
  double-precision projections and LayerNorm, the fp32 head weights within
  fp32 accumulation error;
* the MXFP8 query and the key rows written into the paged index cache bit for
  bit equal to the oracle's quantizer applied to the GPU's own bf16 values
  (quantization codes are decided on the same bf16 inputs), every other cache
  row untouched;
* three streams give the same bits as one stream."""
import numpy as np
import pytest
import torch

import indexer_top_sparse_02_amd as sia
import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _case(batch, ctx, dq=1536, dh=7168, heads=64, seed=31):
    s = W.spec("spec_decode_128k", batch=batch, ctx_lo=ctx, ctx_hi=ctx)
    wl = W.make(s, device="cuda", with_attn=False)
    mx = W.make_mx(wl)
    g = torch.Generator(device="cuda").manual_seed(seed)
    M = wl.num_q
    xq = torch.randn(M, dq, generator=g, device="cuda").to(torch.bfloat16)
    xh = torch.randn(M, dh, generator=g, device="cuda").to(torch.bfloat16)
    wq = (torch.randn(heads * 128, dq, generator=g, device="cuda") / dq ** 0.5).to(torch.bfloat16)
    wk = (torch.randn(128, dh, generator=g, device="cuda") / dh ** 0.5).to(torch.bfloat16)
    ww = (torch.randn(heads, dh, generator=g, device="cuda") / dh ** 0.5).to(torch.bfloat16)
    gamma = torch.rand(128, generator=g, device="cuda") + 0.5
    beta = torch.randn(128, generator=g, device="cuda") * 0.1
    return wl, mx, (xq, xh, wq, wk, gamma, beta, ww)


def _prepare(wl, mx, args, streams=None):
    k_codes, k_scales = wl.idx_k.clone(), mx.k_scales.clone()
    M = wl.num_q
    q_bf16 = torch.empty((M, 64, 128), dtype=torch.bfloat16, device="cuda")
    k_bf16 = torch.empty((M, 128), dtype=torch.bfloat16, device="cuda")
    xq, xh, wq, wk, gamma, beta, ww = args
    qc, qs, w = sia.indexer_prepare(xq, xh, wq, wk, gamma, beta, ww, wl.page_table, wl.seq_lens, k_codes, k_scales,
                                    wl.q_seq, wl.q_pos, eps=1e-6, streams=streams, q_bf16=q_bf16, k_bf16=k_bf16)
    torch.cuda.synchronize()
    return qc, qs, w, q_bf16, k_bf16, k_codes, k_scales


@pytest.mark.parametrize("batch,ctx", [(3, 5037), (64, 300)])
def test_prepare_matches_oracle(batch, ctx):
    wl, mx, args = _case(batch, ctx)
    print(f"prepare: {wl.num_q} tokens", flush=True)
    qc, qs, w, q_bf16, k_bf16, k_codes, k_scales = _prepare(wl, mx, args)
    xq, xh, wq, wk, gamma, beta, ww = args
    q_ref, k_ref, w_ref = oracle.indexer_prepare(xq, xh, wq, wk, gamma, beta, ww, 1e-6)
    qg = q_bf16.double().cpu().numpy().reshape(q_ref.shape)
    assert np.all(np.abs(qg - q_ref) <= 2.0 ** -8 * np.abs(q_ref) + 1e-4 * np.sqrt((q_ref ** 2).mean()))
    kg = k_bf16.double().cpu().numpy()
    assert np.all(np.abs(kg - k_ref) <= 2.0 ** -8 * np.abs(k_ref) + 1e-3)
    wg = w.double().cpu().numpy()
    assert np.allclose(wg, w_ref, rtol=1e-4, atol=1e-4 * np.sqrt((w_ref ** 2).mean()))
    # MXFP8 codes decided on the GPU's own bf16 values
    rc, rs = oracle.quantize_mxfp8(q_bf16.cpu())
    assert np.array_equal(qc.cpu().numpy(), rc) and np.array_equal(qs.cpu().numpy(), rs)
    kc_ref, ks_ref = oracle.quantize_mxfp8(k_bf16.cpu())
    table = wl.page_table.cpu().numpy()
    pos = wl.q_pos.cpu().numpy()
    seq = wl.q_seq.cpu().numpy()
    rows = table[seq, pos // 64].astype(np.int64) * 64 + pos % 64
    kc = k_codes.view(-1, 128).cpu().numpy()
    ks = k_scales.view(-1, 4).cpu().numpy()
    assert np.array_equal(kc[rows], kc_ref) and np.array_equal(ks[rows], ks_ref)
    other = np.setdiff1d(np.arange(kc.shape[0]), rows)
    assert np.array_equal(kc[other], wl.idx_k.view(-1, 128).cpu().numpy()[other])
    assert np.array_equal(ks[other], mx.k_scales.view(-1, 4).cpu().numpy()[other])


def test_three_streams_equal_one():
    wl, mx, args = _case(64, 300)
    one = _prepare(wl, mx, args)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    three = _prepare(wl, mx, args, streams=streams)
    for a, b in zip(one, three):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)
