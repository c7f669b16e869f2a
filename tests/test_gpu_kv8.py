"""Sparse MLA attention over the FP8 latent cache (656-byte rows: 512 e4m3
codes with one fp32 scale per 128, and the 64 bf16 rope values) on the GPU,
through the C ABI, against the oracle on the dequantized rows: per (query,
head) output within 2e-2 relative L2, LSE within 1e-4 relative, for 16, 32 and
128 heads (the three workgroup shapes), index lists in any order with
duplicates and interior padding, rows split over several workgroups, and the
128K speculative-decode workload at full size on sampled queries."""
import numpy as np
import pytest
import torch

import indexer_top_sparse_02_amd as sia
import oracle
import workloads as W
from _paths import check_attention, gpu_topk

pytestmark = pytest.mark.gpu


def _run(wl, kv8, idx, ws=None):
    out, lse = sia.sparse_mla_attention(wl.page_table, wl.seq_lens, kv8, wl.q_seq, wl.q_attn, idx,
                                        wl.spec.sm_scale, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


def _ref(wl, kv8, idx_np, rows=None):
    c = wl.to("cpu")
    q_seq, q = c.q_seq, c.q_attn
    if rows is not None:
        q_seq, q = q_seq[rows], q[rows]
    return oracle.sparse_mla_fp8(q_seq, c.seq_lens.numel(), c.page_table, kv8.cpu(), q, idx_np,
                                 wl.spec.sm_scale)


@pytest.mark.parametrize("heads,batch,topk", [(16, 1, 300), (32, 3, 512), (128, 4, 2048), (128, 64, 256)])
def test_kv8_attention_matches_oracle(heads, batch, topk):
    s = W.spec("decode_b32", batch=batch, ctx_lo=2500, ctx_hi=6000, topk=topk, heads_attn=heads)
    wl = W.make(s, device="cuda", poison=True)
    kv8 = W.make_kv8(wl, poison=True)
    idx, _ = gpu_topk(wl)
    print(f"kv8 attention: {heads} heads, {wl.num_q} queries, Top-{topk}", flush=True)
    out, lse = _run(wl, kv8, idx)
    ref_out, ref_lse = _ref(wl, kv8, idx.cpu().numpy())
    check_attention(out, ref_out, lse, ref_lse)


def test_kv8_attention_any_order_duplicates_padding():
    s = W.spec("decode_b32", batch=3, ctx_lo=2000, ctx_hi=4000, topk=300, heads_attn=64)
    wl = W.make(s, device="cuda", poison=True)
    kv8 = W.make_kv8(wl, poison=True)
    g = np.random.default_rng(12)
    n = wl.seq_lens.cpu().numpy()
    ia = np.stack([g.integers(0, int(n[j]), size=300) for j in range(wl.num_q)]).astype(np.int32)
    ia[:, 50:90] = -1
    ia[:, 100:110] = ia[:, :1]
    out, lse = _run(wl, kv8, torch.from_numpy(ia).cuda())
    ref_out, ref_lse = _ref(wl, kv8, ia)
    check_attention(out, ref_out, lse, ref_lse)


def test_kv8_attention_full_size_speculative_decode():
    s = W.spec("spec_decode_128k")
    wl = W.make(s, device="cuda", poison=True)
    kv8 = W.make_kv8(wl, poison=True)
    idx, _ = sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq, wl.q_pos,
                                     wl.q_idx, wl.w, s.topk, group=2)
    out, lse = _run(wl, kv8, idx)
    rows = np.array([0, 1, 63, 64, 126, 127])
    ref_out, ref_lse = _ref(wl, kv8, idx.cpu().numpy()[rows], rows)
    sel = torch.from_numpy(rows).cuda()
    check_attention(out[sel], ref_out, lse[sel], ref_lse)
