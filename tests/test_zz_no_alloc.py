"""sparse_mla_attention_noalloc (the library's static scratch instead of a
caller workspace) against sparse_mla_attention on the same inputs, bit for
bit, on two calls in a row: the first splits each query's rows over several
workgroups (its partials fill most of the scratch), the second is smaller, so
that whatever the first left in the scratch must not leak into it."""
import pytest
import torch

import indexer_top_sparse_02_amd as sia
import workloads as W
from _paths import gpu_topk

pytestmark = pytest.mark.gpu


def _both(wl, idx):
    s = wl.spec
    need = sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk)
    ref_out, ref_lse = sia.sparse_mla_attention(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn,
                                                idx, s.sm_scale, want_lse=True)
    out, lse = sia.sparse_mla_attention_noalloc(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn,
                                                idx, s.sm_scale, want_lse=True)
    torch.cuda.synchronize()
    return need, (ref_out, ref_lse), (out, lse)


def test_noalloc_attention_matches_workspace_form_twice():
    big = W.spec("decode_b32", batch=4, ctx_lo=9000, ctx_hi=12000)
    wl = W.make(big, device="cuda", poison=True)
    idx, _ = gpu_topk(wl)
    print("no-alloc attention: first call (4 queries, 128 heads, Top-2048)", flush=True)
    need, (ro, rl), (o, l) = _both(wl, idx)
    assert need > 16 << 20   # the first call really uses the scratch for split partials
    assert need <= sia.MLA_NOALLOC_MAX_BYTES
    assert torch.equal(o.view(torch.int16), ro.view(torch.int16))
    assert torch.equal(l, rl)
    small = W.spec("decode_b32", batch=2, ctx_lo=3000, ctx_hi=4000, topk=512, heads_attn=64)
    wl2 = W.make(small, device="cuda", poison=True)
    idx2, _ = gpu_topk(wl2)
    print("no-alloc attention: second call (2 queries, 64 heads, Top-512)", flush=True)
    need2, (ro2, rl2), (o2, l2) = _both(wl2, idx2)
    assert 256 < need2 < need
    assert torch.equal(o2.view(torch.int16), ro2.view(torch.int16))
    assert torch.equal(l2, rl2)
