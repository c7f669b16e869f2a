"""Pins of the oracle's attention over the FP8 latent cache (CPU only):

* with power-of-two block scales every dequantized value is exact in bf16, so
  the FP8 form must give exactly the bf16-cache oracle's results on a bf16
  cache holding those values (a wrong block index, code byte or rope offset
  changes them);
* a single selected row returns that row's dequantized latent part, with
  LSE = its logit (closed form);
* numpy softmax attention over the dequantized rows (torch's e4m3fn decoder
  times the row's fp32 block scales, bf16 rope)."""
import numpy as np
import torch

import oracle
import workloads as W


def _case(seed=5):
    s = W.spec("decode_b32", batch=2, ctx_lo=300, ctx_hi=400, topk=64, heads_attn=16, seed=seed)
    wl = W.make(s, device="cpu")
    return s, wl, W.make_kv8(wl)


def _dequant(kv8):
    rows = kv8.reshape(-1, 656)
    codes = rows[:, :512].contiguous().view(torch.float8_e4m3fn).double()
    sc = rows[:, 512:528].contiguous().view(torch.float32).double()
    rope = rows[:, 528:].contiguous().view(torch.bfloat16).double()
    lat = codes * sc.repeat_interleave(128, dim=1)
    return torch.cat([lat, rope], dim=1).numpy()


def test_power_of_two_scales_equal_the_bf16_cache_oracle():
    s, wl, kv8 = _case()
    g = torch.Generator().manual_seed(1)
    pw = torch.randint(-6, 4, (kv8.shape[0] * 64, 4), generator=g).double()
    flat = kv8.view(-1, 656)
    flat[:, 512:528] = (2.0 ** pw).float().view(torch.uint8).view(-1, 16)
    vals = torch.from_numpy(_dequant(kv8))
    kv_bf16 = vals.to(torch.bfloat16)
    assert torch.equal(kv_bf16.double(), vals)                 # exact in bf16
    wl16 = W.Workload(**{**wl.__dict__, "kv": kv_bf16.view(wl.kv.shape)})
    idx = np.stack([np.random.default_rng(j).choice(int(wl.seq_lens[j]), 64, replace=False)
                    for j in range(wl.num_q)]).astype(np.int32)
    a_out, a_lse = oracle.sparse_mla_fp8(wl.q_seq, 2, wl.page_table, kv8, wl.q_attn, idx, s.sm_scale)
    b_out, b_lse = oracle.sparse_mla(wl16.q_seq, 2, wl16.page_table, wl16.kv, wl16.q_attn, idx, s.sm_scale)
    assert np.array_equal(a_out, b_out) and np.array_equal(a_lse, b_lse)


def test_single_row_returns_its_latent_values():
    s, wl, kv8 = _case(seed=8)
    idx = np.full((wl.num_q, 64), -1, dtype=np.int32)
    idx[:, 17] = [5, 250]
    out, lse = oracle.sparse_mla_fp8(wl.q_seq, 2, wl.page_table, kv8, wl.q_attn, idx, s.sm_scale)
    vals = _dequant(kv8)
    table = wl.page_table.numpy()
    for j, pos in enumerate([5, 250]):
        r = int(table[j, pos // 64]) * 64 + pos % 64
        q = wl.q_attn[j].double().numpy()
        assert np.array_equal(out[j], np.broadcast_to(vals[r, :512], out[j].shape))
        assert np.allclose(lse[j], s.sm_scale * (q @ vals[r]), rtol=1e-13, atol=1e-13)


def test_matches_numpy_attention_on_dequantized_rows():
    s, wl, kv8 = _case(seed=11)
    vals = _dequant(kv8)
    table = wl.page_table.numpy()
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(int(wl.seq_lens[j]), 64, replace=False) for j in range(wl.num_q)]).astype(np.int32)
    idx[0, 10:20] = -1
    out, lse = oracle.sparse_mla_fp8(wl.q_seq, 2, wl.page_table, kv8, wl.q_attn, idx, s.sm_scale)
    for j in range(wl.num_q):
        sel = idx[j][idx[j] >= 0]
        rows = table[j][sel // 64].astype(np.int64) * 64 + sel % 64
        c = vals[rows]
        z = s.sm_scale * (wl.q_attn[j].double().numpy() @ c.T)          # [H, m]
        p = np.exp(z - z.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ c[:, :512]
        assert np.allclose(out[j], ref, rtol=1e-10, atol=1e-12)
        assert np.allclose(lse[j], z.max(axis=1) + np.log(p.sum(axis=1)), rtol=1e-12)
