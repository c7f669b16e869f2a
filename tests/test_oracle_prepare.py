"""Pins of the oracle's indexer input preparation (CPU only), none of which
calls the matrix product the oracle uses:

* one-hot inputs pick out one column of each weight matrix (written out by
  indexing);
* the normalized key has mean beta and, with beta = 0, mean square gamma^2
  times var / (var + eps) (closed forms of LayerNorm);
* a key projection taking two values a, b in alternation normalizes to
  +-1 times gamma (up to eps), the sign following a vs b;
* scaling the hidden state scales q and w and leaves the normalized key
  unchanged (positive homogeneity of the projections, invariance of LayerNorm)."""
import numpy as np
import torch

import oracle


def _weights(dq=64, dh=96, heads=3, dim=128, seed=0):
    g = torch.Generator().manual_seed(seed)
    wq = torch.randn(heads * dim, dq, generator=g).to(torch.bfloat16)
    wk = torch.randn(dim, dh, generator=g).to(torch.bfloat16)
    ww = torch.randn(heads, dh, generator=g).to(torch.bfloat16)
    gamma = torch.rand(dim, generator=g) + 0.5
    beta = torch.randn(dim, generator=g) * 0.1
    return wq, wk, ww, gamma, beta


def test_one_hot_inputs_select_weight_columns():
    wq, wk, ww, gamma, beta = _weights()
    xq = torch.zeros(2, 64, dtype=torch.bfloat16)
    xh = torch.zeros(2, 96, dtype=torch.bfloat16)
    xq[0, 5] = 1
    xq[1, 63] = 1
    xh[0, 7] = 1
    xh[1, 0] = 1
    q, k, w = oracle.indexer_prepare(xq, xh, wq, wk, gamma, beta, ww, 1e-6)
    assert np.array_equal(q[0], wq[:, 5].double().numpy()) and np.array_equal(q[1], wq[:, 63].double().numpy())
    assert np.array_equal(w[0], ww[:, 7].double().numpy()) and np.array_equal(w[1], ww[:, 0].double().numpy())
    col = wk[:, 7].double().numpy()
    ref = (col - col.mean()) / np.sqrt(col.var() + 1e-6) * gamma.double().numpy() + beta.double().numpy()
    assert np.allclose(k[0], ref, rtol=1e-13, atol=1e-13)


def test_layernorm_closed_forms():
    wq, wk, ww, gamma, beta = _weights(seed=1)
    g = torch.Generator().manual_seed(2)
    xh = torch.randn(5, 96, generator=g).to(torch.bfloat16)
    xq = torch.randn(5, 64, generator=g).to(torch.bfloat16)
    _, k, _ = oracle.indexer_prepare(xq, xh, wq, wk, gamma, beta, ww, 1e-6)
    gm, bt = gamma.double().numpy(), beta.double().numpy()
    z = (k - bt) / gm                          # the normalized values
    assert np.allclose(z.mean(axis=1), 0.0, atol=1e-12)
    kp = xh.double().numpy() @ wk.double().numpy().T
    var = kp.var(axis=1)
    assert np.allclose((z ** 2).mean(axis=1), var / (var + 1e-6), rtol=1e-12)


def test_alternating_key_normalizes_to_plus_minus_one():
    wq, wk, ww, gamma, beta = _weights(seed=3)
    wk = torch.zeros_like(wk)
    wk[0::2, 0] = 3.0
    wk[1::2, 0] = -1.0
    xh = torch.zeros(1, 96, dtype=torch.bfloat16)
    xh[0, 0] = 1.0
    xq = torch.zeros(1, 64, dtype=torch.bfloat16)
    _, k, _ = oracle.indexer_prepare(xq, xh, wq, wk, gamma, torch.zeros(128), ww, 0.0)
    sign = np.where(np.arange(128) % 2 == 0, 1.0, -1.0)
    assert np.allclose(k[0], sign * gamma.double().numpy(), rtol=1e-14, atol=1e-14)


def test_scaling_the_hidden_state():
    wq, wk, ww, gamma, beta = _weights(seed=4)
    g = torch.Generator().manual_seed(5)
    xh = torch.randn(3, 96, generator=g).to(torch.bfloat16)
    xq = torch.randn(3, 64, generator=g).to(torch.bfloat16)
    q1, k1, w1 = oracle.indexer_prepare(xq, xh, wq, wk, gamma, beta, ww, 0.0)
    q2, k2, w2 = oracle.indexer_prepare(xq * 4, xh * 4, wq, wk, gamma, beta, ww, 0.0)
    assert np.array_equal(q2, 4 * q1) and np.array_equal(w2, 4 * w1)
    assert np.allclose(k2, k1, rtol=1e-12, atol=1e-12)
