"""CPU checks of the benchmark's contract and of its work accounting: more than
one GPU is refused with a message, and the algorithmic flops and bytes it
divides by equal their closed forms for the workloads it times."""
import json
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_prefill_flops_closed_form():
    # causal prefill of n tokens: the indexer sees sum_{t<n} (t+1) = n(n+1)/2
    # positions, attention selects sum_t min(t+1, K) rows
    s = W.spec("prefill_16k")
    n, K = 16384, s.topk

    class Q:   # only the query positions are read
        q_pos = torch.arange(n, dtype=torch.int32)
    f_idx, f_att = bench.prefill_flops(s, Q)
    assert f_idx == 2 * 64 * 128 * n * (n + 1) // 2
    sel = K * (K + 1) // 2 + (n - K) * K
    assert f_att == 2 * 128 * (576 + 512) * sel
    assert abs(f_idx / 1e12 - 2.19916) < 1e-4 and abs(f_att / 1e12 - 8.76202) < 1e-4


def test_decode_bytes_closed_form():
    # speculative decode, 64 x 131072 positions, 2 draft tokens, fp8 index rows
    # (128 B + a 4 B scale) read once per sequence; latent rows counted once per
    # sequence even when both draft tokens select them
    s = W.spec("spec_decode_128k", batch=2, ctx_lo=4096, ctx_hi=4096, topk=8)

    class WL:
        spec = s
        seq_lens = torch.tensor([4096, 4096], dtype=torch.int32)
        q_seq = torch.tensor([0, 0, 1, 1], dtype=torch.int32)
        num_q = 4
    idx = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7], [4, 5, 6, 7, 8, 9, 10, -1],
                        [0, 1, 2, 3, 4, 5, 6, 7], [0, 1, 2, 3, 4, 5, 6, 7]], dtype=torch.int32)
    by = bench.algorithmic_bytes(WL, idx)
    assert by["index_k"] == 2 * 4096 * 132
    assert by["latent"] == (11 + 8) * 1152          # union per sequence: 11 and 8 rows
    full = 64 * 131072 * 132 + 128 * (64 * 128 * 2 + 64 * 4) + 64 * 2048 * 4 + 128 * 2048 * 4
    assert abs(full / 1e6 - 1111.0) < 0.1
