"""CPU model of the streaming Top-K's candidate buffer (host logic, no GPU).

The fused prefill indexer keeps, per query, a buffer of at most `cap` candidate
keys in position order. A position is appended when its key beats the running
threshold tau (strictly). When the buffer is full it is re-selected: the first
time to exactly the Top-K (tau = the K-th key), later to a superset found in one
histogram pass (every key >= L, where L is the bits all buffered keys share
followed by the digit of the K-th largest key; tau = L), unless that superset is
too large, in which case the exact threshold is taken. The four queries of a
workgroup re-select together: at a tile boundary where any of them might
overflow, every one holding more than K keys re-selects, so a buffer may also be
re-selected before it is full. The final selection over the buffer is exact,
ties going to the lower position.

This model restates those rules in plain Python and checks, on random rows with
many ties and on rising and falling rows, that the result equals the brute-force
Top-K: a dropped position never belongs to the final Top-K.
"""
from __future__ import annotations

import numpy as np
import pytest


def brute_topk(keys: np.ndarray, k: int) -> list[int]:
    """Positions of the k largest nonzero keys, ties to the lower position,
    listed ascending."""
    order = sorted((i for i in range(len(keys)) if keys[i] != 0), key=lambda i: (-int(keys[i]), i))
    return sorted(order[:k])


def exact_threshold(buf: list[tuple[int, int]], k: int) -> tuple[int, int]:
    """(T, ties): the K-th largest key and how many keys equal to it to keep."""
    ks = sorted((key for key, _ in buf), reverse=True)
    t = ks[k - 1]
    above = sum(1 for x in ks if x > t)
    return t, k - above


def keep_exact(buf, k):
    t, ties = exact_threshold(buf, k)
    out, eq = [], 0
    for key, pos in buf:
        if key > t:
            out.append((key, pos))
        elif key == t and eq < ties:
            out.append((key, pos))
            eq += 1
    return out, t


def superset_floor(buf, k):
    """(L, kept): one 8-bit digit below the bits shared by all keys."""
    a, o = 0xFFFFFFFF, 0
    for key, _ in buf:
        a &= key
        o |= key
    diff = a ^ o
    lead = 32 if diff == 0 else 32 - diff.bit_length()
    width = min(8, 32 - lead)
    shift = 32 - lead - width
    dmask = (1 << width) - 1
    pmask = 0 if lead == 0 else (0xFFFFFFFF << (32 - lead)) & 0xFFFFFFFF
    hist = [0] * 256
    for key, _ in buf:
        hist[(key >> shift) & dmask] += 1
    above = 0
    for b in range(255, -1, -1):
        if above + hist[b] >= k:
            return (a & pmask) | (b << shift), above + hist[b]
        above += hist[b]
    raise AssertionError("fewer keys than k")


def stream_topk(keys: np.ndarray, k: int, cap: int, votes=frozenset()) -> list[int]:
    """`votes`: positions before which a partner's vote makes this buffer
    re-select although it is not full (only if it holds more than k keys)."""
    buf: list[tuple[int, int]] = []
    tau = 0
    for p, key in enumerate(int(x) for x in keys):
        if len(buf) > cap - 1 or (p in votes and len(buf) > k):
            if tau != 0:
                L, kept = superset_floor(buf, k)
                if L != 0 and kept <= k + (cap - k) // 2:
                    buf = [(x, q) for x, q in buf if x >= L]
                    assert len(buf) == kept
                    tau = L
                else:
                    buf, tau = keep_exact(buf, k)
            else:
                buf, tau = keep_exact(buf, k)
        if key > tau:
            buf.append((key, p))
    if len(buf) <= k:
        return sorted(q for _, q in buf)
    final, _ = keep_exact(buf, k)
    return sorted(q for _, q in final)


@pytest.mark.parametrize("pattern", ["random", "few_values", "rising", "falling", "rising_steps"])
@pytest.mark.parametrize("k,cap", [(8, 32), (16, 40), (64, 160)])
def test_stream_buffer_rules_give_exact_topk(pattern, k, cap):
    rng = np.random.default_rng(1234 + k)
    n = 3000
    if pattern == "random":
        keys = rng.integers(1, 1 << 32, size=n, dtype=np.uint64)
    elif pattern == "few_values":   # heavy ties
        keys = rng.choice(np.array([0x80000000 + v for v in (1, 2, 3, 5, 8, 13)], dtype=np.uint64), size=n)
    elif pattern == "rising":
        keys = np.arange(1, n + 1, dtype=np.uint64) * 7919 + 0x80000000
    elif pattern == "falling":
        keys = (np.arange(n, 0, -1, dtype=np.uint64) * 7919) + 0x80000000
    else:                           # rising in steps of seven equal keys
        keys = (np.arange(n, dtype=np.uint64) // 7) * 3 + 0xBF000000
    keys[rng.integers(0, n, size=n // 10)] = 0   # non-candidates (invisible positions)
    assert stream_topk(keys, k, cap) == brute_topk(keys, k)
    # partners' votes at random tile boundaries (32 positions)
    votes = frozenset(int(v) * 32 for v in rng.integers(1, n // 32, size=n // 128))
    assert stream_topk(keys, k, cap, votes) == brute_topk(keys, k)


def test_model_detects_a_wrong_tie_rule():
    """The superset must keep the keys equal to L: a variant that keeps only the
    keys above L loses Top-K members on rows whose keys sit on digit boundaries
    (heavy ties), while the rule as built stays exact on the same rows."""
    k, cap = 16, 40

    def dropping_ties(keys):
        buf, tau = [], 0
        for p, key in enumerate(int(x) for x in keys):
            if len(buf) > cap - 1:
                if tau != 0:
                    L, _ = superset_floor(buf, k)
                    buf = [(x, q) for x, q in buf if x > L]   # loses the keys equal to L
                    tau = L
                else:
                    buf, tau = keep_exact(buf, k)
            if key > tau:
                buf.append((key, p))
        final = keep_exact(buf, k)[0] if len(buf) > k else buf
        return sorted(q for _, q in final)

    caught = 0
    for seed in (2, 4):
        rng = np.random.default_rng(seed)
        keys = (0x80000000 + (rng.integers(1, 40, size=600).astype(np.uint64) << 8)).astype(np.uint64)
        assert stream_topk(keys, k, cap) == brute_topk(keys, k)
        caught += dropping_ties(keys) != brute_topk(keys, k)
    assert caught == 2
