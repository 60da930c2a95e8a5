"""Pins of the lossless top-k pruning bound (oracle_w2_l1_bound): it equals its definition
evaluated by numpy in fp32, and it bounds the exact bias of every row for any W1 row, so a
certificate built on it can never exclude the true argmax (checked against brute force)."""
import numpy as np
import pytest

import oracle


def _q(V, seed, std=0.02):
    rng = np.random.default_rng(seed)
    return oracle.quantize_w2((rng.normal(0, std, (V, 256))).astype(np.float32))


@pytest.mark.parametrize("V,seed", [(1, 0), (1000, 1), (4097, 2)])
def test_bound_matches_numpy_fp32(V, seed):
    q, s = _q(V, seed)
    want = np.max(s * np.abs(q.astype(np.int32)).sum(axis=1).astype(np.float32))
    assert np.float32(oracle.w2_l1_bound(q, s)) == want


def test_bound_zero_rows_and_special_rows():
    q = np.zeros((3, 256), np.int8)
    s = np.zeros(3, np.float32)
    assert oracle.w2_l1_bound(q, s) == 0.0
    q[1, :] = -127
    s[1] = np.float32(0.5)
    assert oracle.w2_l1_bound(q, s) == np.float32(0.5) * np.float32(256 * 127)


def test_bound_covers_every_bias_and_certifies_the_argmax():
    """For random W2 / W1 / base rows: |bias(v)| <= B * max|w| for every v (fp64 exact bias);
    and whenever best candidate logit - k-th base > B * max|w|, the dense argmax is a candidate."""
    V, k = 3000, 40
    q, s = _q(V, 5, std=0.05)
    B = oracle.w2_l1_bound(q, s)
    deq = s[:, None].astype(np.float64) * q.astype(np.float64)
    rng = np.random.default_rng(6)
    certified = 0
    for trial in range(60):
        w = rng.normal(0, 0.05 * (1 + trial % 4), 256)
        if trial % 5 == 0:
            w[rng.integers(0, 256)] *= 25.0                 # a heavy entry
        bias = deq @ w
        assert np.all(np.abs(bias) <= B * np.abs(w).max() * (1 + 1e-12))
        base = rng.normal(0, 3.0 if trial % 3 else 0.05, V)
        cand = np.lexsort((np.arange(V), -base))[:k]
        logits = base + bias
        lstar = logits[cand].max()
        kth = base[cand].min()
        if lstar - kth > B * np.abs(w).max():
            certified += 1
            assert int(np.argmax(logits)) in set(cand.tolist())
    assert 10 < certified < 60                            # both outcomes occur
