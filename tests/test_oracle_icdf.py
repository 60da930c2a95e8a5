"""Pins of the oracle's inverse-CDF sampler (sample == 2): its uniform is the documented Philox
word through the pinned uniform map; the draw equals numpy's fp64 cumulative-sum search on
random rows and exact binary-fraction rows at their boundaries; token frequencies over many
seeds follow softmax(lb / temp) (chi-squared); the walk stores the same bf16 row as the Gumbel
walk; and the token-feedback walk is unchanged."""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
from tests import structured

RANK = 256


def bf16_bits(x):
    return (torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16)
            .numpy().view(np.uint16))


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_uniform_is_the_documented_philox_word():
    """u = uniform(word 0 of Philox4x32-10 at counter (0, lo32 P, hi32 P, 1), key seed)."""
    for seed, P in [(0, 0), (1, 7), (2**64 - 1, 15), (0x0123456789ABCDEF, (3 << 32) | 9)]:
        w = oracle.philox4x32_10([0, P & 0xFFFFFFFF, P >> 32, 1], [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.icdf_uniform(seed, P) == oracle.uniform(int(w[0]))
        assert oracle.icdf_uniform(seed, P) == (2 * (int(w[0]) >> 9) + 1) / 2.0 ** 24


def _numpy_draw(bits, temp, u):
    z = bf16_value(bits).astype(np.float64) / temp
    e = np.exp(z - z.max())
    c = np.cumsum(e)
    hit = np.flatnonzero(c > u * e.sum())
    return int(hit[0]) if hit.size else int(np.flatnonzero(e > 0)[-1])


def test_draw_matches_numpy_cumsum():
    rng = np.random.default_rng(3)
    for trial in range(300):
        V = int(rng.integers(1, 3000))
        bits = bf16_bits(rng.normal(0, 3.0, V))
        if trial % 7 == 0:
            bits[rng.random(V) < 0.5] = 0xFF80                  # -inf entries
            bits[0] = 0x3F80
        temp = float(rng.uniform(0.3, 2.0))
        u = float(rng.random())
        assert oracle.icdf_draw(bits, temp, u) == _numpy_draw(bits, temp, u)


def test_draw_exact_boundaries_and_zero_mass():
    uni = bf16_bits([0.0, 0.0, 0.0, 0.0])
    for u, want in [(0.5, 2), (0.49999997, 1), (0.25, 1), (0.2499999, 0), (0.9999999, 3)]:
        assert oracle.icdf_draw(uni, 1.0, u) == want
    holes = bf16_bits([-np.inf, 0.0, -np.inf, 0.0])
    for u, want in [(2.0 ** -24, 1), (0.5, 3), (0.4999999, 1)]:
        assert oracle.icdf_draw(holes, 1.0, u) == want
    assert oracle.icdf_draw(bf16_bits([-np.inf, -np.inf]), 1.0, 0.5) == -1
    assert oracle.icdf_draw(bf16_bits([0.0, np.nan]), 1.0, 0.5) == -1


@pytest.mark.parametrize("temp", [1.0, 0.5, 2.0])
def test_frequencies_are_softmax(temp):
    base_row = np.array([0.0, 0.5, -1.0, 1.25, 2.0, -0.75, 0.25, 1.0], np.float32)
    V, n = base_row.size, 100_000
    q = np.zeros((V, RANK), np.int8)
    s = np.zeros(V, np.float32)
    w1 = np.zeros((V, RANK), np.float32)
    base = np.broadcast_to(base_row, (n, 1, V)).copy()
    seeds = np.arange(n, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15) + np.uint64(77)
    tokens, _, _ = oracle.walk(q, s, w1, base, np.zeros(n, np.int32), sample=2, seeds=seeds,
                               temps=np.full(n, temp, np.float32))
    counts = np.bincount(tokens[:, 0], minlength=V)
    p = np.exp(base_row.astype(np.float64) / temp)
    p /= p.sum()
    assert stats.chisquare(counts, p * n).pvalue > 1e-3


def test_stored_row_is_the_gumbel_walks_and_position_matters():
    rng = np.random.default_rng(8)
    V, T = 500, 3
    q, s = oracle.quantize_w2(rng.normal(0, 0.05, (V, RANK)).astype(np.float32))
    w1 = rng.normal(0, 0.05, (V, RANK)).astype(np.float32)
    base = rng.normal(0, 2.0, (2, T, V)).astype(np.float32)
    start = np.array([3, 400], np.int32)
    seeds = np.array([11, 12], np.uint64)
    temps = np.ones(2, np.float32)
    tg, lg, lbg = oracle.walk(q, s, w1, base, start, sample=True, seeds=seeds, temps=temps,
                              want_logits=True)
    ti, li, lbi = oracle.walk(q, s, w1, base, start, sample=2, seeds=seeds, temps=temps,
                              want_logits=True)
    # teacher-forced: same previous token gives the same logits and stored row
    for b in range(2):
        prev = int(start[b])
        for t in range(T):
            tok, l, lb, _ = oracle.step(q, s, w1, base[b, t], prev, sample=2, seed=int(seeds[b]), P=t)
            assert np.array_equal(lb, bf16_bits(l))
            assert tok == oracle.icdf_draw(lb, 1.0, oracle.icdf_uniform(int(seeds[b]), t))
            prev = int(ti[b, t])
    t0 = [oracle.walk(q, s, w1, base[:1], start[:1], sample=2, seeds=seeds[:1], temps=temps[:1],
                      positions=np.array([p], np.int64))[0][0, 0] for p in range(40)]
    assert len(set(t0)) > 1                                 # the position changes the draw


def test_token_feedback_cycle():
    c = structured.feedback_cycle()
    bs = c["base"].shape[0]
    tokens, _, _ = oracle.walk(*oracle.quantize_w2(c["w2"]), c["w1"], c["base"], c["start"],
                               sample=2, seeds=np.arange(bs, dtype=np.uint64) + 5,
                               temps=np.ones(bs, np.float32))
    assert np.array_equal(tokens[0], c["expected"])
