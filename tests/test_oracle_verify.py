"""Pins of the verification oracle (oracle_verify) against what fixes it independently of its
own code: a case worked by hand (tests/golden/verify_hand_v2.json), the defining property of
both algorithms (the verified output, continued by the target model, is distributed exactly as
the target model's own samples: a chi-squared test over every sequence of a tiny vocabulary,
with a control that a biased verifier fails it), the reduction of block verification to token
verification at T = 1, identical draft and target (everything kept), exact inverse-CDF draws at
probability boundaries, and the support of the replacement token.

Sources: speculative sampling, Leviathan, Kalman, Matias, ICML 2023, Algorithm 1; block
verification, Sun et al., ICLR 2025, Algorithm 2 (Theorem: the output keeps the target
distribution; block verification keeps at least as many tokens on average). The pages ask for
exactly this property: vLLM PR #64476, Validation (block verification keeps the target
distribution across draft steps) and PR #62958, Details (rejection sampling on the stored bf16
distribution)."""
import json
import os

import numpy as np
import pytest
import torch
from scipy.stats import chi2

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_hand_v2.json")
MODES = {"token": oracle.VERIFY_TOKEN, "block": oracle.VERIFY_BLOCK}


def bf16_bits(x):
    return (torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16)
            .numpy().view(np.uint16))


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def softmax64(z):
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------------------------
# worked by hand
# ----------------------------------------------------------------------------------------------
def _golden():
    g = json.load(open(GOLDEN))
    f = lambda v: -np.inf if v == "-inf" else float(v)  # noqa: E731
    lb = bf16_bits([[f(v) for v in row] for row in g["draft_logits"]])[None]
    X = np.array([g["draft_tokens"]], np.int32)
    tg = np.array([g["target_logits"]], np.float32)
    tp = np.array([g["temperature"]], np.float32)
    return g, lb, X, tg, tp


@pytest.mark.parametrize("mode", ["token", "block"])
def test_hand_worked_two_token_block(mode):
    g, lb, X, tg, tp = _golden()
    for case in g["cases"]:
        u = np.array([case["uniforms"]], np.float32)
        acc, out, prob = oracle.verify(lb, X, tg, tp, u, MODES[mode])
        assert int(acc[0]) == case[mode]["accepted"]
        assert out[0].tolist() == case[mode]["out_tokens"]
        assert np.allclose(prob[0], g["accept_prob"][mode], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------------------------
# the defining property: verified output, continued by the target, ~ the target's own samples
# ----------------------------------------------------------------------------------------------
def _prefix_tables(V, T, seed, scale):
    """Logits of the target and the draft for every prefix of length 0..T (draft: 0..T-1),
    indexed by the prefix read as a base-V number; draft logits rounded to bf16 (the stored
    rows the draft samples from)."""
    rng = np.random.default_rng(seed)
    tp = [rng.normal(0.0, scale, (V ** L, V)).astype(np.float32) for L in range(T + 1)]
    tq = [bf16_bits(rng.normal(0.0, scale, (V ** L, V))) for L in range(T)]
    return tp, tq


def _sample_rows(probs, u):
    """One index per row of probs by inverse CDF with uniforms u (test-side drafting)."""
    c = np.cumsum(probs, axis=1)
    return np.minimum((c <= u[:, None] * c[:, -1:]).sum(axis=1), probs.shape[1] - 1)


def _simulate(V, T, n, seed, mode, temp=1.0, scale=1.2, accept_all=False):
    tp, tq = _prefix_tables(V, T, seed, scale)
    rng = np.random.default_rng(seed + 1)
    idx = np.zeros(n, np.int64)
    X = np.zeros((n, T), np.int32)
    lb = np.zeros((n, T, V), np.uint16)
    tg = np.zeros((n, T + 1, V), np.float32)
    for t in range(T):
        lb[:, t] = tq[t][idx]
        tg[:, t] = tp[t][idx]
        q = softmax64(bf16_value(lb[:, t]).astype(np.float64) / temp)
        X[:, t] = _sample_rows(q, rng.random(n))
        idx = idx * V + X[:, t]
    tg[:, T] = tp[T][idx]
    u = rng.random((n, T + 1)).astype(np.float32)
    u = np.maximum(u, np.float32(2.0 ** -24))
    temps = np.full(n, temp, np.float32)
    if accept_all:                      # control: keep every draft token, then a target draw
        acc = np.full(n, T, np.int32)
        out = np.concatenate([X, _sample_rows(softmax64(tg[:, T] / temp), u[:, T])[:, None]], 1)
    else:
        acc, out, _ = oracle.verify(lb, X, tg, temps, u, mode)
    # continue every output to T + 1 tokens with the target model
    seq = out.astype(np.int64).copy()
    pidx = np.zeros(n, np.int64)
    for t in range(T + 1):
        need = seq[:, t] < 0
        if need.any():
            p = softmax64(tp[t][pidx[need]] / temp)
            seq[need, t] = _sample_rows(p, rng.random(int(need.sum())))
        pidx = pidx * V + seq[:, t]
    # exact joint of the target over V^(T+1) sequences
    joint = np.ones(1)
    for t in range(T + 1):
        p = softmax64(tp[t] / temp)                       # [V^t, V]
        joint = (joint[:, None] * p).reshape(-1)
    counts = np.bincount(pidx, minlength=V ** (T + 1))
    return counts, joint * n, acc


def _chi2_p(counts, expected):
    """Pearson chi-squared p-value; cells expected below 5 are pooled into one."""
    small = expected < 5.0
    c = np.append(counts[~small], counts[small].sum())
    e = np.append(expected[~small], expected[small].sum())
    if e[-1] == 0.0:
        c, e = c[:-1], e[:-1]
    stat = float(((c - e) ** 2 / e).sum())
    return chi2.sf(stat, len(e) - 1)


# Sizes: with V <= 3 the replacement distributions max(w p - q, 0) and max(p - q, 0) put their
# mass on nearly the same tokens, so an oracle that dropped the weight w would go unnoticed
# there; V = 6 (T = 2) and V = 5 (T = 3) at a million draws tell them apart, and tell apart
# h_i without its 1 - w_i term and a block verifier that stops at the first failed step.
@pytest.mark.parametrize("mode", ["token", "block"])
@pytest.mark.parametrize("V,T,temp,seed,scale,n", [(3, 2, 1.0, 11, 1.2, 120_000),
                                                   (2, 3, 0.7, 12, 1.2, 120_000),
                                                   (4, 1, 1.3, 13, 1.2, 120_000),
                                                   (6, 2, 1.0, 31, 2.0, 1_000_000),
                                                   (5, 3, 1.0, 33, 2.0, 1_000_000)])
def test_verified_output_keeps_target_distribution(mode, V, T, temp, seed, scale, n):
    counts, expected, _ = _simulate(V, T, n, seed, MODES[mode], temp=temp, scale=scale)
    assert _chi2_p(counts, expected) > 1e-4


def test_chi2_rejects_a_verifier_that_keeps_every_draft_token():
    counts, expected, _ = _simulate(3, 2, 120_000, 11, 0, accept_all=True)
    assert _chi2_p(counts, expected) < 1e-12
    counts, expected, _ = _simulate(6, 2, 1_000_000, 31, 0, scale=2.0, accept_all=True)
    assert _chi2_p(counts, expected) < 1e-12


def test_block_keeps_at_least_as_many_tokens_on_average():
    """Sun et al.: block verification is optimal among valid verifiers; on the same inputs it
    keeps at least as many tokens in expectation as token verification (here, within noise)."""
    for V, T, seed in [(3, 2, 21), (2, 3, 22), (4, 3, 23)]:
        _, _, acc_t = _simulate(V, T, 60_000, seed, oracle.VERIFY_TOKEN)
        _, _, acc_b = _simulate(V, T, 60_000, seed, oracle.VERIFY_BLOCK)
        se = np.sqrt((acc_t.var() + acc_b.var()) / len(acc_t))
        assert acc_b.mean() >= acc_t.mean() - 4 * se


# ----------------------------------------------------------------------------------------------
# special cases
# ----------------------------------------------------------------------------------------------
def _random_inputs(bs, T, V, seed, noise=1.0):
    rng = np.random.default_rng(seed)
    draft = rng.normal(0.0, 2.0, (bs, T, V)).astype(np.float32)
    lb = bf16_bits(draft)
    tg = (np.concatenate([draft, rng.normal(0.0, 2.0, (bs, 1, V))], 1) +
          rng.normal(0.0, noise, (bs, T + 1, V))).astype(np.float32)
    X = rng.integers(0, V, (bs, T)).astype(np.int32)
    u = np.maximum(rng.random((bs, T + 1)).astype(np.float32), np.float32(2.0 ** -24))
    temps = rng.uniform(0.5, 1.5, bs).astype(np.float32)
    return lb, X, tg, temps, u


def test_one_step_block_is_token_verification():
    lb, X, tg, temps, u = _random_inputs(400, 1, 50, 3)
    a = oracle.verify(lb, X, tg, temps, u, oracle.VERIFY_TOKEN)
    b = oracle.verify(lb, X, tg, temps, u, oracle.VERIFY_BLOCK)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.allclose(a[2], b[2], rtol=0, atol=1e-15)


@pytest.mark.parametrize("mode", ["token", "block"])
def test_identical_draft_and_target_keep_everything(mode):
    """p = q at every step: every ratio is 1 (w_i = 1, R_i = 0, h_i = 1), so all T tokens are
    kept for any u < 1 and the next token is the inverse-CDF draw from p_T."""
    bs, T, V = 50, 4, 33
    rng = np.random.default_rng(5)
    lb = bf16_bits(rng.normal(0.0, 2.0, (bs, T, V)))
    tg = np.concatenate([bf16_value(lb), rng.normal(0.0, 2.0, (bs, 1, V)).astype(np.float32)], 1)
    X = rng.integers(0, V, (bs, T)).astype(np.int32)
    u = rng.random((bs, T + 1)).astype(np.float32) * np.float32(0.999)
    acc, out, prob = oracle.verify(lb, X, tg, np.ones(bs, np.float32), u, MODES[mode])
    assert (acc == T).all()
    assert np.allclose(prob, 1.0, rtol=0, atol=1e-12)
    assert np.array_equal(out[:, :T], X)
    p = softmax64(tg[:, T])
    assert np.array_equal(out[:, T], _sample_rows(p, u[:, T].astype(np.float64)))


@pytest.mark.parametrize("mode", ["token", "block"])
def test_inverse_cdf_at_exact_boundaries(mode):
    """Final draws from rows whose probabilities are exact binary fractions (logits 0 and -inf):
    the draw is the first index whose cumulative mass exceeds u * mass, never an index of zero
    mass. Draft = target, so every step is kept and the draw is from p_T."""
    V = 4
    rows = {  # target row T -> (u, expected index)
        "uniform": ([0.0, 0.0, 0.0, 0.0], [(0.5, 2), (0.49999997, 1), (0.25, 1), (0.2499999, 0),
                                          (0.9999999, 3), (2.0 ** -24, 0)]),
        "holes": ([-np.inf, 0.0, -np.inf, 0.0], [(2.0 ** -24, 1), (0.5, 3), (0.4999999, 1),
                                                  (0.9999999, 3)]),
    }
    for tgt, cases in rows.values():
        for uT, want in cases:
            lb = bf16_bits(np.zeros((1, 1, V)))
            tg = np.stack([np.zeros(V), np.asarray(tgt)]).astype(np.float32)[None]
            u = np.array([[0.5, uT]], np.float32)
            acc, out, _ = oracle.verify(lb, np.array([[2]], np.int32), tg,
                                        np.ones(1, np.float32), u, MODES[mode])
            assert int(acc[0]) == 1 and out[0].tolist() == [2, want], (tgt, uT)


def test_replacement_token_support():
    """After a rejection at step tau the new token lies where the replacement distribution has
    mass: p_tau > q_tau (token mode), w_tau p_tau > q_tau (block mode)."""
    lb, X, tg, temps, u = _random_inputs(300, 3, 40, 8, noise=2.0)
    for mode in (oracle.VERIFY_TOKEN, oracle.VERIFY_BLOCK):
        acc, out, prob = oracle.verify(lb, X, tg, temps, u, mode)
        for b in range(len(acc)):
            tau = int(acc[b])
            if tau == X.shape[1]:
                continue
            y = int(out[b, tau])
            p = softmax64(tg[b, tau] / temps[b])
            q = softmax64(bf16_value(lb[b, tau]).astype(np.float64) / temps[b])
            w = 1.0
            if mode == oracle.VERIFY_BLOCK:
                for i in range(tau):
                    pi = softmax64(tg[b, i] / temps[b])[X[b, i]]
                    qi = softmax64(bf16_value(lb[b, i]).astype(np.float64) / temps[b])[X[b, i]]
                    w = min(w * pi / qi, 1.0)
            assert w * p[y] > q[y], (mode, b, tau)
        assert (out[np.arange(len(acc)), acc] >= 0).all()
        assert all((out[b, int(acc[b]) + 1:] == -1).all() for b in range(len(acc)))


def test_token_mode_acceptance_probability_is_min_one_ratio():
    lb, X, tg, temps, u = _random_inputs(100, 3, 64, 9)
    _, _, prob = oracle.verify(lb, X, tg, temps, u, oracle.VERIFY_TOKEN)
    for b in range(100):
        for t in range(3):
            p = softmax64(tg[b, t] / np.float64(temps[b]))[X[b, t]]
            q = softmax64(bf16_value(lb[b, t]).astype(np.float64) / np.float64(temps[b]))[X[b, t]]
            assert abs(prob[b, t] - min(1.0, p / q)) < 1e-12


def test_rejects_bad_inputs():
    lb, X, tg, temps, u = _random_inputs(2, 2, 8, 1)
    bad = tg.copy(); bad[1, 0, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.verify(lb, X, bad, temps, u)
    bx = X.copy(); bx[0, 1] = 8
    with pytest.raises(oracle.OracleError):
        oracle.verify(lb, bx, tg, temps, u)
    with pytest.raises(oracle.OracleError):
        oracle.verify(lb, X, tg, np.array([1.0, 0.0], np.float32), u)
