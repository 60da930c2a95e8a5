"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle function to a value or law fixed outside the oracle: published
known-answer vectors, an independent installed implementation (rocRAND, compiled and run), a
library routine (numpy / torch on CPU), a closed form, an invariant, or a hand-worked example.
The cases are chosen so that a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a wrong rounding) fails at least one of them.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
from scipy import stats

from tests import structured

RANK = 256
HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------------------------
# Philox4x32-10
# ----------------------------------------------------------------------------------------------
def _kat_rows():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answer_vectors(orc):
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, out in rows:
        assert list(orc.philox4x32_10(ctr, key)) == out


def test_philox_matches_rocrand(orc, tmp_path):
    """rocRAND's philox4x32_10 engine, built from its installed header and run on the host."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "rr"
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", "-I/opt/rocm/include",
                    os.path.join(HERE, "rocrand_philox_words.cpp"), "-o", str(exe)], check=True)
    rng = np.random.default_rng(11)
    triples = []
    for _ in range(300):
        seed = int(rng.integers(0, 2**64, dtype=np.uint64))
        P = int(rng.integers(0, 2**20))          # keeps rocRAND's 64-bit offset in range
        v = int(rng.integers(0, 270336))
        triples.append((seed, P, v))
    triples += [(0, 0, 0), (0, 0, 3), (2**64 - 1, 15, 270335), (1, 2**32 - 1 >> 12, 4)]
    inp = "".join(f"{s} {p} {v}\n" for s, p, v in triples)
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout
    got = [int(x) for x in out.split()]
    want = [orc.noise_word(s, p, v) for s, p, v in triples]
    assert got == want


def test_noise_word_mapping(orc):
    """Counter (v >> 2, lo32(P), hi32(P), 0), key (lo32(seed), hi32(seed)), word v & 3."""
    seed, P = 0x0123456789ABCDEF, (5 << 32) | 77
    for v in [0, 1, 2, 3, 4, 7, 151935]:
        words = orc.philox4x32_10([v >> 2, P & 0xFFFFFFFF, P >> 32, 0],
                                  [seed & 0xFFFFFFFF, seed >> 32])
        assert orc.noise_word(seed, P, v) == int(words[v & 3])


# ----------------------------------------------------------------------------------------------
# uniform / Gumbel
# ----------------------------------------------------------------------------------------------
def test_uniform_closed_form(orc):
    assert orc.uniform(0) == 2.0 ** -24
    assert orc.uniform(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert orc.uniform(0x80000000) == 0.5 + 2.0 ** -24
    assert orc.uniform(0x1FF) == 2.0 ** -24          # the low 9 bits are dropped
    for x in [0, 1 << 9, 12345678, 0xDEADBEEF, 0xFFFFFFFF]:
        u = orc.uniform(x)
        assert float(np.float32(u)) == u             # exact in fp32
        assert 0.0 < u < 1.0


def test_gumbel_closed_form(orc):
    # g = -log(-log u) inverts the Gumbel CDF exp(-exp(-g)).
    for x in [0, 0x40000000, 0x80000000, 0xC0000000, 0xFFFFFFFF]:
        u = orc.uniform(x)
        g = orc.gumbel(x)
        assert abs(np.exp(-np.exp(-g)) - u) <= 1e-12
    # the median of the standard Gumbel is -log(log 2)
    assert abs(orc.gumbel(0x80000000) - (-np.log(np.log(2.0)))) < 1e-6


# ----------------------------------------------------------------------------------------------
# bf16 rounding and argmax order
# ----------------------------------------------------------------------------------------------
def test_bf16_matches_torch(orc):
    rng = np.random.default_rng(3)
    xs = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 7,
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38, 1e-40, -1e-40,
                  1.00390625, 1.01171875, 1.0 + 2 ** -8 + 2 ** -20], np.float32),
    ])
    # exact ties of the rounding: mantissa pattern ...x 1000 0000 0000 0000
    ties = (rng.integers(0, 2**15, 500).astype(np.uint32) << 16) | 0x8000
    xs = np.concatenate([xs, ties.view(np.float32)])
    xs = xs[np.isfinite(xs) | np.isinf(xs)]
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_rne(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, want)
    assert np.isnan(orc.bf16_to_f32(orc.bf16_rne(float("nan"))))


def test_argmax_matches_torch(orc):
    rng = np.random.default_rng(4)
    cases = []
    for _ in range(200):
        n = int(rng.integers(1, 50))
        x = rng.integers(-3, 4, n).astype(np.float32)  # many exact ties
        if rng.random() < 0.3:
            x[rng.integers(0, n, 2)] = np.nan
        if rng.random() < 0.3:
            x[rng.integers(0, n)] = -0.0
        cases.append(x)
    cases.append(np.array([-0.0, 0.0, -1.0], np.float32))
    cases.append(np.array([0.0, -0.0], np.float32))
    cases.append(np.array([-np.inf, -np.inf], np.float32))
    cases.append(np.array([1.0, np.nan, 2.0, np.nan], np.float32))
    for x in cases:
        assert orc.argmax_f32(x) == int(torch.argmax(torch.from_numpy(x)))


# ----------------------------------------------------------------------------------------------
# Quantisation
# ----------------------------------------------------------------------------------------------
def test_quantize_numpy_f32_and_bounds(orc):
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((300, RANK)) * 0.02).astype(np.float32)
    w[7] = 0.0
    w[8, :] = 0.0
    w[8, 3] = -1e-30
    q, s = orc.quantize_w2(w)
    a = np.abs(w).max(axis=1)
    s_np = a / np.float32(127)
    assert np.array_equal(s.view(np.uint32), s_np.view(np.uint32))
    nz = a > 0
    q_np = np.zeros_like(q)
    q_np[nz] = np.clip(np.rint(w[nz] / s_np[nz, None]), -127, 127).astype(np.int8)
    assert np.array_equal(q, q_np)
    # round trip within half a step; the absmax element maps to +-127
    err = np.abs(w.astype(np.float64) - s.astype(np.float64)[:, None] * q)
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 * (1 + 2 ** -20))
    am = np.abs(w).argmax(axis=1)
    assert np.all(np.abs(q[nz, am[nz]].astype(int)) == 127)
    assert s[7] == 0 and np.all(q[7] == 0)


def test_quantize_representable_rows_exact(orc):
    # rows that are s * integer with s = 2^-e and max |code| = 127 quantise with no error
    rng = np.random.default_rng(6)
    codes = rng.integers(-127, 128, (64, RANK))
    codes[:, 0] = 127
    scale = 2.0 ** -rng.integers(2, 12, 64)
    w = (codes * scale[:, None]).astype(np.float32)
    q, s = orc.quantize_w2(w)
    assert np.array_equal(s.astype(np.float64), scale)
    assert np.array_equal(q.astype(np.int64), codes)


def test_quantize_rejects_nonfinite(orc):
    w = np.zeros((3, RANK), np.float32)
    w[1, 5] = np.inf
    with pytest.raises(orc.OracleError):
        orc.quantize_w2(w)
    w[1, 5] = np.nan
    with pytest.raises(orc.OracleError):
        orc.quantize_w2(w)


# ----------------------------------------------------------------------------------------------
# One step: logits by brute force, special cases
# ----------------------------------------------------------------------------------------------
def _rand_model(V, seed, w_std=0.05, base_std=2.0):
    rng = np.random.default_rng(seed)
    w1 = (rng.standard_normal((V, RANK)) * w_std).astype(np.float32)
    w2 = (rng.standard_normal((V, RANK)) * w_std).astype(np.float32)
    base = (rng.standard_normal(V) * base_std).astype(np.float32)
    return w1, w2, base


@pytest.mark.parametrize("V", [1, 5, 256, 4096])
def test_step_logits_brute_force(orc, V):
    w1, w2, base = _rand_model(V, 10 + V)
    q, s = orc.quantize_w2(w2)
    deq = s.astype(np.float64)[:, None] * q.astype(np.float64)     # [V, R]
    for prev in sorted({0, V // 2, V - 1}):
        want = (base.astype(np.float64) + deq @ w1[prev].astype(np.float64)).astype(np.float32)
        tok, logits, _, _ = orc.step(q, s, w1, base, prev)
        assert np.array_equal(logits, want)
        assert tok == int(torch.argmax(torch.from_numpy(want)))


def test_step_zero_w2_gives_base(orc):
    V = 1000
    w1, _, base = _rand_model(V, 21)
    q = np.zeros((V, RANK), np.int8)
    s = np.zeros(V, np.float32)
    tok, logits, _, _ = orc.step(q, s, w1, base, 17)
    assert np.array_equal(logits, base)
    assert tok == int(np.argmax(base))


def test_hand_worked_two_step_walk(orc):
    h = structured.hand_walk_v4()
    g = h["golden"]
    q, s = orc.quantize_w2(h["w2"])
    assert list(s) == g["w2_scale"]
    for v in range(4):
        assert q[v, (v - 1) % 4] == 127 and q[v, 4] == [1, -2, 3, -4][v]
    tokens, logits, _ = orc.walk(q, s, h["w1"], h["base"], h["start"], want_logits=True)
    assert tokens[0].tolist() == g["tokens"]
    assert logits[0].tolist() == g["logits"]


def test_token_feedback_cycle(orc):
    c = structured.feedback_cycle()
    q, s = orc.quantize_w2(c["w2"])
    tokens, _, _ = orc.walk(q, s, c["w1"], c["base"], c["start"])
    assert np.array_equal(tokens[0], c["expected"])


# ----------------------------------------------------------------------------------------------
# Sampling: Gumbel-max is softmax sampling (closed form), temperature, positions
# ----------------------------------------------------------------------------------------------
def _chi2_tokens(orc, base_row, temp, n, seed0):
    V = base_row.size
    q = np.zeros((V, RANK), np.int8)
    s = np.zeros(V, np.float32)
    w1 = np.zeros((V, RANK), np.float32)
    base = np.broadcast_to(base_row, (n, 1, V)).copy()
    start = np.zeros(n, np.int32)
    seeds = (np.arange(n, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)) + np.uint64(seed0)
    temps = np.full(n, temp, np.float32)
    tokens, _, _ = orc.walk(q, s, w1, base, start, sample=True, seeds=seeds, temps=temps)
    counts = np.bincount(tokens[:, 0], minlength=V)
    p = np.exp(base_row.astype(np.float64) / temp)
    p /= p.sum()
    return stats.chisquare(counts, p * n).pvalue


@pytest.mark.parametrize("temp", [1.0, 0.5, 2.0])
def test_gumbel_max_frequencies_are_softmax(orc, temp):
    # bf16-exact logits so that the stored row equals the row sampled from
    base_row = np.array([0.0, 0.5, -1.0, 1.25, 2.0, -0.75, 0.25, 1.0], np.float32)
    pval = _chi2_tokens(orc, base_row, temp, 200_000, 12345)
    assert pval > 1e-3


def test_sample_stores_bf16_row_and_uses_position(orc):
    V, T, bs = 64, 3, 4
    w1, w2, _ = _rand_model(V, 31)
    rng = np.random.default_rng(32)
    base = (rng.standard_normal((bs, T, V)) * 3).astype(np.float32)
    q, s = orc.quantize_w2(w2)
    start = rng.integers(0, V, bs).astype(np.int32)
    seeds = rng.integers(0, 2**64, bs, dtype=np.uint64)
    temps = np.ones(bs, np.float32)
    pos = np.array([0, 5, 100, 2**33], np.int64)
    tokens, logits, lb = orc.walk(q, s, w1, base, start, sample=True, seeds=seeds,
                                  positions=pos, temps=temps, want_logits=True)
    want_lb = torch.from_numpy(logits).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(lb, want_lb)
    # step t of request b uses draft position pos[b] + t
    for b in range(bs):
        prev = start[b]
        for t in range(T):
            tok, _, _, _ = orc.step(q, s, w1, base[b, t], prev, sample=True, seed=int(seeds[b]),
                                    P=int(pos[b]) + t, temp=1.0)
            assert tok == tokens[b, t]
            prev = tok


# ----------------------------------------------------------------------------------------------
# Top-k
# ----------------------------------------------------------------------------------------------
def test_topk_matches_lexsort(orc):
    rng = np.random.default_rng(40)
    for V, k in [(10, 1), (1000, 37), (5000, 512), (600, 600)]:
        row = rng.integers(-20, 20, V).astype(np.float32) * 0.5     # many ties
        row[rng.integers(0, V)] = -0.0
        cand = orc.topk(row, k)
        key = np.where(row == 0, 0.0, row)
        order = np.lexsort((np.arange(V), -key.astype(np.float64)))[:k]
        assert np.array_equal(cand, order.astype(np.int32))


def test_topk_k_equals_v_is_dense(orc):
    V, T, bs = 300, 4, 3
    w1, w2, _ = _rand_model(V, 41)
    rng = np.random.default_rng(42)
    base = (rng.standard_normal((bs, T, V)) * 3).astype(np.float32)
    q, s = orc.quantize_w2(w2)
    start = rng.integers(0, V, bs).astype(np.int32)
    seeds = rng.integers(0, 2**64, bs, dtype=np.uint64)
    temps = np.ones(bs, np.float32)
    for sample in (False, True):
        kw = dict(sample=sample, seeds=seeds, temps=temps, want_logits=True)
        d = orc.walk(q, s, w1, base, start, **kw)
        t = orc.walk(q, s, w1, base, start, k=V, **kw)
        assert np.array_equal(d[0], t[0])
        assert np.array_equal(d[1], t[1])
        if sample:
            assert np.array_equal(d[2], t[2])


def test_topk_zero_w2_greedy_is_base_argmax(orc):
    V, T = 2000, 5
    w1, _, _ = _rand_model(V, 43)
    rng = np.random.default_rng(44)
    base = (rng.standard_normal((1, T, V)) * 3).astype(np.float32)
    q = np.zeros((V, RANK), np.int8)
    s = np.zeros(V, np.float32)
    for k in (1, 7, 512):
        tokens, logits, _ = orc.walk(q, s, w1, base, np.array([3], np.int32), k=k,
                                     want_logits=True)
        assert np.array_equal(tokens[0], base[0].argmax(axis=1).astype(np.int32))
        # exactly k finite entries per row, -inf elsewhere
        assert np.all(np.isfinite(logits[0]).sum(axis=1) == k)


def test_topk_off_candidate_is_minus_inf(orc):
    V = 500
    w1, w2, base = _rand_model(V, 45)
    q, s = orc.quantize_w2(w2)
    cand = orc.topk(base, 20)
    tok, logits, _, _ = orc.step(q, s, w1, base, 9, cand=cand)
    mask = np.zeros(V, bool)
    mask[cand] = True
    assert np.all(np.isneginf(logits[~mask]))
    full = orc.step(q, s, w1, base, 9)[1]
    assert np.array_equal(logits[mask], full[mask])
    assert tok in set(cand.tolist())


def test_sample_depends_only_on_stored_bf16_row(orc):
    """The sampler draws from the bf16 row it stores (PR #62958, Details), so two fp32 logit
    rows with the same bf16 rounding must give identical scores and tokens."""
    V = 256
    rng = np.random.default_rng(46)
    # bf16-exact values, then a perturbation below half a bf16 step (7 explicit mantissa bits)
    b0 = torch.from_numpy((rng.standard_normal(V) * 3).astype(np.float32)).to(torch.bfloat16)
    b0 = b0.float().numpy()
    ulp = np.abs(b0) * 2.0 ** -8
    b1 = (b0 + ulp * rng.uniform(-0.45, 0.45, V)).astype(np.float32)
    assert not np.array_equal(b0, b1)
    q = np.zeros((V, RANK), np.int8)
    s = np.zeros(V, np.float32)
    w1 = np.zeros((V, RANK), np.float32)
    for seed in range(20):
        r0 = orc.step(q, s, w1, b0, 0, sample=True, seed=seed, P=3)
        r1 = orc.step(q, s, w1, b1, 0, sample=True, seed=seed, P=3)
        assert np.array_equal(r0[2], r1[2])
        assert np.array_equal(r0[3].view(np.uint32), r1[3].view(np.uint32))
        assert r0[0] == r1[0]
