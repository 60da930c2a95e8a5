"""GPU parity with heavy-tailed W1 rows. The kernels code each gathered W1 row per step with an
absmax scale, so a row with a few entries far above the rest gets a coarse step; the two-digit
codes (C = 16 hi + lo, step absmax / 2032) keep the logit error of such rows inside the 2e-3
tolerance. Inputs: the tiny configuration (V 4096, T 4, W1 and W2 ~ N(0, 0.05^2) in fp32, base
~ N(0, 2^2)) with 4 entries of every W1 row set to +-10 sigma (and +-20 sigma), on every dense
kernel, the top-k walk and the sampling walks; the oracle uses W1 as given (fp64 sums)."""
import numpy as np
import pytest
import torch

import dspark_markov_draft_amd as dm
from dspark_markov_draft_amd import binding as B
from dspark_markov_draft_amd.synth import CASES, make_inputs, with_heavy_entries
from tests.gpu_helpers import Problem

pytestmark = pytest.mark.gpu

SIGMA = 0.05


def _problem(bs, mult, per_row=4, seed=0):
    inp = make_inputs(CASES["tiny_v4096_t4_bs1"], bs=bs)
    w1 = with_heavy_entries(inp.w1, per_row, mult, SIGMA, seed=100 + seed)
    return Problem(w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                   temps=inp.temperature.numpy())


@pytest.fixture(autouse=True)
def _reset_debug():
    yield
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, 0)


@pytest.mark.parametrize("mult", [10.0, 20.0])
@pytest.mark.parametrize("bs,path", [(1, B.PATH_MFMA1), (1, B.PATH_DOT4), (2, B.PATH_DOT4),
                                     (16, B.PATH_MFMA), (64, B.PATH_MFMA)])
def test_greedy_heavy_w1(bs, path, mult, parity_log):
    p = _problem(bs, mult)
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    tok, logits = p.greedy()
    rep = p.check_greedy(tok, logits)
    parity_log(f"heavy_w1_x{int(mult)}_bs{bs}_path{path}_greedy", rep)
    assert rep.ok, rep.summary()


@pytest.mark.parametrize("bs,path", [(1, B.PATH_MFMA1), (3, B.PATH_DOT4), (16, B.PATH_MFMA)])
def test_sample_heavy_w1(bs, path, parity_log):
    p = _problem(bs, 10.0, seed=1)
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    tok, lb = p.sample()
    rep = p.check_sample(tok, lb)
    parity_log(f"heavy_w1_x10_bs{bs}_path{path}_sample", rep)
    assert rep.ok, rep.summary()


def test_paths_agree_bitwise_heavy_w1():
    """Every dense kernel forms the same integer from the two-digit codes: bit-identical logits
    and tokens at 16 requests (the one-request kernel at bs 1)."""
    p = _problem(16, 10.0, seed=2)
    qs = p.quantize()
    outs = []
    for path in (B.PATH_DOT4, B.PATH_MFMA):
        dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
        outs.append(p.greedy(qs=qs))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    p1 = _problem(1, 10.0, seed=2)
    q1 = p1.quantize()
    one = []
    for path in (B.PATH_DOT4, B.PATH_MFMA1):
        dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
        one.append(p1.greedy(qs=q1))
    assert np.array_equal(one[0][0], one[1][0])
    assert np.array_equal(one[0][1].view(np.uint32), one[1][1].view(np.uint32))


@pytest.mark.parametrize("k", [64, 2048])
def test_topk_heavy_w1(k, parity_log):
    p = _problem(8, 10.0, seed=3)
    tok, logits = p.topk(k)
    rep = p.check_topk(k, tok, logits)
    parity_log(f"heavy_w1_x10_topk{k}_bs8", rep)
    assert rep.ok, rep.summary()
