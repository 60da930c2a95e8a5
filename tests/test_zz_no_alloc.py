"""The no-allocation greedy walk (library-held scratch) against the greedy walk with a caller
workspace, through the C ABI: the same tokens and the same logit bits, on two calls in a row,
the second smaller than the first; a timeout is reported through the caller's error word and
leaves nothing behind for the next call."""
import numpy as np
import pytest
import torch

import dspark_markov_draft_amd as dm
import dspark_markov_draft_amd.binding as B
from dspark_markov_draft_amd.synth import CASES, make_inputs
from tests.gpu_helpers import DEV, Problem, random_problem

pytestmark = pytest.mark.gpu


def _noalloc(p, qs, want_logits=True):
    bs, T, V = p.shape
    q, s = qs
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    logits = torch.empty((bs, T, V), dtype=torch.float32, device=DEV) if want_logits else None
    tok = dm.dspark_walk_greedy_noalloc(q, s, p.w1, p.base, p.start, out_logits=logits,
                                        error_word=err)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), (None if logits is None else logits.cpu().numpy()), int(err.item())


def test_noalloc_matches_workspace_walk_twice_shrinking():
    big = make_inputs(CASES["v151936_t7_bs16"])
    p1 = Problem(big.w1, big.w2, big.base, big.start)
    p2 = random_problem(30000, 3, 1, seed=5)          # smaller in every dimension
    for p in (p1, p2):
        qs = p.quantize()
        ref_tok, ref_logits = p.greedy(qs=qs)
        tok, logits, err = _noalloc(p, qs)
        assert err == 0
        assert np.array_equal(tok, ref_tok)
        assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32))
        tok2, _, err2 = _noalloc(p, qs, want_logits=False)
        assert err2 == 0 and np.array_equal(tok2, ref_tok)


def test_noalloc_timeout_reported_and_next_call_clean():
    p = random_problem(8192, 3, 2, seed=31)
    qs = p.quantize()
    ref_tok, ref_logits = p.greedy(qs=qs)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 200)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 1)
    try:
        _, _, err = _noalloc(p, qs)
    finally:
        dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 0)
        dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 0)
    assert err == -B.ERR_TIMEOUT
    tok, logits, err = _noalloc(p, qs)                 # the stale keys were cleared
    assert err == 0
    assert np.array_equal(tok, ref_tok)
    assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32))


def test_noalloc_out_of_range_start_reported():
    p = random_problem(5000, 2, 2, seed=41)
    qs = p.quantize()
    p.start = torch.tensor([7, 5000], dtype=torch.int32, device=DEV)
    _, _, err = _noalloc(p, qs)
    assert err == -B.ERR_INVALID_ARG
