"""The lossless top-k pruned greedy walk (dspark_walk_greedy_pruned) against the dense greedy
walk and the CPU oracle, through the C ABI. Its result is by definition the dense greedy walk's:
tokens equal to the dense walk's bit for bit and teacher-forced equal to the oracle's; every
logit it evaluates bit-identical to the dense walk's. Steps the load-time bound certifies use
only the k candidates; the others (flat base rows, infinities) fall back to every row."""
import numpy as np
import pytest
import torch

import dspark_markov_draft_amd as dm
import dspark_markov_draft_amd.binding as B
import oracle
from dspark_markov_draft_amd.synth import CASES, make_inputs
from oracle.check import check_walk
from tests.gpu_helpers import DEV, Problem, random_problem

pytestmark = pytest.mark.gpu


def _bound(p, qs):
    return dm.dspark_w2_prune_bound(*qs)


def _pruned(p, k, qs, bound, want_logits=True):
    bs, T, V = p.shape
    ws = dm.new_workspace(bs, T, V, k)
    logits = torch.empty((bs, T, V), dtype=torch.float32, device=DEV) if want_logits else None
    dense = torch.full((bs,), -1, dtype=torch.int32, device=DEV)
    tok = dm.dspark_walk_greedy_pruned(qs[0], qs[1], p.w1, p.base, p.start, k, bound, ws,
                                       out_logits=logits, dense_steps=dense)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    return (tok.cpu().numpy(), None if logits is None else logits.cpu().numpy(),
            dense.cpu().numpy())


def _check_against_dense(p, k, qs, bound):
    tok, logits, dense_steps = _pruned(p, k, qs, bound)
    dtok, dlog = p.greedy(qs=qs)
    assert np.array_equal(tok, dtok)
    ev = ~np.isneginf(logits)
    assert np.array_equal(logits[ev].view(np.uint32), dlog[ev].view(np.uint32))
    for b in range(p.shape[0]):
        for t in range(p.shape[1]):
            assert ev[b, t].sum() >= min(k, p.shape[2])         # at least the candidates
    q_o, s_o = p.oracle_q()
    rep = check_walk(q_o, s_o, p.w1_np(), p.base_np, p.start_np, tok)
    assert rep.ok, rep.summary()
    tk, _ = p.greedy(want_logits=False, qs=qs)
    t2, _, _ = _pruned(p, k, qs, bound, want_logits=False)
    assert np.array_equal(t2, tk)
    return dense_steps, rep


@pytest.mark.parametrize("V", [1, 4097, 151936])
def test_bound_bit_exact(V):
    g = torch.Generator().manual_seed(V)
    w2 = (torch.randn(V, 256, generator=g) * 0.02).to(torch.bfloat16)
    if V > 2:
        w2[1] = 0.0
        w2[2, :] = 3.0
    q, s = dm.dspark_quantize_w2(w2.to(DEV))
    b = dm.dspark_w2_prune_bound(q, s)
    want = oracle.w2_l1_bound(q.cpu().numpy(), s.cpu().numpy())
    assert np.float32(b.item()).view(np.uint32) == np.float32(want).view(np.uint32)


SMALL = [  # V, T, bs, dtype, k, base std
    (4096, 4, 1, torch.float32, 64, 3.0),
    (5001, 3, 3, torch.bfloat16, 100, 3.0),
    (20000, 5, 17, torch.bfloat16, 512, 3.0),
    (30000, 3, 4, torch.float16, 1000, 3.0),       # more than 512 candidates per step
    (9000, 2, 2, torch.bfloat16, 7, 3.0),
]


@pytest.mark.parametrize("V,T,bs,dtype,k,bstd", SMALL)
def test_pruned_equals_dense(V, T, bs, dtype, k, bstd):
    p = random_problem(V, T, bs, dtype=dtype, w_std=0.05 if dtype == torch.float32 else 0.02,
                       base_std=bstd, seed=V + k)
    qs = p.quantize()
    dense_steps, _ = _check_against_dense(p, k, qs, _bound(p, qs))
    assert dense_steps.sum() < T * bs, dense_steps          # most steps certified here


def test_flat_rows_fall_back_to_every_row():
    """Base logits with a spread far below the bias: no step can be certified, every step is
    computed over the whole row, and the result is still the dense walk's."""
    p = random_problem(6000, 4, 3, w_std=0.05, base_std=0.01, seed=3)
    qs = p.quantize()
    dense_steps, _ = _check_against_dense(p, 64, qs, _bound(p, qs))
    assert (dense_steps == 4).all(), dense_steps


def test_some_steps_certified_some_not():
    V, T, bs = 8000, 6, 5
    p = random_problem(V, T, bs, w_std=0.05, seed=4)
    base = p.base_np.copy()
    base[:, 1::2] *= 0.003                                # odd steps: flat rows
    p = Problem(p.w1_cpu, p.w2_cpu, base, p.start_np)
    qs = p.quantize()
    dense_steps, _ = _check_against_dense(p, 128, qs, _bound(p, qs))
    assert (dense_steps == 3).all(), dense_steps


def test_infinities_fall_back():
    """+inf among the candidates, -inf rows: such steps are not certified (not finite) and are
    computed over every row, with torch.argmax's order."""
    V, T = 5000, 3
    p = random_problem(V, T, 2, seed=5)
    base = p.base_np.copy()
    base[0, 0, [10, 4000]] = np.inf
    base[1, 1, :] = -np.inf
    base[1, 2, 77] = np.inf
    p = Problem(p.w1_cpu, p.w2_cpu, base, p.start_np)
    qs = p.quantize()
    tok, logits, dense_steps = _pruned(p, 32, qs, _bound(p, qs))
    dtok, _ = p.greedy(qs=qs)
    assert np.array_equal(tok, dtok)
    assert tok[0, 0] == 10 and tok[1, 1] == 0 and tok[1, 2] == 77
    assert dense_steps.tolist() == [1, 2]


@pytest.fixture
def split_knob_reset():
    yield
    dm.dspark_debug_set(B.DEBUG_TOPK_SPLIT, 0)


def _flat_odd_steps(p):
    base = p.base_np.copy()
    base[:, 1::2] *= 0.003                                # odd steps: flat rows
    return Problem(p.w1_cpu, p.w2_cpu, base, p.start_np)


@pytest.mark.parametrize("case", ["random", "flat", "flat_odd", "inf"])
def test_pruned_one_launch(case, split_knob_reset):
    """More (request, step) rows than compute units: the pruned walk runs in one launch with
    the select. Against the dense walk and the oracle (as everywhere here), and bit for bit
    against the two-launch form, dense_steps included; with steps that fall back to every row
    (flat rows, infinities) as well as certified ones."""
    if case == "random":
        p, k = random_problem(20000, 5, 60, w_std=0.02, base_std=3.0, seed=61), 512
    elif case == "flat":
        p, k = random_problem(4096, 5, 64, w_std=0.05, base_std=0.01, seed=62), 64
    elif case == "flat_odd":
        p, k = _flat_odd_steps(random_problem(8000, 6, 48, w_std=0.05, seed=63)), 128
    else:
        p = random_problem(5000, 6, 50, seed=64)
        base = p.base_np.copy()
        base[0, 0, [10, 4000]] = np.inf
        base[1, 1, :] = -np.inf
        base[7, 2, 77] = np.inf
        p, k = Problem(p.w1_cpu, p.w2_cpu, base, p.start_np), 32
    qs = p.quantize()
    bound = _bound(p, qs)
    if case == "inf":
        # (a -inf row has no finite logit to count, so the per-row count of _check_against_dense
        # does not apply: tokens against the dense walk and the oracle)
        tok, _, dense_steps = _pruned(p, k, qs, bound)
        dtok, _ = p.greedy(qs=qs)
        assert np.array_equal(tok, dtok)
        q_o, s_o = p.oracle_q()
        rep = check_walk(q_o, s_o, p.w1_np(), p.base_np, p.start_np, tok)
        assert rep.ok, rep.summary()
        assert tok[0, 0] == 10 and tok[1, 1] == 0 and tok[7, 2] == 77
    else:
        dense_steps, _ = _check_against_dense(p, k, qs, bound)
    if case == "flat":
        assert (dense_steps == p.shape[1]).all(), dense_steps
    elif case == "flat_odd":
        assert (dense_steps == 3).all(), dense_steps
    elif case == "inf":
        assert dense_steps[0] >= 1 and dense_steps[1] >= 1 and dense_steps[7] >= 1
    one = _pruned(p, k, qs, bound)
    dm.dspark_debug_set(B.DEBUG_TOPK_SPLIT, 1)
    two = _pruned(p, k, qs, bound)
    assert np.array_equal(one[0], two[0])
    assert np.array_equal(one[1].view(np.uint32), two[1].view(np.uint32))
    assert np.array_equal(one[2], two[2])


@pytest.mark.parametrize("name,k", [("v151936_t7_bs1", 512), ("v151936_t7_bs16", 512),
                                    ("v151936_t7_bs64", 512), ("v151936_t7_bs16", 2048)])
def test_pruned_full_size(name, k, parity_log):
    inp = make_inputs(CASES[name])
    p = Problem(inp.w1, inp.w2, inp.base, inp.start)
    qs = p.quantize()
    dense_steps, rep = _check_against_dense(p, k, qs, _bound(p, qs))
    parity_log(f"pruned{k}_{name}:greedy", rep)
    assert (dense_steps == 0).all(), dense_steps
