"""GPU parity of the top-k walk (candidate selection + walk over the candidates) against the
CPU oracle, through the C ABI.

The oracle's candidates are the k largest base logits ordered by (value desc, index asc); its
step fills -inf outside them and runs the unchanged greedy / Gumbel-max rule over the dense row.
Checked: the -inf pattern of the dense output (the candidate set, exactly), candidate logits
within 2e-3, bf16 rows under the dense walk's rule, tokens teacher-forced; k = V against the
dense walk bit for bit; boundary ties, +-0, -inf rows and the large-bin path of the select.
"""
import numpy as np
import pytest
import torch

import dspark_markov_draft_amd as dm
import dspark_markov_draft_amd.binding as B
from dspark_markov_draft_amd.synth import CASES, make_inputs
from tests.gpu_helpers import DEV, Problem, random_problem

pytestmark = pytest.mark.gpu


def _run_check(p, k, mode, requests=None):
    sample = mode == "sample"
    tok, out = p.topk(k, sample=sample)
    rep = p.check_topk(k, tok, out, sample=sample, requests=requests)
    return tok, out, rep


SMALL = [  # V, T, bs, dtype, k
    (4096, 4, 1, torch.float32, 64),
    (5001, 3, 3, torch.bfloat16, 100),      # V % 4 != 0: element-wise select path
    (20000, 3, 5, torch.bfloat16, 512),
    (3000, 5, 16, torch.float16, 2048),
    (257, 4, 2, torch.float32, 257),        # k = V
    (1, 2, 1, torch.bfloat16, 1),
    (9000, 2, 64, torch.bfloat16, 1),
    (12345, 3, 7, torch.bfloat16, 777),
    (6000, 1, 4, torch.bfloat16, 300),      # a single step
]


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("V,T,bs,dtype,k", SMALL)
def test_topk_parity_small(V, T, bs, dtype, k, mode):
    p = random_problem(V, T, bs, dtype=dtype, seed=V + 7 * k + bs,
                       temps=np.linspace(0.5, 1.5, bs).astype(np.float32),
                       positions=np.arange(bs, dtype=np.int64) * 3)
    _, _, rep = _run_check(p, k, mode)
    print(V, T, bs, k, mode, rep.summary())
    assert rep.ok, rep.summary()


def test_topk_candidate_set_is_exact():
    """Finite entries of the greedy dense output are exactly the k best base logits
    (lexicographic: value desc, index asc), for every row."""
    V, T, bs, k = 30000, 3, 4, 700
    p = random_problem(V, T, bs, seed=3)
    _, dense = p.topk(k)
    for b in range(bs):
        for t in range(T):
            row = p.base_np[b, t]
            want = np.lexsort((np.arange(V), -row))[:k]
            got = np.flatnonzero(np.isfinite(dense[b, t]))
            assert np.array_equal(np.sort(want), got), (b, t)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_topk_k_equals_V_is_the_dense_walk(mode):
    """k = V selects every entry: tokens and dense outputs equal the dense walk's bit for bit
    (V = 2048, the largest k the library takes)."""
    p = random_problem(2048, 4, 3, seed=11, temps=np.array([1.0, 0.7, 1.3], np.float32))
    qs = p.quantize()
    V = p.shape[2]
    if mode == "greedy":
        d_tok, d_out = p.greedy(qs=qs)
        k_tok, k_out = p.topk(V, qs=qs)
        assert np.array_equal(d_out.view(np.uint32), k_out.view(np.uint32))
    else:
        d_tok, d_out = p.sample(qs=qs)
        k_tok, k_out = p.topk(V, sample=True, qs=qs)
        assert np.array_equal(d_out, k_out)
    assert np.array_equal(d_tok, k_tok)


def _zero_w_problem(base, start=None):
    base = np.asarray(base, np.float32)
    bs, T, V = base.shape
    w = torch.zeros(V, 256, dtype=torch.bfloat16)
    start = np.zeros(bs, np.int32) if start is None else np.asarray(start, np.int32)
    return Problem(w, w.clone(), base, start)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_topk_boundary_ties_take_lower_indices(mode):
    """Rows of few distinct values (many equal keys across the k-th position, +0 and -0 mixed):
    the lower indices win at the boundary."""
    rng = np.random.default_rng(5)
    V, T = 3000, 3
    base = rng.integers(-3, 4, size=(2, T, V)).astype(np.float32)
    base[base == 0] = np.where(rng.random(int((base == 0).sum())) < 0.5, 0.0, -0.0)
    p = _zero_w_problem(base)
    for k in (1, 5, 400, 1234):
        tok, out = p.topk(k, sample=mode == "sample")
        rep = p.check_topk(k, tok, out, sample=mode == "sample")
        assert rep.ok, (k, rep.summary())


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_topk_large_bin_path(mode):
    """A row whose k-th key shares its top bits with more elements than the select keeps in LDS
    (constant rows; a narrow band) takes the global-memory levels; the result is unchanged."""
    V, T, k = 20000, 3, 300
    base = np.zeros((1, T, V), np.float32)
    base[0, 1] = 1.0 + np.arange(V, dtype=np.float32) * 1e-7   # ~20000 keys in one top bin
    base[0, 2, ::7] = 2.0                                        # ties above a constant floor
    p = _zero_w_problem(base)
    tok, out = p.topk(k, sample=mode == "sample")
    rep = p.check_topk(k, tok, out, sample=mode == "sample")
    assert rep.ok, rep.summary()
    if mode == "greedy":
        assert np.array_equal(np.flatnonzero(np.isfinite(out[0, 0])), np.arange(k))


@pytest.mark.parametrize("n_bin", [40, 1500, 5000])
@pytest.mark.parametrize("k", [17, 300])
def test_topk_select_kth_bin_sizes(n_bin, k):
    """Rows whose k-th key shares its top 12 bits with n_bin keys spread along the row (distinct
    values 1 + j 2^-20 in [1, 1.125)): a small bin is ranked directly, a medium one takes radix
    levels over a compacted list, a large one radix levels over the whole buffer."""
    V, T = 24000, 2
    base = np.zeros((1, T, V), np.float32)
    rng = np.random.default_rng(n_bin + k)
    for t in range(T):
        pos = np.sort(rng.choice(V, n_bin, replace=False))
        base[0, t, pos] = 1.0 + rng.permutation(n_bin).astype(np.float32) * 2.0 ** -20
        base[0, t, rng.choice(V, 5, replace=False)] = 3.0 + t   # a few keys above the bin
    p = _zero_w_problem(base)
    tok, dense = p.topk(k)
    rep = p.check_topk(k, tok, dense)
    assert rep.ok, rep.summary()
    for t in range(T):
        row = base[0, t]
        want = np.sort(np.lexsort((np.arange(V), -row))[:k])
        assert np.array_equal(np.flatnonzero(np.isfinite(dense[0, t])), want), t


@pytest.mark.parametrize("k", [100, 512])
def test_topk_bound_from_ordered_rows(k):
    """The select bounds each row by a key of its first 18432-element chunk, chosen to let about
    2k keys through on an unordered row. Rows in descending order put the whole top of the row in
    that chunk, so fewer than k keys reach the bound; rows in ascending order let nearly all
    through. Both take the exact fallback; a random row takes the main path. The candidate set
    is the k largest (lower index first among equals) in every case."""
    V, T = 60000, 3
    rng = np.random.default_rng(k)
    base = np.zeros((1, T, V), np.float32)
    base[0, 0] = -np.arange(V, dtype=np.float32) * 1e-3        # descending
    base[0, 1] = np.arange(V, dtype=np.float32) * 1e-3         # ascending
    base[0, 2] = rng.normal(0.0, 3.0, V).astype(np.float32)
    p = _zero_w_problem(base)
    for mode in ("greedy", "sample"):
        tok, dense = p.topk(k, sample=mode == "sample")
        rep = p.check_topk(k, tok, dense, sample=mode == "sample")
        assert rep.ok, rep.summary()
        # greedy: fp32 logits; sample: bf16 bits, -inf being 0xFF80
        kept = np.isfinite(dense[0]) if mode == "greedy" else dense[0] != 0xFF80
        for t in range(T):
            row = base[0, t]
            want = np.sort(np.lexsort((np.arange(V), -row))[:k])
            assert np.array_equal(np.flatnonzero(kept[t]), want), (mode, t)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_topk_all_candidates_neg_inf_gives_token_zero(mode):
    """A step whose candidates are all -inf: the dense row is -inf everywhere, and torch.argmax
    of such a row is 0 (the first maximum), whether or not 0 is a candidate."""
    V, T, k = 4096, 2, 16
    base = np.full((1, T, V), -np.inf, np.float32)
    base[0, 1, 100:200] = np.linspace(-1, 1, 100)
    p = _zero_w_problem(base, start=[7])
    tok, out = p.topk(k, sample=mode == "sample")
    assert tok[0, 0] == 0
    rep = p.check_topk(k, tok, out, sample=mode == "sample")
    assert rep.ok, rep.summary()


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_topk_full_size(mode, parity_log):
    """The benchmarked top-k workload, every request checked."""
    case = CASES["topk512_v151936_t7_bs64"]
    inp = make_inputs(case)
    p = Problem(inp.w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                temps=inp.temperature.numpy())
    _, _, rep = _run_check(p, case.k, mode)
    parity_log(f"{case.name}:{mode}", rep)
    assert rep.ok, rep.summary()


def test_topk_leaves_workspace_zeroed_for_dense_walks():
    """The candidate lists live in the workspace; the walk clears them, so a dense walk on the
    same workspace afterwards is unaffected."""
    p = random_problem(10000, 4, 8, seed=17)
    qs = p.quantize()
    bs, T, V = p.shape
    ws = dm.new_workspace(bs, T, V, 1000)
    tk = p.topk(1000, ws=ws, qs=qs)
    assert int(ws.count_nonzero()) == 0
    dense = p.greedy(ws=ws, qs=qs)
    assert p.check_greedy(*dense).ok
    tk2 = p.topk(1000, ws=ws, qs=qs)
    assert np.array_equal(tk[0], tk2[0]) and np.array_equal(tk[1].view(np.uint32),
                                                            tk2[1].view(np.uint32))
    assert dm.dspark_workspace_status(ws) == 0


@pytest.fixture
def split_knob_reset():
    yield
    dm.dspark_debug_set(B.DEBUG_TOPK_SPLIT, 0)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 0)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 0)


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("V,T,bs,k", [(20000, 5, 60, 512), (9000, 16, 20, 100), (6000, 9, 32, 300),
                                      (151936, 7, 64, 512), (12000, 16, 40, 256),
                                      (3000, 5, 64, 1), (512, 6, 60, 512)])
def test_topk_one_launch_equals_two_launches(V, T, bs, k, mode, split_knob_reset):
    """The one-launch form (select and walk together, walks waiting for their rows; used for more
    (request, step) rows than compute units: all shapes here) gives the two-launch form's tokens
    and dense rows bit for bit, and leaves the workspace zeroed."""
    sample = mode == "sample"
    p = random_problem(V, T, bs, seed=V + T + k, temps=np.linspace(0.6, 1.4, bs).astype(np.float32),
                       positions=np.arange(bs, dtype=np.int64) * 5)
    qs = p.quantize()
    ws = dm.new_workspace(bs, T, V, k)
    one = p.topk(k, sample=sample, ws=ws, qs=qs)
    assert int(ws.count_nonzero()) == 0
    dm.dspark_debug_set(B.DEBUG_TOPK_SPLIT, 1)
    two = p.topk(k, sample=sample, ws=ws, qs=qs)
    assert dm.dspark_workspace_status(ws) == 0
    assert np.array_equal(one[0], two[0])
    assert np.array_equal(one[1].view(np.uint8), two[1].view(np.uint8))


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("V,T,bs,k", [(5000, 5, 64, 64), (512, 6, 60, 512)])
def test_topk_one_launch_parity(V, T, bs, k, mode):
    """The one-launch form (more rows than compute units) against the oracle, every request."""
    p = random_problem(V, T, bs, seed=V + 3 * k, temps=np.linspace(0.5, 1.5, bs).astype(np.float32),
                       positions=np.arange(bs, dtype=np.int64) * 7)
    _, _, rep = _run_check(p, k, mode)
    assert rep.ok, rep.summary()


def test_topk_one_launch_wait_timeout_is_reported_and_recovers(split_knob_reset):
    """The walks' waits for their rows are bounded: forced never to end, each runs into its
    (small) bound, the kernel completes and records DSPARK_ERR_TIMEOUT (check_workspace raises
    it and zeroes the workspace); the next call is exact."""
    p = random_problem(4096, 5, 64, seed=23)      # 320 rows: the one-launch form
    qs = p.quantize()
    ws = dm.new_workspace(64, 5, 4096, 64)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 200)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 1)
    p.topk(64, ws=ws, qs=qs)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 0)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 0)
    with pytest.raises(B.DsparkError) as e:
        dm.check_workspace(ws)
    assert e.value.status == B.ERR_TIMEOUT
    assert int(ws.count_nonzero()) == 0
    tok, out = p.topk(64, ws=ws, qs=qs)
    assert dm.dspark_workspace_status(ws) == 0
    assert p.check_topk(64, tok, out).ok


def test_topk_out_of_range_start_is_contained():
    p = random_problem(5000, 2, 2, seed=19)
    p.start = torch.tensor([3, 5000], dtype=torch.int32, device=DEV)
    ws = dm.new_workspace(2, 2, 5000, 50)
    p.topk(50, ws=ws)
    assert dm.dspark_workspace_status(ws) == B.ERR_INVALID_ARG
