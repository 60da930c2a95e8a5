"""The inverse-CDF walk (dspark_walk_sample_icdf) against the CPU oracle, through the C ABI:
bf16 rows by the interval rule, tokens teacher-forced (a token differing from the oracle's must
be a draw of the walk's own stored row for a uniform within 1e-5 of the step's); oracle-sized
shapes over all three kernels (one-request MFMA, lane-per-row, batched MFMA with static and
dynamic LDS), ragged slices, grid caps and single steps; the benchmarked shapes;
token frequencies against softmax (chi-squared); the token-feedback walk; timeouts and a
workspace left zeroed."""
import numpy as np
import pytest
import torch
from scipy import stats

import dspark_markov_draft_amd as dm
import dspark_markov_draft_amd.binding as B
from dspark_markov_draft_amd.synth import CASES, make_inputs
from oracle.check import check_walk
from tests import structured
from tests.gpu_helpers import DEV, Problem, lb_bits, random_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_knobs():
    yield
    for key in (B.DEBUG_MAX_WORKGROUPS, B.DEBUG_SPIN_LIMIT, B.DEBUG_WAIT_UNSET_FLAG,
                B.DEBUG_FORCE_PATH, B.DEBUG_MFMA_WAVES):
        dm.dspark_debug_set(key, 0)


def _icdf(p, ws=None, qs=None):
    bs, T, V = p.shape
    q, s = qs if qs is not None else p.quantize()
    ws = dm.new_workspace(bs, T, V) if ws is None else ws
    tok, lb = dm.dspark_walk_sample_icdf(q, s, p.w1, p.base, p.start, p.seeds, p.temps, ws,
                                         positions=p.pos)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lb_bits(lb), ws


def _check(p, tok, lb):
    q, s = p.oracle_q()
    return check_walk(q, s, p.w1_np(), p.base_np, p.start_np, tok, sample=2, seeds=p.seeds_np,
                      temps=p.temps_np, positions=p.pos_np, lb=lb)


SMALL = [  # V, T, bs, dtype, grid cap, path (0: chosen)
    (4096, 4, 1, torch.float32, 0, 0),
    (5000, 3, 1, torch.bfloat16, 0, B.PATH_DOT4),
    (5001, 3, 2, torch.bfloat16, 0, 0),       # odd V
    (20000, 3, 3, torch.float16, 16, 0),      # large slices: LDS row sets, several scan passes
    (30000, 2, 17, torch.bfloat16, 0, B.PATH_DOT4),   # 17 requests on the lane-per-row kernel
    (30000, 2, 17, torch.bfloat16, 0, 0),     # the same on the batched MFMA kernel (2 tiles)
    (4096, 3, 5, torch.float32, 0, 0),        # batched: one partial request tile
    (20000, 3, 20, torch.float16, 24, 0),     # batched, 848-row slices: dynamic LDS variant
    (3000, 5, 64, torch.bfloat16, 0, 0),      # full batch, 12 workgroups: several reducers each
    (20000, 3, 1, torch.bfloat16, 20, 0),     # one request, 1000-row slices (LDS tiles)
    (30000, 1, 1, torch.bfloat16, 0, 0),      # a single step
    (6000, 1, 20, torch.float32, 0, 0),       # a single step, batched
    (257, 16, 2, torch.float32, 0, 0),        # one workgroup, 16 steps
]


@pytest.mark.parametrize("V,T,bs,dtype,cap,path", SMALL)
def test_icdf_parity_small(V, T, bs, dtype, cap, path):
    dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    temps = np.linspace(0.5, 2.0, bs).astype(np.float32) if bs > 1 else None
    pos = np.arange(bs, dtype=np.int64) * 1000 + 3 if bs > 2 else None
    p = random_problem(V, T, bs, dtype=dtype, w_std=0.05 if dtype == torch.float32 else 0.02,
                       seed=V * 3 + bs, temps=temps, positions=pos)
    tok, lb, ws = _icdf(p)
    rep = _check(p, tok, lb)
    assert rep.ok, rep.summary()
    assert int(ws.count_nonzero()) == 0
    assert dm.dspark_workspace_status(ws) == 0


@pytest.mark.parametrize("name", ["v151936_t7_bs1", "v151936_t7_bs16", "v151936_t7_bs64",
                                  "v151936_t16_bs1", "v129280_t5_bs1"])
def test_icdf_full_size(name, parity_log):
    inp = make_inputs(CASES[name])
    p = Problem(inp.w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                temps=inp.temperature.numpy())
    tok, lb, ws = _icdf(p)
    rep = _check(p, tok, lb)
    parity_log(f"{name}:sample_icdf", rep)
    assert rep.ok, rep.summary()
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("case", [(10000, 3, 19, 20), "v151936_t7_bs16"])
def test_icdf_mfma_wave_layouts_agree_bitwise(case):
    """The batched kernel's inverse-CDF builds with 8 waves (the default) and 4 (forced): the
    same tokens and bf16 rows (the per-wave softmax pairs merge in a different grouping, so the
    uniform's target in a slice may move by rounding: tokens are compared through the oracle's
    interval check, rows bit for bit)."""
    if isinstance(case, str):
        inp = make_inputs(CASES[case])
        p = Problem(inp.w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                    temps=inp.temperature.numpy())
    else:
        V, T, bs, cap = case
        dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
        p = random_problem(V, T, bs, dtype=torch.bfloat16, seed=V + bs,
                           temps=np.linspace(0.5, 2.0, bs).astype(np.float32))
    qs = p.quantize()
    res = []
    for waves in (8, 4):
        dm.dspark_debug_set(B.DEBUG_MFMA_WAVES, waves)
        assert dm.dspark_walk_plan_query(*p.shape)["waves_per_workgroup"] == waves
        tok, lb, _ = _icdf(p, qs=qs)
        rep = _check(p, tok, lb)
        assert rep.ok, rep.summary()
        res.append((tok, lb))
    # the rows of a step depend on the tokens before it: compared where the walks took the
    # same tokens (a rounding-moved draw is allowed, and each walk passed the oracle's check)
    same = (res[0][0] == res[1][0]).all(axis=1)
    assert same.mean() > 0.5
    assert np.array_equal(res[0][1][same], res[1][1][same])


@pytest.mark.parametrize("path", [0, B.PATH_DOT4])
@pytest.mark.parametrize("temp", [1.0, 0.6])
def test_icdf_frequencies_are_softmax(temp, path):
    """W2 = 0 and bf16-exact base logits: each step draws from softmax(base / temp). 64 requests
    x 2 steps x 600 calls with fresh seeds: the token counts match it (chi-squared). On the
    batched MFMA kernel (chosen) and the lane-per-row kernel."""
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    V, T, bs, calls = 8, 2, 64, 600
    row = np.array([0.0, 0.5, -1.0, 1.25, 2.0, -0.75, 0.25, 1.0], np.float32)
    w = torch.zeros(V, 256, dtype=torch.bfloat16)
    base = np.broadcast_to(row, (bs, T, V)).copy()
    p = Problem(w, w.clone(), base, np.zeros(bs, np.int32),
                temps=np.full(bs, temp, np.float32))
    qs = p.quantize()
    ws = dm.new_workspace(bs, T, V)
    rng = np.random.default_rng(5)
    counts = np.zeros(V, np.int64)
    for c in range(calls):
        p.seeds = torch.from_numpy(rng.integers(0, 2**63, bs, dtype=np.int64)).to(DEV)
        tok, _, _ = _icdf(p, ws=ws, qs=qs)
        counts += np.bincount(tok.reshape(-1), minlength=V)
    prob = np.exp(row.astype(np.float64) / temp)
    prob /= prob.sum()
    assert stats.chisquare(counts, prob * counts.sum()).pvalue > 1e-4


def test_icdf_token_feedback_cycle():
    c = structured.feedback_cycle()
    p = Problem(torch.from_numpy(c["w1"]).to(torch.bfloat16),
                torch.from_numpy(c["w2"]).to(torch.bfloat16), c["base"], c["start"])
    tok, _, _ = _icdf(p)
    assert np.array_equal(tok[0], c["expected"])


def test_icdf_timeout_is_reported_and_recovers():
    p = random_problem(8192, 3, 2, seed=31)
    qs = p.quantize()
    ws = dm.new_workspace(2, 3, 8192)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 200)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 1)
    _icdf(p, ws=ws, qs=qs)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 0)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 0)
    with pytest.raises(B.DsparkError) as e:
        dm.check_workspace(ws)
    assert e.value.status == B.ERR_TIMEOUT
    tok, lb, _ = _icdf(p, ws=ws, qs=qs)
    assert _check(p, tok, lb).ok
    assert int(ws.count_nonzero()) == 0


def test_icdf_and_gumbel_share_a_workspace():
    a = random_problem(9000, 4, 3, seed=21)
    ws = dm.new_workspace(64, 16, 1)
    r1 = _icdf(a, ws=ws)
    g = a.sample(ws=ws)
    r2 = _icdf(a, ws=ws)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    assert np.array_equal(r1[1][:, 0], g[1][:, 0])   # step 0 stores the Gumbel walk's row
    assert a.check_sample(*g).ok
    assert int(ws.count_nonzero()) == 0
