"""GPU parity of the dense walk, quantisation and Philox against the CPU oracle.

All calls go through the C ABI (libdspark.so) via its thin binding. Bars: quantised W2 and
Philox words bit-exact; logits within 2e-3; bf16 draft logits equal or a neighbour at a rounding
midpoint; tokens teacher-forced, equal except at the oracle's near ties (oracle/check.py).
"""
import numpy as np
import pytest
import torch

import dspark_markov_draft_amd as dm
import dspark_markov_draft_amd.binding as B
import oracle
from dspark_markov_draft_amd.synth import CASES, make_inputs
from tests import structured
from tests.gpu_helpers import DEV, Problem, lb_bits, random_problem

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_knobs():
    yield
    for key in (B.DEBUG_MAX_WORKGROUPS, B.DEBUG_SPIN_LIMIT, B.DEBUG_WAIT_UNSET_FLAG,
                B.DEBUG_FORCE_PATH, B.DEBUG_MFMA_WAVES):
        dm.dspark_debug_set(key, 0)


PATHS = [0, B.PATH_DOT4, B.PATH_MFMA, B.PATH_MFMA1]   # 0: chosen by batch size (MFMA1: 1 request)


# ----------------------------------------------------------------------------------------------
# quantisation and Philox: bit-exact
# ----------------------------------------------------------------------------------------------
def _special_rows(dtype):
    w = torch.zeros(6, 256)
    w[1, 0] = 127.0
    w[1, 1:9] = torch.tensor([2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5, -1.5])  # exact .5 ties
    w[2, 3] = -1e-3                                                         # single element
    w[3] = torch.linspace(-1, 1, 256)
    w[4, :] = 7.0                                                           # constant row
    return w.to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("V", [1, 4097, 151936])
def test_quantize_bit_exact(dtype, V):
    g = torch.Generator().manual_seed(V)
    w2 = (torch.randn(V, 256, generator=g) * 0.02).to(dtype)
    if V > 10:
        w2[:6] = _special_rows(dtype)
    q, s = dm.dspark_quantize_w2(w2.to(DEV))
    q_o, s_o = oracle.quantize_w2(w2.float().numpy())
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_o)


def test_quantize_rejects_nonfinite():
    w2 = torch.zeros(10, 256)
    w2[3, 7] = float("nan")
    with pytest.raises(B.DsparkError) as e:
        dm.dspark_quantize_w2(w2.to(DEV))
    assert e.value.status == B.ERR_NONFINITE
    q, s = dm.dspark_quantize_w2(torch.ones(10, 256, device=DEV))   # the flag is cleared again
    assert float(s[0]) == np.float32(1.0) / np.float32(127.0)


@pytest.mark.parametrize("seed,pos", [(0, 0), (1, 7), (2**64 - 1, 15), (0x0123456789ABCDEF, 2**33 + 5)])
def test_philox_words_bit_exact(seed, pos):
    v0, n = 151936 - 1000, 1200
    got = dm.dspark_philox_words(seed, pos, v0, n)
    want = np.array([oracle.noise_word(seed, pos, v0 + i) for i in range(n)], np.uint32)
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------------------------
# structured walks with exact answers
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_hand_worked_walk(dtype):
    h = structured.hand_walk_v4()
    g = h["golden"]
    p = Problem(torch.from_numpy(h["w1"]).to(dtype), torch.from_numpy(h["w2"]).to(dtype),
                h["base"], h["start"])
    tok, logits = p.greedy()
    assert tok[0].tolist() == g["tokens"]
    assert logits[0].tolist() == g["logits"]


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_token_feedback_cycle(mode):
    c = structured.feedback_cycle()
    p = Problem(torch.from_numpy(c["w1"]).to(torch.bfloat16),
                torch.from_numpy(c["w2"]).to(torch.bfloat16), c["base"], c["start"])
    tok = p.greedy()[0] if mode == "greedy" else p.sample()[0]
    assert np.array_equal(tok[0], c["expected"])


# ----------------------------------------------------------------------------------------------
# teacher-forced parity, oracle-sized problems spanning several workgroups and ragged tails
# ----------------------------------------------------------------------------------------------
SMALL = [  # V, T, bs, dtype, grid cap (0 = one workgroup per CU)
    (4096, 4, 1, torch.float32, 0),
    (5000, 3, 3, torch.bfloat16, 0),        # ragged last workgroup
    (70001, 2, 2, torch.float16, 0),        # two register row sets, odd V
    (20000, 3, 5, torch.bfloat16, 16),      # LDS-resident and streamed row sets
    (3000, 5, 64, torch.bfloat16, 0),       # full batch
    (257, 16, 2, torch.float32, 0),         # one workgroup, 16 steps
    (1, 2, 1, torch.bfloat16, 0),           # a single-entry vocabulary
    (40000, 2, 17, torch.bfloat16, 8),      # MFMA, dynamic LDS: LDS and streamed tiles, ragged
                                            # request tile
    (4099, 3, 33, torch.float16, 0),        # V % 4 != 0: scalar base / draft-logit accesses
    (12288, 3, 21, torch.bfloat16, 0),      # MFMA, static LDS: two request tiles (5 in the
                                            # second), W1 gather of four groups with idle ones
    (8192, 2, 40, torch.float16, 0),        # MFMA, static LDS: three request tiles
    (12480, 2, 24, torch.float32, 20),      # MFMA, static LDS: 624-row slices (the largest)
    (10000, 3, 19, torch.bfloat16, 20),     # MFMA, static LDS, 8-slot build: 512-row slices (its
                                            # largest, with the sampling kernel's LDS slot), ragged
    (12000, 3, 1, torch.float16, 24),       # one request, 500-row slices: the 8-slot build
    (15000, 2, 1, torch.bfloat16, 24),      # one request, 628-row slices: the 10-slot build
    (20000, 3, 1, torch.bfloat16, 20),      # one request, 1000-row slices: LDS tiles (MFMA1)
    (9000, 2, 1, torch.float16, 8),         # one request, 1128-row slices: 8 LDS tiles, ragged
    (30000, 1, 1, torch.bfloat16, 0),       # a single step: the first step is also the last
    (6000, 1, 20, torch.float32, 0),        # a single step, batched
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V,T,bs,dtype,cap", SMALL)
def test_greedy_parity_small(V, T, bs, dtype, cap, path):
    dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    p = random_problem(V, T, bs, dtype=dtype, w_std=0.05 if dtype == torch.float32 else 0.02,
                       seed=V + T + bs)
    tok, logits = p.greedy()
    rep = p.check_greedy(tok, logits)
    assert rep.ok, rep.summary()
    print(rep.summary())


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("V,T,bs,dtype,cap", SMALL)
def test_sample_parity_small(V, T, bs, dtype, cap, path):
    dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    temps = np.linspace(0.5, 2.0, bs).astype(np.float32) if bs > 1 else None
    pos = np.arange(bs, dtype=np.int64) * 1000 + 3 if bs > 2 else None
    p = random_problem(V, T, bs, dtype=dtype, seed=V * 7 + bs, temps=temps, positions=pos)
    tok, lb = p.sample()
    rep = p.check_sample(tok, lb)
    assert rep.ok, rep.summary()
    print(rep.summary())


# ----------------------------------------------------------------------------------------------
# full-size workloads (the pages' kernel-table shapes), sampled requests
# ----------------------------------------------------------------------------------------------
# Every workload and mode the benchmark times, plus the tiny case exactly as specified (V 4096,
# 4 steps, one request, fp32 W ~ N(0, 0.05^2), base ~ N(0, 2^2)) and the largest supported shape
# (V = 270336, 16 steps: 1056-row slices, so the 64-request walk runs the MFMA kernel with dynamic
# LDS, one staging buffer and streamed tiles, and the one-request walk holds LDS tiles). Every
# request of every case is checked against the oracle, teacher-forced.
FULL = [(name, mode) for name in
        ["tiny_v4096_t4_bs1", "v151936_t7_bs1", "v151936_t7_bs16", "v151936_t7_bs64",
         "v151936_t16_bs1", "v129280_t5_bs1", "v129280_t5_bs64", "v248320_t16_bs1",
         "vmax270336_t16_bs64", "vmax270336_t16_bs1"]
        for mode in ("greedy", "sample")]


@pytest.mark.parametrize("name,mode", FULL)
def test_parity_full_size(name, mode, parity_log):
    inp = make_inputs(CASES[name])
    p = Problem(inp.w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                temps=inp.temperature.numpy())
    if mode == "greedy":
        tok, logits = p.greedy()
        rep = p.check_greedy(tok, logits)
    else:
        tok, lb = p.sample()
        rep = p.check_sample(tok, lb)
    parity_log(f"{name}:{mode}", rep)
    assert rep.ok, rep.summary()


@pytest.mark.parametrize("name,mode,reqs", [("v151936_t7_bs1", "greedy", None),
                                            ("v151936_t7_bs1", "sample", None),
                                            ("v248320_t16_bs1", "greedy", None),
                                            ("v151936_t7_bs16", "sample", [3, 12])])
def test_paths_agree_bitwise(name, mode, reqs):
    """All kernels form each logit with the same exact int32 sum and the same fp32 operations,
    so they must agree bit for bit; each is also checked against the oracle. (The one-request
    MFMA kernel only takes one request: at bs 16 forcing it leaves the batched kernel.)"""
    inp = make_inputs(CASES[name])
    p = Problem(inp.w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                temps=inp.temperature.numpy())
    qs = p.quantize()
    outs = []
    for path in (B.PATH_DOT4, B.PATH_MFMA, B.PATH_MFMA1):
        dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
        outs.append(p.greedy(qs=qs) if mode == "greedy" else p.sample(qs=qs))
    for o in outs[1:]:
        assert np.array_equal(outs[0][0], o[0])
        assert np.array_equal(outs[0][1].view(np.uint32 if mode == "greedy" else np.uint16),
                              o[1].view(np.uint32 if mode == "greedy" else np.uint16))
    for o in outs[1:]:
        rep = (p.check_greedy(*o, requests=reqs) if mode == "greedy"
               else p.check_sample(*o, requests=reqs))
        assert rep.ok, rep.summary()


@pytest.mark.parametrize("path", [B.PATH_DOT4, B.PATH_MFMA])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_special_values_both_paths(mode, path):
    """W2 = 0 makes every logit its base logit exactly, so special values reach the argmax as
    planted: NaN (the first NaN wins), rows that are -inf throughout (row 0 wins), +inf next to
    -inf, all-zero rows with -0 and +0 mixed (ties: the first index), a NaN after a +inf. Both
    kernels, 20 requests (two 16-request tiles on the MFMA path)."""
    V, T, bs = 4096, 3, 20
    rng = np.random.default_rng(77)
    base = rng.normal(0.0, 3.0, (bs, T, V)).astype(np.float32)
    base[0, 0, [100, 2000, 3000]] = np.nan
    base[1, 1, :] = -np.inf
    base[2, 0, 50], base[2, 0, 51] = np.inf, -np.inf
    base[3, 0, :] = np.where(rng.random(V) < 0.5, 0.0, -0.0)
    base[4, 2, 7], base[4, 2, 8], base[4, 2, 3] = np.nan, np.inf, np.inf
    base[17, 1, :] = -np.inf
    base[17, 1, 4095] = np.nan
    base[19, 2, 1000:1010] = np.inf
    w = torch.zeros(V, 256, dtype=torch.bfloat16)
    p = Problem(w, w.clone(), base, np.zeros(bs, np.int32))
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    if mode == "greedy":
        tok, logits = p.greedy()
        rep = p.check_greedy(tok, logits)
        assert tok[0, 0] == 100 and tok[1, 1] == 0 and tok[2, 0] == 50 and tok[3, 0] == 0
        assert tok[4, 2] == 7 and tok[17, 1] == 4095 and tok[19, 2] == 1000
    else:
        tok, lb = p.sample()
        rep = p.check_sample(tok, lb)
        assert tok[0, 0] == 100 and tok[1, 1] == 0 and tok[4, 2] == 7 and tok[17, 1] == 4095
    assert rep.ok, rep.summary()


def _zero_w2_problem(base_rows, start=0):
    V = base_rows.shape[-1]
    w = torch.zeros(V, 256, dtype=torch.bfloat16)
    base = np.asarray(base_rows, np.float32)[None]
    return Problem(w, w.clone(), base, np.array([start], np.int32))


@pytest.mark.parametrize("path", [B.PATH_DOT4, B.PATH_MFMA1])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_special_values_one_request(mode, path):
    """One request (the MFMA1 kernel's shape): W2 = 0, so each step's logits are its base row
    exactly and planted values reach the grid-wide argmax as they are. V = 39990 gives 157
    workgroups of 256 rows, the last holding 54 (three full 16-row tiles and a partial one); the
    specials sit in the first, middle and last workgroups."""
    V = 39990
    rng = np.random.default_rng(78)
    rows, want = [], []
    r = rng.normal(0.0, 3.0, V).astype(np.float32); r[[100, 20000, V - 1]] = np.nan
    rows.append(r); want.append(100)
    rows.append(np.full(V, -np.inf, np.float32)); want.append(0)
    r = rng.normal(0.0, 3.0, V).astype(np.float32); r[25050], r[25051] = np.inf, -np.inf
    rows.append(r); want.append(25050)
    rows.append(np.where(rng.random(V) < 0.5, 0.0, -0.0).astype(np.float32)); want.append(0)
    r = rng.normal(0.0, 3.0, V).astype(np.float32); r[30007], r[30008], r[30003] = np.nan, np.inf, np.inf
    rows.append(r); want.append(30007)          # a NaN outranks the +inf before it
    r = np.full(V, -np.inf, np.float32); r[V - 1] = np.nan
    rows.append(r); want.append(V - 1)
    r = rng.normal(0.0, 3.0, V).astype(np.float32); r[V - 10:] = np.inf
    rows.append(r); want.append(V - 10)
    base = np.stack(rows)
    for t, row in enumerate(rows):
        assert want[t] == int(torch.argmax(torch.from_numpy(row)))
    p = _zero_w2_problem(base, start=5)
    assert B.dspark_walk_plan_query(1, len(rows), V)["path"] == B.PATH_MFMA1
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    if mode == "greedy":
        tok, logits = p.greedy()
        assert np.array_equal(logits[0], base, equal_nan=True)
        assert list(tok[0]) == want
    else:
        tok, lb = p.sample()
        rep = p.check_sample(tok, lb)
        assert rep.ok, rep.summary()
        assert tok[0, 0] == 100 and tok[0, 1] == 0 and tok[0, 5] == V - 1


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_one_request_grid_invariant(mode):
    """One request on MFMA1 at several grid sizes: 27 workgroups of 1112 rows (640 in register
    tiles, 472 in LDS tiles), a cap of 117 (116 workgroups of 260 rows, a partial tile each)
    and the device's own grid. Every grid gives the same bits, and the workspace ends zeroed."""
    V = 30000
    p = random_problem(V, 5, 1, seed=12)
    qs = p.quantize()
    ws = dm.new_workspace(1, 5, V)
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, B.PATH_MFMA1)
    ref = None
    for cap in (27, 117, 0):
        dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
        assert B.dspark_walk_plan_query(1, 5, V)["path"] == B.PATH_MFMA1, cap
        out = p.greedy(qs=qs, ws=ws) if mode == "greedy" else p.sample(qs=qs, ws=ws)
        bits = (out[0], out[1].view(np.uint32 if mode == "greedy" else np.uint16))
        if ref is None:
            ref = bits
            rep = p.check_greedy(*out) if mode == "greedy" else p.check_sample(*out)
            assert rep.ok, rep.summary()
        else:
            assert np.array_equal(bits[0], ref[0]) and np.array_equal(bits[1], ref[1]), cap
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("name", ["v151936_t7_bs1", "v151936_t7_bs16", "v151936_t7_bs64",
                                  "v129280_t5_bs64"])
def test_full_size_without_out_logits_same_tokens(name):
    """The timed configuration (greedy, no logits output: a build of its own on the batched
    kernel) emits the tokens of the run whose logits were checked against the oracle."""
    inp = make_inputs(CASES[name])
    p = Problem(inp.w1, inp.w2, inp.base, inp.start)
    qs = p.quantize()
    a, _ = p.greedy(want_logits=True, qs=qs)
    b, _ = p.greedy(want_logits=False, qs=qs)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("case", [(10000, 3, 19, 20), (12480, 2, 24, 20), "v151936_t7_bs64"])
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_mfma_wave_layouts_agree_bitwise(case, mode):
    """The batched kernel's static-LDS builds with 8 waves (two per SIMD, the default) and with 4
    (forced by the test hook) form every logit with the same exact sums and fp32 operations: the
    same tokens and bit-identical logits or bf16 rows. Slices of 512 rows (the builds with 8 and
    4 slots per wave), of 624 rows (10 and 5) and the full-size 64-request walk; the 4-wave run is
    also checked against the oracle."""
    if isinstance(case, str):
        inp = make_inputs(CASES[case])
        p = Problem(inp.w1, inp.w2, inp.base, inp.start, seeds=inp.seeds,
                    temps=inp.temperature.numpy())
    else:
        V, T, bs, cap = case
        dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
        temps = np.linspace(0.5, 2.0, bs).astype(np.float32)
        p = random_problem(V, T, bs, dtype=torch.bfloat16, seed=V + bs, temps=temps)
    qs = p.quantize()
    outs = []
    for waves in (8, 4):
        dm.dspark_debug_set(B.DEBUG_MFMA_WAVES, waves)
        plan = dm.dspark_walk_plan_query(*p.shape)
        assert plan["path"] == B.PATH_MFMA and plan["waves_per_workgroup"] == waves
        outs.append(p.greedy(qs=qs) if mode == "greedy" else p.sample(qs=qs))
    view = np.uint32 if mode == "greedy" else np.uint16
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(view), outs[1][1].view(view))
    rep = p.check_greedy(*outs[1]) if mode == "greedy" else p.check_sample(*outs[1])
    assert rep.ok, rep.summary()


# ----------------------------------------------------------------------------------------------
# torch.argmax order through the grid-wide combine (ties and NaN in different workgroups)
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_argmax_order_across_workgroups(mode):
    V = 151936      # 255 workgroups of 596 rows
    rows = []
    r = np.full(V, -1.0, np.float32); r[100000] = 5.0; r[3] = 5.0; rows.append((r, 3))
    r = np.full(V, -1.0, np.float32); r[90000] = np.nan; r[150000] = np.nan; r[7] = 9.0
    rows.append((r, 90000))
    r = np.full(V, -np.inf, np.float32); rows.append((r, 0))
    r = np.full(V, -1.0, np.float32); r[60000] = -0.0; r[120000] = 0.0; rows.append((r, 60000))
    r = np.full(V, -1.0, np.float32); r[V - 1] = 2.0; rows.append((r, V - 1))
    base = np.stack([x for x, _ in rows])
    p = _zero_w2_problem(base)
    if mode == "greedy":
        tok, logits = p.greedy()
        assert np.array_equal(logits[0], base, equal_nan=True)
        for t, (_, want) in enumerate(rows):
            assert tok[0, t] == want == int(torch.argmax(torch.from_numpy(base[t])))
    else:
        tok, lb = p.sample()
        rep = p.check_sample(tok, lb)
        assert rep.ok, rep.summary()
        assert tok[0, 1] == 90000 and tok[0, 2] == 0


# ----------------------------------------------------------------------------------------------
# determinism, grid-size invariance, workspace hygiene, back-to-back calls
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("path", [B.PATH_DOT4, B.PATH_MFMA])
def test_repeatable_and_grid_invariant(path):
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    p = random_problem(30000, 5, 4, seed=11)
    qs = p.quantize()
    ref_tok, ref_logits = p.greedy(qs=qs)
    ws = dm.new_workspace(4, 5, 30000)
    for _ in range(5):
        tok, logits = p.greedy(qs=qs, ws=ws)
        assert np.array_equal(tok, ref_tok)
        assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32))
    assert int(ws.count_nonzero()) == 0
    for cap in (3, 8, 37, 117, 0):
        dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
        tok, logits = p.greedy(qs=qs, ws=ws)
        assert np.array_equal(tok, ref_tok), cap
        assert np.array_equal(logits.view(np.uint32), ref_logits.view(np.uint32)), cap
        stok, slb = p.sample(qs=qs, ws=ws)
        if cap == 3:
            ref_s = (stok, slb)
        else:
            assert np.array_equal(stok, ref_s[0]) and np.array_equal(slb, ref_s[1])
    assert int(ws.count_nonzero()) == 0


def test_back_to_back_calls_share_workspace():
    a = random_problem(9000, 6, 8, seed=21)
    b = random_problem(40000, 3, 2, seed=22)
    ws = dm.new_workspace(64, 16, 1)
    ra = a.greedy(ws=ws)
    rb = b.sample(ws=ws)
    ra2 = a.greedy(ws=ws)
    rb2 = b.sample(ws=ws)
    assert np.array_equal(ra[0], ra2[0]) and np.array_equal(ra[1], ra2[1])
    assert np.array_equal(rb[0], rb2[0]) and np.array_equal(rb[1], rb2[1])
    assert a.check_greedy(*ra).ok and b.check_sample(*rb).ok
    assert dm.dspark_workspace_status(ws) == 0
    assert int(ws.count_nonzero()) == 0


def test_kernel_timing_hook():
    """Dispatch-recorded kernel times: one positive duration per launch, results unchanged."""
    p = random_problem(30000, 4, 2, seed=23)
    qs = p.quantize()
    ws = dm.new_workspace(2, 4, 30000)
    ref = p.greedy(qs=qs, ws=ws)
    dm.dspark_debug_set(B.DEBUG_KERNEL_TIMING, 3)
    try:
        outs = [p.greedy(qs=qs, ws=ws) for _ in range(5)]
        times = dm.dspark_kernel_times()
    finally:
        dm.dspark_debug_set(B.DEBUG_KERNEL_TIMING, 0)
    assert len(times) == 3 and all(0.0 < t < 1e5 for t in times)
    assert dm.dspark_kernel_times() == []
    for tok, logits in outs:
        assert np.array_equal(tok, ref[0]) and np.array_equal(logits, ref[1])
    assert dm.dspark_workspace_status(ws) == 0


def test_timeout_is_reported_and_recovers():
    """The host makes every grid-wide wait also wait for a flag it never sets; each wait runs
    into its (small) time bound, the kernel still completes, and the error word says so."""
    p = random_problem(8192, 3, 2, seed=31)
    qs = p.quantize()
    ws = dm.new_workspace(2, 3, 8192)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 200)
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 1)
    p.greedy(qs=qs, ws=ws)
    assert dm.dspark_workspace_status(ws) == B.ERR_TIMEOUT
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 0)
    dm.dspark_debug_set(B.DEBUG_SPIN_LIMIT, 0)
    ws.zero_()                      # after a timeout the workspace is zeroed again
    tok, logits = p.greedy(qs=qs, ws=ws)
    assert dm.dspark_workspace_status(ws) == 0
    assert p.check_greedy(tok, logits).ok
    assert int(ws.count_nonzero()) == 0


def test_default_time_bound_ends_waits_within_milliseconds():
    """With the default bound (10 ms of device clock per wait) a walk whose waits can never be
    satisfied still finishes in a few tens of milliseconds; check_workspace() then raises the
    timeout and leaves the workspace zeroed for the next call."""
    import time
    p = random_problem(8192, 3, 1, seed=37)
    qs = p.quantize()
    ws = dm.new_workspace(1, 3, 8192)
    p.greedy(qs=qs, ws=ws)                       # warm: the kernel is loaded
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 1)
    t0 = time.perf_counter()
    p.greedy(qs=qs, ws=ws)
    wall = time.perf_counter() - t0
    dm.dspark_debug_set(B.DEBUG_WAIT_UNSET_FLAG, 0)
    assert 0.02 < wall < 0.5, wall               # three waits of about 10 ms each
    with pytest.raises(B.DsparkError) as e:
        dm.check_workspace(ws)
    assert e.value.status == B.ERR_TIMEOUT
    assert int(ws.count_nonzero()) == 0
    tok, logits = p.greedy(qs=qs, ws=ws)
    dm.check_workspace(ws)
    assert p.check_greedy(tok, logits).ok


def test_out_of_range_start_token_is_contained():
    p = random_problem(5000, 2, 2, seed=41)
    p.start = torch.tensor([7, 5000], dtype=torch.int32, device=DEV)   # 5000 is out of range
    ws = dm.new_workspace(2, 2, 5000)
    p.greedy(ws=ws)
    assert dm.dspark_workspace_status(ws) == B.ERR_INVALID_ARG


def test_graph_capture_replay():
    p = random_problem(20000, 4, 3, seed=51)
    q, s = p.quantize()
    bs, T, V = p.shape
    ws = dm.new_workspace(bs, T, V)
    tokens = torch.empty((bs, T), dtype=torch.int32, device=DEV)
    logits = torch.empty((bs, T, V), dtype=torch.float32, device=DEV)
    dm.dspark_walk_greedy(q, s, p.w1, p.base, p.start, ws, draft_tokens=tokens,
                          out_logits=logits)
    torch.cuda.synchronize()
    ref_t, ref_l = tokens.clone(), logits.clone()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        tokens.zero_()
        with torch.cuda.graph(g, stream=stream):
            dm.dspark_walk_greedy(q, s, p.w1, p.base, p.start, ws, draft_tokens=tokens,
                                  out_logits=logits)
    torch.cuda.synchronize()
    for i in range(4):
        tokens.fill_(-1)
        logits.zero_()
        scratch = torch.randn(1000, device=DEV) * 2          # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(tokens, ref_t), i
        assert torch.equal(logits, ref_l), i
        assert float(scratch.abs().sum()) > 0
    assert int(ws.count_nonzero()) == 0


# ----------------------------------------------------------------------------------------------
# the one- and two-request combine (every workgroup reads all keys from one of 16 / bs
# replicas; one reducer per request at the last step)
# ----------------------------------------------------------------------------------------------
SMALL_COMBINE = [  # V, T, bs, grid cap (0 = one workgroup per CU)
    (9000, 1, 1, 0),      # the last step is the only step: reducer only
    (9000, 1, 2, 0),
    (9000, 2, 1, 0),      # one all-poll step, then the reducer clears both steps
    (9000, 5, 1, 3),      # three workgroups: replicas read by fewer workgroups than exist
    (9000, 5, 2, 2),
    (20000, 16, 1, 0),    # the deepest walk
    (20000, 16, 2, 0),
]


@pytest.mark.parametrize("mode", ["greedy", "sample"])
@pytest.mark.parametrize("V,T,bs,cap", SMALL_COMBINE)
def test_small_batch_combine(V, T, bs, cap, mode):
    """Two calls on one workspace: both match the oracle and leave the workspace all zero (a key
    left behind would let the next call's wait finish early)."""
    dm.dspark_debug_set(B.DEBUG_MAX_WORKGROUPS, cap)
    p = random_problem(V, T, bs, seed=V + 31 * T + bs + cap)
    qs = p.quantize()
    ws = dm.new_workspace(bs, T, V)
    for _ in range(2):
        if mode == "greedy":
            tok, out = p.greedy(qs=qs, ws=ws)
            rep = p.check_greedy(tok, out)
        else:
            tok, out = p.sample(qs=qs, ws=ws)
            rep = p.check_sample(tok, out)
        assert rep.ok, rep.summary()
        assert dm.dspark_workspace_status(ws) == 0
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("path", PATHS)
def test_single_step_leaves_workspace_zeroed(path):
    """T = 1: the first step is also the last one, whose combine clears what it used. Greedy
    and sample in turn on one workspace, at one request and at 20; the workspace ends zeroed
    after every call, and the tokens match the oracle's."""
    dm.dspark_debug_set(B.DEBUG_FORCE_PATH, path)
    ws = dm.new_workspace(20, 1, 30000)
    for bs, seed in ((1, 31), (20, 32)):
        p = random_problem(30000, 1, bs, seed=seed)
        qs = p.quantize()
        tok, logits = p.greedy(qs=qs, ws=ws)
        assert int(ws.count_nonzero()) == 0
        rep = p.check_greedy(tok, logits)
        assert rep.ok, rep.summary()
        stok, lb = p.sample(qs=qs, ws=ws)
        assert int(ws.count_nonzero()) == 0
        rep = p.check_sample(stok, lb)
        assert rep.ok, rep.summary()


def test_workspace_shared_across_batch_sizes():
    """One workspace (sized for the largest call) serves walks of 3, 1, 2 and 3 requests in turn:
    the two key layouts (per-workgroup slots, per-request replicas) both leave it zero."""
    V, T = 7000, 4
    ws = dm.new_workspace(3, T, V)
    for bs in (3, 1, 2, 3):
        p = random_problem(V, T, bs, seed=500 + bs)
        tok, logits = p.greedy(ws=ws)
        rep = p.check_greedy(tok, logits)
        assert rep.ok, rep.summary()
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("V,T,bs", [(12288, 3, 20), (12288, 3, 40), (12288, 4, 64), (8192, 2, 48)])
def test_batched_greedy_without_logits_same_tokens(V, T, bs):
    """The timed greedy configuration (no fp32 logits output) is its own kernel build for batched
    walks (it holds no logits between its tile slots). Its tokens equal those of the run with
    logits, which is checked against the oracle: two, three and four 16-request tiles."""
    p = random_problem(V, T, bs, seed=V + bs)
    qs = p.quantize()
    tok, logits = p.greedy(want_logits=True, qs=qs)
    rep = p.check_greedy(tok, logits)
    assert rep.ok, rep.summary()
    for _ in range(2):
        tok2, _ = p.greedy(want_logits=False, qs=qs)
        assert np.array_equal(tok, tok2)
