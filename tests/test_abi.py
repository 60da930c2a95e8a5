"""The C ABI on the CPU: the library loads, exports every entry point its header declares, and
rejects invalid arguments before any device work. No compute call is made here: every call
below is invalid in at least one way that the host checks first, so it is safe on any machine.
"""
import ctypes
import os
import re

import pytest
import torch

import dspark_markov_draft_amd.binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

FAKE = 0x100000          # 16-byte aligned, never dereferenced: every call fails validation first
VP = ctypes.c_void_p


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s+(dspark_\w+)\s*\(",
                                 text, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 10
    L = B.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in dspark.h but not exported"


def test_status_strings():
    for code in [0, -1, -2, -3, -4, -5, -6, -7, 99]:
        s = B.dspark_status_string(code)
        assert isinstance(s, str) and s


def test_workspace_bytes():
    # 16 copies of the result words + a key region of 256 workgroups x 16 keys per step
    one = B.dspark_walk_workspace_bytes(1, 1, 10, 0)
    assert one >= 4096 + 16 * 16 * 64 * 8 + 256 * 128 and one % 256 == 0
    big = B.dspark_walk_workspace_bytes(64, 16, 270336, 0)
    assert big >= 16 * 256 * 64 * 8 and big % 256 == 0
    assert B.dspark_walk_workspace_bytes(64, 16, 4096, 0) == big      # independent of V
    assert B.dspark_walk_workspace_bytes(17, 3, 10, 0) == B.dspark_walk_workspace_bytes(32, 3, 10, 0)
    k = B.dspark_walk_workspace_bytes(64, 7, 151936, 512)
    assert k >= 64 * 7 * 513 * 4 and k >= B.dspark_walk_workspace_bytes(64, 7, 151936, 0)


@pytest.mark.parametrize("bs", [1, 4, 64])
@pytest.mark.parametrize("cus", [1, 8, 32, 80, 256, 304])
@pytest.mark.parametrize("V", [1, 3, 255, 256, 257, 4096, 5000, 70000, 129280, 151936, 248320,
                               270336])
def test_plan_partition(bs, cus, V):
    try:
        p = B.dspark_walk_plan_for(cus, 163840, bs, 7, V)
    except B.DsparkError as e:
        assert e.status == B.ERR_UNSUPPORTED
        return
    mfma_ok = bs >= 3 and V % 4 == 0                 # the greedy plan
    rpw4 = -(-max(-(-V // min(cus, 256)), min(V, 256)) // 4) * 4
    if bs == 1:
        # one request: the matrix-core kernel when a slice fits its 640 register rows and 512
        # LDS rows
        assert p["path"] == (B.PATH_MFMA1 if rpw4 <= 1152 else B.PATH_DOT4)
    elif not mfma_ok:
        assert p["path"] == B.PATH_DOT4
    elif p["path"] == B.PATH_DOT4:
        # the MFMA kernel was refused only because one staging buffer (16 request rows of the
        # slice, padded) does not fit next to its fixed LDS
        rpw16 = -(-max(-(-V // min(cus, 256)), min(V, 256)) // 16) * 16
        u16 = rpw16 // 4 + (1 - (rpw16 // 4) % 2)
        fixed = 64 * 256 + 64 * 4 + rpw16 * 4 + 4 * 4 * 64 * 8 + 64 * 4
        assert fixed + 16 * u16 * 16 > 163840
    mfma = p["path"] == B.PATH_MFMA
    quantum = 16 if mfma else 4                      # rows: 16-row tiles vs lane-per-row sets
    nwg, rpw = p["num_workgroups"], p["rows_per_workgroup"]
    cus = min(cus, 256)                          # the grid is capped at 256 workgroups
    assert 1 <= nwg <= cus
    assert nwg * rpw >= V > (nwg - 1) * rpw          # every row owned exactly once
    assert rpw % quantum == 0
    assert p["rows_in_registers"] + p["rows_in_lds"] + p["rows_streamed"] == rpw
    assert p["resident_bytes"] + p["streamed_bytes"] == V * 256
    if p["path"] == B.PATH_MFMA1:
        assert p["rows_in_registers"] == min(rpw, 640) and p["rows_streamed"] == 0
        assert p["rows_in_lds"] == rpw - min(rpw, 640) <= 512
        assert p["total_units"] == -(-(-(-rpw // 16)) // 4) <= 18
        assert p["reg_units"] == min(p["total_units"], 10)
    elif not mfma:
        assert p["rows_in_registers"] <= 3 * 256 and p["rows_in_lds"] <= 512
        assert p["total_units"] == -(-rpw // 256)
    else:
        # 4 waves, or 8 (5 register tiles each) for slices with static LDS
        w = p["waves_per_workgroup"]
        stat = rpw <= 624 and p["stage_stride"] <= 628
        assert w == 4 or (w == 8 and stat)
        assert p["rows_in_registers"] <= (8 if w == 4 else 5) * 16 * w
        assert p["total_units"] == -(-(rpw // 16) // w)
        assert p["stage_bufs"] == (2 if bs > 16 else 1) or p["stage_bufs"] >= 1
        assert p["stage_stride"] >= rpw and (p["stage_stride"] // 4) % 2 == 1
    if not mfma:
        assert p["waves_per_workgroup"] == 4
    assert p["reg_units"] + p["lds_units"] <= p["total_units"]
    assert 96 * 1024 <= p["lds_bytes"] <= 163840
    if V >= 256 * cus:
        # big vocabularies: the smallest multiple of the quantum that covers V with every CU
        assert (rpw - quantum) * cus < V <= rpw * cus


@pytest.mark.parametrize("waves", [4, 8])
def test_plan_mfma_waves_hook(waves):
    """The test hook forces the waves per workgroup of the static-LDS MFMA kernel; the tiles per
    wave follow, and the kernel with dynamic LDS keeps 4."""
    try:
        assert B.lib().dspark_debug_set(B.DEBUG_MFMA_WAVES, waves) == 0
        p = B.dspark_walk_plan_for(256, 163840, 64, 7, 151936)   # 608-row slices: static
        assert p["path"] == B.PATH_MFMA and p["waves_per_workgroup"] == waves
        assert p["total_units"] == -(-38 // waves)
        assert p["rows_in_registers"] + p["rows_in_lds"] == 608
        p = B.dspark_walk_plan_for(256, 163840, 64, 7, 200000)   # 784-row slices: dynamic
        assert p["path"] == B.PATH_MFMA and p["waves_per_workgroup"] == 4
        assert B.lib().dspark_debug_set(B.DEBUG_MFMA_WAVES, 5) == B.ERR_INVALID_ARG
    finally:
        B.lib().dspark_debug_set(B.DEBUG_MFMA_WAVES, 0)


@pytest.mark.parametrize("bs", [1, 16, 64])
def test_plan_pages_shapes_fit_on_chip(bs):
    """On a 256-CU MI355X the W2 of every shape in the pages' kernel table stays on chip (the
    V = 248320 walks there are single-request; with several requests the MFMA kernel gives its
    LDS to the base-logit staging first and streams part of that W2)."""
    for V in (129280, 151936, 248320, 270336):
        p = B.dspark_walk_plan_for(256, 163840, bs, 7, V)
        if V <= 151936 or (bs == 1 and V <= 248320):
            assert p["streamed_bytes"] == 0, (bs, V, p)
        assert p["resident_bytes"] + p["streamed_bytes"] == V * 256


def _greedy(**kw):
    a = dict(q=FAKE, s=FAKE, w1=FAKE, dt=B.BF16, base=FAKE, start=FAKE, bs=1, T=7, V=151936,
             rank=256, tokens=FAKE, logits=None, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return B.lib().dspark_walk_greedy(a["q"], a["s"], a["w1"], a["dt"], a["base"], a["start"],
                                      a["bs"], a["T"], a["V"], a["rank"], a["tokens"],
                                      a["logits"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), B.ERR_INVALID_ARG),
    (dict(w1=None), B.ERR_INVALID_ARG),
    (dict(base=None), B.ERR_INVALID_ARG),
    (dict(tokens=None), B.ERR_INVALID_ARG),
    (dict(ws=None), B.ERR_INVALID_ARG),
    (dict(q=FAKE + 4), B.ERR_INVALID_ARG),
    (dict(w1=FAKE + 8), B.ERR_INVALID_ARG),
    (dict(bs=0), B.ERR_INVALID_ARG),
    (dict(T=0), B.ERR_INVALID_ARG),
    (dict(V=0), B.ERR_INVALID_ARG),
    (dict(V=-5), B.ERR_INVALID_ARG),
    (dict(rank=128), B.ERR_UNSUPPORTED),
    (dict(T=17), B.ERR_UNSUPPORTED),
    (dict(bs=65), B.ERR_UNSUPPORTED),
    (dict(V=270337), B.ERR_UNSUPPORTED),
    (dict(dt=7), B.ERR_UNSUPPORTED),
    (dict(wsb=100), B.ERR_WORKSPACE),
])
def test_greedy_validation(kw, code):
    assert _greedy(**kw) == code


def _noalloc(**kw):
    a = dict(q=FAKE, s=FAKE, w1=FAKE, dt=B.BF16, base=FAKE, start=FAKE, bs=1, T=7, V=151936,
             rank=256, tokens=FAKE, logits=None, err=None, stream=None)
    a.update(kw)
    return B.lib().dspark_walk_greedy_noalloc(a["q"], a["s"], a["w1"], a["dt"], a["base"],
                                              a["start"], a["bs"], a["T"], a["V"], a["rank"],
                                              a["tokens"], a["logits"], a["err"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), B.ERR_INVALID_ARG),
    (dict(s=None), B.ERR_INVALID_ARG),
    (dict(tokens=None), B.ERR_INVALID_ARG),
    (dict(q=FAKE + 4), B.ERR_INVALID_ARG),
    (dict(err=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(logits=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(bs=0), B.ERR_INVALID_ARG),
    (dict(rank=128), B.ERR_UNSUPPORTED),
    (dict(T=17), B.ERR_UNSUPPORTED),
    (dict(bs=65), B.ERR_UNSUPPORTED),
    (dict(V=270337), B.ERR_UNSUPPORTED),
    (dict(dt=7), B.ERR_UNSUPPORTED),
])
def test_noalloc_validation(kw, code):
    """The no-allocation walk checks its arguments on the host like the greedy walk (its
    largest shape, bs 64 x 16 steps, fits its scratch by construction)."""
    assert _noalloc(**kw) == code


def _verify(**kw):
    a = dict(lb=FAKE, X=FAKE, tg=FAKE, temp=FAKE, u=FAKE, bs=4, T=7, V=151936, mode=0,
             acc=FAKE, out=FAKE, prob=None, ws=FAKE, wsb=1 << 24, stream=None)
    a.update(kw)
    return B.lib().dspark_verify(a["lb"], a["X"], a["tg"], a["temp"], a["u"], a["bs"], a["T"],
                                 a["V"], a["mode"], a["acc"], a["out"], a["prob"], a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(lb=None), B.ERR_INVALID_ARG),
    (dict(tg=None), B.ERR_INVALID_ARG),
    (dict(u=None), B.ERR_INVALID_ARG),
    (dict(out=None), B.ERR_INVALID_ARG),
    (dict(ws=None), B.ERR_INVALID_ARG),
    (dict(lb=FAKE + 1), B.ERR_INVALID_ARG),
    (dict(tg=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(prob=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(ws=FAKE + 8), B.ERR_INVALID_ARG),
    (dict(mode=2), B.ERR_INVALID_ARG),
    (dict(bs=0), B.ERR_INVALID_ARG),
    (dict(T=17), B.ERR_UNSUPPORTED),
    (dict(bs=65), B.ERR_UNSUPPORTED),
    (dict(V=270337), B.ERR_UNSUPPORTED),
    (dict(wsb=1000), B.ERR_WORKSPACE),
])
def test_verify_validation(kw, code):
    assert _verify(**kw) == code


def test_verify_workspace_bytes():
    n = B.lib().dspark_verify_workspace_bytes
    assert n(64, 7, 151936) % 256 == 0
    assert n(64, 7, 151936) >= 64 * 8 * 75 * 16          # chunk statistics at the smallest chunk
    assert n(1, 1, 1) <= n(64, 16, 270336) < 8 << 20
    assert n(64, 16, 270336) == n(65, 17, 300000)       # clamped to the envelope


def _pruned(**kw):
    a = dict(q=FAKE, s=FAKE, w1=FAKE, dt=B.BF16, base=FAKE, start=FAKE, bs=1, T=7, V=151936,
             rank=256, k=512, bound=FAKE, tokens=FAKE, logits=None, dense=None, ws=FAKE,
             wsb=1 << 24, stream=None)
    a.update(kw)
    return B.lib().dspark_walk_greedy_pruned(a["q"], a["s"], a["w1"], a["dt"], a["base"],
                                             a["start"], a["bs"], a["T"], a["V"], a["rank"],
                                             a["k"], a["bound"], a["tokens"], a["logits"],
                                             a["dense"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(bound=None), B.ERR_INVALID_ARG),
    (dict(bound=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(q=None), B.ERR_INVALID_ARG),
    (dict(logits=FAKE + 4), B.ERR_INVALID_ARG),
    (dict(dense=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(k=0), B.ERR_INVALID_ARG),
    (dict(k=151937), B.ERR_INVALID_ARG),
    (dict(k=2049), B.ERR_UNSUPPORTED),
    (dict(T=17), B.ERR_UNSUPPORTED),
    (dict(wsb=100), B.ERR_WORKSPACE),
])
def test_pruned_validation(kw, code):
    assert _pruned(**kw) == code


def test_prune_bound_validation():
    L = B.lib()
    assert L.dspark_w2_prune_bound(None, FAKE, 10, 256, FAKE, None) == B.ERR_INVALID_ARG
    assert L.dspark_w2_prune_bound(FAKE, FAKE, 0, 256, FAKE, None) == B.ERR_INVALID_ARG
    assert L.dspark_w2_prune_bound(FAKE + 4, FAKE, 10, 256, FAKE, None) == B.ERR_INVALID_ARG
    assert L.dspark_w2_prune_bound(FAKE, FAKE, 10, 128, FAKE, None) == B.ERR_UNSUPPORTED


def _sample(**kw):
    a = dict(q=FAKE, s=FAKE, w1=FAKE, dt=B.BF16, base=FAKE, start=FAKE, bs=1, T=7, V=151936,
             rank=256, seeds=FAKE, pos=None, temp=FAKE, tokens=FAKE, lb=FAKE, ws=FAKE,
             wsb=1 << 20, stream=None)
    a.update(kw)
    return B.lib().dspark_walk_sample(a["q"], a["s"], a["w1"], a["dt"], a["base"], a["start"],
                                      a["bs"], a["T"], a["V"], a["rank"], a["seeds"], a["pos"],
                                      a["temp"], a["tokens"], a["lb"], a["ws"], a["wsb"],
                                      a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(seeds=None), B.ERR_INVALID_ARG),
    (dict(temp=None), B.ERR_INVALID_ARG),
    (dict(lb=None), B.ERR_INVALID_ARG),
    (dict(seeds=FAKE + 4), B.ERR_INVALID_ARG),
    (dict(pos=FAKE + 4), B.ERR_INVALID_ARG),
    (dict(lb=FAKE + 1), B.ERR_INVALID_ARG),
    (dict(T=99), B.ERR_UNSUPPORTED),
    (dict(wsb=0), B.ERR_WORKSPACE),
])
def test_sample_validation(kw, code):
    assert _sample(**kw) == code


def _topk(**kw):
    a = dict(q=FAKE, s=FAKE, w1=FAKE, dt=B.BF16, base=FAKE, start=FAKE, bs=64, T=7, V=151936,
             rank=256, k=512, sample=1, seeds=FAKE, pos=None, temp=FAKE, tokens=FAKE, dl=FAKE,
             ws=FAKE, wsb=1 << 24, stream=None)
    a.update(kw)
    return B.lib().dspark_walk_topk(a["q"], a["s"], a["w1"], a["dt"], a["base"], a["start"],
                                    a["bs"], a["T"], a["V"], a["rank"], a["k"], a["sample"],
                                    a["seeds"], a["pos"], a["temp"], a["tokens"], a["dl"],
                                    a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), B.ERR_INVALID_ARG),
    (dict(k=151937), B.ERR_INVALID_ARG),
    (dict(k=4096), B.ERR_UNSUPPORTED),
    (dict(sample=2), B.ERR_INVALID_ARG),
    (dict(seeds=None), B.ERR_INVALID_ARG),
    (dict(dl=None), B.ERR_INVALID_ARG),
    (dict(dl=FAKE + 2), B.ERR_INVALID_ARG),
    (dict(wsb=4096), B.ERR_WORKSPACE),
    (dict(rank=255), B.ERR_UNSUPPORTED),
])
def test_topk_validation(kw, code):
    assert _topk(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(w2=None), B.ERR_INVALID_ARG),
    (dict(V=0), B.ERR_INVALID_ARG),
    (dict(rank=64), B.ERR_UNSUPPORTED),
    (dict(dt=3), B.ERR_UNSUPPORTED),
    (dict(q=FAKE + 2), B.ERR_INVALID_ARG),
])
def test_quantize_validation(kw, code):
    a = dict(w2=FAKE, dt=B.BF16, V=10, rank=256, q=FAKE, s=FAKE)
    a.update(kw)
    assert B.lib().dspark_quantize_w2(a["w2"], a["dt"], a["V"], a["rank"], a["q"], a["s"],
                                      None) == code


def test_misc_validation():
    L = B.lib()
    assert L.dspark_philox_words(1, 2, 0, 10, None, None) == B.ERR_INVALID_ARG
    assert L.dspark_philox_words(1, 2, -1, 10, FAKE, None) == B.ERR_INVALID_ARG
    assert L.dspark_workspace_status(None, None) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(99, 1) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(B.DEBUG_SPIN_LIMIT, -1) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(B.DEBUG_FORCE_PATH, 4) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(B.DEBUG_STAMPS, 12) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(B.DEBUG_KERNEL_TIMING, 4097) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(B.DEBUG_TOPK_SPLIT, -1) == B.ERR_INVALID_ARG
    assert L.dspark_debug_set(B.DEBUG_TOPK_SPLIT, 1) == B.OK
    assert L.dspark_debug_set(B.DEBUG_TOPK_SPLIT, 0) == B.OK
    n = ctypes.c_int32(-1)
    buf = (ctypes.c_float * 4)()
    assert L.dspark_kernel_times(None, 4, ctypes.byref(n)) == B.ERR_INVALID_ARG
    assert L.dspark_kernel_times(buf, -1, ctypes.byref(n)) == B.ERR_INVALID_ARG
    assert L.dspark_kernel_times(buf, 4, None) == B.ERR_INVALID_ARG
    assert L.dspark_kernel_times(buf, 4, ctypes.byref(n)) == B.OK and n.value == 0
    assert L.dspark_walk_plan_query(1, 1, 10, None) == B.ERR_INVALID_ARG
    assert L.dspark_walk_plan_for(0, 163840, 1, 1, 10, ctypes.byref(B.WalkPlan())) == \
        B.ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible")
def test_no_device_without_gpu():
    """Valid arguments on a machine with no GPU: the device check refuses the call."""
    assert _greedy() == B.ERR_NO_DEVICE
    assert _sample() == B.ERR_NO_DEVICE
    assert _noalloc() == B.ERR_NO_DEVICE
    assert _verify() == B.ERR_NO_DEVICE
    assert _pruned() == B.ERR_NO_DEVICE
    assert _noalloc(bs=64, T=16, V=270336) == B.ERR_NO_DEVICE
    p = B.WalkPlan()
    assert B.lib().dspark_walk_plan_query(1, 7, 151936, ctypes.byref(p)) == B.ERR_NO_DEVICE
