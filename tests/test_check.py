"""The teacher-forced checker's own rules (CPU): the bf16 rounding intervals it uses agree with
torch's bf16 rounding, and a planted token error is caught."""
import numpy as np
import torch

from oracle.check import _bf16_interval, _bf16_within_tol, bf16_bits_to_f32, check_walk


def test_bf16_interval_matches_torch_rounding():
    rng = np.random.default_rng(0)
    h = rng.integers(0, 0x7F7F, 3000).astype(np.uint16)
    h = np.concatenate([h, h | np.uint16(0x8000), np.array([1, 0x8001, 0x3F80], np.uint16)])
    lo, hi = _bf16_interval(h)
    for f in (0.01, 0.25, 0.5, 0.75, 0.99):      # interior points (endpoints are ties)
        x = (lo + (hi - lo) * f).astype(np.float32)
        xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(xb, h)
    # just outside the interval rounds elsewhere
    out = (hi + (hi - lo) * 0.01).astype(np.float32)
    ob = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert not np.any(ob == h)


def test_bf16_tolerance_rule():
    l = np.array([0.02367045, 5.0, 5.0], np.float32)
    lb_o = torch.from_numpy(l).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # one bf16 step up at 0.0237 (1.2e-4 away): within 2e-3; 5.0 -> 5.0625: not within 2e-3
    lb_t = lb_o.copy()
    lb_t[0] += 1
    lb_t[1] += 2
    diff, ok = _bf16_within_tol(l, lb_o, lb_t, 2e-3)
    assert diff.tolist() == [0, 1] and ok.tolist() == [True, False]
    assert bf16_bits_to_f32(lb_t[1:2])[0] == np.float32(5.0625)


def test_checker_catches_wrong_token(orc):
    rng = np.random.default_rng(1)
    V, T = 300, 3
    w1 = (rng.standard_normal((V, 256)) * 0.05).astype(np.float32)
    w2 = (rng.standard_normal((V, 256)) * 0.05).astype(np.float32)
    base = (rng.standard_normal((1, T, V)) * 3).astype(np.float32)
    q, s = orc.quantize_w2(w2)
    start = np.array([4], np.int32)
    tokens, logits, _ = orc.walk(q, s, w1, base, start, want_logits=True)
    assert check_walk(q, s, w1, base, start, tokens, logits=logits).ok
    bad = tokens.copy()
    bad[0, 1] = (bad[0, 1] + 1) % V
    assert not check_walk(q, s, w1, base, start, bad).ok
    off = logits.copy()
    off[0, 2, 17] += 3e-3
    assert not check_walk(q, s, w1, base, start, tokens, logits=off).ok
