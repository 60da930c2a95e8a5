"""The teacher-forced checker's own rules (CPU): the bf16 rounding intervals it uses agree with
torch's bf16 rounding, and a planted token error is caught."""
import numpy as np
import torch

import oracle
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


def test_verify_checker_catches_planted_mistakes():
    """The verification checker accepts the oracle's own outputs and rejects a wrong next token,
    a wrong kept length away from any near tie, a kept prefix that is not the draft, and an
    acceptance probability off by more than its tolerance."""
    import torch
    from oracle.check import check_verify
    from dspark_markov_draft_amd.synth import make_verify_inputs
    v = make_verify_inputs(16, 4, 700, 5, temperature=None)
    lb = v.draft_lb.view(torch.int16).numpy().view(np.uint16)
    args = (lb, v.draft_tokens.numpy(), v.target.numpy(), v.temperature.numpy(),
            v.uniforms.numpy())
    for mode in (0, 1):
        acc, out, prob = oracle.verify(*args, mode)
        prob = prob.astype(np.float32)
        assert check_verify(*args, mode, acc, out, prob).ok
        b = int(np.argmax(acc < 4))                      # a request with a drawn next token
        bad = out.copy(); bad[b, acc[b]] = (bad[b, acc[b]] + 7) % 700
        assert not check_verify(*args, mode, acc, bad, prob).ok
        u = v.uniforms.numpy()
        far = [i for i in range(16) if acc[i] < 4 and
               (np.abs(u[i, :4] - oracle.verify(*args, mode)[2][i]) > 1e-2).all()]
        i = far[0]
        acc2, out2 = acc.copy(), out.copy()
        acc2[i] += 1
        out2[i, :acc2[i]] = args[1][i, :acc2[i]]
        out2[i, acc2[i]] = 0
        out2[i, acc2[i] + 1:] = -1
        assert not check_verify(*args, mode, acc2, out2, prob).ok
        bad = out.copy(); bad[b, 0] = (bad[b, 0] + 1) % 700 if acc[b] > 0 else bad[b, 0]
        if acc[b] > 0:
            assert not check_verify(*args, mode, acc, bad, prob).ok
        p2 = prob.copy(); p2[3, 1] += 5e-4
        assert not check_verify(*args, mode, acc, out, p2).ok
