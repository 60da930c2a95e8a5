"""Teacher-forced comparison of a walk's outputs with the CPU oracle.

TEST INFRASTRUCTURE ONLY (tests, ``__graft_entry__.smoke()``, the CPU leg of ``bench.py``).

The walk is sequential, so one legitimate near-tie flip would change every later step. Each
step is therefore re-run in the oracle with the previous token the walk under test actually
chose (teacher forcing), and compared element by element:

  * fp32 logits: |l_test - l_oracle| <= tol wherever the oracle is finite, and the -inf
    entries of a top-k row match exactly;
  * bf16 draft logits: equal, or the bf16 rounding of some value within tol of the oracle's
    fp32 logit (the logit tolerance carried through the rounding; where |l| is small a bf16
    step is far below tol, so a legitimate logit difference can move it by several steps);
  * tokens: equal, or a near tie: the oracle's argmaxed quantity (logits for greedy, scores for
    sampling) at the chosen token is within tol of its maximum; for sampling the allowance grows
    by the stored bf16 difference / temperature at the two tokens.

The tolerance 2e-3 (absolute, on logits) is the one the measured target names; the walk under
test quantises the gathered W1 row to int8, which the oracle does not.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import icdf_draw as oracle_icdf_draw
from . import icdf_uniform as oracle_icdf_uniform
from . import step as oracle_step
from . import topk as oracle_topk

TOL = 2e-3
TOL_ICDF_U = 1e-5   # inverse-CDF sampling: any draw of the stored row for u +- this


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Report:
    steps: int = 0
    max_abs_logit_err: float = 0.0
    lb_mismatch: int = 0            # bf16 entries that differ (each within the tolerance)
    near_ties: List[tuple] = field(default_factory=list)   # (b, t, oracle tok, test tok, gap)
    failures: List[str] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        return (f"steps={self.steps} max|dlogit|={self.max_abs_logit_err:.3g} "
                f"bf16 diffs={self.lb_mismatch} near-ties={len(self.near_ties)} "
                f"failures={len(self.failures)}" +
                ("" if self.ok else "\n  " + "\n  ".join(self.failures[:10])))


def _bf16_interval(h: np.ndarray):
    """[lo, hi] of the fp32 values that round (nearest even) to each finite bf16 h: halfway to
    the neighbouring bf16 values on either side."""
    h = np.asarray(h, np.uint16).astype(np.int64)
    v = bf16_bits_to_f32(h).astype(np.float64)
    sign = np.where(h & 0x8000, -1, 1)
    mag = h & 0x7FFF
    up = bf16_bits_to_f32(((mag + 1) | (h & 0x8000)).astype(np.uint16)).astype(np.float64)
    dn_mag = np.maximum(mag - 1, 0)
    dn = bf16_bits_to_f32((dn_mag | (h & 0x8000)).astype(np.uint16)).astype(np.float64)
    dn = np.where(mag == 0, -v - (up - v), dn)          # around zero the step is symmetric
    a, b = (v + dn) / 2, (v + up) / 2                    # away-from-zero neighbour is `up`
    lo = np.where(sign > 0, a, b)
    hi = np.where(sign > 0, b, a)
    return np.minimum(lo, hi), np.maximum(lo, hi)


def _bf16_within_tol(l_orc: np.ndarray, lb_orc: np.ndarray, lb_test: np.ndarray, tol: float):
    """Entries where lb_test != lb_orc are allowed if lb_test is the bf16 rounding of some value
    within tol of the oracle's fp32 logit (its rounding interval meets [l - tol, l + tol])."""
    diff = np.nonzero(lb_orc != lb_test)[0]
    if diff.size == 0:
        return diff, np.ones(0, bool)
    l = l_orc[diff].astype(np.float64)
    t = lb_test[diff]
    tv = bf16_bits_to_f32(t).astype(np.float64)
    lo, hi = _bf16_interval(t)
    ok = np.isfinite(tv) & np.isfinite(l) & (lo <= l + tol) & (hi >= l - tol)
    return diff, ok


def check_walk(q, s, w1, base, start, tokens, *, sample=False, seeds=None, temps=None,
               positions=None, k=0, logits=None, lb=None, requests=None, tol=TOL) -> Report:
    """Compare a walk's outputs with the oracle, teacher-forced.

    q, s: the ORACLE's own quantisation of W2; w1 fp32 [V, R]; base [bs, T, V] fp32; start [bs];
    tokens [bs, T] from the walk under test; logits fp32 [bs, T, V] (greedy, optional);
    lb uint16 [bs, T, V] (sample, optional); requests: subset of request indices to check.
    sample: False (greedy), True or 1 (Gumbel), 2 (inverse CDF). For the inverse-CDF sampler a
    token that differs from the oracle's is accepted if it is a draw of the row the walk stored
    (already checked against the oracle's logits) for some uniform within TOL_ICDF_U of the
    step's: the draw is monotone in u, so between the draws at the two ends.
    """
    bs, T, V = base.shape
    rep = Report()
    reqs = range(bs) if requests is None else requests
    for b in reqs:
        prev = int(start[b])
        for t in range(T):
            cand = oracle_topk(base[b, t], k) if k else None
            P = (int(positions[b]) if positions is not None else 0) + t
            seed = int(seeds[b]) if sample else 0
            temp = float(temps[b]) if sample else 1.0
            tok, l_o, lb_o, sc_o = oracle_step(q, s, w1, base[b, t], prev, cand=cand,
                                               sample=sample, seed=seed, P=P, temp=temp)
            got = int(tokens[b, t])
            rep.steps += 1
            where = f"b={b} t={t}"
            if not (0 <= got < V):
                rep.failures.append(f"{where}: token {got} out of range")
                break
            if logits is not None:
                l_t = np.asarray(logits[b, t], np.float32)
                fin = np.isfinite(l_o)
                if not np.array_equal(np.isneginf(l_o), np.isneginf(l_t)):
                    rep.failures.append(f"{where}: -inf pattern differs")
                err = np.abs(l_t[fin].astype(np.float64) - l_o[fin].astype(np.float64))
                m = float(err.max()) if err.size else 0.0
                rep.max_abs_logit_err = max(rep.max_abs_logit_err, m)
                if not m <= tol:
                    rep.failures.append(f"{where}: max |dlogit| {m:.3g} > {tol}")
            lb_t = None
            if sample and lb is not None:
                lb_t = np.asarray(lb[b, t], np.uint16)
                diff, ok = _bf16_within_tol(l_o, lb_o, lb_t, tol)
                rep.lb_mismatch += int(diff.size)
                if diff.size and not ok.all():
                    bad = diff[~ok][:3]
                    rep.failures.append(
                        f"{where}: bf16 draft logits differ at {bad.tolist()} "
                        f"(oracle {bf16_bits_to_f32(lb_o[bad])}, test {bf16_bits_to_f32(lb_t[bad])},"
                        f" l {l_o[bad]})")
            if got != tok and sample == 2:
                u = oracle_icdf_uniform(seed, P)
                row = lb_t if lb_t is not None else lb_o
                lo = oracle_icdf_draw(row, temp, max(u - TOL_ICDF_U, 2.0 ** -24))
                hi = oracle_icdf_draw(row, temp, min(u + TOL_ICDF_U, 1.0 - 2.0 ** -24))
                if lo <= got <= hi:
                    rep.near_ties.append((b, t, tok, got, 0.0))
                else:
                    rep.failures.append(f"{where}: token {got} vs oracle {tok} (draws of the "
                                        f"stored row for u +- {TOL_ICDF_U}: {lo}..{hi})")
            elif got != tok:
                qty = sc_o if sample else l_o
                gap = float(qty[tok]) - float(qty[got])
                allow = tol
                if sample and lb_t is not None:
                    for v in (tok, got):
                        allow += abs(float(bf16_bits_to_f32(lb_t[v:v + 1])[0]) -
                                     float(bf16_bits_to_f32(lb_o[v:v + 1])[0])) / temp
                if np.isnan(qty[tok]) or not (gap <= allow):
                    rep.failures.append(f"{where}: token {got} vs oracle {tok} (gap {gap:.3g})")
                else:
                    rep.near_ties.append((b, t, tok, got, gap))
            prev = got
    return rep


# ----------------------------------------------------------------------------------------------
# verification of drafted blocks
# ----------------------------------------------------------------------------------------------
TOL_PROB = 1e-4     # acceptance probabilities (fp32 softmax and sums against fp64)
TOL_U = 1e-5        # inverse-CDF draws: the next token may be any the oracle draws for u +- this


@dataclass
class VerifyReport:
    requests: int = 0
    max_prob_err: float = 0.0
    kept_total: int = 0
    near_ties: List[tuple] = field(default_factory=list)     # (b, what)
    failures: List[str] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        return (f"requests={self.requests} kept={self.kept_total} "
                f"max|dprob|={self.max_prob_err:.3g} near-ties={len(self.near_ties)} "
                f"failures={len(self.failures)}" +
                ("" if self.ok else "\n  " + "\n  ".join(self.failures[:10])))


def _implied_decisions(mode, tau, T):
    """Per step i (0-based), the accept/reject decision a verifier must have taken to end with
    kept length tau (None where the outcome does not depend on it)."""
    d = [None] * T
    if mode == 0:
        for i in range(T):
            if i < tau:
                d[i] = True
            elif i == tau:
                d[i] = False
    else:       # block: tau = largest i with u_{i-1} <= h_i
        for i in range(1, T + 1):
            if i == tau:
                d[i - 1] = True
            elif i > tau:
                d[i - 1] = False
    return d


def check_verify(lb, X, tg, temps, u, mode, acc, out, prob=None, tol_prob=TOL_PROB,
                 tol_u=TOL_U) -> VerifyReport:
    """Compare a verification's outputs (acc [bs], out [bs, T + 1], prob [bs, T] or None) with
    the oracle on the same inputs. The kept length must equal the oracle's unless every step
    whose decision differs has its uniform within tol_prob of the oracle's acceptance
    probability (a near tie; then the next token is not compared). The next token must lie
    among the oracle's draws for uniforms in [u - tol_u, u + tol_u] (the draw is monotone in
    u, so between the draws at the two ends)."""
    from . import verify as oracle_verify
    lb = np.asarray(lb, np.uint16)
    u = np.asarray(u, np.float32)
    bs, T, V = lb.shape
    acc_o, out_o, prob_o = oracle_verify(lb, X, tg, temps, u, mode)
    lo_u, hi_u = u.copy(), u.copy()
    lo_u[:, T] = np.maximum(u[:, T] - np.float32(tol_u), np.float32(2.0 ** -24))
    hi_u[:, T] = np.minimum(u[:, T] + np.float32(tol_u), np.float32(1.0 - 2.0 ** -24))
    _, out_lo, _ = oracle_verify(lb, X, tg, temps, lo_u, mode)
    _, out_hi, _ = oracle_verify(lb, X, tg, temps, hi_u, mode)
    rep = VerifyReport(requests=bs)
    if prob is not None:
        err = np.abs(np.asarray(prob, np.float64) - prob_o)
        rep.max_prob_err = float(err.max())
        if not rep.max_prob_err <= tol_prob:
            b, t = np.unravel_index(int(err.argmax()), err.shape)
            rep.failures.append(f"b={b} t={t}: accept prob {prob[b, t]} vs oracle {prob_o[b, t]}")
    for b in range(bs):
        tau = int(acc[b])
        rep.kept_total += max(tau, 0)
        if not 0 <= tau <= T:
            rep.failures.append(f"b={b}: kept length {tau} out of range")
            continue
        if not np.array_equal(out[b, :tau], X[b, :tau]) or (out[b, tau + 1:] != -1).any():
            rep.failures.append(f"b={b}: output {out[b].tolist()} is not the kept prefix, a token, -1s")
            continue
        if not 0 <= int(out[b, tau]) < V:
            rep.failures.append(f"b={b}: next token {int(out[b, tau])} out of range")
            continue
        if tau != int(acc_o[b]):
            want = _implied_decisions(mode, tau, T)
            orc = [bool(u[b, i] <= prob_o[b, i]) for i in range(T)]
            bad = [i for i in range(T) if want[i] is not None and want[i] != orc[i] and
                   not abs(float(u[b, i]) - float(prob_o[b, i])) <= tol_prob]
            if bad:
                rep.failures.append(f"b={b}: kept {tau} vs oracle {int(acc_o[b])} (steps {bad})")
            else:
                rep.near_ties.append((b, f"kept {tau} vs {int(acc_o[b])}"))
            continue
        y, y_lo, y_hi = int(out[b, tau]), int(out_lo[b, tau]), int(out_hi[b, tau])
        if y != int(out_o[b, tau]):
            if min(y_lo, y_hi) <= y <= max(y_lo, y_hi):
                rep.near_ties.append((b, f"next token {y} vs {int(out_o[b, tau])}"))
            else:
                rep.failures.append(f"b={b}: next token {y} vs oracle {int(out_o[b, tau])} "
                                    f"(draws for u +- {tol_u}: {y_lo}..{y_hi})")
    return rep
