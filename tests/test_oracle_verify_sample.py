"""Pins of the stochastic-verification oracle (oracle/verify_sample.py).

Each pin checks the oracle against something other than itself: published
known-answer vectors of the random generator, and distributional properties
that the mathematics fixes (checked by Monte Carlo with chi-square bounds at
a 1e-4 false-alarm level; all seeds are fixed, so the tests are
deterministic), plus the low-temperature limit, which must reproduce the
greedy oracle.
"""
import math
import os

import numpy as np
import pytest

import oracle.verify_sample as vs
from oracle import verify_ref
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
CHI2_99_99 = {2: 18.42, 3: 21.11, 4: 23.51}  # chi-square quantile 0.9999 by degrees of freedom


def test_philox_known_answers():
    for line in open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")):
        if line.startswith("#") or not line.strip():
            continue
        w = [int(x, 16) for x in line.split()]
        out = vs.philox4x32_10(w[0:4], (w[4], w[5]))
        assert [int(x) for x in out] == w[6:10]


def _chi2(counts, probs):
    n = counts.sum()
    e = n * np.asarray(probs)
    return float(((counts - e) ** 2 / e).sum())


def test_uniforms_are_uniform_and_in_open_interval():
    u = vs.row_uniforms(seed=7, step=3, b=0, j=1, V=40000)
    assert u.min() > 0.0 and u.max() < 1.0
    counts = np.histogram(u, bins=5, range=(0, 1))[0]
    assert _chi2(counts, [0.2] * 5) < CHI2_99_99[4]


def test_uniform_grid_is_exact_in_fp32_at_both_ends():
    # the GPU forms the same uniforms in fp32: every grid value, the extremes
    # included, must survive a round trip through float32 and stay inside (0, 1)
    x = np.array([0, 1 << 9, 0x7FFFFFFF, 0x80000000, 0xFFFFFDFF, 0xFFFFFFFF], dtype=np.uint64)
    u = vs.to_uniform(x)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    assert u[0] == 2.0 ** -24 and u[-1] == 1.0 - 2.0 ** -24
    assert (u > 0).all() and (u < 1).all()


def test_gumbel_draw_follows_the_weights():
    w = np.array([0.1, 0.2, 0.3, 0.4])
    n = 20000
    counts = np.zeros(4)
    for b in range(n):
        idx, _ = vs.gumbel_draw(w, vs.row_uniforms(seed=11, step=0, b=b, j=2, V=4))
        counts[idx] += 1
    assert _chi2(counts, w) < CHI2_99_99[3]


def test_first_token_is_distributed_as_the_target():
    """Speculative sampling's defining property: drawing the candidate from q
    and keeping or resampling it gives a token distributed exactly as p."""
    rng = np.random.default_rng(5)
    V, n = 5, 20000
    lp = rng.normal(size=V) * 1.5
    lq = rng.normal(size=V) * 1.5
    p, q = vs.softmax(lp, 1.0), vs.softmax(lq, 1.0)
    # candidate 0 ~ q, drawn with an independent Gumbel stream (row 9)
    cand = np.array([[vs.gumbel_draw(q, vs.row_uniforms(3, 1, b, 9, V))[0]] for b in range(n)], np.int32)
    ar = np.broadcast_to(lp, (n, 2, V))
    ql = np.broadcast_to(lq, (n, 1, V))
    a, nxt = vs.verify_sample_ref(ar, ql, None, cand, 1.0, seed=3, step=1)
    first = np.where(a == 1, cand[:, 0], nxt[:, 0])
    counts = np.bincount(first, minlength=V).astype(float)
    assert _chi2(counts, p) < CHI2_99_99[4]
    kept = float((a == 1).mean())
    expect = float(np.minimum(p, q).sum())
    assert abs(kept - expect) < 4.0 * np.sqrt(expect * (1 - expect) / n)


def test_low_temperature_with_one_hot_proposals_is_the_greedy_rule():
    """T -> 0 with proposals peaked at the candidates: a candidate is kept
    iff it is the target argmax, the resample is the target argmax and the
    drafts are argmaxes -- the greedy oracle's outputs."""
    B, k, V = 6, 4, 300
    v = W.verify_inputs(B, k, V, seed=21, accept="uniform")
    ar, dr, cand = v["ar_logits"].astype(np.float64), v["draft_logits"].astype(np.float64), v["cand"]
    # make every row's maximum stand clear of the rest (gap >= 1) so T = 1e-3 is one-hot
    for arr in (ar.reshape(-1, V), dr.reshape(-1, V)):
        top = arr.argmax(axis=1)
        arr[np.arange(len(arr)), top] = arr.max(axis=1) + 1.0
    ql = np.zeros((B, k, V))
    ql[np.arange(B)[:, None], np.arange(k)[None, :], cand] = 100.0
    a_g, n_g = verify_ref(ar, dr, cand)
    a_s, n_s = vs.verify_sample_ref(ar, ql, dr, cand, 1e-3, seed=1, step=0)
    assert a_s.tolist() == a_g.tolist()
    assert n_s.tolist() == n_g.tolist()


def test_proposal_equal_to_target_keeps_every_candidate():
    rng = np.random.default_rng(2)
    B, k, V = 3, 5, 50
    ar = rng.normal(size=(B, k + 1, V))
    cand = rng.integers(0, V, size=(B, k)).astype(np.int32)
    a, _ = vs.verify_sample_ref(ar, ar[:, :k], rng.normal(size=(B, k, k, V)), cand, 0.7, seed=4, step=2)
    assert a.tolist() == [k] * B


# --- _residual_margin: the gap of a residual draw under the worst-case
# precision loss of p - q (the decision the sampling parity test may exempt)

def test_residual_margin_hand_value():
    """w = max(0, p - q) = (0.5, 0.25) with u = e^-1 (Gumbel noise 0 for both
    entries): the drawn entry 0 loses 1e-4 * (p0 + q0) = 1e-4, entry 1 gains
    1e-4 * (p1 + q1) = 2.5e-5, so the margin is ln(0.4999 / 0.250025)."""
    p = np.array([0.75, 0.25])
    q = np.array([0.25, 0.0])
    w = np.maximum(0.0, p - q)
    u = np.full(2, np.exp(-1.0))
    got = vs._residual_margin(w, p, q, u, 0)
    assert abs(got - math.log(0.4999 / 0.250025)) < 1e-12


def test_residual_margin_is_worst_case_brute_force():
    """Positive exactly when the drawn entry stays the Gumbel argmax after
    every weight moves by up to eps*(p+q) against it; never above the plain
    gap; and random perturbations inside that box never change a draw the
    margin calls safe."""
    rng = np.random.default_rng(3)
    eps = vs.RESIDUAL_EPS
    for trial in range(300):
        V = int(rng.integers(2, 7))
        p = rng.dirichlet(np.ones(V))
        q = p + rng.normal(0, 10 ** rng.uniform(-6, -1), V)  # near-cancelling at times
        q = np.abs(q) / np.abs(q).sum()
        w = np.maximum(0.0, p - q)
        if not w.sum() > 0:
            continue
        u = rng.uniform(0.01, 0.99, V)
        G = -np.log(-np.log(u))
        with np.errstate(divide="ignore"):
            first = int(np.argmax(np.log(w) + G))
        m = vs._residual_margin(w, p, q, u, first)
        # worst case written out entry by entry
        wc = w + eps * (p + q)
        wc[first] = w[first] - eps * (p[first] + q[first])
        if wc[first] > 0:
            with np.errstate(divide="ignore"):
                s = np.log(wc) + G
            survives = all(s[first] > s[v] for v in range(V) if v != first)
        else:
            survives = False
        assert (m > 0) == survives, (trial, m, survives)
        _, _, plain = vs.gumbel_top2(w, u)
        assert m <= plain + 1e-12
        if m > 0:
            for _ in range(20):
                wp = np.maximum(w + rng.uniform(-1, 1, V) * eps * (p + q), 0.0)
                with np.errstate(divide="ignore"):
                    assert int(np.argmax(np.log(wp) + G)) == first


def test_residual_margin_without_slack_is_the_plain_gap(monkeypatch):
    rng = np.random.default_rng(4)
    monkeypatch.setattr(vs, "RESIDUAL_EPS", 0.0)
    for _ in range(50):
        V = 9
        p = rng.dirichlet(np.ones(V))
        q = rng.dirichlet(np.ones(V))
        w = np.maximum(0.0, p - q)
        if not w.sum() > 0:
            continue
        u = rng.uniform(0.01, 0.99, V)
        first, _, gap = vs.gumbel_top2(w, u)
        assert abs(vs._residual_margin(w, p, q, u, first) - gap) < 1e-12
