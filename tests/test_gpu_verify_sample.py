"""GPU parity of tidar_verify_sample (stochastic verification at T > 0)
against the oracle on the same seeded inputs and the same Philox stream.

Accept lengths and every drawn token must be identical.  The oracle decides
in float64, the kernels in float32, so a decision whose oracle margin is
below MARGIN (a relative 1e-4, two orders above fp32 rounding at these
sizes) may legitimately go either way: such a sequence is compared up to
that decision only, and those must stay rare."""
import numpy as np
import pytest

import workloads as W
from oracle.verify_sample import verify_sample_ref

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import to_dev  # noqa: E402

MARGIN = 1e-4


def _run(d, T, seed, step):
    a, n = tidar.verify_sample(to_dev(d["ar_logits"]), to_dev(d["q_logits"]),
                               None if d["draft_logits"] is None else to_dev(d["draft_logits"]),
                               to_dev(d["cand"]), T, seed, step)
    return a.cpu().numpy(), n.cpu().numpy()


def _compare(d, T, seed, step, what):
    """Compare with the oracle; returns the number of sequences that held a
    decision within MARGIN of its threshold."""
    a, n = _run(d, T, seed, step)
    ra, rn, mg = verify_sample_ref(d["ar_logits"], d["q_logits"], d["draft_logits"], d["cand"], T, seed, step,
                                   margins=True)
    k = d["cand"].shape[1]
    near = 0
    for b in range(len(ra)):
        m = mg[b]
        n_tests = len(m) - k  # keep tests taken: a+1, or k when all were kept
        first_near = next((i for i, x in enumerate(m) if x < MARGIN), None)
        if first_near is None:
            assert a[b] == ra[b], f"{what} b={b}: accept {a[b]} != {ra[b]}"
            assert n[b].tolist() == rn[b].tolist(), f"{what} b={b}: next {n[b].tolist()} != {rn[b].tolist()}"
            continue
        near += 1
        if first_near < n_tests:  # a keep test near its threshold: only the tests before it are fixed
            assert a[b] >= first_near, f"{what} b={b}: accept {a[b]} below the first close test {first_near}"
        else:  # the accept length is fixed, and so is every draw that is not close
            assert a[b] == ra[b], f"{what} b={b}: accept {a[b]} != {ra[b]}"
            far = [j for j in range(k) if m[n_tests + j] >= MARGIN]
            assert n[b, far].tolist() == rn[b, far].tolist(), f"{what} b={b}: draws {far}"
        assert 0 <= n[b].min() and n[b].max() < d["ar_logits"].shape[2], f"{what} b={b}: token out of range"
    return near


@pytest.mark.parametrize("B,k,V,T,kw", [
    (16, 8, 128256, 1.0, {}),                       # 8B-shaped step
    (8, 4, 151936, 0.7, {}),                        # 1.5B-shaped step
    (4, 16, 128256, 1.3, {"shift": (-1.0, 3.0)}),   # long-context step, deeper accepts
    (32, 8, 128256, 1.0, {"shift": (0.0, 4.0)}),    # mostly kept: bonus rows from p_k
    (5, 1, 1001, 0.9, {}),                          # no drafts, V not a multiple of 4
    (3, 3, 4097, 1.0, {}),                          # one entry past a chunk boundary
    (9, 5, 64, 1.0, {"carried": False}),            # tiny vocab, candidate 0 may be rejected
    (12, 4, 5003, 1.0, {"masked": 0.5}),            # filtered vocabulary (-inf logits)
    (12, 4, 5000, 1.0, {"masked": 0.9, "carried": False}),
    (6, 6, 32000, 0.05, {}),                        # near-greedy temperature
    (6, 6, 32000, 20.0, {}),                        # near-uniform temperature
])
def test_verify_sample_matches_oracle(B, k, V, T, kw):
    d = W.sample_inputs(B, k, V, seed=1000 + B * 17 + k, **kw)
    near = 0
    for seed, step in ((12345, 0), (2 ** 40 + 7, 3)):
        near += _compare(d, T, seed, step, f"B={B} k={k} V={V} T={T} {kw} seed={seed} step={step}")
    assert near <= max(1, B // 8), f"{near} sequences with a decision within {MARGIN}"


def test_zero_probability_candidate_takes_the_fallback_draw():
    # the carried candidate's logit is -inf: p(x) = q(x) = 0, it is rejected
    # and p_0 - q_0 is zero everywhere, so next_cand[0] is drawn from p_0
    d = W.sample_inputs(4, 3, 3000, seed=5)
    for b in range(4):
        d["ar_logits"][b, 0, d["cand"][b, 0]] = -np.inf
    d["q_logits"][:, 0] = d["ar_logits"][:, 0]
    a, n = _run(d, 1.0, 9, 1)
    ra, rn = verify_sample_ref(d["ar_logits"], d["q_logits"], d["draft_logits"], d["cand"], 1.0, 9, 1)
    assert a.tolist() == [0] * 4 == ra.tolist()
    assert n.tolist() == rn.tolist()


def test_same_seed_and_step_repeat_and_others_differ():
    d = W.sample_inputs(16, 8, 20000, seed=3)
    a0, n0 = _run(d, 1.0, 77, 5)
    a1, n1 = _run(d, 1.0, 77, 5)
    assert a0.tolist() == a1.tolist() and n0.tolist() == n1.tolist()
    _, n2 = _run(d, 1.0, 77, 6)
    _, n3 = _run(d, 1.0, 78, 5)
    assert (n2 != n0).mean() > 0.5 and (n3 != n0).mean() > 0.5


CHI2_15_9999 = 44.26  # chi-square 99.99% point, 15 degrees of freedom


def test_emitted_token_follows_the_ar_distribution():
    # B independent trials of one step (the Philox counter holds b): the token
    # emitted after candidate 0 is cand[1] when kept, else the residual draw;
    # together they must be distributed as p_1 = softmax(ar[1] / T).  The
    # kept fraction must be sum_v min(p_1, q_1)
    B, k, V, T = 16000, 2, 16, 1.0
    rng = np.random.default_rng(4)
    ar1 = rng.standard_normal((k + 1, V)).astype(np.float32)
    q1 = rng.standard_normal((k, V)).astype(np.float32)
    q1[0] = ar1[0]
    ar = np.ascontiguousarray(np.broadcast_to(ar1, (B, k + 1, V)))
    q = np.ascontiguousarray(np.broadcast_to(q1, (B, k, V)))
    dr = rng.standard_normal((B, k, k, V)).astype(np.float32)
    # the rule's premise: candidate 1 is a draw from q_1 (candidate 0 is kept whatever it is)
    zq = q1[1].astype(np.float64) / T
    q_1 = np.exp(zq - zq.max())
    cand = np.stack([np.full(B, 3), rng.choice(V, size=B, p=q_1 / q_1.sum())], axis=1).astype(np.int32)
    a, n = _run({"ar_logits": ar, "q_logits": q, "draft_logits": dr, "cand": cand}, T, 2024, 0)
    assert (a >= 1).all()  # candidate 0 was drawn from the carried row itself
    tok = np.where(a == 2, cand[:, 1], n[:, 0])
    z = ar1[1].astype(np.float64) / T
    p = np.exp(z - z.max())
    p /= p.sum()
    counts = np.bincount(tok, minlength=V)
    chi2 = float(((counts - B * p) ** 2 / (B * p)).sum())
    assert chi2 < CHI2_15_9999, (chi2, counts.tolist(), (B * p).round(1).tolist())
    kept = float(np.minimum(p, q_1 / q_1.sum()).sum())
    assert abs((a == 2).mean() - kept) < 4 * np.sqrt(kept * (1 - kept) / B)
