"""Stochastic verification (temperature > 0) of the carried candidates and
sampling of the next drafts.  TEST INFRASTRUCTURE ONLY (see oracle/__init__).

The pages state that TiDAR's final tokens are sampled autoregressively and
that the result is mathematically the same as sampling the AR model alone
("TiDAR：Nvidia 的擴散＋自回歸混合架構", engineer-news.pages.dev, section on
what TiDAR does, "Talk in Autoregression"), and that accepted text is
rescored under the strict distribution ("TiDAR : l'hybride de NVIDIA qui
rédige par diffusion et parle de manière autorégressive", nodesdaily.com,
paragraph on the reported numbers).  They give no rule; the reading taken is
the standard speculative-sampling rule, which has exactly that property:

* p_i = softmax(ar_logits[b][i] / T) is the target at candidate i's
  position, q_i = softmax(q_logits[b][i] / T) the distribution candidate i
  was drawn from (for candidate 0 the carried AR row, so it is always kept).
* Candidates are tested left to right: candidate i (token x) is kept when
  u_i * q_i(x) < p_i(x), i.e. with probability min(1, p_i(x) / q_i(x)).
* At the first rejection a = i the next token is drawn from the residual
  max(0, p_a - q_a) (normalised); if all k are kept (a = k) it is drawn
  from p_k.  That token is next_cand[b][0].
* g = max(a, 1) - 1 as in the greedy rule; next_cand[b][m] for m >= 1 is
  drawn from softmax(draft_logits[b][g][m] / T).

Randomness (passed as a seed and a step number, so both sides draw the same
numbers): Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011), key = (seed low, seed high 32 bits),
counter = (c0, purpose, b, step).  A 32-bit output x gives the uniform
u = ((x >> 9) + 0.5) * 2^-23 in (0, 1): 23 random bits, so that every u is
exactly representable in fp32 (with 24 bits and the half offset, the upper
half of the grid falls between fp32 values and its top rounds to 1.0).
* accept test of candidate i: counter (i, 0xFFFFFFFF, b, step), word 0;
* draw for row j (0 = next_cand[0], m = next_cand[m]): Gumbel-max,
  argmax_v (log w_v + G_v) with G_v = -log(-log u_v) and u_v from counter
  (v // 4, j, b, step), word v % 4.  (Gumbel-max draws index v with
  probability w_v / sum(w), for any nonnegative weights w.)

Everything is float64 here; the GPU computes the same quantities in fp32,
so a decision may differ only where the two compared values are within
rounding of each other.  With margins=True the oracle reports, for each
decision, how far it is from flipping: the keep test's |u q - p| /
max(u q, p) and a draw's gap between the best and runner-up Gumbel scores
(a relative change e of the weights moves a score by at most e); for the
residual draw, the gap left after a worst-case move of 1e-4 (p + q) of
every weight.

Pins (tests/test_oracle_verify_sample.py): the published Philox4x32-10
known-answer vectors; the first emitted token is distributed as p (the
defining property of the rule, by Monte Carlo with a chi-square bound); the
Gumbel-max draw is distributed as softmax (the same way); the kept fraction
is sum_x min(p(x), q(x)); and the limit of a low temperature with one-hot
proposals reproduces the greedy oracle.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
ACCEPT_PURPOSE = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.  ctr: uint32 array [..., 4]; key: 2 ints.
    Each round multiplies words 0 and 2 by the two multipliers, swaps the
    halves into the next counter with the key xored into the high parts,
    and the key is bumped by the two Weyl constants between rounds."""
    c = np.array(ctr, dtype=np.uint64) & 0xFFFFFFFF
    k0, k1 = np.uint64(key[0] & 0xFFFFFFFF), np.uint64(key[1] & 0xFFFFFFFF)
    mask = np.uint64(0xFFFFFFFF)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(PHILOX_W1)) & mask
        p0 = np.uint64(PHILOX_M0) * c[..., 0]
        p1 = np.uint64(PHILOX_M1) * c[..., 2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & mask
        hi1, lo1 = p1 >> np.uint64(32), p1 & mask
        c = np.stack([hi1 ^ c[..., 1] ^ k0, lo1, hi0 ^ c[..., 3] ^ k1, lo0], axis=-1)
    return c.astype(np.uint32)


def _key(seed):
    return (int(seed) & 0xFFFFFFFF, (int(seed) >> 32) & 0xFFFFFFFF)


def to_uniform(x):
    """uint32 -> uniform in (0, 1) from the top 23 bits (exact in fp32)."""
    return ((np.asarray(x, dtype=np.uint64) >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def accept_uniform(seed, step, b, i):
    out = philox4x32_10([i, ACCEPT_PURPOSE, b, step], _key(seed))
    return float(to_uniform(out[0]))


def row_uniforms(seed, step, b, j, V):
    """Uniforms u_v, v = 0..V-1, of draw row j of sequence b."""
    n = (V + 3) // 4
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n)
    ctr[:, 1] = j
    ctr[:, 2] = b
    ctr[:, 3] = step
    out = philox4x32_10(ctr, _key(seed)).reshape(-1)[:V]
    return to_uniform(out)


def softmax(logits, T):
    z = np.asarray(logits, dtype=np.float64) / T
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def gumbel_top2(weights, u):
    """Gumbel-max scores argmax_v (log w_v + G(u_v)); zero weights never win.
    Returns (best index, runner-up index, gap between their scores)."""
    with np.errstate(divide="ignore"):
        score = np.log(np.asarray(weights, dtype=np.float64)) - np.log(-np.log(u))
    order = np.argsort(-score, kind="stable")
    if len(score) == 1:
        return int(order[0]), int(order[0]), np.inf
    return int(order[0]), int(order[1]), float(score[order[0]] - score[order[1]])


def gumbel_draw(weights, u):
    """(index drawn with probability w / sum(w), gap to the runner-up score)."""
    first, _, gap = gumbel_top2(weights, u)
    return first, gap


RESIDUAL_EPS = 1e-4


def _residual_margin(w, p, q, u, first):
    """Score gap of a residual draw that survives moving every weight w_v by
    RESIDUAL_EPS * (p_v + q_v) against the drawn entry (p - q loses relative
    precision where p and q nearly cancel); <= 0 when it does not survive."""
    G = -np.log(-np.log(u))
    slack = RESIDUAL_EPS * (p + q)
    lo = w[first] - slack[first]
    if not lo > 0:
        return 0.0
    with np.errstate(divide="ignore"):
        hi = np.log(w + slack) + G
    hi[first] = -np.inf
    return float(np.log(lo) + G[first] - hi.max())


def verify_sample_ref(ar_logits, q_logits, draft_logits, cand, T, seed, step, margins=False):
    """Returns (accept_len [B], next_cand [B][k]) and, with margins=True, a
    list per sequence of the relative margins of its decisions."""
    ar_logits = np.asarray(ar_logits)
    q_logits = np.asarray(q_logits)
    draft_logits = np.asarray(draft_logits) if draft_logits is not None else None
    cand = np.asarray(cand)
    B, k = cand.shape
    V = ar_logits.shape[2]
    accept = np.zeros(B, dtype=np.int32)
    nxt = np.zeros((B, k), dtype=np.int32)
    all_margins = []
    for b in range(B):
        mg = []
        a = k
        for i in range(k):
            p = softmax(ar_logits[b, i], T)
            q = softmax(q_logits[b, i], T)
            x = int(cand[b, i])
            u = accept_uniform(seed, step, b, i)
            lhs, rhs = u * q[x], p[x]
            # p(x) == 0 (a -inf logit) rejects exactly in any precision
            mg.append(np.inf if rhs == 0 else abs(lhs - rhs) / max(lhs, rhs))
            if not lhs < rhs:
                a = i
                break
        accept[b] = a
        u0 = row_uniforms(seed, step, b, 0, V)
        if a < k:
            p = softmax(ar_logits[b, a], T)
            q = softmax(q_logits[b, a], T)
            w = np.maximum(0.0, p - q)
            if not w.sum() > 0:  # p == q: every draw would have been kept
                nxt[b, 0], gap = gumbel_draw(p, u0)
            else:
                nxt[b, 0], _ = gumbel_draw(w, u0)
                gap = _residual_margin(w, p, q, u0, nxt[b, 0])
        else:
            nxt[b, 0], gap = gumbel_draw(softmax(ar_logits[b, k], T), u0)
        mg.append(gap)
        g = max(a, 1) - 1
        for m in range(1, k):
            w = softmax(draft_logits[b, g, m], T)
            nxt[b, m], gap = gumbel_draw(w, row_uniforms(seed, step, b, m, V))
            mg.append(gap)
        all_margins.append(mg)
    if margins:
        return accept, nxt, all_margins
    return accept, nxt
