"""Greedy verification of the carried candidates and selection of the next drafts.

"TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
autorégressive" (nodesdaily.com), paragraph on drafting for every outcome:
the carried candidates are scored strictly left to right, and whichever
outcome verification confirms, the guess prepared for that outcome is taken
as the next drafts.  The paragraph on the reported numbers (and the
engineer-news.pages.dev section on what TiDAR does) state that accepted text
is rescored under the strict AR distribution, so the output equals AR
sampling; greedy decoding is the deterministic case of that.

Readings of what the pages leave open:

* ar_logits[b][0] is the AR distribution at candidate 0's position (carried
  from the previous pass); ar_logits[b][i] for i >= 1 is the output of
  candidate row i-1 (the distribution at candidate i's position); row k
  follows the last candidate.
* t_i = argmax ar_logits[b][i] (lowest index wins ties, -0.0 ties +0.0).
  accept_len a = the largest j <= k with cand[b][i] == t_i for all i < j.
* next_cand[b][0] = t_a (the exact AR token after the accepted prefix).
* group g = max(a, 1) - 1 (group g stands for "candidates 0..g survive";
  there is no group for a = 0, which a real loop never produces because
  candidate 0 is always the exact AR token).
* next_cand[b][m] = argmax draft_logits[b][g][m] for m = 1..k-1; slot 0 of
  the group sits at the same position as t_a and is superseded by it.

Pins: planted accept lengths (exact answer by construction), hand-written
cases in tests/golden (ties, a = 0, a = k), and argmax_first against a plain
scan.
"""
from __future__ import annotations

import numpy as np


def argmax_first(row) -> int:
    """Index of the largest value; the lowest index wins ties.  Inputs must be
    finite (NaN behaviour is left unspecified)."""
    row = np.asarray(row)
    assert np.all(np.isfinite(row)), "logits must be finite"
    return int(np.argmax(row))  # numpy returns the first occurrence of the max


def verify_ref(ar_logits, draft_logits, cand):
    """Returns (accept_len [B] int32, next_cand [B][k] int32)."""
    ar_logits = np.asarray(ar_logits)
    cand = np.asarray(cand)
    B, k = cand.shape
    assert ar_logits.shape[:2] == (B, k + 1)
    accept = np.zeros(B, dtype=np.int32)
    nxt = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        t = [argmax_first(ar_logits[b, i]) for i in range(k + 1)]
        a = 0
        while a < k and int(cand[b, a]) == t[a]:
            a += 1
        accept[b] = a
        nxt[b, 0] = t[a]
        g = max(a, 1) - 1
        for m in range(1, k):
            nxt[b, m] = argmax_first(draft_logits[b, g, m])
    return accept, nxt
