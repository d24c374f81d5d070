"""LM head fused with greedy verification.  TEST INFRASTRUCTURE ONLY (see
oracle/__init__).

"TiDAR: Think in Diffusion, Talk in Autoregression" (mauroscia.it), section
"2. Single Forward Pass & Structured Attention Mask": the one pass yields
the joint distribution used to verify and the marginals used to draft.
"TiDAR : l'hybride de NVIDIA ..." (nodesdaily.com), paragraphs on scoring
the whispered tokens strictly left to right and on drafting for every
outcome.  Both distributions are the LM head applied to the pass's final
hidden states; verification only needs each row's argmax, so the fused form
never keeps a row of logits.

Reading: logits = h . W^T with W [V][d] (one row per vocabulary entry); then
exactly the greedy rule of oracle.verify_ref: t_i = argmax of AR row i
(lowest index on ties), a = the longest prefix with cand[i] == t_i,
next[0] = t_a, g = max(a, 1) - 1, next[m] = argmax of draft row (g, m).
Only the selected group's draft rows are evaluated.

Pins (tests/test_oracle_lmhead.py): with W = I (V = d) the logits are the
hidden states and the result equals the greedy oracle on them; a head whose
rows are permuted unit vectors permutes the argmax accordingly; a positive
rescaling of W changes nothing; a hand-computed 3-token example.
"""
from __future__ import annotations

import numpy as np

from .verify import argmax_first


def _row_logits(h_row, w64):
    return w64 @ np.asarray(h_row, dtype=np.float64)


def _top2_gap(z):
    i = argmax_first(z)
    rest = np.delete(z, i)
    return float(z[i] - rest.max()) if rest.size else np.inf


def lmhead_verify_ref(h_ar, h_draft, w, cand, margins=False):
    """h_ar [B][k+1][d], h_draft [B][k][k][d] (None when k == 1), w [V][d],
    cand [B][k].  Returns (accept_len [B], next_cand [B][k]) and, with
    margins=True, per sequence the top-2 logit gap of every row it decided
    on (AR rows 0..a, then the k-1 draft rows)."""
    w64 = np.asarray(w, dtype=np.float64)
    h_ar = np.asarray(h_ar)
    cand = np.asarray(cand)
    B, k = cand.shape
    acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros((B, k), dtype=np.int32)
    all_mg = []
    for b in range(B):
        mg = []
        a = k
        t_a = None
        for i in range(k + 1):
            z = _row_logits(h_ar[b, i], w64)
            t = argmax_first(z)
            mg.append(_top2_gap(z))
            if i == k or int(cand[b, i]) != t:
                a, t_a = i, t
                break
        acc[b] = a
        nxt[b, 0] = t_a
        g = max(a, 1) - 1
        for m in range(1, k):
            z = _row_logits(h_draft[b, g, m], w64)
            nxt[b, m] = argmax_first(z)
            mg.append(_top2_gap(z))
        all_mg.append(mg)
    if margins:
        return acc, nxt, all_mg
    return acc, nxt
