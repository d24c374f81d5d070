"""Step attention of one TiDAR decode step, written as its dense definition.

What the pages fix ("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et
parle de manière autorégressive", nodesdaily.com):

* paragraph on the three zones: each step splits the sequence into the
  settled prefix (its keys/values are cached and reused), the candidates
  carried over from the previous step, and blank slots reserved for the next
  round of guesses;
* paragraph on drafting for every outcome: in the same pass that scores the
  carried candidates strictly left to right, fresh guesses are prepared for
  every possible verification outcome (only the first candidate survives, two
  survive, ..., all survive);
* paragraph on masking: settled tokens keep strictly causal visibility, each
  block of guesses sees all of itself and the whole settled past.

"TiDAR: Think in Diffusion, Talk in Autoregression" (mauroscia.it), section
"2. Single Forward Pass & Structured Attention Mask", names the same three
sections (prefix causal, previously drafted tokens under verification,
pre-drafted tokens with bidirectional attention).

Readings of what the pages leave open (slot layout and positions):

* the step block holds R = k + n_groups*k query rows, n_groups in {0, k};
* rows 0..k-1 are candidates; candidate i sits at position L+i;
* row k + g*k + s is slot s of group g, the group for the outcome "candidates
  0..g survive"; it sits at position L+g+1+s;
* candidate i sees the prefix and candidates 0..i;
* slot (g, s) sees the prefix, candidates 0..g and all k slots of group g.

Parity: candidate rows are pinned against textbook causal attention
(library routine) and a brute-force full-sequence pass; slot rows against
library attention over the reduced sequence [prefix, accepted candidates,
own group] and hand-written masks in tests/golden.
"""
from __future__ import annotations

import numpy as np


def step_mask_ref(k: int, n_groups: int, L: int) -> np.ndarray:
    """Explicit visibility matrix M[r, c] of the step block, R x (L + R).

    Key column c < L is settled prefix position c; column L + j is step row j.
    Built by enumerating each row's visible set (three-zone paragraph and the
    masking paragraph of the nodesdaily.com page), not by a closed formula."""
    assert n_groups in (0, k)
    R = k + n_groups * k
    M = np.zeros((R, L + R), dtype=bool)
    M[:, :L] = True  # every row sees the whole settled past
    for i in range(k):  # candidate i: strictly causal among candidates
        visible = {L + j for j in range(i + 1)}
        for c in visible:
            M[i, c] = True
    for g in range(n_groups):  # group g: outcome "candidates 0..g survive"
        own_group = {L + k + g * k + s2 for s2 in range(k)}
        accepted = {L + j for j in range(g + 1)}
        for s in range(k):
            r = k + g * k + s
            for c in accepted | own_group:
                M[r, c] = True
    return M


def _gather_kv(k_step, v_step, k_cache, v_cache, b, kv, L):
    """Concatenated [prefix ; step] keys and values (float64), (L+R) x D.
    v_cache holds pages of 64 positions, each stored transposed:
    value of position p = v_cache[b, kv, p // 64, :, p % 64]."""
    K = np.concatenate([np.asarray(k_cache[b, kv, :L, :], dtype=np.float64),
                        np.asarray(k_step[b, :, kv, :], dtype=np.float64)], axis=0)
    pages = np.asarray(v_cache[b, kv], dtype=np.float64)          # [S/64][D][64]
    prefix_v = pages.transpose(0, 2, 1).reshape(-1, pages.shape[1])[:L]
    V = np.concatenate([prefix_v, np.asarray(v_step[b, :, kv, :], dtype=np.float64)], axis=0)
    return K, V


def _pairs(B, Hq, pairs):
    if pairs is None:
        return [(b, h) for b in range(B) for h in range(Hq)]
    return [(int(b), int(h)) for b, h in pairs]


def attention_ref(q, k_step, v_step, k_cache, v_cache, lens, k, n_groups, sm_scale, pairs=None):
    """Dense masked softmax attention of the step block, float64.

    q [B][R][Hq][D]; k_step/v_step [B][R][Hkv][D]; k_cache [B][Hkv][S][D];
    v_cache [B][Hkv][S/64][D][64] (pages of 64 positions, transposed); lens [B].  Query head h reads KV head h // (Hq/Hkv).
    Returns out [B][R][Hq][D] and lse [B][Hq][R] (natural log of the softmax
    denominator of sm_scale*q.k over visible keys).  With ``pairs`` (a list of
    (b, h)), only those heads are computed; other entries are NaN."""
    q = np.asarray(q)
    B, R, Hq, D = q.shape
    Hkv = k_step.shape[2]
    G = Hq // Hkv
    assert R == k + n_groups * k
    out = np.full((B, R, Hq, D), np.nan)
    lse = np.full((B, Hq, R), np.nan)
    masks = {}
    for b, h in _pairs(B, Hq, pairs):
        L = int(lens[b])
        if L not in masks:
            masks[L] = step_mask_ref(k, n_groups, L)
        M = masks[L]
        K, V = _gather_kv(k_step, v_step, k_cache, v_cache, b, h // G, L)
        S = sm_scale * (np.asarray(q[b, :, h, :], dtype=np.float64) @ K.T)
        S = np.where(M, S, -np.inf)
        mx = S.max(axis=1, keepdims=True)
        P = np.exp(S - mx)
        den = P.sum(axis=1, keepdims=True)
        out[b, :, h, :] = (P / den) @ V
        lse[b, h, :] = mx[:, 0] + np.log(den[:, 0])
    return out, lse


def attention_split_ref(q, k_step, v_step, k_cache, v_cache, lens, k, n_groups, sm_scale, chunk,
                        pairs=None):
    """The same attention computed over key chunks of ``chunk`` columns of the
    [prefix ; step] sequence, each chunk with its own running max m_s, sum l_s
    and unnormalised output O_s, then merged:
    M = max_s m_s,  O = sum_s e^(m_s-M) O_s / sum_s e^(m_s-M) l_s,
    lse = M + ln sum_s e^(m_s-M) l_s.  A chunk with no visible key contributes
    nothing (m_s = -inf, l_s = 0)."""
    q = np.asarray(q)
    B, R, Hq, D = q.shape
    Hkv = k_step.shape[2]
    G = Hq // Hkv
    out = np.full((B, R, Hq, D), np.nan)
    lse = np.full((B, Hq, R), np.nan)
    for b, h in _pairs(B, Hq, pairs):
        L = int(lens[b])
        M = step_mask_ref(k, n_groups, L)
        K, V = _gather_kv(k_step, v_step, k_cache, v_cache, b, h // G, L)
        S = sm_scale * (np.asarray(q[b, :, h, :], dtype=np.float64) @ K.T)
        S = np.where(M, S, -np.inf)
        parts = []
        for c0 in range(0, L + R, chunk):
            Sc = S[:, c0:c0 + chunk]
            m = Sc.max(axis=1)
            ok = np.isfinite(m)
            P = np.where(ok[:, None], np.exp(Sc - np.where(ok, m, 0.0)[:, None]), 0.0)
            parts.append((np.where(ok, m, -np.inf), P.sum(axis=1), P @ V[c0:c0 + chunk]))
        Mx = np.max([p[0] for p in parts], axis=0)
        num = np.zeros((R, D))
        den = np.zeros(R)
        for m, l, O in parts:
            w = np.where(np.isfinite(m), np.exp(m - Mx), 0.0)
            num += w[:, None] * O
            den += w * l
        out[b, :, h, :] = num / den[:, None]
        lse[b, h, :] = Mx + np.log(den)
    return out, lse


def causal_attention_ref(q, k, v, sm_scale):
    """Plain causal softmax attention over one full sequence, float64.
    q, k, v: [T][H][D].  Row t sees positions 0..t (the triangular mask of
    ordinary next-token training, engineer-news.pages.dev, section on the
    causal-mask training trick)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, D = q.shape
    tri = np.tril(np.ones((T, T), dtype=bool))
    out = np.empty_like(q)
    for h in range(H):
        S = sm_scale * (q[:, h, :] @ k[:, h, :].T)
        S = np.where(tri, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        out[:, h, :] = (P / P.sum(axis=1, keepdims=True)) @ v[:, h, :]
    return out
