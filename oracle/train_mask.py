"""Training-mask attention: the duplicated training sequence.  TEST
INFRASTRUCTURE ONLY (see oracle/__init__).

"TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
autorégressive" (nodesdaily.com), paragraph on training: every example is
laid out twice in one long sequence, once for ordinary next-token
supervision and once as a fully masked block to be filled in parallel, and
the two losses are added with equal weight.  "TiDAR: Think in Diffusion,
Talk in Autoregression" (mauroscia.it), section "3. Training Recipe": the
AR and diffusion losses come from the same data in the same pass, the
diffusion part being masked.  "TiDAR：Nvidia 的擴散＋自回歸混合架構"
(engineer-news.pages.dev), section recalling AR training: one forward pass
under a triangular mask yields a loss at every position.

The pages give no mask matrix.  Reading taken (the one that matches what a
draft group sees at decode time, where a group sees the prefix, the accepted
candidates and its own group):

* the sequence is [x_0 .. x_{N-1} ; m_0 .. m_{N-1}], T = 2N positions: the
  clean copy, then the masked copy (the caller fills it with the MASK
  embedding);
* clean row r < N sees clean keys c <= r (causal, next-token supervision);
* masked row N + j belongs to block b = j // bs, covering clean indices
  lo = b*bs .. hi = min(lo + bs, N) - 1; it sees the clean prefix c < lo and
  every masked key of its own block, N + lo <= c < N + hi (bidirectional
  inside the block, nothing of other blocks, nothing of the clean copy at or
  past lo).

Pins (tests/test_oracle_train_mask.py): a hand-typed 8 x 8 mask for N = 4,
bs = 2 (tests/golden/train_mask_n4_b2.txt); clean rows equal library causal
attention and ignore the masked copy; a block's rows equal unmasked library
attention over [clean prefix ; own block]; with bs = N the masked copy is
plain bidirectional attention over itself; permuting tokens inside a block
permutes its outputs.
"""
from __future__ import annotations

import numpy as np


def train_mask_ref(N: int, bs: int) -> np.ndarray:
    """Visibility matrix M[r, c] (T x T, T = 2N), built by enumerating each
    row's visible set."""
    T = 2 * N
    M = np.zeros((T, T), dtype=bool)
    for r in range(N):
        for c in range(r + 1):
            M[r, c] = True
    for j in range(N):
        lo = (j // bs) * bs
        hi = min(lo + bs, N)
        visible = set(range(lo)) | set(range(N + lo, N + hi))
        for c in visible:
            M[N + j, c] = True
    return M


def train_attention_ref(q, k, v, N, bs, sm_scale, rows=None):
    """Dense masked softmax attention over the training sequence, float64.

    q [B][T][Hq][D]; k [B][T][Hkv][D]; v [B][T][Hkv][D] (natural layout);
    query head h reads KV head h // (Hq/Hkv).  Returns out [B][T][Hq][D] and
    lse [B][Hq][T].  With ``rows`` (a list of (b, h, r)), only those rows
    are computed; everything else is NaN."""
    q = np.asarray(q)
    B, T, Hq, D = q.shape
    Hkv = np.asarray(k).shape[2]
    G = Hq // Hkv
    assert T == 2 * N
    M = train_mask_ref(N, bs)
    out = np.full((B, T, Hq, D), np.nan)
    lse = np.full((B, Hq, T), np.nan)
    if rows is None:
        for b in range(B):
            for h in range(Hq):
                K = np.asarray(k[b, :, h // G, :], dtype=np.float64)
                V = np.asarray(v[b, :, h // G, :], dtype=np.float64)
                S = sm_scale * (np.asarray(q[b, :, h, :], dtype=np.float64) @ K.T)
                S = np.where(M, S, -np.inf)
                mx = S.max(axis=1, keepdims=True)
                P = np.exp(S - mx)
                den = P.sum(axis=1, keepdims=True)
                out[b, :, h, :] = (P / den) @ V
                lse[b, h, :] = mx[:, 0] + np.log(den[:, 0])
        return out, lse
    for b, h, r in rows:
        vis = np.nonzero(M[r])[0]
        K = np.asarray(k[b, vis, h // G, :], dtype=np.float64)
        V = np.asarray(v[b, vis, h // G, :], dtype=np.float64)
        s = sm_scale * (K @ np.asarray(q[b, r, h, :], dtype=np.float64))
        mx = s.max()
        p = np.exp(s - mx)
        out[b, r, h, :] = (p / p.sum()) @ V
        lse[b, h, r] = mx + np.log(p.sum())
    return out, lse
