"""KV-cache commit / evict after verification.

"TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
autorégressive" (nodesdaily.com), paragraph on the three zones: the settled
cache is reused and rejected entries are evicted.  "TiDAR: Think in
Diffusion, Talk in Autoregression" (mauroscia.it), section "KV Cache", and
the abstract on fugumt.com: the method keeps an exact KV cache.

Reading: the step block's keys/values live in their own buffers; committing
appends the rows of the a accepted candidates (step rows 0..a-1) at settled
positions lens[b]..lens[b]+a-1 and advances lens[b] by a.  Rejected
candidates and every slot row are evicted by never being written.  A
sequence whose cache would overflow (lens + a > S_max) or whose a lies
outside 0..k is left untouched and flagged (1 = overflow, 2 = bad length).

Pins: brute-force concatenation and len_final = len_0 + sum(a) in tests.
"""
from __future__ import annotations

import numpy as np


def commit_ref(k_cache, v_cache, lens, k_step, v_step, accept_len, k):
    """k_cache [B][Hkv][S][D], v_cache [B][Hkv][S/64][D][64] (pages of 64
    positions, each stored transposed),
    k_step/v_step [B][R][Hkv][D], lens/accept_len [B].  Works on any element
    type (it is a copy).  Returns new (k_cache, v_cache, lens, err_flags)."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ln = np.array(lens, dtype=np.int32, copy=True)
    err = np.zeros(len(ln), dtype=np.int32)
    S = kc.shape[2]
    for b in range(len(ln)):
        a = int(accept_len[b])
        L = int(ln[b])
        if a < 0 or a > k:
            err[b] = 2
            continue
        if L + a > S:
            err[b] = 1
            continue
        for i in range(a):
            pos = L + i
            kc[b, :, pos, :] = k_step[b, i, :, :]
            vc[b, :, pos // 64, :, pos % 64] = v_step[b, i, :, :]
        ln[b] = L + a
    return kc, vc, ln, err
