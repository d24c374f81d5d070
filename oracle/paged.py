"""Paged (block-table) KV cache: step attention and commit over shared page
pools.  TEST INFRASTRUCTURE ONLY (see oracle/__init__).

The abstract on the fugumt.com page ("論文の概要: TiDAR: Think in Diffusion,
Talk in Autoregression") calls the design serving-friendly as a standalone
model with exact KV-cache support, and the "KV Cache" section of the
mauroscia.it page says the cache is managed without wasting memory.  The
pages give no layout; the reading taken is the block table used by serving
systems:

* position p of sequence b lives in page ``table[b][p // 64]`` of the pools,
  at row ``p % 64``: key ``k_pool[page, h, p % 64, :]``, value
  ``v_pool[page, h, :, p % 64]`` (value pages stored transposed, as in the
  contiguous cache);
* attention over a paged cache is attention over the positions gathered by
  that rule; a sequence whose table names a page outside the pools for a
  settled position gets NaN outputs (the same contract as a violated length
  bound);
* commit writes accepted row i of sequence b to position lens[b] + i by the
  same rule and advances lens[b]; flags: 1 capacity (lens + a > 64 *
  max_pages), 2 a outside 0..k, 3 a page entry outside the pools for one of
  the positions written.  A flagged sequence is left untouched.

Pins (tests/test_oracle_paged.py): pools whose every element encodes its own
(page, head, row, column) show that the gather puts page table[b][p // 64],
row p % 64 at position p; with pages laid out in sequence order the paged
attention equals the contiguous oracle exactly; paged commit followed by the
gather equals the contiguous commit of the gathered cache, and pages outside
the written positions are untouched.
"""
from __future__ import annotations

import numpy as np

from .step_attention import attention_ref

PAGE = 64


def gather_paged(k_pool, v_pool, table, lens, S):
    """Per-sequence contiguous caches of capacity S (a multiple of 64) read
    position by position from the pools: k [B][Hkv][S][D], v [B][Hkv][S/64][D][64].
    Positions >= lens[b] are zero."""
    k_pool = np.asarray(k_pool)
    v_pool = np.asarray(v_pool)
    B = len(lens)
    _, Hkv, _, D = k_pool.shape
    kc = np.zeros((B, Hkv, S, D), dtype=k_pool.dtype)
    vc = np.zeros((B, Hkv, S // PAGE, D, PAGE), dtype=v_pool.dtype)
    for b in range(B):
        for p in range(int(lens[b])):
            page = int(table[b][p // PAGE])
            row = p % PAGE
            kc[b, :, p, :] = k_pool[page, :, row, :]
            vc[b, :, p // PAGE, :, row] = v_pool[page, :, :, row]
    return kc, vc


def pages_valid(table, lens, n_pages):
    """Per sequence: every page holding a settled position lies in the pools."""
    ok = []
    for b in range(len(lens)):
        L = int(lens[b])
        ok.append(L >= 0 and all(0 <= int(table[b][t]) < n_pages for t in range((L + PAGE - 1) // PAGE)))
    return np.array(ok)


def paged_attention_ref(q, k_step, v_step, k_pool, v_pool, table, lens, k, n_groups, sm_scale, pairs=None):
    """attention_ref over the positions the block table names.  Sequences
    with an invalid page entry get NaN rows."""
    n_pages = np.asarray(k_pool).shape[0]
    valid = pages_valid(table, lens, n_pages)
    lens_ok = np.where(valid, np.asarray(lens), 0)
    S = max(PAGE, -(-int(max(lens_ok, default=0)) // PAGE) * PAGE)
    kc, vc = gather_paged(k_pool, v_pool, table, lens_ok, S)
    out, lse = attention_ref(q, k_step, v_step, kc, vc, lens_ok, k, n_groups, sm_scale, pairs)
    for b in np.nonzero(~valid)[0]:
        out[b] = np.nan
        lse[b] = np.nan
    return out, lse


def commit_paged_ref(k_pool, v_pool, table, lens, k_step, v_step, accept_len, k):
    """Returns new (k_pool, v_pool, lens, err_flags)."""
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    ln = np.array(lens, dtype=np.int32, copy=True)
    err = np.zeros(len(ln), dtype=np.int32)
    n_pages = kp.shape[0]
    max_pages = np.asarray(table).shape[1]
    for b in range(len(ln)):
        a = int(accept_len[b])
        L = int(ln[b])
        if a < 0 or a > k:
            err[b] = 2
            continue
        if L < 0 or L + a > max_pages * PAGE:
            err[b] = 1
            continue
        if any(not 0 <= int(table[b][(L + i) // PAGE]) < n_pages for i in range(a)):
            err[b] = 3
            continue
        for i in range(a):
            p = L + i
            page = int(table[b][p // PAGE])
            kp[page, :, p % PAGE, :] = k_step[b, i, :, :]
            vp[page, :, :, p % PAGE] = v_step[b, i, :, :]
        ln[b] = L + a
    return kp, vp, ln, err
