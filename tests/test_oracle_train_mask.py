"""Pins of the training-mask oracle: hand-typed masks, library attention on
the causal half and on each block, the one-block special case, and
permutation within a block."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.train_mask import train_attention_ref, train_mask_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = [l.split() for l in open(os.path.join(GOLDEN, name)) if l.strip() and not l.startswith("#")]
    return np.array(rows, dtype=int).astype(bool)


@pytest.mark.parametrize("N,bs,name", [(4, 2, "train_mask_n4_b2.txt"), (5, 2, "train_mask_n5_b2.txt")])
def test_mask_matches_hand_typed(N, bs, name):
    assert np.array_equal(train_mask_ref(N, bs), _golden(name))


def _inputs(B, T, Hq, Hkv, D, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, T, Hq, D)), g.standard_normal((B, T, Hkv, D)), g.standard_normal((B, T, Hkv, D)))


def _sdpa(q, k, v, scale, causal=False):
    """Library attention over one head: q [Tq][D], k/v [Tk][D], float64."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("N,bs,G", [(16, 4, 2), (13, 5, 1), (24, 8, 3)])
def test_clean_half_is_causal_attention_and_ignores_the_masked_copy(N, bs, G):
    q, k, v = _inputs(1, 2 * N, 2 * G, 2, 8, seed=N)
    out, _ = train_attention_ref(q, k, v, N, bs, 0.3)
    for h in range(2 * G):
        ref = _sdpa(q[0, :N, h], k[0, :N, h // G], v[0, :N, h // G], 0.3, causal=True)
        np.testing.assert_allclose(out[0, :N, h], ref, rtol=0, atol=1e-12)
    k2, v2 = k.copy(), v.copy()
    k2[:, N:] += 5.0
    v2[:, N:] -= 3.0
    out2, _ = train_attention_ref(q, k2, v2, N, bs, 0.3)
    assert np.array_equal(out2[:, :N], out[:, :N])


@pytest.mark.parametrize("N,bs", [(16, 4), (13, 5), (10, 10)])
def test_each_block_is_plain_attention_over_prefix_and_itself(N, bs):
    q, k, v = _inputs(2, 2 * N, 3, 3, 8, seed=bs)
    out, lse = train_attention_ref(q, k, v, N, bs, 0.25)
    for b in range(2):
        for h in range(3):
            for lo in range(0, N, bs):
                hi = min(lo + bs, N)
                cols = list(range(lo)) + list(range(N + lo, N + hi))
                ref = _sdpa(q[b, N + lo:N + hi, h], k[b, cols, h], v[b, cols, h], 0.25)
                np.testing.assert_allclose(out[b, N + lo:N + hi, h], ref, rtol=0, atol=1e-12)
                s = 0.25 * q[b, N + lo:N + hi, h] @ k[b, cols, h].T
                ref_lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
                np.testing.assert_allclose(lse[b, h, N + lo:N + hi], ref_lse, rtol=0, atol=1e-12)


def test_one_block_is_bidirectional_attention_over_the_masked_copy():
    N = 12
    q, k, v = _inputs(1, 2 * N, 2, 2, 8, seed=3)
    out, _ = train_attention_ref(q, k, v, N, N, 0.5)
    for h in range(2):
        ref = _sdpa(q[0, N:, h], k[0, N:, h], v[0, N:, h], 0.5)
        np.testing.assert_allclose(out[0, N:, h], ref, rtol=0, atol=1e-12)


def test_permuting_inside_a_block_permutes_its_outputs():
    N, bs = 12, 4
    q, k, v = _inputs(1, 2 * N, 2, 2, 8, seed=5)
    out, _ = train_attention_ref(q, k, v, N, bs, 0.5)
    perm = np.arange(2 * N)
    perm[N + 4:N + 8] = N + np.array([6, 4, 7, 5])  # block 1 of the masked copy
    out_p, _ = train_attention_ref(q[:, perm], k[:, perm], v[:, perm], N, bs, 0.5)
    np.testing.assert_allclose(out_p, out[:, perm], rtol=0, atol=1e-12)


def test_sampled_rows_equal_the_dense_result():
    N, bs = 10, 3
    q, k, v = _inputs(2, 2 * N, 4, 2, 8, seed=9)
    out, lse = train_attention_ref(q, k, v, N, bs, 0.4)
    rows = [(0, 0, 0), (1, 3, 9), (0, 2, 10), (1, 1, 19), (0, 3, 15)]
    o2, l2 = train_attention_ref(q, k, v, N, bs, 0.4, rows=rows)
    for b, h, r in rows:
        np.testing.assert_allclose(o2[b, r, h], out[b, r, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2[b, h, r], lse[b, h, r], rtol=0, atol=1e-12)
