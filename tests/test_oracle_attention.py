"""Pins of the oracle's step attention against what the pages and mathematics fix.

* hand-typed masks (tests/golden/step_mask_*.txt) and hand-worked attention
  values (tests/golden/attention_worked_examples.json);
* zero drafts: textbook causal attention from a library routine
  (torch scaled_dot_product_attention in float64 on the CPU);
* candidate rows of a full step: causal rows of a brute-force full-sequence
  pass (library routine);
* slot rows of group g: unmasked library attention over the reduced
  sequence [prefix ; candidates 0..g ; own group];
* invariances (candidate rows ignore slots; groups ignore each other and
  later candidates; permutation within a group), closed forms, and the
  split-K merge equal to the unsplit result.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W


def _inputs(B, Hq, Hkv, D, k, n_groups, lens, seed=0, S_max=None, scale=None):
    S_max = S_max or ((max(lens) + 8 + 63) // 64 * 64)
    shape = W.AttnShape(B=B, Hq=Hq, Hkv=Hkv, D=D, k=k, n_groups=n_groups, lens=tuple(lens),
                        S_max=S_max, dtype="f32", sm_scale=scale or 1.0 / math.sqrt(D))
    d = W.attention_inputs(shape, seed=seed, tail="nan")
    d = {n: (np.asarray(a, dtype=np.float64) if n != "lens" else a) for n, a in d.items()}
    return shape, d


def _run(shape, d, **kw):
    return oracle.attention_ref(d["q"], d["k_step"], d["v_step"], d["k_cache"], d["v_cache"], d["lens"],
                                shape.k, shape.n_groups, shape.sm_scale, **kw)


def _read_mask(path):
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    return np.array([[c == "1" for c in r] for r in rows])


@pytest.mark.parametrize("fname,k,L", [("step_mask_k2_L3.txt", 2, 3), ("step_mask_k3_L0.txt", 3, 0)])
def test_mask_matches_hand_typed(golden_dir, fname, k, L):
    want = _read_mask(os.path.join(golden_dir, fname))
    got = oracle.step_mask_ref(k, k, L)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("k,L", [(1, 0), (4, 5), (8, 33)])
def test_mask_zero_groups_is_causal(k, L):
    # with no draft groups the step block is the last k rows of a triangular mask
    tri = np.tril(np.ones((L + k, L + k), dtype=bool))[L:]
    assert np.array_equal(oracle.step_mask_ref(k, 0, L), tri)


def test_mask_counts():
    # visible step-block entries: candidates k(k+1)/2; group g: k*(g+1) + k*k
    for k in (1, 2, 4, 8, 16):
        M = oracle.step_mask_ref(k, k, 0)
        want = k * (k + 1) // 2 + sum(k * (g + 1) + k * k for g in range(k))
        assert int(M.sum()) == want


def test_worked_examples(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "attention_worked_examples.json")))
    for case in doc["cases"]:
        D = case["D"]
        q = np.array(case["q"]).reshape(1, 2, 1, D)
        ks = np.array(case["k_step"]).reshape(1, 2, 1, D)
        vs = np.array(case["v_step"]).reshape(1, 2, 1, D)
        kc = np.zeros((1, 1, 64, D))
        kc[0, 0, 0] = case["k_prefix"][0]
        vc = np.zeros((1, 1, 1, D, 64))  # one value page, stored transposed
        vc[0, 0, 0, :, 0] = case["v_prefix"][0]
        out, lse = oracle.attention_ref(q, ks, vs, kc, vc, [1], 1, 1, case["sm_scale"])
        np.testing.assert_allclose(out[0, :, 0, :], np.array(case["out"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0], np.array(case["lse"]), rtol=0, atol=1e-14)


def _sdpa(q, k, v, scale, mask=None, causal=False, gqa=False):
    """Library attention; q [T][H][D] etc. as float64 numpy."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(np.asarray(x).transpose(1, 0, 2)))[None]
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
                                       is_causal=causal, scale=scale, enable_gqa=gqa)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("B,Hq,Hkv,D,k,lens", [
    (2, 4, 4, 16, 1, (0, 7)),
    (2, 8, 2, 32, 4, (5, 40)),
    (1, 6, 1, 64, 8, (129,)),
])
def test_zero_drafts_is_causal_attention(B, Hq, Hkv, D, k, lens):
    shape, d = _inputs(B, Hq, Hkv, D, k, 0, lens)
    out, _ = _run(shape, d)
    rng = np.random.default_rng(7)
    for b in range(B):
        L = lens[b]
        keys = np.concatenate([d["k_cache"][b, :, :L, :].transpose(1, 0, 2), d["k_step"][b]], axis=0)
        vals = np.concatenate([W.v_natural(d["v_cache"][b])[:, :L, :].transpose(1, 0, 2), d["v_step"][b]], axis=0)
        qfull = np.concatenate([rng.standard_normal((L, Hq, D)), d["q"][b]], axis=0)
        ref = _sdpa(qfull, keys, vals, shape.sm_scale, causal=True, gqa=True)[L:]
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,k,L", [(4, 2, 3, 10), (4, 4, 5, 0), (8, 2, 8, 65)])
def test_full_step_candidates_and_slots(Hq, Hkv, k, L):
    D = 32
    shape, d = _inputs(1, Hq, Hkv, D, k, k, (L,))
    out, _ = _run(shape, d)
    keys_pre = d["k_cache"][0, :, :L, :].transpose(1, 0, 2)
    vals_pre = W.v_natural(d["v_cache"][0])[:, :L, :].transpose(1, 0, 2)
    ks, vs, q = d["k_step"][0], d["v_step"][0], d["q"][0]
    # candidate rows == causal rows of a brute-force pass over [prefix ; candidates]
    rng = np.random.default_rng(3)
    qfull = np.concatenate([rng.standard_normal((L, Hq, D)), q[:k]], axis=0)
    ref = _sdpa(qfull, np.concatenate([keys_pre, ks[:k]]), np.concatenate([vals_pre, vs[:k]]),
                shape.sm_scale, causal=True, gqa=True)[L:]
    np.testing.assert_allclose(out[0, :k], ref, rtol=1e-12, atol=1e-12)
    # slot rows of group g == unmasked attention over [prefix ; c_0..c_g ; own group]
    for g in range(k):
        rows = slice(k + g * k, k + g * k + k)
        kk = np.concatenate([keys_pre, ks[:g + 1], ks[rows]])
        vv = np.concatenate([vals_pre, vs[:g + 1], vs[rows]])
        ref = _sdpa(q[rows], kk, vv, shape.sm_scale, gqa=True)
        np.testing.assert_allclose(out[0, rows], ref, rtol=1e-12, atol=1e-12)


def test_candidates_ignore_slots_and_groups_ignore_each_other():
    k, L = 4, 9
    shape, d = _inputs(1, 4, 2, 16, k, k, (L,), seed=5)
    out0, _ = _run(shape, d)
    # perturb every slot row's K/V: candidate outputs unchanged (bit-identical)
    d2 = {n: a.copy() for n, a in d.items()}
    d2["k_step"][0, k:] += 3.0
    d2["v_step"][0, k:] -= 2.0
    out1, _ = _run(shape, d2)
    assert np.array_equal(out0[0, :k], out1[0, :k])
    # perturb group 2's K/V and candidate 3: group 1 unchanged, group 2 changes
    d3 = {n: a.copy() for n, a in d.items()}
    g2 = slice(k + 2 * k, k + 3 * k)
    d3["k_step"][0, g2] += 1.0
    d3["v_step"][0, 3] += 1.0
    out2, _ = _run(shape, d3)
    g1 = slice(k + k, k + 2 * k)
    assert np.array_equal(out0[0, g1], out2[0, g1])
    assert not np.allclose(out0[0, g2], out2[0, g2])


def test_permutation_within_group_is_equivariant():
    k, L = 5, 6
    shape, d = _inputs(1, 2, 1, 16, k, k, (L,), seed=11)
    out0, _ = _run(shape, d)
    g = 3
    base = k + g * k
    perm = np.array([2, 0, 4, 1, 3])
    d2 = {n: a.copy() for n, a in d.items()}
    for name in ("q", "k_step", "v_step"):
        d2[name][0, base:base + k] = d[name][0, base + perm]
    out1, _ = _run(shape, d2)
    np.testing.assert_allclose(out1[0, base:base + k], out0[0, base + perm], rtol=1e-13, atol=1e-13)


def test_closed_forms():
    k = 3
    shape, d = _inputs(1, 2, 2, 8, k, k, (0,), seed=2)
    out, lse = _run(shape, d)
    # L = 0: candidate row 0 sees only its own key -> O = v_step[0], lse = its score
    np.testing.assert_array_equal(out[0, 0], d["v_step"][0, 0])
    s = shape.sm_scale * np.einsum("hd,hd->h", d["q"][0, 0], d["k_step"][0, 0])
    np.testing.assert_allclose(lse[0, :, 0], s, rtol=1e-14, atol=1e-14)
    # constant V -> O equals the constant in every row
    shape, d = _inputs(2, 4, 2, 8, 4, 4, (3, 17), seed=4)
    d["v_step"][:] = 0.625
    d["v_cache"][:] = 0.625
    out, _ = _run(shape, d)
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-15)
    # q = 0 -> uniform weights: lse = ln(number of visible keys)
    d["q"][:] = 0.0
    _, lse = _run(shape, d)
    for b, L in enumerate((3, 17)):
        n_vis = oracle.step_mask_ref(4, 4, L).sum(axis=1)
        np.testing.assert_allclose(lse[b], np.broadcast_to(np.log(n_vis), lse[b].shape), rtol=1e-14)


@pytest.mark.parametrize("chunk", [1, 7, 32, 64, 1000])
def test_split_merge_equals_unsplit(chunk):
    shape, d = _inputs(2, 4, 2, 16, 4, 4, (45, 0), seed=9)
    out, lse = _run(shape, d)
    out2, lse2 = oracle.attention_split_ref(d["q"], d["k_step"], d["v_step"], d["k_cache"], d["v_cache"],
                                            d["lens"], 4, 4, shape.sm_scale, chunk)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)


def test_pairs_subset_matches_full():
    shape, d = _inputs(3, 4, 2, 16, 2, 2, (5, 9, 1), seed=12)
    out, lse = _run(shape, d)
    pairs = [(2, 1), (0, 3)]
    out2, lse2 = _run(shape, d, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(out2[b, :, h], out[b, :, h])
        assert np.array_equal(lse2[b, h], lse[b, h])
    assert np.isnan(out2[1]).all()


def test_never_reads_past_settled_length():
    # the cache tail holds NaN; any read past lens[b] would poison the result
    shape, d = _inputs(2, 4, 2, 16, 4, 4, (5, 0), seed=1, S_max=64)
    assert np.isnan(d["k_cache"][0, :, 5:]).all()
    out, lse = _run(shape, d)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
