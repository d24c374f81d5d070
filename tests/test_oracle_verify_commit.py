"""Pins of the oracle's greedy verify and KV commit.

* verify: hand-worked cases (tests/golden/verify_cases.json, including
  ties and -0.0 vs +0.0), planted accept lengths (the exact answer by
  construction), and argmax_first against a plain Python scan;
* commit: brute-force concatenation of the accepted rows, len_final =
  len_0 + sum(a) over several steps, untouched rows past the new length,
  overflow and bad-length flags.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W


def _scan_argmax(row):
    best, bi = None, -1
    for i, x in enumerate(row):
        if best is None or x > best:
            best, bi = x, i
    return bi


def test_golden_cases(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "verify_cases.json")))
    for case in doc["cases"]:
        a, nxt = oracle.verify_ref(np.array(case["ar_logits"], dtype=np.float32),
                                   np.array(case["draft_logits"], dtype=np.float32),
                                   np.array(case["cand"], dtype=np.int32))
        assert a.tolist() == case["accept_len"], case["name"]
        assert nxt.tolist() == case["next_cand"], case["name"]


def test_argmax_first_matches_scan_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(50):
        row = rng.integers(-3, 4, size=rng.integers(1, 300)).astype(np.float32)  # many ties
        if trial % 3 == 0:
            row[row == 0] = -0.0
        assert oracle.argmax_first(row) == _scan_argmax(row.tolist())


@pytest.mark.parametrize("kind,k,V,B", [("uniform", 8, 1000, 12), ("geometric", 16, 513, 10),
                                        ("uniform", 1, 64, 5), ("uniform", 4, 4096, 9)])
def test_planted_accept_lengths(kind, k, V, B):
    d = W.verify_inputs(B, k, V, seed=3, accept=kind)
    a, nxt = oracle.verify_ref(d["ar_logits"], d["draft_logits"], d["cand"])
    assert a.tolist() == d["planted"].tolist()
    for b in range(B):
        assert nxt[b, 0] == _scan_argmax(d["ar_logits"][b, a[b]].tolist())
        g = max(int(a[b]), 1) - 1
        for m in range(1, k):
            assert nxt[b, m] == _scan_argmax(d["draft_logits"][b, g, m].tolist())


def test_boost_mode_gives_varied_lengths():
    d = W.verify_inputs(64, 4, 2000, seed=1, accept="boost")
    a, _ = oracle.verify_ref(d["ar_logits"], d["draft_logits"], d["cand"])
    assert len(set(a.tolist())) >= 2


def test_commit_equals_concatenation_over_steps():
    rng = np.random.default_rng(5)
    B, H, S, D, k, R = 3, 2, 64, 8, 4, 20
    kc = rng.standard_normal((B, H, S, D))
    vc = rng.standard_normal((B, H, S // 64, D, 64))
    lens0 = np.array([0, 5, 17], dtype=np.int32)
    lens = lens0.copy()
    k_start, v_start = kc.copy(), vc.copy()
    step_rows, accepted = [], [[] for _ in range(B)]
    for step in range(4):
        ks = rng.standard_normal((B, R, H, D))
        vs = rng.standard_normal((B, R, H, D))
        a = rng.integers(0, k + 1, size=B).astype(np.int32)
        kc, vc, lens_new, err = oracle.commit_ref(kc, vc, lens, ks, vs, a, k)
        assert (err == 0).all()
        assert (lens_new == lens + a).all()
        lens = lens_new
        step_rows.append((ks, vs, a))
    assert (lens == lens0 + sum(r[2] for r in step_rows)).all()
    for b in range(B):
        for h in range(H):
            want_k = np.concatenate([k_start[b, h, :lens0[b]]] + [ks[b, :a[b], h] for ks, _, a in step_rows])
            v0, v1 = W.v_natural(v_start[b, h]), W.v_natural(vc[b, h])
            want_v = np.concatenate([v0[:lens0[b]]] + [vs[b, :a[b], h] for _, vs, a in step_rows])
            assert np.array_equal(kc[b, h, :lens[b]], want_k)
            assert np.array_equal(v1[:lens[b]], want_v)
            # rows past the new length are untouched
            assert np.array_equal(kc[b, h, lens[b]:], k_start[b, h, lens[b]:])
            assert np.array_equal(v1[lens[b]:], v0[lens[b]:])


def test_commit_flags():
    B, H, S, D, k = 3, 1, 64, 4, 4
    kc = np.zeros((B, H, S, D), dtype=np.uint16)
    vc = np.zeros((B, H, S // 64, D, 64), dtype=np.uint16)
    ks = np.ones((B, 20, H, D), dtype=np.uint16)
    vs = np.ones((B, 20, H, D), dtype=np.uint16)
    lens = np.array([62, 62, 2], dtype=np.int32)
    a = np.array([2, 3, 5], dtype=np.int32)  # fits, overflows (65 > 64), a > k
    kc2, vc2, lens2, err = oracle.commit_ref(kc, vc, lens, ks, vs, a, k)
    assert err.tolist() == [0, 1, 2]
    assert lens2.tolist() == [64, 62, 2]
    assert kc2[0, 0, 62:64].sum() == 2 * D and kc2[1].sum() == 0 and kc2[2].sum() == 0
    assert vc2[0, 0, 0, :, 62:64].sum() == 2 * D and vc2[0, 0, 0, :, :62].sum() == 0
