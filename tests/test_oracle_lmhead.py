"""Pins of the fused LM-head + greedy verify oracle."""
import numpy as np
import pytest

import oracle
from oracle.lmhead import lmhead_verify_ref


def test_hand_computed_three_token_head():
    # W rows: v0 = (1, 0), v1 = (0, 1), v2 = (1, 1)
    w = np.array([[1, 0], [0, 1], [1, 1]], dtype=np.float32)
    h_ar = np.array([[[2, 1], [1, 3], [3, -1]]], dtype=np.float32)  # logits (2,1,3) (1,3,4) (3,-1,2)
    h_draft = np.zeros((1, 2, 2, 2), dtype=np.float32)
    h_draft[0, 0, 1] = (-1, 2)  # logits (-1, 2, 1): token 1
    h_draft[0, 1, 1] = (1, 0)   # logits (1, 0, 1): tie of v0 and v2, the lower index wins
    # cand (2, 1): t0 = 2 kept, t1 = 2 != 1 -> a = 1, bonus t1 = 2, group 0's slot 1 -> 1
    a, n = lmhead_verify_ref(h_ar, h_draft, w, np.array([[2, 1]]))
    assert a.tolist() == [1] and n.tolist() == [[2, 1]]
    # cand (2, 2): both kept -> a = 2, bonus t2 = 0, group 1's slot 1 -> 0 (tie)
    a, n = lmhead_verify_ref(h_ar, h_draft, w, np.array([[2, 2]]))
    assert a.tolist() == [2] and n.tolist() == [[0, 0]]


def _case(B, k, d, seed):
    g = np.random.default_rng(seed)
    h_ar = g.standard_normal((B, k + 1, d)).astype(np.float32)
    h_draft = g.standard_normal((B, k, k, d)).astype(np.float32)
    return h_ar, h_draft, g


@pytest.mark.parametrize("B,k,d", [(3, 4, 32), (2, 1, 16), (4, 8, 64)])
def test_identity_head_reduces_to_greedy_verify_on_the_hidden_states(B, k, d):
    h_ar, h_draft, g = _case(B, k, d, seed=B * k)
    # plant matches: candidate i < a copies the argmax of hidden row i
    cand = g.integers(0, d, size=(B, k)).astype(np.int32)
    for b in range(B):
        for i in range(int(g.integers(0, k + 1))):
            cand[b, i] = int(np.argmax(h_ar[b, i]))
    a, n = lmhead_verify_ref(h_ar, h_draft, np.eye(d, dtype=np.float32), cand)
    ra, rn = oracle.verify_ref(h_ar, h_draft, cand)
    assert a.tolist() == ra.tolist() and n.tolist() == rn.tolist()


def test_permuted_unit_rows_permute_the_argmax():
    B, k, d = 3, 5, 40
    h_ar, h_draft, g = _case(B, k, d, seed=7)
    perm = g.permutation(d)
    w = np.eye(d, dtype=np.float32)[perm]  # logit v = h[perm[v]]
    inv = np.argsort(perm)
    cand = g.integers(0, d, size=(B, k)).astype(np.int32)
    cand[:, 0] = inv[np.argmax(h_ar[:, 0], axis=1)]  # candidate 0 always matches
    a, n = lmhead_verify_ref(h_ar, h_draft, w, cand)
    ra, rn = oracle.verify_ref(h_ar, h_draft, perm[cand])  # the same test in hidden-state coordinates
    assert a.tolist() == ra.tolist()
    assert n.tolist() == inv[rn].tolist()
    assert (a >= 1).all()


def test_positive_rescaling_changes_nothing():
    B, k, d, V = 4, 4, 24, 50
    h_ar, h_draft, g = _case(B, k, d, seed=3)
    w = g.standard_normal((V, d)).astype(np.float32)
    cand = g.integers(0, V, size=(B, k)).astype(np.int32)
    a, n = lmhead_verify_ref(h_ar, h_draft, w, cand)
    a2, n2 = lmhead_verify_ref(h_ar, h_draft, w * 3.5, cand)
    assert a.tolist() == a2.tolist() and n.tolist() == n2.tolist()
