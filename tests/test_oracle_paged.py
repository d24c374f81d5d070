"""Pins of the paged-cache oracle (block-table placement, attention over
pages, commit into pages) against closed forms and the contiguous oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle.paged import gather_paged, pages_valid


def _encoded_pools(n_pages, Hkv, D):
    # every element names its own (page, head, row, column)
    pg = np.arange(n_pages)[:, None, None, None]
    h = np.arange(Hkv)[None, :, None, None]
    r = np.arange(64)[None, None, :, None]
    d = np.arange(D)[None, None, None, :]
    code = pg * 1e6 + h * 1e4 + r * 100 + d                     # [page][h][row][d]
    return code.astype(np.float64), -np.swapaxes(code, 2, 3).astype(np.float64)  # v: [page][h][d][row]


def test_gather_places_page_table_row_at_each_position():
    table = np.array([[5, 0, 3], [6, 2, 1]], dtype=np.int32)
    lens = [130, 64]
    kp, vp = _encoded_pools(7, 2, 3)
    kc, vc = gather_paged(kp, vp, table, lens, 192)
    for b, L in enumerate(lens):
        p = np.arange(192)
        want = table[b][p // 64][None, :, None] * 1e6 + np.arange(2)[:, None, None] * 1e4 \
            + (p % 64)[None, :, None] * 100 + np.arange(3)[None, None, :]
        want = np.where(p[None, :, None] < L, want, 0.0)
        assert np.array_equal(kc[b], want)
        v_nat = vc[b].transpose(0, 1, 3, 2).reshape(2, 192, 3)  # [h][position][d]
        assert np.array_equal(v_nat, -want)


def _contiguous_case(dtype="f32"):
    s = W.AttnShape(B=3, Hq=4, Hkv=2, D=64, k=3, n_groups=3, lens=(70, 0, 191), S_max=256,
                    sm_scale=0.125, dtype=dtype)
    return s, W.attention_inputs(s, seed=4, tail="zero")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("shuffled", [False, True])
def test_paged_attention_equals_contiguous(shuffled):
    s, d = _contiguous_case()
    B, Hkv, S, D = d["k_cache"].shape
    P = S // 64
    if shuffled:
        pg = W.to_pages(d["k_cache"], d["v_cache"], seed=9, spare=5)
        kp, vp, table = pg["k_pool"], pg["v_pool"], pg["block_table"]
    else:  # pages in sequence order: page b*P + t is tile t of sequence b
        kp = d["k_cache"].reshape(B, Hkv, P, 64, D).transpose(0, 2, 1, 3, 4).reshape(B * P, Hkv, 64, D)
        vp = d["v_cache"].transpose(0, 2, 1, 3, 4).reshape(B * P, Hkv, D, 64)
        table = np.arange(B * P, dtype=np.int32).reshape(B, P)
    out, lse = oracle.paged_attention_ref(d["q"], d["k_step"], d["v_step"], kp, vp, table, d["lens"], s.k,
                                          s.n_groups, s.sm_scale)
    ref, ref_lse = oracle.attention_ref(d["q"], d["k_step"], d["v_step"], d["k_cache"], d["v_cache"], d["lens"],
                                        s.k, s.n_groups, s.sm_scale)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def test_bad_page_entry_gives_nan_rows_only_there():
    s, d = _contiguous_case()
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=2)
    table = pg["block_table"].copy()
    table[2, 1] = 10 ** 6  # a settled position of sequence 2 (lens 191 covers pages 0..2)
    table[0, 3] = -1       # past sequence 0's pages (lens 70 covers 0..1): never read
    assert pages_valid(table, d["lens"], pg["k_pool"].shape[0]).tolist() == [True, True, False]
    out, lse = oracle.paged_attention_ref(d["q"], d["k_step"], d["v_step"], pg["k_pool"], pg["v_pool"], table,
                                          d["lens"], s.k, s.n_groups, s.sm_scale)
    assert np.isnan(out[2]).all() and np.isnan(lse[2]).all()
    assert np.isfinite(out[:2]).all()


def test_paged_commit_commutes_with_the_gather():
    s, d = _contiguous_case()
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=3, spare=4)
    kp, vp, table = pg["k_pool"], pg["v_pool"], pg["block_table"]
    acc = np.array([3, 0, 2], dtype=np.int32)
    kp2, vp2, ln2, err = oracle.commit_paged_ref(kp, vp, table, d["lens"], d["k_step"], d["v_step"], acc, s.k)
    kc, vc = gather_paged(kp, vp, table, d["lens"], s.S_max)
    kc_ref, vc_ref, ln_ref, err_ref = oracle.commit_ref(kc, vc, d["lens"], d["k_step"], d["v_step"], acc, s.k)
    assert err.tolist() == err_ref.tolist() == [0, 0, 0]
    assert ln2.tolist() == ln_ref.tolist() == [73, 0, 193]
    kc2, vc2 = gather_paged(kp2, vp2, table, ln2, s.S_max)
    assert np.array_equal(kc2, kc_ref) and np.array_equal(_f64(vc2), _f64(vc_ref))
    # outside the written positions every pool element is unchanged (NaN spares included)
    written = np.zeros(kp.shape[:1] + kp.shape[2:3], dtype=bool)  # [page][row]
    for b in range(3):
        for p in range(int(d["lens"][b]), int(ln2[b])):
            written[table[b][p // 64], p % 64] = True
    same_k = (kp2 == kp) | (np.isnan(kp2) & np.isnan(kp))
    same_v = (vp2 == vp) | (np.isnan(vp2) & np.isnan(vp))
    assert same_k.transpose(0, 2, 1, 3)[~written].all()
    assert same_v.transpose(0, 3, 1, 2)[~written].all()
    assert not same_k.all()  # something was written


def test_paged_commit_flags():
    s, d = _contiguous_case()
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=3)
    table = pg["block_table"].copy()
    lens = np.array([70, 254, 127], dtype=np.int32)
    table[2, 1] = 99999   # positions 127.. fall in page 1 then 2: page 1 is outside the pools
    acc = np.array([4, 3, 2], dtype=np.int32)  # 4 > k=3 -> 2; 254 + 3 > 256 -> 1; bad page -> 3
    kp2, vp2, ln2, err = oracle.commit_paged_ref(pg["k_pool"], pg["v_pool"], table, lens, d["k_step"],
                                                 d["v_step"], acc, s.k)
    assert err.tolist() == [2, 1, 3]
    assert ln2.tolist() == lens.tolist()
    same = (kp2 == pg["k_pool"]) | (np.isnan(kp2) & np.isnan(pg["k_pool"]))
    assert same.all()
