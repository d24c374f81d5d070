"""GPU tests of the checked build (libtidar_checked.so): every kernel family
runs through it with no failed bounds test on valid inputs and gives the
oracle's results (attention within the bf16 tolerance, verification and
commits bit-exact), and contract violations planted from the host -- a
length past max_len, a page outside the pools, a commit past the cache, an
accept length above k, a logit row with nothing above -inf, a verify +
commit state that was not cleared -- are recorded with their code while
every kernel runs to its end (the outcomes the release library documents
for them are unchanged)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle.train_mask import train_attention_ref

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, attn_f32, attn_to_dev, bits, check_attention, to_dev  # noqa: E402

CODE = {name: code for code, name in tidar.CHECK_CODES.items()}


def _clean():
    rec = tidar.check_read()
    assert rec[0] == 0, f"failed bounds test {tidar.CHECK_CODES.get(rec[0], rec[0])}: {rec}"


def _shape(B, Hq, Hkv, k, ng, lens, D=128, dtype="bf16", S_max=None):
    S_max = S_max or ((max(lens) + k + ng * k + 63) // 64 * 64)
    return W.AttnShape(B=B, Hq=Hq, Hkv=Hkv, D=D, k=k, n_groups=ng, lens=tuple(lens), S_max=S_max,
                       sm_scale=1.0 / math.sqrt(D), dtype=dtype)


ATTN = {
    # name: (kernel restriction, shape, kv_chunk)
    "eight_wave_nine_tiles": ("pp", _shape(16, 32, 8, 8, 8, tuple(64 + 37 * i for i in range(16))), 0),
    "eight_wave_split": ("pp", _shape(2, 8, 2, 4, 4, (383, 70)), 128),
    "four_wave_ragged": ("pipe", _shape(3, 8, 2, 4, 4, (0, 37, 300)), 0),
    "four_wave_split": ("pipe", _shape(4, 12, 2, 4, 4, (2048, 5, 64, 1000)), 256),
    "f32_split": (None, _shape(2, 8, 2, 3, 3, (200, 70), dtype="f32"), 64),
}


@pytest.mark.parametrize("name", list(ATTN))
def test_checked_attention_matches_oracle(monkeypatch, name):
    kern, s, chunk = ATTN[name]
    if kern:
        monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    print(f"checked attention {name}", flush=True)
    d = W.attention_inputs(s, seed=len(name), tail="nan")
    t = attn_to_dev(d, s.dtype)
    with tidar.checked_library():
        out, lse = tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], s.k,
                                        s.n_groups, s.sm_scale, max_len=s.max_len, kv_chunk=chunk)
        _clean()
    f = attn_f32(d, s.dtype)
    ref, ref_lse = oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"],
                                        s.k, s.n_groups, s.sm_scale)
    check_attention(out, lse, ref, ref_lse, s.dtype, what=f"checked {name}")


@pytest.mark.parametrize("kern", ["pp", "pipe"])
def test_checked_paged_attention_and_bad_page(monkeypatch, kern):
    monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    s = _shape(3, 8, 2, 3, 3, (70, 0, 191), S_max=256)
    d = W.attention_inputs(s, seed=3, tail="nan")
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=4, spare=8)
    t = attn_to_dev(d, "bf16")
    kp, vp = to_dev(pg["k_pool"], True), to_dev(pg["v_pool"], True)
    table = pg["block_table"].copy()
    print(f"checked paged {kern}", flush=True)
    with tidar.checked_library():
        out, lse = tidar.step_attention_paged(t["q"], t["k_step"], t["v_step"], kp, vp, to_dev(table), t["lens"],
                                              s.k, s.n_groups, s.sm_scale, max_len=s.max_len)
        _clean()
        bad = table.copy()
        bad[2, 1] = pg["k_pool"].shape[0] + 7  # a settled page of sequence 2 outside the pools
        out2, _ = tidar.step_attention_paged(t["q"], t["k_step"], t["v_step"], kp, vp, to_dev(bad), t["lens"],
                                             s.k, s.n_groups, s.sm_scale, max_len=s.max_len)
        rec = tidar.check_read()
    f = attn_f32(d, "bf16")
    ref, ref_lse = oracle.paged_attention_ref(f["q"], f["k_step"], f["v_step"], W.bf16_to_f32(pg["k_pool"]),
                                              W.bf16_to_f32(pg["v_pool"]), table, d["lens"], s.k, s.n_groups,
                                              s.sm_scale)
    check_attention(out, lse, ref, ref_lse, "bf16", what=f"checked paged {kern}")
    assert rec[0] == CODE["page"] and rec[3] == pg["k_pool"].shape[0] + 7, rec
    o2 = out2.float().cpu().numpy()
    assert np.isnan(o2[2]).all() and np.isfinite(o2[:2]).all()


@pytest.mark.parametrize("kern", ["pp", "pipe"])
def test_checked_records_length_past_max_len(monkeypatch, kern):
    monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    s = _shape(3, 8, 2, 4, 4, (100, 200, 50))
    d = W.attention_inputs(s, seed=8, tail="nan")
    t = attn_to_dev(d, "bf16")
    t["lens"][1] = s.max_len + 5  # the kernels write NaN rows for it and read nothing of it
    print(f"checked planted length {kern}", flush=True)
    with tidar.checked_library():
        out, _ = tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], s.k,
                                      s.n_groups, s.sm_scale, max_len=s.max_len)
        rec = tidar.check_read()
    assert rec[0] == CODE["lens"] and rec[3] == s.max_len + 5, rec
    o = out.float().cpu().numpy()
    assert np.isnan(o[1]).all() and np.isfinite(o[[0, 2]]).all()


def test_checked_train_attention_matches_oracle():
    B, Hq, Hkv, D, N, bs = 1, 8, 2, 128, 256, 8
    d = W.train_inputs(B, Hq, Hkv, D, N, seed=2)
    scale = 1.0 / math.sqrt(D)
    with tidar.checked_library():
        out, lse = tidar.train_attention(to_dev(d["q"], True), to_dev(d["k"], True), to_dev(d["v"], True), N, bs,
                                         scale)
        _clean()
    ref, ref_lse = train_attention_ref(W.bf16_to_f32(d["q"]), W.bf16_to_f32(d["k_nat"]), W.bf16_to_f32(d["v_nat"]),
                                       N, bs, scale)
    got = out.float().cpu().numpy()
    assert np.abs(got - ref).max() <= 2e-2
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= 1e-2


def _cache(B, Hkv, D, S, k, lens, seed):
    s = W.AttnShape(B=B, Hq=Hkv, Hkv=Hkv, D=D, k=k, n_groups=k, lens=tuple(lens), S_max=S, dtype="bf16")
    d = W.kv_cache(s, seed=seed, tail="random")
    d.update(W.step_rows(s, seed=seed))
    return d


def _dev_cache(d):
    return {"kc": to_dev(d["k_cache"], True), "vc": to_dev(d["v_cache"], True), "ln": to_dev(d["lens"]),
            "ks": to_dev(d["k_step"], True), "vs": to_dev(d["v_step"], True)}


def test_checked_verify_and_commit_paths_match_oracle():
    B, k, V, Hkv, D, S = 5, 4, 6000, 2, 128, 256
    v = W.verify_inputs(B, k, V, seed=11, accept="uniform")
    d = _cache(B, Hkv, D, S, k, (0, 60, 63, 100, 190), seed=11)
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    rk, rv, rl, re = oracle.commit_ref(d["k_cache"], d["v_cache"], d["lens"], d["k_step"], d["v_step"], ra, k)
    ar, dr, cand = to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"])
    with tidar.checked_library():
        a, n = tidar.verify_greedy(ar, dr, cand)
        _clean()
        assert a.cpu().numpy().tolist() == ra.tolist() and n.cpu().numpy().tolist() == rn.tolist()
        t = _dev_cache(d)
        err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        tidar.kv_commit(t["kc"], t["vc"], t["ln"], t["ks"], t["vs"], a, k, err)
        _clean()
        assert err.cpu().numpy().tolist() == re.tolist() and t["ln"].cpu().numpy().tolist() == rl.tolist()
        assert np.array_equal(bits(t["kc"]), rk) and np.array_equal(bits(t["vc"]), rv)
        t = _dev_cache(d)
        st = tidar.verify_commit_state(B, k, DEV)
        a2, n2 = tidar.verify_commit_greedy(ar, dr, cand, t["kc"], t["vc"], t["ln"], t["ks"], t["vs"], state=st)
        _clean()
        assert a2.cpu().numpy().tolist() == ra.tolist() and n2.cpu().numpy().tolist() == rn.tolist()
        assert t["ln"].cpu().numpy().tolist() == rl.tolist()
        assert np.array_equal(bits(t["kc"]), rk) and np.array_equal(bits(t["vc"]), rv)
        assert int(st.abs().sum()) == 0


def test_checked_paged_commits_match_oracle():
    B, k, V, Hkv, D, S = 5, 4, 3000, 2, 128, 256
    v = W.verify_inputs(B, k, V, seed=12, accept="uniform")
    d = _cache(B, Hkv, D, S, k, (0, 60, 63, 100, 190), seed=12)
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=12, spare=3)
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    kp2, vp2, ln2, err2 = oracle.commit_paged_ref(pg["k_pool"], pg["v_pool"], pg["block_table"], d["lens"],
                                                  d["k_step"], d["v_step"], ra, k)
    with tidar.checked_library():
        for fused in (False, True):
            kp, vp, ln = to_dev(pg["k_pool"], True), to_dev(pg["v_pool"], True), to_dev(d["lens"])
            tbl, ks, vs = to_dev(pg["block_table"]), to_dev(d["k_step"], True), to_dev(d["v_step"], True)
            err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
            if fused:
                st = tidar.verify_commit_state(B, k, DEV)
                a, n = tidar.verify_commit_greedy_paged(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]),
                                                        to_dev(v["cand"]), kp, vp, tbl, ln, ks, vs, err_flags=err,
                                                        state=st)
                assert n.cpu().numpy().tolist() == rn.tolist()
            else:
                a = to_dev(ra)
                tidar.kv_commit_paged(kp, vp, tbl, ln, ks, vs, a, k, err)
            _clean()
            assert a.cpu().numpy().tolist() == ra.tolist() and err.cpu().numpy().tolist() == err2.tolist()
            assert ln.cpu().numpy().tolist() == ln2.tolist()
            assert np.array_equal(bits(kp), kp2.view(np.uint16)) and np.array_equal(bits(vp), vp2.view(np.uint16))


def test_checked_sampling_and_lmhead_match_the_release_library():
    ds = W.sample_inputs(4, 3, 3000, seed=5)
    dl = W.lmhead_inputs(3, 4, 2000, 256, seed=7, accept="uniform")

    def run():
        a, n = tidar.verify_sample(to_dev(ds["ar_logits"]), to_dev(ds["q_logits"]), to_dev(ds["draft_logits"]),
                                   to_dev(ds["cand"]), 0.8, 1234, 7)
        a2, n2 = tidar.lmhead_verify_greedy(to_dev(dl["h_ar"], True), to_dev(dl["h_draft"], True),
                                            to_dev(dl["w"], True), to_dev(dl["cand"]))
        return [x.cpu().numpy().tolist() for x in (a, n, a2, n2)]

    release = run()
    with tidar.checked_library():
        checked = run()
        _clean()
    assert checked == release


def test_checked_records_commit_violations():
    B, k, Hkv, D, S = 3, 4, 2, 128, 128
    d = _cache(B, Hkv, D, S, k, (10, 126, 40), seed=13)
    acc = np.array([2, 4, 1], dtype=np.int32)  # sequence 1: 126 + 4 > 128
    with tidar.checked_library():
        t = _dev_cache(d)
        err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        tidar.kv_commit(t["kc"], t["vc"], t["ln"], t["ks"], t["vs"], to_dev(acc), k, err)
        rec = tidar.check_read()
        assert err.cpu().numpy().tolist() == [0, 1, 0]
        assert rec[0] == CODE["capacity"] and rec[3] == 130, rec
        acc2 = np.array([1, 0, k + 3], dtype=np.int32)  # sequence 2: accept length above k
        err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        tidar.kv_commit(t["kc"], t["vc"], t["ln"], t["ks"], t["vs"], to_dev(acc2), k, err)
        rec = tidar.check_read()
        assert err.cpu().numpy().tolist() == [0, 0, 2]
        assert rec[0] == CODE["accept"] and rec[3] == k + 3, rec


def test_checked_records_a_row_with_no_token():
    B, k, V = 3, 4, 5000
    v = W.verify_inputs(B, k, V, seed=14, accept="uniform")
    v["ar_logits"][1, 0, :] = -np.inf  # AR row 0 of sequence 1 has no argmax
    with tidar.checked_library():
        a, n = tidar.verify_greedy(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"]))
        rec = tidar.check_read()
    assert rec[0] == CODE["token"], rec
    assert int(a[1]) == 0


def test_checked_records_a_state_that_was_not_cleared():
    B, k, V, Hkv, D, S = 2, 4, 3000, 2, 128, 256
    v = W.verify_inputs(B, k, V, seed=15, accept="uniform")
    d = _cache(B, Hkv, D, S, k, (30, 90), seed=15)
    t = _dev_cache(d)
    st = tidar.verify_commit_state(B, k, DEV)
    st.fill_(255)  # every counter and key set: a state some earlier call left behind
    with tidar.checked_library():
        tidar.verify_commit_greedy(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"]), t["kc"],
                                   t["vc"], t["ln"], t["ks"], t["vs"], state=st)
        rec = tidar.check_read()
    assert rec[0] == CODE["state"], rec


@pytest.mark.skipif(os.environ.get("TIDAR_LIBRARY") == "checked", reason="the whole run uses the checked build")
def test_release_library_reports_no_checks():
    assert tidar.lib().tidar_check_enabled() == 0
    assert tidar.check_read() == (0, 0, 0, 0)
