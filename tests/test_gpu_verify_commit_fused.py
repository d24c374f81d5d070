"""GPU parity of the fused greedy verification + KV commit
(tidar_verify_commit_greedy[_paged]): bit-exact against the oracle's verify
and commit, and against the separate tidar_verify_greedy + tidar_kv_commit
calls, on the golden tie cases, planted accept lengths at every k from 1 to
16, ragged vocabularies, the full 8B-shaped step, capacity and bad-page
flags, paged caches, and a many-step loop that reuses one state buffer.
The state must be left zeroed by every call; that is checked too."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, bits, to_dev  # noqa: E402


def _cache(B, Hkv, D, S, k, lens, dtype, seed):
    shape = W.AttnShape(B=B, Hq=Hkv, Hkv=Hkv, D=D, k=k, n_groups=k, lens=tuple(lens), S_max=S, dtype=dtype)
    d = W.kv_cache(shape, seed=seed, tail="random")
    d.update(W.step_rows(shape, seed=seed))
    return shape, d


def _fused(v, d, dtype, state=None, err=None):
    bf = dtype == "bf16"
    t = {"kc": to_dev(d["k_cache"], bf), "vc": to_dev(d["v_cache"], bf), "ln": to_dev(d["lens"]),
         "ks": to_dev(d["k_step"], bf), "vs": to_dev(d["v_step"], bf)}
    B, k = v["cand"].shape
    err = torch.full((B,), -1, dtype=torch.int32, device=DEV) if err is None else err
    st = tidar.verify_commit_state(B, k, DEV) if state is None else state
    a, n = tidar.verify_commit_greedy(to_dev(v["ar_logits"]),
                                      None if v["draft_logits"] is None else to_dev(v["draft_logits"]),
                                      to_dev(v["cand"]), t["kc"], t["vc"], t["ln"], t["ks"], t["vs"],
                                      err_flags=err, state=st)
    torch.cuda.synchronize()
    assert int(st.abs().sum()) == 0, "the state must be left zeroed"
    return a.cpu().numpy(), n.cpu().numpy(), t, err.cpu().numpy()


def _raw(x):
    """Element bits of a host cache (f32 caches are float arrays, bf16 ones bits)."""
    x = np.asarray(x)
    return x.view(np.uint32) if x.dtype == np.float32 else x


def _check_against_oracle(v, d, k, dtype, a, n, t, err):
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    assert a.tolist() == ra.tolist()
    assert n.tolist() == rn.tolist()
    rk, rv, rl, re = oracle.commit_ref(d["k_cache"], d["v_cache"], d["lens"], d["k_step"], d["v_step"], ra, k)
    assert err.tolist() == re.tolist()
    assert t["ln"].cpu().numpy().tolist() == rl.tolist()
    assert np.array_equal(bits(t["kc"]), _raw(rk)) and np.array_equal(bits(t["vc"]), _raw(rv))
    return ra


def test_golden_cases(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "verify_cases.json")))
    for case in doc["cases"]:
        v = {"ar_logits": np.array(case["ar_logits"], dtype=np.float32),
             "draft_logits": np.array(case["draft_logits"], dtype=np.float32),
             "cand": np.array(case["cand"], dtype=np.int32)}
        B, k = v["cand"].shape
        _, d = _cache(B, 2, 64, 128, k, [5] * B, "bf16", seed=3)
        a, n, t, err = _fused(v, d, "bf16")
        assert a.tolist() == case["accept_len"], case["name"]
        assert n.tolist() == case["next_cand"], case["name"]
        _check_against_oracle(v, d, k, "bf16", a, n, t, err)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 7, 8, 12, 16])
def test_every_k_matches_oracle(k):
    B, V = 6, 5000
    v = W.verify_inputs(B, k, V, seed=40 + k, accept="uniform", with_drafts=k > 1)
    _, d = _cache(B, 4, 128, 256, k, (0, 1, 63, 64, 120, 200), "bf16", seed=k)
    a, n, t, err = _fused(v, d, "bf16")
    ra = _check_against_oracle(v, d, k, "bf16", a, n, t, err)
    assert ra.tolist() == v["planted"].tolist()


@pytest.mark.parametrize("B,k,V,kind,dtype", [
    (16, 8, 128256, "uniform", "bf16"),   # 8B-shaped step
    (8, 4, 151936, "boost", "bf16"),      # 1.5B-shaped step
    (4, 16, 128256, "geometric", "bf16"),  # long-context step
    (5, 1, 1001, "uniform", "f32"),       # no drafts, V not a multiple of 4
    (3, 3, 4097, "uniform", "f32"),       # one element past a chunk boundary
    (7, 5, 64, "none", "bf16"),           # tiny vocabulary, one chunk
])
def test_matches_oracle_and_separate_calls(B, k, V, kind, dtype):
    v = W.verify_inputs(B, k, V, seed=B * 100 + k, accept=kind, with_drafts=k > 1)
    lens = [(37 * i) % 150 for i in range(B)]
    _, d = _cache(B, 8, 128, 256, k, lens, dtype, seed=B)
    a, n, t, err = _fused(v, d, dtype)
    _check_against_oracle(v, d, k, dtype, a, n, t, err)
    # the separate calls on copies of the same inputs give the same bits
    bf = dtype == "bf16"
    kc, vc, ln = to_dev(d["k_cache"], bf), to_dev(d["v_cache"], bf), to_dev(d["lens"])
    a2, n2 = tidar.verify_greedy(to_dev(v["ar_logits"]), None if k == 1 else to_dev(v["draft_logits"]),
                                 to_dev(v["cand"]))
    e2 = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    tidar.kv_commit(kc, vc, ln, to_dev(d["k_step"], bf), to_dev(d["v_step"], bf), a2, k, e2)
    torch.cuda.synchronize()
    assert a2.cpu().numpy().tolist() == a.tolist() and n2.cpu().numpy().tolist() == n.tolist()
    assert np.array_equal(bits(kc), bits(t["kc"])) and np.array_equal(bits(vc), bits(t["vc"]))
    assert ln.cpu().numpy().tolist() == t["ln"].cpu().numpy().tolist() and e2.cpu().numpy().tolist() == err.tolist()


def test_ties_everywhere():
    rng = np.random.default_rng(0)
    B, k, V = 6, 4, 9000
    ar = rng.integers(-2, 3, size=(B, k + 1, V)).astype(np.float32)
    ar[ar == 0] = -0.0
    ar[:, :, 5000] = 2.0
    ar[:, :, 4095:4097] = 2.0  # equal maxima on both sides of the 4096 chunk boundary
    dr = rng.integers(-1, 2, size=(B, k, k, V)).astype(np.float32)
    cand = np.zeros((B, k), dtype=np.int32)
    cand[:3, 0] = 4095
    cand[::2, 1] = 0
    v = {"ar_logits": ar, "draft_logits": dr, "cand": cand}
    _, d = _cache(B, 2, 64, 64, k, [10] * B, "bf16", seed=9)
    a, n, t, err = _fused(v, d, "bf16")
    _check_against_oracle(v, d, k, "bf16", a, n, t, err)


def test_capacity_flag():
    B, k, V = 4, 8, 3000
    v = W.verify_inputs(B, k, V, seed=5, accept="uniform")
    # sequence 1 overflows the 128-position cache when it accepts 3 or more
    _, d = _cache(B, 2, 128, 128, k, (0, 126, 10, 60), "bf16", seed=5)
    a, n, t, err = _fused(v, d, "bf16")
    ra = _check_against_oracle(v, d, k, "bf16", a, n, t, err)
    assert (err[1] == 1) == (ra[1] >= 3)


def test_paged_matches_oracle_with_bad_page():
    B, Hkv, D, k, V = 5, 4, 128, 8, 4000
    S = 256
    v = W.verify_inputs(B, k, V, seed=6, accept="uniform")
    shape, d = _cache(B, Hkv, D, S, k, (0, 60, 63, 100, 190), "bf16", seed=6)
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=6, spare=3)
    table = pg["block_table"].copy()
    table[3, 100 // 64] = pg["k_pool"].shape[0] + 5  # sequence 3's next page is outside the pools
    kp, vp = to_dev(pg["k_pool"], True), to_dev(pg["v_pool"], True)
    ln = to_dev(d["lens"])
    err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    st = tidar.verify_commit_state(B, k, DEV)
    a, n = tidar.verify_commit_greedy_paged(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"]), kp,
                                            vp, to_dev(table), ln, to_dev(d["k_step"], True),
                                            to_dev(d["v_step"], True), err_flags=err, state=st)
    # the separate paged commit on a copy of the pools is the reference for the pages
    kp2, vp2, ln2 = to_dev(pg["k_pool"], True), to_dev(pg["v_pool"], True), to_dev(d["lens"])
    e2 = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    a2, n2 = tidar.verify_greedy(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"]))
    tidar.kv_commit_paged(kp2, vp2, to_dev(table), ln2, to_dev(d["k_step"], True), to_dev(d["v_step"], True), a2, k,
                          e2)
    torch.cuda.synchronize()
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    assert a.cpu().numpy().tolist() == ra.tolist() and n.cpu().numpy().tolist() == rn.tolist()
    assert err.cpu().numpy().tolist() == e2.cpu().numpy().tolist()
    assert int(err[3]) == 3 or ra[3] == 0
    assert ln.cpu().numpy().tolist() == ln2.cpu().numpy().tolist()
    assert np.array_equal(bits(kp), bits(kp2)) and np.array_equal(bits(vp), bits(vp2))
    assert int(st.abs().sum()) == 0


def test_loop_reuses_one_state():
    """Twenty consecutive steps on one cache and one state buffer, with the
    batch shrinking half-way (the second shape reads the same state)."""
    B, Hkv, D, k, V, S = 8, 2, 128, 4, 2000, 256
    shape, d = _cache(B, Hkv, D, S, k, (0, 3, 17, 40, 64, 65, 100, 130), "bf16", seed=11)
    kc, vc, ln = to_dev(d["k_cache"], True), to_dev(d["v_cache"], True), to_dev(d["lens"])
    rk, rv, rl = d["k_cache"], d["v_cache"], d["lens"]
    st = tidar.verify_commit_state(B, k, DEV)
    for step in range(20):
        b = B if step < 10 else B // 2
        v = W.verify_inputs(b, k, V, seed=step, step=step, accept="uniform")
        rows = W.step_rows(shape, seed=11, step=step)
        ks, vs = rows["k_step"][:b], rows["v_step"][:b]
        a, n = tidar.verify_commit_greedy(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"]),
                                          kc[:b], vc[:b], ln[:b], to_dev(ks, True), to_dev(vs, True), state=st)
        ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
        nk, nv, nl, _ = oracle.commit_ref(rk[:b], rv[:b], rl[:b], ks, vs, ra, k)
        rk, rv, rl = rk.copy(), rv.copy(), rl.copy()
        rk[:b], rv[:b], rl[:b] = nk, nv, nl
        torch.cuda.synchronize()
        assert a.cpu().numpy().tolist() == ra.tolist() and n.cpu().numpy().tolist() == rn.tolist(), step
        assert int(st.abs().sum()) == 0, step
    assert ln.cpu().numpy().tolist() == rl.tolist()
    assert np.array_equal(bits(kc), _raw(rk)) and np.array_equal(bits(vc), _raw(rv))
