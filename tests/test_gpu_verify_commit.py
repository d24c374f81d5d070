"""GPU parity of tidar_verify_greedy and tidar_kv_commit: bit-exact against the oracle."""
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


def _verify(v):
    a, n = tidar.verify_greedy(to_dev(v["ar_logits"]), None if v["draft_logits"] is None else to_dev(v["draft_logits"]),
                               to_dev(v["cand"]))
    return a.cpu().numpy(), n.cpu().numpy()


def test_golden_cases(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "verify_cases.json")))
    for case in doc["cases"]:
        v = {"ar_logits": np.array(case["ar_logits"], dtype=np.float32),
             "draft_logits": np.array(case["draft_logits"], dtype=np.float32),
             "cand": np.array(case["cand"], dtype=np.int32)}
        a, n = _verify(v)
        assert a.tolist() == case["accept_len"], case["name"]
        assert n.tolist() == case["next_cand"], case["name"]


@pytest.mark.parametrize("B,k,V,kind", [
    (16, 8, 128256, "uniform"),   # 8B-shaped step
    (8, 4, 151936, "boost"),      # 1.5B-shaped step
    (4, 16, 128256, "geometric"), # long-context step
    (5, 1, 1001, "uniform"),      # no drafts, V not a multiple of 4
    (3, 3, 4097, "uniform"),      # one element past a chunk boundary
    (7, 5, 64, "none"),           # tiny vocab, one chunk
])
def test_verify_matches_oracle(B, k, V, kind):
    v = W.verify_inputs(B, k, V, seed=B * 100 + k, accept=kind, with_drafts=k > 1)
    a, n = _verify(v)
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    assert a.tolist() == ra.tolist()
    assert n.tolist() == rn.tolist()
    if v["planted"] is not None:
        assert a.tolist() == v["planted"].tolist()


def test_verify_ties_everywhere():
    # integer-valued logits: many exact ties, also across chunk boundaries and -0.0/+0.0
    rng = np.random.default_rng(0)
    B, k, V = 6, 4, 9000
    ar = rng.integers(-2, 3, size=(B, k + 1, V)).astype(np.float32)
    ar[ar == 0] = -0.0
    ar[:, :, 5000] = 2.0
    ar[:, :, 4095:4097] = 2.0  # equal maxima both sides of the 4096 boundary
    dr = rng.integers(-1, 2, size=(B, k, k, V)).astype(np.float32)
    cand = np.zeros((B, k), dtype=np.int32)
    cand[:3, 0] = 4095  # lowest maximal index of row 0 is 4095 or lower
    cand[::2, 1] = 0
    v = {"ar_logits": ar, "draft_logits": dr, "cand": cand}
    a, n = _verify(v)
    ra, rn = oracle.verify_ref(ar, dr, cand)
    assert a.tolist() == ra.tolist() and n.tolist() == rn.tolist()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_commit_matches_oracle_over_steps(dtype):
    rng = np.random.default_rng(1)
    B, Hkv, D, S, k = 5, 4, 128, 128, 8
    R = k + k * k
    shape = W.AttnShape(B=B, Hq=Hkv, Hkv=Hkv, D=D, k=k, n_groups=k, lens=(0, 7, 60, 110, 124), S_max=S, dtype=dtype)
    d = W.kv_cache(shape, seed=2, tail="random")
    kc, vc, ln = d["k_cache"], d["v_cache"], d["lens"]
    t_kc, t_vc, t_ln = to_dev(kc, dtype == "bf16"), to_dev(vc, dtype == "bf16"), to_dev(ln)
    for step in range(3):
        rows = W.step_rows(shape, seed=3, step=step)
        a = rng.integers(0, k + 1, size=B).astype(np.int32)
        if step == 2:
            a[4] = 9   # bad length -> flag 2
        ef = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        tidar.kv_commit(t_kc, t_vc, t_ln, to_dev(rows["k_step"], dtype == "bf16"),
                        to_dev(rows["v_step"], dtype == "bf16"), to_dev(a), k, ef)
        kc, vc, ln, ref_ef = oracle.commit_ref(kc, vc, ln, rows["k_step"], rows["v_step"], a, k)
        torch.cuda.synchronize()
        assert ef.cpu().numpy().tolist() == ref_ef.tolist()
        assert t_ln.cpu().numpy().tolist() == ln.tolist()
        assert np.array_equal(bits(t_kc), kc.view(np.uint16) if dtype == "bf16" else kc.view(np.uint32))
        assert np.array_equal(bits(t_vc), vc.view(np.uint16) if dtype == "bf16" else vc.view(np.uint32))


def test_commit_overflow_flag():
    B, Hkv, D, S, k = 2, 1, 64, 64, 4
    kc = torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros((B, Hkv, S // 64, D, 64), dtype=torch.bfloat16, device=DEV)
    ks = torch.ones((B, k + k * k, Hkv, D), dtype=torch.bfloat16, device=DEV)
    lens = torch.tensor([62, 60], dtype=torch.int32, device=DEV)
    a = torch.tensor([3, 4], dtype=torch.int32, device=DEV)
    ef = torch.empty(B, dtype=torch.int32, device=DEV)
    tidar.kv_commit(kc, vc, lens, ks, ks, a, k, ef)
    assert ef.cpu().tolist() == [1, 0]
    assert lens.cpu().tolist() == [62, 64]
    assert float(kc[0].float().abs().sum()) == 0.0 and float(kc[1, 0, 60:64].float().sum()) == 4 * D
    assert float(vc[1, 0, 0, :, 60:64].float().sum()) == 4 * D and float(vc[1].float().sum()) == 4 * D
