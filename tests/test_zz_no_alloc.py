"""GPU check of the allocation-free fused verification + KV commit
(tidar_verify_commit_greedy_noalloc): called through the C ABI, its results
must equal those of tidar_verify_commit_greedy (bit for bit: accept lengths,
next drafts, flags, settled lengths and both caches) on consecutive calls
of different sizes, which share the library's per-GPU state; a size whose
state exceeds the array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, bits, to_dev  # noqa: E402


def _inputs(B, k, V, Hkv, D, S, lens, dtype, seed):
    v = W.verify_inputs(B, k, V, seed=seed, accept="uniform", with_drafts=k > 1)
    shape = W.AttnShape(B=B, Hq=Hkv, Hkv=Hkv, D=D, k=k, n_groups=k, lens=tuple(lens), S_max=S, dtype=dtype)
    d = W.kv_cache(shape, seed=seed, tail="random")
    d.update(W.step_rows(shape, seed=seed))
    return v, d


def _dev(v, d, dtype):
    bf = dtype == "bf16"
    B, k = v["cand"].shape
    return {"ar": to_dev(v["ar_logits"]), "dr": None if k == 1 else to_dev(v["draft_logits"]),
            "cand": to_dev(v["cand"]), "kc": to_dev(d["k_cache"], bf), "vc": to_dev(d["v_cache"], bf),
            "ln": to_dev(d["lens"]), "ks": to_dev(d["k_step"], bf), "vs": to_dev(d["v_step"], bf),
            "a": torch.full((B,), -7, dtype=torch.int32, device=DEV),
            "n": torch.full((B, k), -7, dtype=torch.int32, device=DEV),
            "err": torch.full((B,), -7, dtype=torch.int32, device=DEV)}


def _results(t):
    return {"accept_len": t["a"].cpu().numpy(), "next_cand": t["n"].cpu().numpy(), "err": t["err"].cpu().numpy(),
            "lens": t["ln"].cpu().numpy(), "k_cache": bits(t["kc"]), "v_cache": bits(t["vc"])}


def _one_call(B, k, V, Hkv, D, S, dtype, seed):
    lens = [(41 * i + 3) % (S - k) for i in range(B)]
    v, d = _inputs(B, k, V, Hkv, D, S, lens, dtype, seed)
    ref = _dev(v, d, dtype)
    tidar.verify_commit_greedy(ref["ar"], ref["dr"], ref["cand"], ref["kc"], ref["vc"], ref["ln"], ref["ks"],
                               ref["vs"], accept_len=ref["a"], next_cand=ref["n"], err_flags=ref["err"])
    got = _dev(v, d, dtype)
    tidar.verify_commit_greedy_noalloc(got["ar"], got["dr"], got["cand"], got["kc"], got["vc"], got["ln"],
                                       got["ks"], got["vs"], got["a"], got["n"], got["err"])
    torch.cuda.synchronize()
    r, g = _results(ref), _results(got)
    for name in r:
        assert np.array_equal(r[name], g[name]), f"{name} differs (B={B}, k={k}, V={V})"
    assert (r["accept_len"] >= 0).all() and (r["err"] >= 0).all()


def test_noalloc_matches_the_state_entry_point_on_consecutive_calls():
    # an 8B-shaped step, then a smaller one, then the first size again: the
    # calls share the per-GPU state, which each leaves cleared
    _one_call(16, 8, 128256, 8, 128, 256, "bf16", seed=1)
    _one_call(5, 3, 4097, 2, 64, 128, "f32", seed=2)
    _one_call(16, 8, 128256, 8, 128, 256, "bf16", seed=3)


def test_noalloc_refuses_a_state_beyond_the_array():
    B, k, V, Hkv, D, S = 1024, 16, 64, 1, 64, 64
    n_state = tidar.verify_commit_state_bytes(B, k)
    assert n_state > 2 * 1024 * 1024
    t = {"ar": torch.zeros((B, k + 1, V), dtype=torch.float32, device=DEV),
         "dr": torch.zeros((B, k, k, V), dtype=torch.float32, device=DEV),
         "cand": torch.zeros((B, k), dtype=torch.int32, device=DEV),
         "kc": torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16, device=DEV),
         "vc": torch.zeros((B, Hkv, S // 64, D, 64), dtype=torch.bfloat16, device=DEV),
         "ln": torch.zeros((B,), dtype=torch.int32, device=DEV),
         "ks": torch.zeros((B, k + k * k, Hkv, D), dtype=torch.bfloat16, device=DEV),
         "vs": torch.zeros((B, k + k * k, Hkv, D), dtype=torch.bfloat16, device=DEV),
         "a": torch.full((B,), -7, dtype=torch.int32, device=DEV),
         "n": torch.full((B, k), -7, dtype=torch.int32, device=DEV)}
    with pytest.raises(tidar.TidarError) as e:
        tidar.verify_commit_greedy_noalloc(t["ar"], t["dr"], t["cand"], t["kc"], t["vc"], t["ln"], t["ks"],
                                           t["vs"], t["a"], t["n"])
    assert e.value.status == tidar.TIDAR_EWORKSPACE
    torch.cuda.synchronize()
    assert int((t["a"] != -7).sum()) == 0 and int(t["ln"].abs().sum()) == 0  # nothing ran
