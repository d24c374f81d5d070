"""GPU parity at the full sizes of the 1.5B-shaped, 8B-shaped and long-context
8B-shaped steps, in the launch configuration bench.py times (the library's
own split plan), and on the 8B step with each of the two attention kernels.
Attention: every (sequence, head) of the 1.5B and 8B steps, and every head
of the first and last sequence of the long-context step (the oracle takes
about a second per 8B step); outputs are pre-filled with NaN so an unwritten
row shows.  Verify and commit bit-exact on the whole batch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, attn_f32, attn_to_dev, bits, check_attention, to_dev  # noqa: E402

NAMES = ["step_1p5b", "step_8b", "step_8b_long"]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,kern", [("step_1p5b", None), ("step_8b", None), ("step_8b", "pipe"),
                                       ("step_8b", "pp"), ("step_8b_long", None)])
def test_full_size_attention(monkeypatch, name, kern):
    wl = W.WORKLOADS[name]()
    s = wl.attn
    if kern:
        monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    plan = tidar.step_attention_plan(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, s.max_len, s.k, s.n_groups)
    print(f"{name} ({kern or 'library plan'}): {wl.description}; plan {plan}", flush=True)
    d = W.attention_inputs(s, seed=7, config_id=wl.config_id, tail="nan")  # NaN past lens: never read
    t = attn_to_dev(d, "bf16")
    out = torch.full(tuple(t["q"].shape), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((s.B, s.Hq, s.R), float("nan"), dtype=torch.float32, device=DEV)
    tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], s.k, s.n_groups,
                         s.sm_scale, max_len=s.max_len, out=out, lse=lse)
    pairs = None
    if name == "step_8b_long":  # every head of two whole sequences
        pairs = [(b, h) for b in (0, s.B - 1) for h in range(s.Hq)]
    f = attn_f32(d, "bf16")
    ref, ref_lse = oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"], s.k,
                                        s.n_groups, s.sm_scale, pairs=pairs)
    check_attention(out, lse, ref, ref_lse, "bf16", pairs=pairs, what=name)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", NAMES)
def test_full_size_verify(name):
    wl = W.WORKLOADS[name]()
    s = wl.attn
    v = W.verify_inputs(s.B, s.k, wl.V, seed=7, config_id=wl.config_id, accept=wl.accept)
    a, n = tidar.verify_greedy(to_dev(v["ar_logits"]), to_dev(v["draft_logits"]), to_dev(v["cand"]))
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    assert a.cpu().numpy().tolist() == ra.tolist()
    assert n.cpu().numpy().tolist() == rn.tolist()
    if v["planted"] is not None:
        assert ra.tolist() == v["planted"].tolist()


@pytest.mark.timeout(300)
def test_full_size_commit_8b():
    wl = W.step_8b()
    s = wl.attn
    d = W.attention_inputs(s, seed=8, config_id=wl.config_id, tail="random")
    a = W.accept_lengths("uniform", s.B, s.k, seed=8, config_id=wl.config_id)
    kc, vc, ln = to_dev(d["k_cache"], True), to_dev(d["v_cache"], True), to_dev(d["lens"])
    ef = torch.full((s.B,), -1, dtype=torch.int32, device=DEV)
    tidar.kv_commit(kc, vc, ln, to_dev(d["k_step"], True), to_dev(d["v_step"], True), to_dev(a), s.k, ef)
    rk, rv, rl, re = oracle.commit_ref(d["k_cache"], d["v_cache"], d["lens"], d["k_step"], d["v_step"], a, s.k)
    assert ef.cpu().numpy().tolist() == re.tolist()
    assert ln.cpu().numpy().tolist() == rl.tolist()
    assert np.array_equal(bits(kc), rk) and np.array_equal(bits(vc), rv)
