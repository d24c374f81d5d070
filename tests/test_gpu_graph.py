"""A whole TiDAR step (attention, greedy verification, KV commit) captured in
a HIP graph and replayed: every replay equals the eager step bit for bit.

The step is what bench.py replays.  Replays are interleaved with eager work
on other buffers and with synchronisations, and each one checks every output
(attention rows and LSE, accept lengths, next candidates, the committed
caches and the advanced lengths).  The commit writes the caches and lengths
in place, so the captured step starts by copying the pristine inputs back."""
import math

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
import torch  # noqa: E402
from _gpu_util import bits, to_dev  # noqa: E402


def _case(seed):
    shape = W.AttnShape(B=3, Hq=8, Hkv=2, D=128, k=4, n_groups=4, lens=(200, 64, 131), S_max=384,
                        sm_scale=1.0 / math.sqrt(128.0))
    d = W.attention_inputs(shape, seed=seed, tail="zero")
    v = W.verify_inputs(shape.B, shape.k, 5003, seed=seed + 1, accept="uniform")
    t = {n: to_dev(x, n != "lens") for n, x in d.items()}
    t.update({"ar_logits": to_dev(v["ar_logits"]), "draft_logits": to_dev(v["draft_logits"]),
              "cand": to_dev(v["cand"])})
    s = shape
    ws_a = tidar.step_attention_workspace_bytes(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, s.max_len, s.k, s.n_groups)
    t.update({
        "k0": t["k_cache"].clone(), "v0": t["v_cache"].clone(), "lens0": t["lens"].clone(),
        "out": torch.empty_like(t["q"]), "lse": torch.empty((s.B, s.Hq, s.R), dtype=torch.float32, device=t["q"].device),
        "ws_a": torch.zeros(max(ws_a, 256), dtype=torch.uint8, device=t["q"].device),
        "ws_v": torch.empty(tidar.verify_workspace_bytes(s.B, s.k, 5003), dtype=torch.uint8, device=t["q"].device),
        "acc": torch.empty(s.B, dtype=torch.int32, device=t["q"].device),
        "next": torch.empty((s.B, s.k), dtype=torch.int32, device=t["q"].device),
        "err": torch.empty(s.B, dtype=torch.int32, device=t["q"].device),
    })
    return shape, t


def _step(s, t):
    t["k_cache"].copy_(t["k0"])
    t["v_cache"].copy_(t["v0"])
    t["lens"].copy_(t["lens0"])
    tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], s.k, s.n_groups,
                         s.sm_scale, max_len=s.max_len, out=t["out"], lse=t["lse"], workspace=t["ws_a"])
    tidar.verify_greedy(t["ar_logits"], t["draft_logits"], t["cand"], accept_len=t["acc"], next_cand=t["next"],
                        workspace=t["ws_v"])
    tidar.kv_commit(t["k_cache"], t["v_cache"], t["lens"], t["k_step"], t["v_step"], t["acc"], s.k, t["err"])


NAMES = ("out", "lse", "acc", "next", "k_cache", "v_cache", "lens", "err")


def _snapshot(t):
    return {n: bits(t[n]).copy() for n in NAMES}


def test_graph_replays_equal_the_eager_step():
    print("graph: capture and replay one step", flush=True)
    s, t = _case(seed=21)
    _step(s, t)
    torch.cuda.synchronize()
    ref = _snapshot(t)
    assert (ref["err"] == 0).all()

    side_s, side = _case(seed=22)  # eager work between replays
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        _step(s, t)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(s, t)
    torch.cuda.synchronize()
    for rep in range(4):
        for n in ("out", "lse", "acc", "next"):
            t[n].fill_(-1 if n in ("acc", "next") else 0)  # poison the outputs the replay must rewrite
        g.replay()
        _step(side_s, side)
        torch.cuda.synchronize()
        got = _snapshot(t)
        for n in NAMES:
            assert np.array_equal(got[n], ref[n]), f"replay {rep}: {n}"
