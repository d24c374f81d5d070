"""GPU parity with KV caches past 4 GiB: every cache address the kernels form
is a 64-bit product (a 64-bit tile base plus a 32-bit offset inside the tile
for the direct loads), so a sequence whose keys start beyond 2^32 bytes must
give the oracle's attention and take its commit at the right place.

The caches (about 4.8 GB of keys and as much of values) are drawn on the
device from a seeded torch generator; the oracle receives copies of the
slices it checks: the last sequence (its K/V start past 4.5 GiB) and the
first one.  Attention, the separate commit and the fused verify + commit
are checked there."""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, bits, check_attention  # noqa: E402

B, HQ, HKV, D, K, NG = 72, 32, 8, 128, 4, 4
S_MAX = 32832  # 513 pages of 64
R = K + NG * K


def _host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f32(x):
    return (x.astype(np.uint32) << 16).view(np.float32)


@pytest.fixture(scope="module")
def big():
    g = torch.Generator(device=DEV)
    g.manual_seed(20241)
    kc = (torch.randn(B, HKV, S_MAX, D, device=DEV, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    vc = torch.randn(B, HKV, S_MAX // 64, D, 64, device=DEV, generator=g).to(torch.bfloat16)
    q = torch.randn(B, R, HQ, D, device=DEV, generator=g).to(torch.bfloat16)
    ks = (torch.randn(B, R, HKV, D, device=DEV, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    vs = torch.randn(B, R, HKV, D, device=DEV, generator=g).to(torch.bfloat16)
    lens_h = np.array([S_MAX - R - 64 * (i % 7) - (i * 13) % 61 for i in range(B)], dtype=np.int32)
    lens_h[-1] = S_MAX - R  # the last sequence: a full cache
    assert kc.numel() * 2 > (1 << 32) and (B - 1) * HKV * S_MAX * D * 2 > (1 << 32)
    yield {"kc": kc, "vc": vc, "q": q, "ks": ks, "vs": vs, "lens_h": lens_h}
    del kc, vc
    torch.cuda.empty_cache()


def _one(t, b):
    """Host copies of sequence b's inputs, as a batch of one."""
    return {"q": _f32(_host_bf16(t["q"][b:b + 1])), "ks": _f32(_host_bf16(t["ks"][b:b + 1])),
            "vs": _f32(_host_bf16(t["vs"][b:b + 1])), "kc": _f32(_host_bf16(t["kc"][b:b + 1])),
            "vc": _f32(_host_bf16(t["vc"][b:b + 1]))}


def test_attention_past_4gib_matches_oracle(big):
    t = big
    lens = torch.from_numpy(t["lens_h"]).to(DEV)
    sm = 1.0
    print(f"large cache: K cache {t['kc'].numel() * 2 / 2**30:.2f} GiB, B={B} S_max={S_MAX}", flush=True)
    out, lse = tidar.step_attention(t["q"], t["ks"], t["vs"], t["kc"], t["vc"], lens, K, NG, sm,
                                    max_len=S_MAX - R)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        h = _one(t, b)
        ref, ref_lse = oracle.attention_ref(h["q"], h["ks"], h["vs"], h["kc"], h["vc"], t["lens_h"][b:b + 1], K, NG,
                                            sm)
        check_attention(out[b:b + 1], lse[b:b + 1], ref, ref_lse, "bf16", what=f"sequence {b} of a >4 GiB cache")
    assert torch.isfinite(out.float()).all()


def test_commit_past_4gib_matches_oracle(big):
    t = big
    b = B - 1
    lens_h = t["lens_h"].copy()
    lens_h[b] = S_MAX - R  # positions S_MAX-R .. S_MAX-R+3: the cache's last page
    acc_h = np.zeros(B, dtype=np.int32)
    acc_h[b] = K
    before = {"kc": _host_bf16(t["kc"][b:b + 1]), "vc": _host_bf16(t["vc"][b:b + 1])}
    lens = torch.from_numpy(lens_h).to(DEV)
    err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    tidar.kv_commit(t["kc"], t["vc"], lens, t["ks"], t["vs"], torch.from_numpy(acc_h).to(DEV), K, err)
    torch.cuda.synchronize()
    rk, rv, rl, re = oracle.commit_ref(before["kc"], before["vc"], lens_h[b:b + 1], _host_bf16(t["ks"][b:b + 1]),
                                       _host_bf16(t["vs"][b:b + 1]), acc_h[b:b + 1], K)
    assert int(err[b]) == int(re[0]) == 0 and int(lens[b]) == int(rl[0])
    assert np.array_equal(bits(t["kc"][b:b + 1]), rk) and np.array_equal(bits(t["vc"][b:b + 1]), rv)
    assert (err.cpu().numpy() == 0).all() and lens.cpu().numpy().tolist()[:-1] == lens_h.tolist()[:-1]


def test_fused_verify_commit_past_4gib_matches_oracle(big):
    import workloads as W
    t = big
    V = 1000
    v = W.verify_inputs(B, K, V, seed=7, accept="uniform")
    lens_h = t["lens_h"].copy()
    lens_h[-1] = S_MAX - R - 64  # the commit lands in one of the cache's last pages
    ra, rn = oracle.verify_ref(v["ar_logits"], v["draft_logits"], v["cand"])
    b = B - 1
    before = {"kc": _host_bf16(t["kc"][b:b + 1]), "vc": _host_bf16(t["vc"][b:b + 1])}
    lens = torch.from_numpy(lens_h).to(DEV)
    err = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    a, n = tidar.verify_commit_greedy(torch.from_numpy(v["ar_logits"]).to(DEV),
                                      torch.from_numpy(v["draft_logits"]).to(DEV),
                                      torch.from_numpy(v["cand"]).to(DEV), t["kc"], t["vc"], lens, t["ks"], t["vs"],
                                      err_flags=err, state=tidar.verify_commit_state(B, K, DEV))
    torch.cuda.synchronize()
    assert a.cpu().numpy().tolist() == ra.tolist() and n.cpu().numpy().tolist() == rn.tolist()
    rk, rv, rl, re = oracle.commit_ref(before["kc"], before["vc"], lens_h[b:b + 1], _host_bf16(t["ks"][b:b + 1]),
                                       _host_bf16(t["vs"][b:b + 1]), ra[b:b + 1], K)
    assert int(err[b]) == int(re[0]) and int(lens[b]) == int(rl[0])
    assert np.array_equal(bits(t["kc"][b:b + 1]), rk) and np.array_equal(bits(t["vc"][b:b + 1]), rv)
