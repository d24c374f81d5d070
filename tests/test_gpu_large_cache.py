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


def test_paged_attention_and_commit_past_4gib_match_oracle():
    """A 4.6 GiB page pool per tensor; the checked sequence's pages lie past
    4 GiB and are scattered; attention against the oracle on those pages,
    then a commit into its last page, bit for bit."""
    Bp, n_pages, max_pages = 8, 36000, 520
    g = torch.Generator(device=DEV)
    g.manual_seed(515)
    kp = (torch.randn(n_pages, HKV, 64, D, device=DEV, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    vp = torch.randn(n_pages, HKV, D, 64, device=DEV, generator=g).to(torch.bfloat16)
    q = torch.randn(Bp, R, HQ, D, device=DEV, generator=g).to(torch.bfloat16)
    ks = (torch.randn(Bp, R, HKV, D, device=DEV, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    vs = torch.randn(Bp, R, HKV, D, device=DEV, generator=g).to(torch.bfloat16)
    assert kp.numel() * 2 > (1 << 32)
    rng = np.random.default_rng(3)
    lens_h = np.array([max_pages * 64 - R - 100 * i for i in range(Bp)], dtype=np.int32)
    table = np.full((Bp, max_pages), -1, dtype=np.int32)
    perm = rng.permutation(n_pages)
    high = perm[perm >= 33000][:max_pages]  # page byte offsets past 4.3 GB
    table[Bp - 1] = rng.permutation(high)
    rest = perm[perm < 33000]
    for i in range(Bp - 1):
        table[i] = rest[i * max_pages:(i + 1) * max_pages]
    lens = torch.from_numpy(lens_h).to(DEV)
    tbl = torch.from_numpy(table).to(DEV)
    out, lse = tidar.step_attention_paged(q, ks, vs, kp, vp, tbl, lens, K, NG, 1.0, max_len=max_pages * 64 - R)
    torch.cuda.synchronize()
    b = Bp - 1
    used = torch.from_numpy(table[b]).to(DEV).long()
    kp_b, vp_b = _f32(_host_bf16(kp.index_select(0, used))), _f32(_host_bf16(vp.index_select(0, used)))
    local = np.arange(max_pages, dtype=np.int32)[None]
    ref, ref_lse = oracle.paged_attention_ref(_f32(_host_bf16(q[b:b + 1])), _f32(_host_bf16(ks[b:b + 1])),
                                              _f32(_host_bf16(vs[b:b + 1])), kp_b, vp_b, local, lens_h[b:b + 1], K,
                                              NG, 1.0)
    check_attention(out[b:b + 1], lse[b:b + 1], ref, ref_lse, "bf16", what="paged sequence on pages past 4 GiB")
    # commit k rows of sequence b at its end (its last used page lies past 4 GiB)
    acc_h = np.zeros(Bp, dtype=np.int32)
    acc_h[b] = K
    last = (int(lens_h[b]) + K - 1) // 64
    pages = sorted({int(lens_h[b]) // 64, last})
    before_k = {p: _host_bf16(kp[int(table[b, p])]) for p in pages}
    before_v = {p: _host_bf16(vp[int(table[b, p])]) for p in pages}
    err = torch.full((Bp,), -1, dtype=torch.int32, device=DEV)
    tidar.kv_commit_paged(kp, vp, tbl, lens, ks, vs, torch.from_numpy(acc_h).to(DEV), K, err)
    torch.cuda.synchronize()
    assert int(err[b]) == 0 and int(lens[b]) == int(lens_h[b]) + K
    ksh, vsh = _host_bf16(ks[b]), _host_bf16(vs[b])  # [R][Hkv][D]
    for p in pages:
        want_k, want_v = before_k[p].copy(), before_v[p].copy()  # [Hkv][64][D], [Hkv][D][64]
        for i in range(K):
            pos = int(lens_h[b]) + i
            if pos // 64 == p:
                want_k[:, pos % 64, :] = ksh[i]
                want_v[:, :, pos % 64] = vsh[i]
        assert np.array_equal(_host_bf16(kp[int(table[b, p])]), want_k)
        assert np.array_equal(_host_bf16(vp[int(table[b, p])]), want_v)
    del kp, vp
    torch.cuda.empty_cache()
