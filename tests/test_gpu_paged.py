"""GPU parity of the paged-cache calls (tidar_step_attention_paged,
tidar_kv_commit_paged): element by element against the oracle at small
sizes, bit for bit against the contiguous calls on the same data at the full
8B and long-context sizes, commit bit-exact against the oracle, and a
serving loop whose commits land in pages."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, attn_f32, attn_to_dev, bits, check_attention, to_dev  # noqa: E402


def _pages(d, seed, spare=8):
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=seed, spare=spare)
    return pg, {"k_pool": to_dev(pg["k_pool"], True), "v_pool": to_dev(pg["v_pool"], True),
                "block_table": to_dev(pg["block_table"])}


def _run_paged(t, p, s, max_len=None, kv_chunk=0):
    return tidar.step_attention_paged(t["q"], t["k_step"], t["v_step"], p["k_pool"], p["v_pool"], p["block_table"],
                                      t["lens"], s.k, s.n_groups, s.sm_scale,
                                      max_len=s.max_len if max_len is None else max_len, kv_chunk=kv_chunk)


def _run_contig(t, s, kv_chunk=0):
    return tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], s.k,
                                s.n_groups, s.sm_scale, max_len=s.max_len, kv_chunk=kv_chunk)


SMALL = [
    # B, Hq, Hkv, D, k, n_groups, lens, S_max, kv_chunk
    (3, 8, 2, 128, 3, 3, (70, 0, 191), 256, 0),
    (4, 12, 2, 128, 4, 4, (2048, 5, 64, 1000), 2112, 0),
    (4, 12, 2, 128, 4, 4, (2048, 5, 64, 1000), 2112, 256),   # split keys + merge
    (2, 4, 4, 64, 2, 2, (100, 300), 320, 0),                  # head dim 64
    (5, 8, 8, 128, 1, 0, (63, 64, 65, 0, 130), 192, 0),       # plain decode rows
]


@pytest.mark.parametrize("B,Hq,Hkv,D,k,ng,lens,S_max,kv_chunk", SMALL)
def test_paged_attention_matches_oracle(B, Hq, Hkv, D, k, ng, lens, S_max, kv_chunk):
    s = W.AttnShape(B=B, Hq=Hq, Hkv=Hkv, D=D, k=k, n_groups=ng, lens=lens, S_max=S_max,
                    sm_scale=1.0 / np.sqrt(D))
    print(f"paged B={B} Hq={Hq} Hkv={Hkv} D={D} k={k} lens={lens} chunk={kv_chunk}", flush=True)
    d = W.attention_inputs(s, seed=B + k, tail="nan")  # NaN past lens, NaN spare pages: any stray read shows
    pg, p = _pages(d, seed=B * 3 + k)
    t = attn_to_dev(d, "bf16")
    out, lse = _run_paged(t, p, s, kv_chunk=kv_chunk)
    f = attn_f32(d, "bf16")
    kp, vp = W.bf16_to_f32(pg["k_pool"]), W.bf16_to_f32(pg["v_pool"])
    ref, ref_lse = oracle.paged_attention_ref(f["q"], f["k_step"], f["v_step"], kp, vp, pg["block_table"],
                                              d["lens"], s.k, s.n_groups, s.sm_scale)
    check_attention(out, lse, ref, ref_lse, "bf16", what=f"paged {lens}")
    c_out, c_lse = _run_contig(t, s, kv_chunk=kv_chunk)
    assert np.array_equal(bits(out), bits(c_out)) and np.array_equal(bits(lse), bits(c_lse))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["step_8b", "step_8b_long"])
def test_paged_full_size_equals_contiguous(name):
    wl = W.WORKLOADS[name]()
    s = wl.attn
    print(f"paged {name}: {wl.description}", flush=True)
    d = W.attention_inputs(s, seed=11, config_id=wl.config_id, tail="nan")
    pg, p = _pages(d, seed=5)
    t = attn_to_dev(d, "bf16")
    out, lse = _run_paged(t, p, s)
    c_out, c_lse = _run_contig(t, s)
    assert np.array_equal(bits(out), bits(c_out)), "paged and contiguous outputs differ"
    assert np.array_equal(bits(lse), bits(c_lse))
    pairs = [(0, 0), (s.B - 1, s.Hq - 1), (s.B // 2, 5)]
    f = attn_f32(d, "bf16")
    kp, vp = W.bf16_to_f32(pg["k_pool"]), W.bf16_to_f32(pg["v_pool"])
    ref, ref_lse = oracle.paged_attention_ref(f["q"], f["k_step"], f["v_step"], kp, vp, pg["block_table"],
                                              d["lens"], s.k, s.n_groups, s.sm_scale, pairs=pairs)
    check_attention(out, lse, ref, ref_lse, "bf16", pairs=pairs, what=f"paged {name}")


@pytest.mark.parametrize("kv_chunk", [0, 128])
def test_bad_page_entry_gives_nan_rows_for_that_sequence_only(kv_chunk):
    s = W.AttnShape(B=4, Hq=8, Hkv=2, D=128, k=3, n_groups=3, lens=(300, 130, 64, 500), S_max=512,
                    sm_scale=0.088)
    d = W.attention_inputs(s, seed=3, tail="nan")
    pg, p = _pages(d, seed=1)
    table = pg["block_table"].copy()
    n_pages = pg["k_pool"].shape[0]
    table[1, 2] = n_pages       # page 2 holds settled positions 128..129 of sequence 1
    table[2, 1] = -7            # sequence 2 (lens 64) reads only page 0: never looked at
    p["block_table"] = to_dev(table)
    t = attn_to_dev(d, "bf16")
    out, lse = _run_paged(t, p, s, kv_chunk=kv_chunk)
    o = out.float().cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(lse[1].cpu().numpy()).all()
    c_out, c_lse = _run_contig(t, s, kv_chunk=kv_chunk)
    for b in (0, 2, 3):
        assert np.array_equal(bits(out[b]), bits(c_out[b]))
        assert np.array_equal(bits(lse[b]), bits(c_lse[b]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_commit_matches_oracle(dtype):
    s = W.AttnShape(B=6, Hq=8, Hkv=4, D=128, k=8, n_groups=8, lens=(0, 60, 127, 250, 200, 1000), S_max=1024,
                    dtype=dtype)
    d = W.attention_inputs(s, seed=21, tail="random")
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=2, spare=3)
    table = pg["block_table"].copy()
    table[4, 3] = 10 ** 6                            # positions 192..255 of sequence 4: flag 3
    acc = np.array([8, 4, 3, 6, 8, 5], dtype=np.int32)  # sequence 5: 1000 + 5 > 1024? no; sequence 3: 256 ok
    acc[5] = 30                                      # above k: flag 2
    bf = dtype == "bf16"
    kp_d, vp_d = to_dev(pg["k_pool"], bf), to_dev(pg["v_pool"], bf)
    ln_d = to_dev(d["lens"])
    ef = torch.full((s.B,), -1, dtype=torch.int32, device=DEV)
    tidar.kv_commit_paged(kp_d, vp_d, to_dev(table), ln_d, to_dev(d["k_step"], bf), to_dev(d["v_step"], bf),
                          to_dev(acc), s.k, ef)
    kp2, vp2, ln2, err = oracle.commit_paged_ref(pg["k_pool"], pg["v_pool"], table, d["lens"], d["k_step"],
                                                 d["v_step"], acc, s.k)
    assert ef.cpu().numpy().tolist() == err.tolist() == [0, 0, 0, 0, 3, 2]
    assert ln_d.cpu().numpy().tolist() == ln2.tolist()
    assert np.array_equal(bits(kp_d), kp2.view(bits(kp_d).dtype))
    assert np.array_equal(bits(vp_d), vp2.view(bits(vp_d).dtype))


@pytest.mark.timeout(600)
def test_paged_serving_loop_tracks_the_contiguous_one():
    """The ragged serving loop (batch 32, lengths U{512..8192}, k = 8), run
    on paged and on contiguous caches side by side for 64 steps: every
    step's attention is bit-identical, and at the end the pages hold exactly
    the contiguous caches' rows, spare pages untouched."""
    wl = W.ragged_8b(seed=0)
    s = wl.attn
    B, k, cid = s.B, s.k, wl.config_id
    steps = 64
    cache = W.kv_cache(s, seed=0, config_id=cid, tail="zero")
    pg = W.to_pages(cache["k_cache"], cache["v_cache"], seed=7, spare=16)
    kc, vc = to_dev(cache["k_cache"], True), to_dev(cache["v_cache"], True)
    kp, vp, tbl = to_dev(pg["k_pool"], True), to_dev(pg["v_pool"], True), to_dev(pg["block_table"])
    lens_c, lens_p = to_dev(cache["lens"]), to_dev(cache["lens"])
    err_c = torch.zeros(B, dtype=torch.int32, device=DEV)
    err_p = torch.zeros(B, dtype=torch.int32, device=DEV)
    ws = torch.zeros(max(tidar.step_attention_workspace_bytes(0, B, s.Hq, s.Hkv, s.D, s.S_max, s.S_max - k, k, k),
                         256), dtype=torch.uint8, device=DEV)
    print(f"paged loop: B={B} lens {min(s.lens)}..{max(s.lens)} pages {pg['k_pool'].shape[0]}", flush=True)
    for t in range(steps):
        rows = W.step_rows_device(s, 0, t, DEV, config_id=cid)
        acc = to_dev(W.accept_lengths("uniform", B, k, 0, t, cid))
        max_len = max(s.lens) + t * k
        o_c, l_c = tidar.step_attention(rows["q"], rows["k_step"], rows["v_step"], kc, vc, lens_c, k, k, s.sm_scale,
                                        max_len=max_len, workspace=ws)
        o_c, l_c = o_c.clone(), l_c.clone()
        o_p, l_p = tidar.step_attention_paged(rows["q"], rows["k_step"], rows["v_step"], kp, vp, tbl, lens_p, k, k,
                                              s.sm_scale, max_len=max_len, workspace=ws)
        assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16)), f"step {t}: outputs differ"
        assert torch.equal(l_p.view(torch.int32), l_c.view(torch.int32)), f"step {t}: lse differs"
        tidar.kv_commit(kc, vc, lens_c, rows["k_step"], rows["v_step"], acc, k, err_c)
        tidar.kv_commit_paged(kp, vp, tbl, lens_p, rows["k_step"], rows["v_step"], acc, k, err_p)
        assert int(err_c.abs().sum()) == 0 and int(err_p.abs().sum()) == 0
    assert torch.equal(lens_c, lens_p)
    lens = lens_c.cpu().numpy()
    kc_h, vc_h = bits(kc), bits(vc)
    kp_h, vp_h = bits(kp), bits(vp)
    g_k, g_v = oracle.gather_paged(kp_h, vp_h, pg["block_table"], lens, s.S_max)
    for b in range(B):
        L = int(lens[b])
        assert np.array_equal(g_k[b, :, :L], kc_h[b, :, :L]), f"sequence {b}: keys differ"
        assert np.array_equal(W.v_natural(g_v[b])[:, :L], W.v_natural(vc_h[b])[:, :L]), f"sequence {b}: values"
    spare = np.setdiff1d(np.arange(kp_h.shape[0]), pg["block_table"].reshape(-1))
    assert len(spare) == 16 and np.array_equal(kp_h[spare], pg["k_pool"][spare])
