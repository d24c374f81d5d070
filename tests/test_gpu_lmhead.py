"""GPU parity of tidar_lmhead_verify_greedy (LM head fused with greedy
verification) against the oracle.

Accept lengths and tokens must be identical, except where the oracle's two
best logits of a decided row lie within MARGIN of each other: the kernel
takes the argmax over fp32 accumulations of bf16 products, the oracle in
float64, so such a row may legitimately go either way.  A close AR row
fixes only the rows before it; a close draft row fixes the others."""
import numpy as np
import pytest

import workloads as W
from oracle.lmhead import lmhead_verify_ref

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import bits, to_dev  # noqa: E402

MARGIN = 1e-3


def _run(d):
    hd = None if d["h_draft"] is None else to_dev(d["h_draft"], True)
    a, n = tidar.lmhead_verify_greedy(to_dev(d["h_ar"], True), hd, to_dev(d["w"], True), to_dev(d["cand"]))
    return a.cpu().numpy(), n.cpu().numpy()


def _run_packed(d):
    hd = None if d["h_draft"] is None else to_dev(d["h_draft"], True)
    w = to_dev(d["w"], True)
    a, n = tidar.lmhead_verify_greedy_packed(to_dev(d["h_ar"], True), hd, tidar.lmhead_pack(w), w.shape[0],
                                             to_dev(d["cand"]))
    return a.cpu().numpy(), n.cpu().numpy()


def _f32(x):
    return None if x is None else W.bf16_to_f32(x)


def _compare(d, a, n, seqs, what):
    k = d["cand"].shape[1]
    sub = lambda x: None if x is None else x[seqs]
    ra, rn, mg = lmhead_verify_ref(_f32(sub(d["h_ar"])), _f32(sub(d["h_draft"])), _f32(d["w"]), d["cand"][seqs],
                                   margins=True)
    near = 0
    for j, b in enumerate(seqs):
        m = mg[j]
        n_ar = len(m) - (k - 1)  # AR rows decided: a + 1
        close_ar = [i for i in range(n_ar) if m[i] < MARGIN]
        close_dr = [i for i in range(k - 1) if m[n_ar + i] < MARGIN]
        near += bool(close_ar or close_dr)
        if close_ar:
            assert a[b] >= close_ar[0], f"{what} b={b}: accept {a[b]} below close row {close_ar[0]}"
            continue
        assert a[b] == ra[j], f"{what} b={b}: accept {a[b]} != {ra[j]}"
        assert n[b, 0] == rn[j, 0], f"{what} b={b}: bonus token"
        far = [1 + i for i in range(k - 1) if i not in close_dr]
        assert n[b, far].tolist() == rn[j, far].tolist(), f"{what} b={b}: drafts"
    return near


SHAPES = [
    (4, 8, 32000, 1024, "uniform"),
    (6, 4, 5003, 256, "uniform"),      # V ends mid-chunk
    (5, 1, 1000, 64, "uniform"),       # no drafts
    (150, 3, 257, 128, "uniform"),     # 600 AR rows: five row groups; a one-entry last chunk
    (3, 16, 4096, 512, "geometric"),   # k = 16
    (18, 3, 3001, 128, "uniform"),     # 72 AR rows: five row tiles per workgroup
    (22, 3, 2049, 64, "uniform"),      # 88 AR rows: six row tiles
    (30, 3, 1024, 192, "geometric"),   # 120 AR rows: eight row tiles
]


@pytest.mark.parametrize("B,k,V,d,accept", SHAPES)
def test_lmhead_verify_matches_oracle(B, k, V, d, accept):
    print(f"lmhead B={B} k={k} V={V} d={d}", flush=True)
    data = W.lmhead_inputs(B, k, V, d, seed=B + k + d, accept=accept)
    a, n = _run(data)
    near = _compare(data, a, n, list(range(B)), f"B={B} k={k} V={V} d={d}")
    assert near <= max(1, B // 8)
    assert a.tolist() == data["planted"].tolist()  # planted rows have wide margins


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,B,k,V,d", [("8B", 16, 8, 128256, 4096), ("1.5B", 8, 4, 151936, 1536)])
def test_lmhead_verify_full_size(name, B, k, V, d):
    """The 8B- and 1.5B-shaped heads on the whole batch; the oracle checks
    three sequences (each row costs it a V x d product in float64), the
    planted accept lengths check all of them."""
    print(f"lmhead full size {name}: B={B} k={k} V={V} d={d}", flush=True)
    data = W.lmhead_inputs(B, k, V, d, seed=5, accept="uniform")
    a, n = _run(data)
    assert a.tolist() == data["planted"].tolist()
    assert ((n >= 0) & (n < V)).all()
    _compare(data, a, n, [0, B // 2, B - 1], name)
    # the packed head gives the same bits: the same products in the same order
    ap, np_ = _run_packed(data)
    assert ap.tolist() == a.tolist() and np_.tolist() == n.tolist()


def _packed_layout(w_bits, V, d):
    """The packed layout as tidar.h states it: tile (c, s) at byte
    (c * (d/64) + s) * 32768 holds, at byte 128 r + 16 j, the 8 elements of
    row 256 c + r from column 64 s + 8 (j ^ (r % 8)); rows past V are zero."""
    nc, ns = -(-V // 256), d // 64
    wp = np.zeros((nc * 256, d), dtype=np.uint16)
    wp[:V] = w_bits
    out = np.empty((nc, ns, 256, 8, 8), dtype=np.uint16)
    r = np.arange(256)
    for j in range(8):
        src = 8 * (j ^ (r % 8))                       # first column of physical piece j, per row
        for s in range(ns):
            cols = 64 * s + src[:, None] + np.arange(8)[None, :]
            out[:, s, :, j, :] = wp.reshape(nc, 256, d)[:, r[:, None], cols]
    return out.reshape(-1)


@pytest.mark.parametrize("V,d", [(3001, 128), (256, 64), (5, 192)])
def test_pack_layout(V, d):
    print(f"lmhead pack V={V} d={d}", flush=True)
    w = W.lmhead_inputs(1, 1, V, d, seed=V + d)["w"]
    got = bits(tidar.lmhead_pack(to_dev(w, True)))
    assert got.tolist() == _packed_layout(w, V, d).tolist()


@pytest.mark.parametrize("B,k,V,d,accept", SHAPES)
def test_packed_head_matches_row_major(B, k, V, d, accept):
    """The packed W changes only where the kernel reads each tile from: the
    results are the row-major head's, bit for bit, and the planted accept
    lengths."""
    print(f"lmhead packed B={B} k={k} V={V} d={d}", flush=True)
    data = W.lmhead_inputs(B, k, V, d, seed=B + k + d, accept=accept)
    a, n = _run(data)
    ap, np_ = _run_packed(data)
    assert ap.tolist() == a.tolist() and np_.tolist() == n.tolist()
    assert ap.tolist() == data["planted"].tolist()


def test_equal_logits_take_the_lowest_index_across_chunks():
    B, k, V, d = 2, 3, 800, 128
    data = W.lmhead_inputs(B, k, V, d, seed=9, accept="uniform")
    w = data["w"].copy()
    w[300] = w[17]
    w[700] = w[17]       # three equal rows in three chunks of 256
    data["w"] = w
    h = data["h_ar"].copy()
    h[:, 0] = W.bf16_bits(np.float32(12.0) * W.bf16_to_f32(w[300]))  # AR row 0 aligned with the tied rows
    data["h_ar"] = h
    data["cand"][:, 0] = 17
    a, n = _run(data)
    ra, rn = lmhead_verify_ref(_f32(data["h_ar"]), _f32(data["h_draft"]), _f32(data["w"]), data["cand"])
    assert (a >= 1).all() and a.tolist() == ra.tolist() and n.tolist() == rn.tolist()
