"""GPU parity of tidar_train_attention (the duplicated training sequence:
causal clean half, masked half in blocks) against the oracle: element by
element at small sizes, on sampled rows at the full training shape, with
each of the two kernels (TIDAR_ATTN_KERNEL: "pipe" four waves, "pp" eight
waves; head dim 64 has the four-wave kernel only)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle.train_mask import train_attention_ref

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import TOL, to_dev  # noqa: E402


def _run(d, N, bs, scale):
    return tidar.train_attention(to_dev(d["q"], True), to_dev(d["k"], True), to_dev(d["v"], True), N, bs, scale)


def _check(out, lse, ref, ref_lse, sel, what):
    """sel: list of (b, h, r) rows compared."""
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    got = np.stack([o[b, r, h] for b, h, r in sel])
    want = np.stack([ref[b, r, h] for b, h, r in sel])
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    err = np.abs(got - want)
    mean_rel = err.sum() / np.abs(want).sum()
    assert err.max() <= TOL["bf16"]["max_abs"], f"{what}: max-abs {err.max():.3e}"
    assert mean_rel <= TOL["bf16"]["mean_rel"], f"{what}: mean-rel {mean_rel:.3e}"
    lerr = max(abs(l[b, h, r] - ref_lse[b, h, r]) for b, h, r in sel)
    assert lerr <= TOL["bf16"]["lse"], f"{what}: lse err {lerr:.3e}"


SMALL = [
    # B, Hq, Hkv, D, N, block
    (2, 4, 2, 128, 64, 8),
    (1, 8, 2, 64, 128, 5),      # blocks cross tile boundaries, partial last block
    (1, 4, 4, 128, 192, 192),   # one block: the masked copy is bidirectional
    (2, 6, 2, 128, 128, 1),     # blocks of one token
    (1, 12, 2, 128, 256, 16),   # 1.5B-shaped heads
]


@pytest.mark.parametrize("kern", ["pipe", "pp"])
@pytest.mark.parametrize("B,Hq,Hkv,D,N,bs", SMALL)
def test_train_attention_matches_oracle(monkeypatch, kern, B, Hq, Hkv, D, N, bs):
    monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    print(f"train {kern} B={B} Hq={Hq} Hkv={Hkv} D={D} N={N} block={bs}", flush=True)
    d = W.train_inputs(B, Hq, Hkv, D, N, seed=N + bs)
    scale = 1.0 / np.sqrt(D)
    out, lse = _run(d, N, bs, scale)
    ref, ref_lse = train_attention_ref(W.bf16_to_f32(d["q"]), W.bf16_to_f32(d["k_nat"]), W.bf16_to_f32(d["v_nat"]),
                                       N, bs, scale)
    sel = [(b, h, r) for b in range(B) for h in range(Hq) for r in range(2 * N)]
    _check(out, lse, ref, ref_lse, sel, f"N={N} block={bs}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kern", ["pipe", "pp"])
def test_train_attention_full_size_sampled(monkeypatch, kern):
    monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    B, Hq, Hkv, D, N, bs = 4, 32, 8, 128, 4096, 8
    print(f"train full size {kern} B={B} N={N} block={bs}", flush=True)
    d = W.train_inputs(B, Hq, Hkv, D, N, seed=1)
    scale = 1.0 / np.sqrt(D)
    out, lse = _run(d, N, bs, scale)
    rng = np.random.default_rng(2)
    rows = [0, 1, 63, 64, N - 1, N, N + 7, N + 8, 2 * N - 9, 2 * N - 8, 2 * N - 1]
    rows += [int(x) for x in rng.integers(0, 2 * N, size=12)]
    sel = [(int(rng.integers(B)), int(rng.integers(Hq)), r) for r in rows]
    ref, ref_lse = train_attention_ref(W.bf16_to_f32(d["q"]), W.bf16_to_f32(d["k_nat"]), W.bf16_to_f32(d["v_nat"]),
                                       N, bs, scale, rows=sel)
    _check(out, lse, ref, ref_lse, sel, "full size")
    assert torch.isfinite(out.float()).all()
