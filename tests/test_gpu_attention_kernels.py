"""GPU parity of both bf16 step-attention kernels against the float64 oracle.

The library has two bf16 kernels: four waves per workgroup (one per SIMD)
and eight waves (two per SIMD, head dim 128).  Its planner picks one per
shape; TIDAR_ATTN_KERNEL restricts the choice, so every case here runs on
each kernel in turn, and the plan query confirms which one ran.  Cases: the
shapes of test_gpu_attention.py with head dim 128, workgroups of exactly
nine row tiles (the eight-wave kernel's shared tile), one row tile, every
split count, paged caches, and scores large enough that the held softmax
reference overflows and the chunk is recomputed exactly.  Cache rows past
every length hold NaN, and the outputs are pre-filled with NaN, so a read of
an unsettled position or an unwritten output shows."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, attn_f32, attn_to_dev, check_attention, to_dev  # noqa: E402

KERNELS = {"pp": "eight_wave", "pipe": "four_wave"}


def _shape(B, Hq, Hkv, k, n_groups, lens, scale=None, k_prescale=1.0, S_max=None):
    S_max = S_max or ((max(lens) + 64 + 63) // 64 * 64)
    return W.AttnShape(B=B, Hq=Hq, Hkv=Hkv, D=128, k=k, n_groups=n_groups, lens=tuple(lens), S_max=S_max,
                       sm_scale=scale or 1.0 / math.sqrt(128), k_prescale=k_prescale)


CASES = {
    "gqa4_k4_ragged": _shape(3, 8, 2, 4, 4, (0, 37, 300)),
    "gqa6_k4": _shape(2, 12, 2, 4, 4, (130, 1)),
    "zero_drafts_k5": _shape(2, 8, 2, 5, 0, (77, 200)),
    "single_token_decode": _shape(3, 8, 8, 1, 0, (1, 64, 65)),
    "k16_rows1088": _shape(1, 8, 2, 16, 16, (700,)),
    # 288 rows per KV head over 128 (sequence, KV head) pairs: two
    # workgroups of nine 16-row tiles each (the 8B step's layout)
    "k8_gqa4_nine_tiles": _shape(16, 32, 8, 8, 8, tuple(64 + 37 * i for i in range(16)), scale=1.0,
                                 k_prescale=1 / math.sqrt(128)),
    # 144 rows per KV head over 256 pairs: one workgroup of nine tiles each
    "k8_gqa2_nine_tiles": _shape(128, 4, 2, 8, 8, tuple((i * 41) % 230 for i in range(128))),
    # a single 16-row tile per KV head (seven idle waves)
    "one_tile": _shape(2, 2, 2, 2, 2, (600, 3)),
    # sm_scale 8: scores far above the reference the step block sets, so the
    # loop's tile sums pass 2^64 and the chunk is recomputed exactly
    "overflow_recompute": _shape(2, 8, 2, 4, 4, (450, 200), scale=8.0),
}


def _use(monkeypatch, kern, shape, kv_chunk=0):
    monkeypatch.setenv("TIDAR_ATTN_KERNEL", kern)
    s = shape
    plan = tidar.step_attention_plan(0, s.B, s.Hq, s.Hkv, s.D, s.S_max, s.max_len, s.k, s.n_groups, kv_chunk)
    assert plan["kernel"] == KERNELS[kern], plan
    return plan


def _nan_outputs(shape):
    s = shape
    out = torch.full((s.B, s.R, s.Hq, s.D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((s.B, s.Hq, s.R), float("nan"), dtype=torch.float32, device=DEV)
    return out, lse


def _ref(shape, d):
    f = attn_f32(d, "bf16")
    return oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"],
                                shape.k, shape.n_groups, shape.sm_scale)


@pytest.mark.parametrize("kern", list(KERNELS))
@pytest.mark.parametrize("name", list(CASES))
def test_kernel_matches_oracle(monkeypatch, kern, name):
    shape = CASES[name]
    plan = _use(monkeypatch, kern, shape)
    print(f"{kern} {name}: {plan}", flush=True)
    if kern == "pp" and "nine_tiles" in name:
        assert plan["shared_tiles"] == 1, plan  # the case exists for the shared tile
    d = W.attention_inputs(shape, seed=zlib.crc32(name.encode()) % 1000, tail="nan")
    t = attn_to_dev(d, "bf16")
    out, lse = _nan_outputs(shape)
    tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], shape.k,
                         shape.n_groups, shape.sm_scale, max_len=shape.max_len, out=out, lse=lse)
    ref, ref_lse = _ref(shape, d)
    check_attention(out, lse, ref, ref_lse, "bf16", what=f"{kern} {name}")


@pytest.mark.parametrize("kern", list(KERNELS))
def test_kernel_every_split_count(monkeypatch, kern):
    shape = _shape(2, 8, 2, 4, 4, (383, 70))
    d = W.attention_inputs(shape, seed=5, tail="nan")
    t = attn_to_dev(d, "bf16")
    ref, ref_lse = _ref(shape, d)
    for c in (64, 128, 192, 448, 4096):
        plan = _use(monkeypatch, kern, shape, c)
        print(f"{kern} kv_chunk={c}: {plan}", flush=True)
        out, lse = _nan_outputs(shape)
        tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], shape.k,
                             shape.n_groups, shape.sm_scale, max_len=shape.max_len, out=out, lse=lse, kv_chunk=c)
        check_attention(out, lse, ref, ref_lse, "bf16", what=f"{kern} kv_chunk={c}")


@pytest.mark.parametrize("kern", list(KERNELS))
@pytest.mark.parametrize("name", ["gqa4_k4_ragged", "k8_gqa4_nine_tiles", "overflow_recompute"])
def test_kernel_paged_matches_oracle(monkeypatch, kern, name):
    shape = CASES[name]
    _use(monkeypatch, kern, shape)
    seed = zlib.crc32(name.encode()) % 1000
    d = W.attention_inputs(shape, seed=seed, tail="nan")
    t = attn_to_dev(d, "bf16")
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=seed, spare=3)
    out, lse = _nan_outputs(shape)
    tidar.step_attention_paged(t["q"], t["k_step"], t["v_step"], to_dev(pg["k_pool"], True),
                               to_dev(pg["v_pool"], True), to_dev(pg["block_table"]), t["lens"], shape.k,
                               shape.n_groups, shape.sm_scale, max_len=shape.max_len, out=out, lse=lse)
    ref, ref_lse = _ref(shape, d)
    check_attention(out, lse, ref, ref_lse, "bf16", what=f"{kern} paged {name}")


@pytest.mark.parametrize("kern", list(KERNELS))
def test_kernel_lens_past_bound(monkeypatch, kern):
    shape = _shape(2, 32, 8, 8, 8, (50, 60))
    _use(monkeypatch, kern, shape)
    d = W.attention_inputs(shape, seed=4, tail="zero")
    t = attn_to_dev(d, "bf16")
    out, lse = tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"],
                                    shape.k, shape.n_groups, shape.sm_scale, max_len=55)
    o = out.float().cpu().numpy()
    assert np.isnan(o[1]).all() and np.isnan(lse.cpu().numpy()[1]).all()
    ref, _ = _ref(shape, d)
    assert np.abs(o[0] - ref[0]).max() <= 2e-2


def test_kernels_agree_bit_for_bit_is_not_required_but_close(monkeypatch):
    """The two kernels order their sums differently; both stay within the
    oracle tolerance of each other on the 8B step's row layout."""
    shape = CASES["k8_gqa4_nine_tiles"]
    d = W.attention_inputs(shape, seed=11, tail="nan")
    t = attn_to_dev(d, "bf16")
    outs = []
    for kern in KERNELS:
        _use(monkeypatch, kern, shape)
        o, _ = tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"],
                                    shape.k, shape.n_groups, shape.sm_scale, max_len=shape.max_len)
        outs.append(o.float().cpu().numpy())
    assert np.abs(outs[0] - outs[1]).max() <= 2e-2
