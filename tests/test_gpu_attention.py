"""GPU parity of tidar_step_attention against the float64 oracle.

Small shapes span several 64-key tiles, several row blocks and a ragged tail;
every split count is exercised through kv_chunk.  bf16: max-abs <= 2e-2 and
mean-rel <= 5e-3; f32: max-abs <= 1e-5 (tolerances in _gpu_util.TOL).
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, attn_f32, attn_to_dev, bits, check_attention  # noqa: E402


def _shape(B, Hq, Hkv, D, k, n_groups, lens, dtype="bf16", S_max=None, scale=None, k_prescale=1.0):
    S_max = S_max or ((max(lens) + 64 + 63) // 64 * 64)
    return W.AttnShape(B=B, Hq=Hq, Hkv=Hkv, D=D, k=k, n_groups=n_groups, lens=tuple(lens), S_max=S_max,
                       dtype=dtype, sm_scale=scale or 1.0 / math.sqrt(D), k_prescale=k_prescale)


def _run_gpu(shape, t, kv_chunk=0, max_len=None):
    return tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"],
                                shape.k, shape.n_groups, shape.sm_scale,
                                max_len=shape.max_len if max_len is None else max_len, kv_chunk=kv_chunk)


def _run_ref(shape, d, pairs=None):
    f = attn_f32(d, shape.dtype)
    return oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"],
                                shape.k, shape.n_groups, shape.sm_scale, pairs=pairs)


CASES = {
    "bf16_gqa4_k4_ragged": _shape(3, 8, 2, 128, 4, 4, (0, 37, 300)),
    "bf16_gqa6_k4": _shape(2, 12, 2, 128, 4, 4, (130, 1)),
    "bf16_mha_d64_k8": _shape(2, 4, 4, 64, 8, 8, (100, 64)),
    "bf16_zero_drafts_k5": _shape(2, 8, 2, 128, 5, 0, (77, 200)),
    "bf16_single_token_decode": _shape(3, 8, 8, 128, 1, 0, (1, 64, 65)),
    "bf16_k16_rows1088": _shape(1, 8, 2, 128, 16, 16, (700,)),
    "bf16_k1_one_group": _shape(2, 4, 1, 64, 1, 1, (5, 191)),
    "bf16_prescaled_keys_scale1": _shape(2, 32, 8, 128, 8, 8, (257, 64), scale=1.0, k_prescale=1 / math.sqrt(128)),
    "f32_tiny_mha_d64_k4": _shape(1, 4, 4, 64, 4, 4, (64,), dtype="f32"),
    # work order: longest sequences first when B <= 256 and B*Hkv is a
    # multiple of 8 (ties broken by sequence index), plain order otherwise
    "bf16_ranked_ties_and_zeros": _shape(8, 8, 2, 64, 4, 4, (300, 0, 300, 65, 0, 129, 64, 300)),
    "bf16_ranked_batch256": _shape(256, 2, 1, 64, 1, 0, tuple((i * 53) % 197 for i in range(256))),
    "bf16_plain_order_batch264": _shape(264, 2, 1, 64, 1, 0, tuple((i * 37) % 131 for i in range(264))),
    "f32_gqa4_d128_k8": _shape(2, 8, 2, 128, 8, 8, (1000, 3), dtype="f32"),
    "f32_zero_drafts": _shape(2, 4, 2, 64, 3, 0, (0, 33), dtype="f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_attention_matches_oracle(name):
    shape = CASES[name]
    d = W.attention_inputs(shape, seed=zlib.crc32(name.encode()) % 1000, tail="nan")
    t = attn_to_dev(d, shape.dtype)
    out, lse = _run_gpu(shape, t)
    ref, ref_lse = _run_ref(shape, d)
    check_attention(out, lse, ref, ref_lse, shape.dtype, what=name)


@pytest.mark.parametrize("dtype,chunks", [("bf16", [64, 128, 192, 448, 4096]), ("f32", [64, 192, 1024])])
def test_every_split_count(dtype, chunks):
    shape = _shape(2, 8, 2, 128 if dtype == "bf16" else 64, 4, 4, (383, 70), dtype=dtype)
    d = W.attention_inputs(shape, seed=5, tail="nan")
    t = attn_to_dev(d, dtype)
    ref, ref_lse = _run_ref(shape, d)
    for c in chunks:
        out, lse = _run_gpu(shape, t, kv_chunk=c)
        check_attention(out, lse, ref, ref_lse, dtype, what=f"kv_chunk={c}")


def test_deterministic_bits():
    shape = CASES["bf16_gqa4_k4_ragged"]
    d = W.attention_inputs(shape, seed=3, tail="nan")
    t = attn_to_dev(d, "bf16")
    o1, l1 = _run_gpu(shape, t)
    o1, l1 = bits(o1), bits(l1)
    o2, l2 = _run_gpu(shape, t)
    assert np.array_equal(o1, bits(o2)) and np.array_equal(l1, bits(l2))


def test_lens_past_bound_gives_nan_not_garbage():
    shape = _shape(2, 4, 2, 128, 2, 2, (50, 60))
    d = W.attention_inputs(shape, seed=4, tail="zero")
    t = attn_to_dev(d, "bf16")
    out, lse = _run_gpu(shape, t, max_len=55)  # sequence 1 violates lens <= max_len
    out = out.float().cpu().numpy()
    assert np.isnan(out[1]).all() and np.isnan(lse.cpu().numpy()[1]).all()
    ref, ref_lse = _run_ref(shape, d, pairs=[(0, h) for h in range(4)])
    assert np.abs(out[0] - ref[0]).max() <= 2e-2


def test_empty_batch_and_bad_arguments():
    shape = _shape(1, 4, 2, 128, 2, 2, (10,))
    d = W.attention_inputs(shape, seed=6)
    t = attn_to_dev(d, "bf16")
    # B = 0 is a no-op
    z = {n: v[:0].contiguous() for n, v in t.items()}
    out, lse = tidar.step_attention(z["q"], z["k_step"], z["v_step"], z["k_cache"], z["v_cache"], z["lens"],
                                    2, 2, 0.1, max_len=0)
    assert out.numel() == 0
    with pytest.raises(tidar.TidarError):  # n_groups not in {0, k}
        tidar.step_attention(t["q"][:, :4].contiguous(), t["k_step"][:, :4].contiguous(),
                             t["v_step"][:, :4].contiguous(), t["k_cache"], t["v_cache"], t["lens"], 2, 1, 0.1,
                             max_len=10)
    with pytest.raises(tidar.TidarError):  # max_len > S_max
        tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"], 2, 2, 0.1,
                             max_len=shape.S_max + 8)
