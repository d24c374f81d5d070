"""Seeded sweep of random small step-attention shapes against the float64
oracle: batch, KV heads, GQA group, head dim, k, with or without draft
groups, ragged lengths (zero included), and sometimes a forced key-chunk
size, on contiguous and paged caches.  Cache rows past every length hold
NaN, so a read of an unsettled position shows in the output.  Tolerances
are those of the other attention tests (bf16: max-abs 2e-2, mean-rel 5e-3)."""
import math

import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import attn_f32, attn_to_dev, check_attention, to_dev  # noqa: E402


def _draw(seed):
    g = np.random.default_rng(1000 + seed)
    B = int(g.integers(1, 5))
    Hkv = int(g.choice([1, 2, 4]))
    G = int(g.choice([1, 2, 4, 6, 8]))
    D = int(g.choice([64, 128]))
    k = int(g.integers(1, 9))
    n_groups = int(g.choice([0, k]))
    lens = tuple(int(x) for x in g.integers(0, 700, size=B))
    S_max = (max(lens) + 64 + 63) // 64 * 64 + 64 * int(g.integers(0, 2))
    shape = W.AttnShape(B=B, Hq=G * Hkv, Hkv=Hkv, D=D, k=k, n_groups=n_groups, lens=lens, S_max=S_max,
                        sm_scale=1.0 / math.sqrt(D))
    kv_chunk = int(g.choice([0, 0, 64, 192, 320]))
    return shape, kv_chunk


def _reference(shape, d):
    f = attn_f32(d, "bf16")
    return oracle.attention_ref(f["q"], f["k_step"], f["v_step"], f["k_cache"], f["v_cache"], d["lens"],
                                shape.k, shape.n_groups, shape.sm_scale)


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_match_oracle(seed):
    shape, kv_chunk = _draw(seed)
    print(f"sweep {seed}: {shape} kv_chunk={kv_chunk}", flush=True)
    d = W.attention_inputs(shape, seed=seed, tail="nan")
    t = attn_to_dev(d, "bf16")
    out, lse = tidar.step_attention(t["q"], t["k_step"], t["v_step"], t["k_cache"], t["v_cache"], t["lens"],
                                    shape.k, shape.n_groups, shape.sm_scale, max_len=shape.max_len, kv_chunk=kv_chunk)
    ref, ref_lse = _reference(shape, d)
    check_attention(out, lse, ref, ref_lse, "bf16", what=f"seed {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_paged_match_oracle(seed):
    shape, kv_chunk = _draw(100 + seed)
    print(f"paged sweep {seed}: {shape} kv_chunk={kv_chunk}", flush=True)
    d = W.attention_inputs(shape, seed=seed, tail="nan")
    t = attn_to_dev(d, "bf16")
    pg = W.to_pages(d["k_cache"], d["v_cache"], seed=seed, spare=2)
    out, lse = tidar.step_attention_paged(t["q"], t["k_step"], t["v_step"], to_dev(pg["k_pool"], True),
                                          to_dev(pg["v_pool"], True), to_dev(pg["block_table"]), t["lens"], shape.k,
                                          shape.n_groups, shape.sm_scale, max_len=shape.max_len, kv_chunk=kv_chunk)
    ref, ref_lse = _reference(shape, d)
    check_attention(out, lse, ref, ref_lse, "bf16", what=f"paged seed {seed}")
