"""Ragged serving-style loop on the GPU against the oracle.

8B shapes (32 query / 8 KV heads of 128), batch 32, k = 8, settled lengths
drawn U{512..8192}, 256 consecutive steps.  Each step runs step attention,
greedy verify with planted accept lengths U{0..8} and the KV commit, which
advances the device-side lengths in place (the host only keeps an upper
bound).  Step rows are redrawn from the seed every step.

The oracle keeps its own copy of every committed row (commit_ref applied to
a window of its own tail cache), so no expected value comes from the GPU:
verify is compared every step; attention on every head of every sequence at
the first and last steps and on 8 sampled heads at every 16th step (against
the initial cache plus the oracle's committed rows); the final caches bit
for bit.  The loop runs once with the separate verify and commit calls and
once with the fused verify + commit call (one state buffer for all steps).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV, TOL, bits, to_dev  # noqa: E402

STEPS = 256
CHECK_ATTN = sorted({0, 1, 2, 127, 255} | set(range(0, STEPS, 16)))
PAGE = 64


def _host_bits(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _pair_cache(init_k, init_v_nat, tail_k, tail_v_nat, b, kvh, L0, n_tail):
    """Settled keys/values of one (b, kvh) as the oracle sees them: the
    initial rows then the rows the oracle itself committed."""
    k = np.concatenate([init_k[b, kvh, :L0], tail_k[b, kvh, :n_tail]])
    v = np.concatenate([init_v_nat[b, kvh, :L0], tail_v_nat[b, kvh, :n_tail]])
    S = (len(k) + PAGE - 1) // PAGE * PAGE
    kp = np.zeros((1, 1, S, k.shape[1]), np.float32)
    vp = np.zeros((1, 1, S, k.shape[1]), np.float32)
    kp[0, 0, :len(k)] = W.bf16_to_f32(k)
    vp[0, 0, :len(v)] = W.bf16_to_f32(v)
    return kp, W.v_paged(vp)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fused", [False, True])
def test_ragged_serving_loop(fused):
    wl = W.ragged_8b(seed=0)
    s = wl.attn
    B, k, V, Hkv, D = s.B, s.k, wl.V, s.Hkv, s.D
    cid = wl.config_id
    print(f"ragged loop: B={B} lens {min(s.lens)}..{max(s.lens)} S_max={s.S_max}", flush=True)

    cache = W.kv_cache(s, seed=0, config_id=cid, tail="zero")
    init_k, init_v = cache["k_cache"], cache["v_cache"]
    lens0 = cache["lens"].copy()
    kc, vc, lens = to_dev(init_k, True), to_dev(init_v, True), to_dev(lens0)
    init_v_nat = W.v_natural(init_v)

    # oracle-side committed rows: tail caches of STEPS*k positions per (b, kvh)
    T = STEPS * k + 2 * PAGE  # room for the last two-page window
    tail_k = np.zeros((B, Hkv, T, D), np.uint16)
    tail_v = np.zeros((B, Hkv, T // PAGE, D, PAGE), np.uint16)
    tail_len = np.zeros(B, np.int32)

    base = W.verify_inputs(B, k, V, seed=0, config_id=cid, accept="none")
    ar_h, dr_h = base["ar_logits"], base["draft_logits"]
    ar_d, dr_d = to_dev(ar_h), to_dev(dr_h)
    ws_a = None
    err = torch.zeros(B, dtype=torch.int32, device=DEV)
    state = tidar.verify_commit_state(B, k, DEV)
    worst = 0.0
    for t in range(STEPS):
        rows = W.step_rows_device(s, 0, t, DEV, config_id=cid)
        cand = W.generator(0, cid, t, 13).integers(0, V, size=(B, k)).astype(np.int32)
        a_plant = W.accept_lengths("uniform", B, k, 0, t, cid)
        edits = W.plant_accept(ar_h, cand, a_plant)
        eb, ei, et = (torch.tensor([e[j] for e in edits], device=DEV) for j in range(3))
        ar_d[eb, ei, et] = torch.from_numpy(ar_h[[e[0] for e in edits], [e[1] for e in edits],
                                                 [e[2] for e in edits]]).to(DEV)
        max_len = int(lens0.max()) + t * k  # host bound: each step adds at most k
        if ws_a is None:
            ws_a = torch.zeros(max(tidar.step_attention_workspace_bytes(0, B, s.Hq, Hkv, D, s.S_max, s.S_max - k,
                                                                       k, k), 256), dtype=torch.uint8, device=DEV)
        out, lse = tidar.step_attention(rows["q"], rows["k_step"], rows["v_step"], kc, vc, lens, k, k, s.sm_scale,
                                        max_len=max_len, workspace=ws_a)
        if fused:
            acc, nxt = tidar.verify_commit_greedy(ar_d, dr_d, to_dev(cand), kc, vc, lens, rows["k_step"],
                                                  rows["v_step"], err_flags=err, state=state)
        else:
            acc, nxt = tidar.verify_greedy(ar_d, dr_d, to_dev(cand))
            tidar.kv_commit(kc, vc, lens, rows["k_step"], rows["v_step"], acc, k, err)

        # oracle: verify
        ra, rn = oracle.verify_ref(ar_h, dr_h, cand)
        assert ra.tolist() == a_plant.tolist()
        assert acc.cpu().numpy().tolist() == ra.tolist(), f"step {t}: accept lengths differ"
        assert nxt.cpu().numpy().tolist() == rn.tolist(), f"step {t}: next drafts differ"

        ks_h, vs_h = _host_bits(rows["k_step"][:, :k]), _host_bits(rows["v_step"][:, :k])
        if t in CHECK_ATTN:  # attention against the cache state before this step's commit
            q_h = W.bf16_to_f32(_host_bits(rows["q"]))
            kst, vst = W.bf16_to_f32(_host_bits(rows["k_step"])), W.bf16_to_f32(_host_bits(rows["v_step"]))
            got = out.float().cpu().numpy()
            got_lse = lse.cpu().numpy()
            rng = np.random.default_rng(t)
            tail_v_nat = W.v_natural(tail_v)
            if t in (0, STEPS - 1):  # every head of every sequence
                heads = {(b, kvh): list(range(s.G)) for b in range(B) for kvh in range(Hkv)}
            else:  # 8 sampled heads
                heads = {}
                for _ in range(8):
                    b, h = int(rng.integers(B)), int(rng.integers(s.Hq))
                    heads.setdefault((b, h // s.G), []).append(h % s.G)
            for (b, kvh), js in heads.items():
                L = int(lens0[b] + tail_len[b])
                kp, vp = _pair_cache(init_k, init_v_nat, tail_k, tail_v_nat, b, kvh, int(lens0[b]),
                                     int(tail_len[b]))
                ref, ref_lse = _ref_pair(q_h, kst, vst, kp, vp, b, kvh, L, s, sorted(set(js)))
                for j in sorted(set(js)):
                    h = kvh * s.G + j
                    e = np.abs(got[b, :, h] - ref[:, j])
                    worst = max(worst, float(e.max()))
                    assert e.max() <= TOL["bf16"]["max_abs"], f"step {t} (b={b}, h={h}) max-abs {e.max()}"
                    assert e.sum() / np.abs(ref[:, j]).sum() <= TOL["bf16"]["mean_rel"]
                    assert abs(got_lse[b, h] - ref_lse[j]).max() <= TOL["bf16"]["lse"]

        # oracle: commit into its own tail, one sequence window at a time
        for b in range(B):
            p0 = int(tail_len[b]) // PAGE * PAGE
            wk = tail_k[b:b + 1, :, p0:p0 + 2 * PAGE].copy()
            wv = tail_v[b:b + 1, :, p0 // PAGE:p0 // PAGE + 2].copy()
            nk, nv, nl, ne = oracle.commit_ref(wk, wv, [int(tail_len[b]) - p0], ks_h[b:b + 1], vs_h[b:b + 1],
                                               ra[b:b + 1], k)
            assert ne[0] == 0
            tail_k[b:b + 1, :, p0:p0 + 2 * PAGE] = nk
            tail_v[b:b + 1, :, p0 // PAGE:p0 // PAGE + 2] = nv
            tail_len[b] = p0 + nl[0]
        assert lens.cpu().numpy().tolist() == (lens0 + tail_len).tolist(), f"step {t}: lengths differ"
        assert int(err.abs().sum()) == 0

        for b_, i_, t_, old in reversed(edits):  # restore the base logits
            ar_h[b_, i_, t_] = old
        ar_d[eb, ei, et] = torch.from_numpy(ar_h[[e[0] for e in edits], [e[1] for e in edits],
                                                 [e[2] for e in edits]]).to(DEV)
        if t % 32 == 31:
            print(f"  step {t + 1}/{STEPS}: mean settled length {float((lens0 + tail_len).mean()):.0f}, "
                  f"worst attention max-abs {worst:.2e}", flush=True)

    # final caches, bit for bit: settled rows untouched, committed rows as the oracle committed them
    gk, gv = bits(kc), W.v_natural(bits(vc))
    tv = W.v_natural(tail_v)
    for b in range(B):
        L0, n = int(lens0[b]), int(tail_len[b])
        assert np.array_equal(gk[b, :, :L0], init_k[b, :, :L0])
        assert np.array_equal(gv[b, :, :L0], init_v_nat[b, :, :L0])
        assert np.array_equal(gk[b, :, L0:L0 + n], tail_k[b, :, :n])
        assert np.array_equal(gv[b, :, L0:L0 + n], tv[b, :, :n])


def _ref_pair(q_h, kst, vst, kp, vp, b, kvh, L, s, js):
    """Oracle attention of query heads kvh*G + j (j in js) against one
    (b, kvh) cache: out [R][G][D], lse [G][R] (rows of other heads NaN)."""
    G = s.G
    q1 = q_h[b:b + 1, :, kvh * G:(kvh + 1) * G]
    ref, ref_lse = oracle.attention_ref(q1, kst[b:b + 1, :, kvh:kvh + 1], vst[b:b + 1, :, kvh:kvh + 1], kp, vp, [L],
                                        s.k, s.n_groups, s.sm_scale, pairs=[(0, j) for j in js])
    return ref[0], ref_lse[0]
