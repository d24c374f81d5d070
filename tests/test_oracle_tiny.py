"""End-to-end pin of the oracle: TiDAR greedy == plain AR greedy, token for token.

The pages state that accepted text is confirmed under the strict causal
distribution, so TiDAR's output equals AR decoding ("TiDAR : l'hybride de
NVIDIA qui rédige par diffusion et parle de manière autorégressive",
nodesdaily.com, paragraph on the reported numbers).  The AR reference
recomputes the full sequence with a plain triangular mask and shares no mask,
cache or verify code with the TiDAR loop.  A planted mistake in the step
mask (a candidate seeing the next candidate) must break the equality.
"""
import numpy as np
import pytest

import oracle
import oracle.step_attention as osa
import oracle.tiny_decoder as otd
import workloads as W

CFG = W.TinyConfig()


@pytest.fixture(scope="module")
def model():
    return oracle.TinyDecoder(W.tiny_weights(CFG, 0), CFG)


@pytest.fixture(scope="module")
def ar_tokens(model):
    toks, stats = oracle.ar_greedy(model, W.tiny_prompt(CFG, 0), CFG.n_new)
    return toks


def test_rope_properties(model):
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    np.testing.assert_allclose(model.rope(q, [0]), q, atol=1e-15)  # position 0 is identity
    assert abs(np.linalg.norm(model.rope(q, [37])) - np.linalg.norm(q)) < 1e-12  # rotation
    dots = [float(np.sum(model.rope(q, [p + 5]) * model.rope(k, [p]))) for p in (0, 11, 90)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)  # depends on the offset only


def test_rmsnorm_unit_rms(model):
    x = np.random.default_rng(1).standard_normal((5, 256)) * 7.0
    np.testing.assert_allclose(np.sqrt(np.mean(model.rms(x) ** 2, axis=-1)), 1.0, rtol=1e-6)


@pytest.mark.parametrize("k", [4, 1, 2])
def test_tidar_equals_ar(model, ar_tokens, k):
    toks, stats = oracle.tidar_greedy(model, W.tiny_prompt(CFG, 0), CFG.n_new, k)
    assert toks == ar_tokens
    assert stats["final_len"] >= CFG.prompt_len + CFG.n_new - 1


def test_tidar_equals_ar_with_injected_drafts(model, ar_tokens):
    prompt = list(W.tiny_prompt(CFG, 0))
    truth = list(ar_tokens) + [0] * 16
    k = CFG.k

    def drafts(step, L, emitted, cand):
        # cand[0] is the exact AR token at position L; feed the true next k-1
        # tokens, each corrupted with probability 0.25
        pos = L - len(prompt)  # index of cand[0] in the generated stream
        return W.corrupt_drafts(truth[pos + 1:pos + k], CFG.vocab, 0.25, seed=0, step=step)

    toks, stats = oracle.tidar_greedy(model, prompt, CFG.n_new, k, draft_fn=drafts)
    assert toks == ar_tokens
    assert sum(stats["accept_hist"][3:]) > 0  # multi-token commits happened
    assert stats["steps"] < CFG.n_new // 2


def test_planted_mask_mistake_breaks_equality(model, ar_tokens, monkeypatch):
    real = osa.step_mask_ref

    def leaky(k, n_groups, L):
        M = real(k, n_groups, L)
        for i in range(k - 1):
            M[i, L + i + 1] = True  # candidate i peeks at candidate i+1
        return M

    monkeypatch.setattr(osa, "step_mask_ref", leaky)
    prompt = list(W.tiny_prompt(CFG, 0))
    truth = list(ar_tokens) + [0] * 16

    def drafts(step, L, emitted, cand):
        pos = L - len(prompt)
        return W.corrupt_drafts(truth[pos + 1:pos + CFG.k], CFG.vocab, 0.25, seed=0, step=step)

    toks, _ = otd.tidar_greedy(model, prompt, CFG.n_new, CFG.k, draft_fn=drafts)
    assert toks != ar_tokens
