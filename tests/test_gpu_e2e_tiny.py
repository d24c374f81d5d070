"""End to end on the GPU: TiDAR greedy decoding of the tiny random-init decoder
equals plain AR greedy decoding token for token.

The pages state that TiDAR's output equals AR sampling because every
emitted token is confirmed under the strict causal distribution
("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
autorégressive", nodesdaily.com, paragraph on the reported numbers).

The reference tokens come from the float64 oracle (full causal recompute on
the CPU).  The GPU run is a float32 test harness: the dense layers are
plain torch ops on the GPU, while every step's attention, verify and KV
commit go through the C ABI (the prompt itself is prefilled one token at a
time with single-candidate steps, i.e. ordinary causal decode).  The model,
bootstrap and loop follow oracle.tiny_decoder.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.tiny_decoder as otd
import workloads as W

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
from _gpu_util import DEV  # noqa: E402

CFG = W.TinyConfig()


class GpuTiny:
    """The tiny decoder in float32 on the GPU; attention through the C ABI."""

    def __init__(self, weights, cfg):
        self.cfg = cfg
        self.w = {n: torch.from_numpy(a).to(DEV) for n, a in weights.items()}
        hd = cfg.head_dim
        self.inv_freq = cfg.rope_base ** (-np.arange(0, hd, 2, dtype=np.float64) / hd)
        self.scale = 1.0 / np.sqrt(hd)
        H, S = cfg.n_heads, cfg.S_max
        self.caches = [(torch.zeros((1, H, S, hd), device=DEV), torch.zeros((1, H, S // 64, hd, 64), device=DEV))
                       for _ in range(cfg.n_layers)]
        self.lens = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.L = 0  # host copy of lens[0]

    def rms(self, x):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + self.cfg.rms_eps)

    def rope(self, x, pos):
        ang = np.asarray(pos, dtype=np.float64)[:, None] * self.inv_freq[None, :]
        c = torch.from_numpy(np.cos(ang)).float().to(DEV)[:, None, :]
        s = torch.from_numpy(np.sin(ang)).float().to(DEV)[:, None, :]
        half = x.shape[-1] // 2
        x1, x2 = x[..., :half], x[..., half:]
        return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)

    def step(self, tokens, positions, k, n_groups):
        cfg = self.cfg
        R = len(tokens)
        h = self.w["emb"][torch.tensor(tokens, device=DEV)]
        step_kv = []
        for l in range(cfg.n_layers):
            xn = self.rms(h)
            q = (xn @ self.w[f"l{l}.wq"]).view(R, cfg.n_heads, cfg.head_dim)
            kk = (xn @ self.w[f"l{l}.wk"]).view(R, cfg.n_heads, cfg.head_dim)
            vv = (xn @ self.w[f"l{l}.wv"]).view(R, cfg.n_heads, cfg.head_dim)
            q, kk = self.rope(q, positions), self.rope(kk, positions)
            kk, vv = kk[None].contiguous(), vv[None].contiguous()
            kc, vc = self.caches[l]
            out, _ = tidar.step_attention(q[None].contiguous(), kk, vv, kc, vc, self.lens, k, n_groups, self.scale,
                                          max_len=self.L, want_lse=False)
            step_kv.append((kk, vv))
            h = h + out[0].reshape(R, -1) @ self.w[f"l{l}.wo"]
            xn = self.rms(h)
            g, u = xn @ self.w[f"l{l}.w_gate"], xn @ self.w[f"l{l}.w_up"]
            h = h + (torch.nn.functional.silu(g) * u) @ self.w[f"l{l}.w_down"]
        return self.rms(h) @ self.w["lm_head"], step_kv

    def commit(self, step_kv, accept, k):
        """Commit the accepted rows in every layer; returns the accept length."""
        a = torch.as_tensor(accept, dtype=torch.int32, device=DEV).reshape(1)
        err = torch.empty(1, dtype=torch.int32, device=DEV)
        lens_before = self.lens.clone()
        for l in range(self.cfg.n_layers):
            kc, vc = self.caches[l]
            ks, vs = step_kv[l]
            self.lens.copy_(lens_before)
            tidar.kv_commit(kc, vc, self.lens, ks, vs, a, k, err)
            assert int(err[0]) == 0
        n = int(a[0])
        self.L += n
        assert int(self.lens[0]) == self.L
        return n


def tidar_greedy_gpu(model: GpuTiny, prompt, n_new, k, draft_fn=None):
    cfg = model.cfg
    MASK, V = cfg.mask_token, cfg.vocab
    prompt = [int(t) for t in prompt]
    for i, tok in enumerate(prompt[:-1]):  # causal prefill, one token per step
        _, kv = model.step([tok], [i], 1, 0)
        model.commit(kv, [1], 1)
    # bootstrap: one step with the last prompt token as candidate 0, forced accepted
    cand = [prompt[-1]] + [MASK] * (k - 1)
    logits, kv = model.step(cand + [MASK] * (k * k), otd.step_positions(model.L, k, k), k, k)
    ar = torch.zeros((1, k + 1, V), device=DEV)
    ar[0, 0, prompt[-1]] = 1.0
    ar[0, 1:] = logits[:k]
    boot = torch.tensor([[prompt[-1]] + [-1] * (k - 1)], dtype=torch.int32, device=DEV)
    a, nxt = tidar.verify_greedy(ar.contiguous(), logits[k:].reshape(1, k, k, V).contiguous(), boot)
    assert int(a[0]) == 1
    model.commit(kv, a, k)
    carried = ar[0, 1].clone()
    cand = nxt[0].cpu().tolist()
    emitted, hist, step = [], [0] * (k + 1), 0
    while len(emitted) < n_new:
        if draft_fn is not None:
            cand[1:] = draft_fn(step, model.L, list(emitted), list(cand))
        logits, kv = model.step(cand + [MASK] * (k * k), otd.step_positions(model.L, k, k), k, k)
        ar = torch.cat([carried[None], logits[:k]], dim=0)[None].contiguous()
        a, nxt = tidar.verify_greedy(ar, logits[k:].reshape(1, k, k, V).contiguous(),
                                     torch.tensor([cand], dtype=torch.int32, device=DEV))
        n = model.commit(kv, a, k)
        assert n >= 1
        emitted += cand[:n]
        hist[n] += 1
        carried = ar[0, n].clone()
        cand = nxt[0].cpu().tolist()
        step += 1
    return emitted[:n_new], {"accept_hist": hist, "steps": step}


@pytest.fixture(scope="module")
def reference():
    weights = W.tiny_weights(CFG, 0)
    m = oracle.TinyDecoder(weights, CFG)
    prompt = W.tiny_prompt(CFG, 0)
    toks, stats = oracle.ar_greedy(m, prompt, CFG.n_new)
    return weights, list(prompt), toks, stats


@pytest.mark.parametrize("k", [4, 2])
def test_tidar_gpu_equals_ar(reference, k):
    weights, prompt, ar_tokens, stats = reference
    assert stats["min_margin"] > 1e-4  # the float32 GPU run cannot flip a near-tie
    toks, st = tidar_greedy_gpu(GpuTiny(weights, CFG), prompt, CFG.n_new, k)
    print(f"k={k}: {st}")
    assert toks == ar_tokens


def test_tidar_gpu_equals_ar_injected_drafts(reference):
    weights, prompt, ar_tokens, _ = reference
    truth = list(ar_tokens) + [0] * 16
    k = CFG.k

    def drafts(step, L, emitted, cand):
        pos = L - len(prompt)
        return W.corrupt_drafts(truth[pos + 1:pos + k], CFG.vocab, 0.25, seed=0, step=step)

    toks, st = tidar_greedy_gpu(GpuTiny(weights, CFG), prompt, CFG.n_new, k, draft_fn=drafts)
    print(f"injected drafts: {st}")
    assert toks == ar_tokens
    assert sum(st["accept_hist"][3:]) > 0
