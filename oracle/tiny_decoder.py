"""Tiny random-init decoder, plain AR greedy decoding and the TiDAR greedy loop (float64).

Used to check the pages' central claim end to end: the output of the TiDAR
loop equals plain autoregressive greedy decoding token for token, because
every emitted token is confirmed under the strict causal distribution
("TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
autorégressive", nodesdaily.com, paragraphs on drafting for every outcome and
on the reported numbers; "TiDAR：Nvidia 的擴散＋自回歸混合架構…"
(engineer-news.pages.dev), section on what TiDAR does).  Random weights give
meaningless drafts, which only lowers the accept length; exactness never
depends on draft quality.

Model (a reading; the pages fix no architecture for this check): pre-norm, 2
layers, RMSNorm with unit gain and eps 1e-6, multi-head attention 4 x 64 with
rotate-half RoPE (base 10000), SwiGLU MLP 1024, untied embedding / LM head, no
biases.  A dedicated MASK embedding row (id = vocab) fills the blank slots;
the LM head has no column for it, so AR decoding can never emit it.

TiDAR loop (readings of what the pages leave open):

* bootstrap: the prompt minus its last token is prefilled causally into the
  cache; then one ordinary step runs with candidate 0 = the last prompt token
  (other candidates MASK), and verification is forced to accept exactly that
  token by a one-hot carried row.  This gives the AR distribution after the
  prompt (candidate row 0) and drafts for the next k positions (group 0).
* each step: query block [cand ; MASK x k*k] at the positions of
  oracle.step_attention, one forward pass, ar_logits = [carried row ;
  candidate rows], greedy verify, commit of the accepted rows' K/V in every
  layer, emit cand[0..a-1], carry ar_logits[a].
"""
from __future__ import annotations

import numpy as np

from .step_attention import attention_ref, causal_attention_ref
from .verify import argmax_first, verify_ref
from .commit import commit_ref


class TinyDecoder:
    def __init__(self, weights: dict, cfg):
        self.cfg = cfg
        self.w = {name: np.asarray(a, dtype=np.float64) for name, a in weights.items()}
        hd = cfg.head_dim
        self.inv_freq = cfg.rope_base ** (-np.arange(0, hd, 2, dtype=np.float64) / hd)
        self.scale = 1.0 / np.sqrt(hd)

    # -- pieces
    def rms(self, x):
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + self.cfg.rms_eps)

    def rope(self, x, pos):
        """x [T][H][hd]; rotate-half RoPE at integer positions pos [T]."""
        ang = np.asarray(pos, dtype=np.float64)[:, None] * self.inv_freq[None, :]
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        half = x.shape[-1] // 2
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)

    def qkv(self, l, h, pos):
        cfg = self.cfg
        T = h.shape[0]
        xn = self.rms(h)
        q = (xn @ self.w[f"l{l}.wq"]).reshape(T, cfg.n_heads, cfg.head_dim)
        k = (xn @ self.w[f"l{l}.wk"]).reshape(T, cfg.n_heads, cfg.head_dim)
        v = (xn @ self.w[f"l{l}.wv"]).reshape(T, cfg.n_heads, cfg.head_dim)
        return self.rope(q, pos), self.rope(k, pos), v

    def mlp(self, l, h):
        xn = self.rms(h)
        g = xn @ self.w[f"l{l}.w_gate"]
        u = xn @ self.w[f"l{l}.w_up"]
        return ((g / (1.0 + np.exp(-g))) * u) @ self.w[f"l{l}.w_down"]

    def head(self, h):
        return self.rms(h) @ self.w["lm_head"]

    # -- full causal recompute (plain AR)
    def forward_full(self, tokens):
        """Logits [T][V] of a full causal pass; also returns per-layer (k, v)."""
        T = len(tokens)
        pos = np.arange(T)
        h = self.w["emb"][np.asarray(tokens)]
        kv = []
        for l in range(self.cfg.n_layers):
            q, k, v = self.qkv(l, h, pos)
            kv.append((k, v))
            a = causal_attention_ref(q, k, v, self.scale)
            h = h + a.reshape(T, -1) @ self.w[f"l{l}.wo"]
            h = h + self.mlp(l, h)
        return self.head(h), kv

    # -- one TiDAR step against the cache
    def forward_step(self, tokens, positions, caches, lens, k, n_groups):
        """tokens/positions of the R step rows; caches[l] = (k_cache, v_cache)
        of shape [1][H][S][hd] / [1][H][S/64][hd][64].  Returns logits [R][V] and the
        per-layer step keys/values [1][R][H][hd]."""
        R = len(tokens)
        h = self.w["emb"][np.asarray(tokens)]
        step_kv = []
        for l in range(self.cfg.n_layers):
            q, kk, vv = self.qkv(l, h, positions)
            kc, vc = caches[l]
            a, _ = attention_ref(q[None], kk[None], vv[None], kc, vc, lens, k, n_groups, self.scale)
            step_kv.append((kk[None], vv[None]))
            h = h + a[0].reshape(R, -1) @ self.w[f"l{l}.wo"]
            h = h + self.mlp(l, h)
        return self.head(h), step_kv


def _margin(row):
    top2 = np.partition(np.asarray(row, dtype=np.float64), -2)[-2:]
    return float(top2[1] - top2[0])


def ar_greedy(model: TinyDecoder, prompt, n_new):
    """Plain AR greedy: recompute the whole sequence for every new token."""
    toks = [int(t) for t in prompt]
    out, margins = [], []
    for _ in range(n_new):
        logits, _ = model.forward_full(toks)
        t = argmax_first(logits[-1])
        margins.append(_margin(logits[-1]))
        toks.append(t)
        out.append(t)
    return out, {"min_margin": min(margins)}


def step_positions(L, k, n_groups):
    """Positions of the step rows: candidate i at L+i, slot (g, s) at L+g+1+s."""
    pos = [L + i for i in range(k)]
    for g in range(n_groups):
        pos += [L + g + 1 + s for s in range(k)]
    return np.asarray(pos)


def tidar_greedy(model: TinyDecoder, prompt, n_new, k, draft_fn=None):
    """TiDAR greedy decoding with the step mask, greedy verify and KV commit.

    draft_fn(step, L, emitted, cand) may replace cand[1..k-1] before a step
    (injected drafts); exactness must not depend on it."""
    cfg = model.cfg
    H, hd, S = cfg.n_heads, cfg.head_dim, cfg.S_max
    MASK = cfg.mask_token
    prompt = [int(t) for t in prompt]
    P = len(prompt)
    caches = []
    _, kv = model.forward_full(prompt[:-1])
    for l in range(cfg.n_layers):
        kc = np.zeros((1, H, S, hd))
        kk, vv = kv[l]
        kc[0, :, :P - 1, :] = kk.transpose(1, 0, 2)
        vn = np.zeros((H, S, hd))
        vn[:, :P - 1, :] = vv.transpose(1, 0, 2)
        vc = vn.reshape(1, H, S // 64, 64, hd).transpose(0, 1, 2, 4, 3).copy()  # pages of 64, transposed
        caches.append((kc, vc))
    lens = np.array([P - 1], dtype=np.int32)

    def run_step(cand):
        toks = list(cand) + [MASK] * (k * k)
        pos = step_positions(int(lens[0]), k, k)
        return model.forward_step(toks, pos, caches, lens, k, k)

    def commit(step_kv, a):
        nonlocal lens
        new_lens = None
        for l in range(cfg.n_layers):
            kc, vc = caches[l]
            ks, vs = step_kv[l]
            kc, vc, new_lens, err = commit_ref(kc, vc, lens, ks, vs, a, k)
            assert err[0] == 0
            caches[l] = (kc, vc)
        lens = new_lens

    # bootstrap: accept exactly the last prompt token
    cand = [prompt[-1]] + [MASK] * (k - 1)
    logits, step_kv = run_step(cand)
    V = cfg.vocab
    ar = np.zeros((1, k + 1, V))
    ar[0, 0, prompt[-1]] = 1.0
    ar[0, 1:] = logits[:k]
    a, nxt = verify_ref(ar, logits[k:].reshape(1, k, k, V), np.array([[prompt[-1]] + [-1] * (k - 1)]))
    assert a[0] == 1
    commit(step_kv, a)
    carried = ar[0, 1].copy()
    cand = [int(x) for x in nxt[0]]
    margins = [_margin(carried)]

    emitted, hist, step = [], [0] * (k + 1), 0
    while len(emitted) < n_new:
        if draft_fn is not None:
            cand[1:] = draft_fn(step, int(lens[0]), list(emitted), list(cand))
        logits, step_kv = run_step(cand)
        ar = np.concatenate([carried[None], logits[:k]], axis=0)[None]
        a, nxt = verify_ref(ar, logits[k:].reshape(1, k, k, V), np.array([cand]))
        ai = int(a[0])
        assert ai >= 1
        margins += [_margin(ar[0, i]) for i in range(1, ai + 1)]
        commit(step_kv, a)
        emitted += cand[:ai]
        hist[ai] += 1
        carried = ar[0, ai].copy()
        cand = [int(x) for x in nxt[0]]
        step += 1
    return emitted[:n_new], {"accept_hist": hist, "steps": step, "min_margin": min(margins),
                             "final_len": int(lens[0])}
