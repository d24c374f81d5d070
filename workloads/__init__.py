"""Seeded synthetic inputs for the TiDAR decode-step hot path.

This module draws random numbers and lays them out in the buffer layouts of
the C-ABI (``include/tidar.h``).  It holds none of the method's arithmetic: no
attention, softmax, argmax, acceptance test or cache update.  The CPU oracle's
tests and the GPU side (tests, ``bench.py``) both take their inputs from here,
so both see the same bytes.

Buffer layouts (row-major, B = batch, R = k + n_groups*k step rows):

=============  ===========================  =====================================
name           shape                        note
=============  ===========================  =====================================
q              [B][R][Hq][D]                query rows of the step block
k_step/v_step  [B][R][Hkv][D]               keys/values of the step block
k_cache        [B][Hkv][S_max][D]           settled keys, rows < lens[b] valid
v_cache        [B][Hkv][S_max/64][D][64]    settled values in pages of 64 positions,
                                            each page stored transposed
lens           [B] int32                    settled prefix length per sequence
k_pool         [n_pages][Hkv][64][D]        paged keys: position p of sequence b is row
                                            p % 64 of page block_table[b][p // 64]
v_pool         [n_pages][Hkv][D][64]        paged values, each page transposed
block_table    [B][max_pages] int32         page of each 64-position tile
ar_logits      [B][k+1][V] float32          row 0 carried, rows 1..k candidates
draft_logits   [B][k][k][V] float32         group g, slot s
cand           [B][k] int32                 carried-over draft candidates
=============  ===========================  =====================================

bf16 tensors are held as uint16 bit patterns (numpy has no bfloat16); they are
produced from float32 draws by round-to-nearest-even.

Every array is drawn from ``numpy.random.Generator(PCG64(SeedSequence([seed,
config_id, step, tensor_id])))`` so any tensor of any step can be regenerated
on its own.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

# tensor ids inside one (seed, config, step) stream
_T_Q, _T_KS, _T_VS, _T_KC, _T_VC, _T_LENS = 1, 2, 3, 4, 5, 6
_T_AR, _T_DRAFT, _T_CAND, _T_ACC, _T_BOOST = 11, 12, 13, 14, 15
_T_TINY_W, _T_PROMPT, _T_INJECT = 21, 22, 23
_T_QLOG, _T_QBOOST, _T_SHIFT, _T_MASK = 31, 32, 33, 34
_T_PAGES = 41
_T_TQ, _T_TK, _T_TV = 51, 52, 53
_T_LW, _T_LH, _T_LD, _T_LN, _T_LT = 61, 62, 63, 64, 65

MASK_TOKEN_TINY = 1024  # extra embedding row of the tiny decoder; outside its LM head
VPAGE = 64  # positions per value-cache page


def v_paged(v: np.ndarray) -> np.ndarray:
    """[..., S, D] values -> [..., S/64, D, 64] pages (layout only)."""
    *lead, S, D = v.shape
    assert S % VPAGE == 0
    p = v.reshape(*lead, S // VPAGE, VPAGE, D)
    return np.ascontiguousarray(np.swapaxes(p, -1, -2))


def v_natural(vp: np.ndarray) -> np.ndarray:
    """[..., S/64, D, 64] pages -> [..., S, D] values (layout only)."""
    *lead, P, D, W = vp.shape
    return np.ascontiguousarray(np.swapaxes(vp, -1, -2)).reshape(*lead, P * W, D)


def generator(seed: int, config_id: int, step: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config_id, step, tensor_id])))


# ----------------------------------------------------------------------------- bf16 bits
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------- shapes
@dataclasses.dataclass(frozen=True)
class AttnShape:
    """Shape of one step-attention call."""
    B: int
    Hq: int
    Hkv: int
    D: int
    k: int
    n_groups: int
    lens: tuple           # per-sequence settled length
    S_max: int
    dtype: str = "bf16"   # "bf16" | "f32"
    sm_scale: float = 1.0
    k_prescale: float = 1.0  # keys are drawn N(0,1) * k_prescale

    @property
    def R(self) -> int:
        return self.k + self.n_groups * self.k

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_len(self) -> int:
        return max(self.lens) if self.lens else 0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the synthetic workloads (shapes of the 1.5B / 8B settings)."""
    name: str
    config_id: int
    attn: AttnShape
    V: int
    accept: str            # "boost" | "uniform" | "geometric"
    steps: int = 1
    description: str = ""
    d_model: int = 4096    # hidden size feeding the LM head (1536 at 1.5B, 4096 at 8B)


def _lens(B, L):
    return tuple([L] * B)


def step_1p5b() -> Workload:
    """1.5B-shaped step: 12 query / 2 KV heads of 128, batch 8, prefix 2048, k=4."""
    return Workload("step_1p5b", 2,
                    AttnShape(B=8, Hq=12, Hkv=2, D=128, k=4, n_groups=4, lens=_lens(8, 2048),
                              S_max=2048 + 64, sm_scale=1.0 / math.sqrt(128.0)),
                    V=151936, accept="boost",
                    description="B8 Hq12 Hkv2 D128 L2048 k4 bf16; verify V=151936, +4 boost at p=0.7", d_model=1536)


def step_8b() -> Workload:
    """8B-shaped step: 32 query / 8 KV heads of 128, batch 16, prefix 4096, k=8.

    Keys are drawn N(0,1)/sqrt(128) and the softmax scale is 1 (the scale is
    folded into K)."""
    return Workload("step_8b", 3,
                    AttnShape(B=16, Hq=32, Hkv=8, D=128, k=8, n_groups=8, lens=_lens(16, 4096),
                              S_max=4096 + 64, sm_scale=1.0, k_prescale=1.0 / math.sqrt(128.0)),
                    V=128256, accept="uniform",
                    description="B16 Hq32 Hkv8 D128 L4096 k8 bf16 (K/sqrt(128), scale 1); "
                                "verify V=128256, planted accept U{0..8}")


def step_8b_long() -> Workload:
    """Long-context 8B-shaped step: batch 4, prefix 32768, k=16."""
    return Workload("step_8b_long", 4,
                    AttnShape(B=4, Hq=32, Hkv=8, D=128, k=16, n_groups=16, lens=_lens(4, 32768),
                              S_max=32768 + 64, sm_scale=1.0 / math.sqrt(128.0)),
                    V=128256, accept="geometric",
                    description="B4 Hq32 Hkv8 D128 L32768 k16 bf16; verify V=128256, "
                                "planted accept min(Geom0(0.3),16)")


def ragged_8b(seed: int = 0) -> Workload:
    """Ragged serving-style loop: batch 32, k=8, prefix U{512..8192}, 256 steps."""
    g = generator(seed, 5, 0, _T_LENS)
    lens = tuple(int(x) for x in g.integers(512, 8192 + 1, size=32))
    return Workload("ragged_8b", 5,
                    AttnShape(B=32, Hq=32, Hkv=8, D=128, k=8, n_groups=8, lens=lens,
                              S_max=8192 + 256 * 8, sm_scale=1.0 / math.sqrt(128.0)),
                    V=128256, accept="uniform", steps=256,
                    description="B32 Hq32 Hkv8 D128 L~U{512..8192} k8 bf16, 256 steps; "
                                "planted accept U{0..8}")


WORKLOADS = {"step_1p5b": step_1p5b, "step_8b": step_8b, "step_8b_long": step_8b_long,
             "ragged_8b": ragged_8b}


# ----------------------------------------------------------------------------- attention inputs
def _normal(g: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _as_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x) if dtype == "bf16" else x


def step_rows(shape: AttnShape, seed: int, step: int = 0, config_id: int = 0) -> dict:
    """q, k_step, v_step for one step (bf16 bits or float32)."""
    s = shape
    q = _normal(generator(seed, config_id, step, _T_Q), (s.B, s.R, s.Hq, s.D))
    ks = _normal(generator(seed, config_id, step, _T_KS), (s.B, s.R, s.Hkv, s.D), s.k_prescale)
    vs = _normal(generator(seed, config_id, step, _T_VS), (s.B, s.R, s.Hkv, s.D))
    return {"q": _as_dtype(q, s.dtype), "k_step": _as_dtype(ks, s.dtype), "v_step": _as_dtype(vs, s.dtype)}


def kv_cache(shape: AttnShape, seed: int, config_id: int = 0, tail: str = "nan") -> dict:
    """Settled caches filled up to lens[b]; rows at or past lens[b] hold ``tail``
    ("nan" poisons any read past the settled length, "zero", or "random")."""
    s = shape
    assert s.S_max % VPAGE == 0, "cache capacity must be a whole number of 64-position pages"
    kc = _normal(generator(seed, config_id, 0, _T_KC), (s.B, s.Hkv, s.S_max, s.D), s.k_prescale)
    vc = _normal(generator(seed, config_id, 0, _T_VC), (s.B, s.Hkv, s.S_max, s.D))
    if tail != "random":
        fill = np.float32(np.nan) if tail == "nan" else np.float32(0.0)
        for b, L in enumerate(s.lens):
            kc[b, :, L:, :] = fill
            vc[b, :, L:, :] = fill
    return {"k_cache": _as_dtype(kc, s.dtype), "v_cache": _as_dtype(v_paged(vc), s.dtype),
            "lens": np.asarray(s.lens, dtype=np.int32)}


def attention_inputs(shape: AttnShape, seed: int = 0, step: int = 0, config_id: int = 0,
                     tail: str = "nan") -> dict:
    d = step_rows(shape, seed, step, config_id)
    d.update(kv_cache(shape, seed, config_id, tail))
    return d


def to_pages(k_cache: np.ndarray, v_cache: np.ndarray, seed: int, spare: int = 8, config_id: int = 0) -> dict:
    """Move contiguous caches (k [B][Hkv][S][D], v [B][Hkv][S/64][D][64])
    into shared pools under a random block table (layout only).

    Every (sequence, 64-position tile) gets its own page, in a seeded random
    order over ``B*S/64 + spare`` pages; the spare pages are filled with NaN
    so that a read of a page no table row names shows up.  Returns k_pool
    [n_pages][Hkv][64][D], v_pool [n_pages][Hkv][D][64] and block_table
    [B][S/64] int32."""
    B, Hkv, S, D = k_cache.shape
    P = S // VPAGE
    n_pages = B * P + spare
    order = generator(seed, config_id, 0, _T_PAGES).permutation(n_pages).astype(np.int32)
    table = order[:B * P].reshape(B, P)
    nan = BF16_NAN if k_cache.dtype == np.uint16 else np.float32(np.nan)
    k_pool = np.full((n_pages, Hkv, VPAGE, D), nan, dtype=k_cache.dtype)
    v_pool = np.full((n_pages, Hkv, D, VPAGE), nan, dtype=v_cache.dtype)
    k_pool[table.reshape(-1)] = k_cache.reshape(B, Hkv, P, VPAGE, D).transpose(0, 2, 1, 3, 4).reshape(B * P, Hkv, VPAGE, D)
    v_pool[table.reshape(-1)] = v_cache.transpose(0, 2, 1, 3, 4).reshape(B * P, Hkv, D, VPAGE)
    return {"k_pool": k_pool, "v_pool": v_pool, "block_table": np.ascontiguousarray(table)}


def train_inputs(B: int, Hq: int, Hkv: int, D: int, N: int, seed: int, config_id: int = 6) -> dict:
    """Training-sequence attention inputs, bf16 bits from N(0,1) draws, T = 2N
    positions: q [B][T][Hq][D]; keys and values in their natural layout
    k_nat / v_nat [B][T][Hkv][D] and in the call's layouts k [B][Hkv][T][D],
    v [B][Hkv][T/64][D][64] (layout only)."""
    T = 2 * N
    q = _normal(generator(seed, config_id, 0, _T_TQ), (B, T, Hq, D))
    k = _normal(generator(seed, config_id, 0, _T_TK), (B, T, Hkv, D))
    v = _normal(generator(seed, config_id, 0, _T_TV), (B, T, Hkv, D))
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    k_l = np.ascontiguousarray(kb.transpose(0, 2, 1, 3))
    v_l = v_paged(np.ascontiguousarray(vb.transpose(0, 2, 1, 3)))
    return {"q": qb, "k_nat": kb, "v_nat": vb, "k": k_l, "v": v_l}


def lmhead_inputs(B: int, k: int, V: int, d: int, seed: int, accept: str = "uniform", config_id: int = 7,
                  strength: float = 12.0) -> dict:
    """Inputs of the fused LM head + verify, bf16 bits: w [V][d] from
    N(0, 1/d), h_draft [B][k][k][d] and h_ar [B][k+1][d] from N(0, 1),
    candidates uniform in [0, V).  Accept lengths are planted (``planted``)
    by aligning hidden rows with rows of w: AR row i < a is strength *
    w[cand[i]] plus N(0, 1) noise, row a (if a < k) is strength * w[t] for
    a t other than cand[a]; the other rows stay random."""
    g_w = generator(seed, config_id, 0, _T_LW)
    w = (g_w.standard_normal(size=(V, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d)))
    h_ar = _normal(generator(seed, config_id, 0, _T_LH), (B, k + 1, d))
    h_dr = _normal(generator(seed, config_id, 0, _T_LD), (B, k, k, d)) if k > 1 else None
    cand = generator(seed, config_id, 0, _T_CAND).integers(0, V, size=(B, k)).astype(np.int32)
    planted = accept_lengths(accept, B, k, seed, 0, config_id)
    other = generator(seed, config_id, 0, _T_LT).integers(1, V, size=B)
    for b in range(B):
        a = int(planted[b])
        for i in range(a):
            h_ar[b, i] += np.float32(strength) * w[cand[b, i]]
        if a < k:
            t = (int(cand[b, a]) + int(other[b])) % V
            h_ar[b, a] = np.float32(strength) * w[t]
    return {"w": bf16_bits(w), "h_ar": bf16_bits(h_ar), "h_draft": None if h_dr is None else bf16_bits(h_dr),
            "cand": cand, "planted": planted}


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of an input tensor (bf16 bits are widened)."""
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------- verify inputs
def accept_lengths(kind: str, B: int, k: int, seed: int, step: int = 0, config_id: int = 0) -> np.ndarray:
    """Planted accept lengths.  "uniform": U{0..k} inclusive.  "geometric":
    min(failures before the first success at p=0.3, k)."""
    g = generator(seed, config_id, step, _T_ACC)
    if kind == "uniform":
        return g.integers(0, k + 1, size=B).astype(np.int32)
    if kind == "geometric":
        return np.minimum(g.geometric(0.3, size=B) - 1, k).astype(np.int32)
    raise ValueError(kind)


def plant_accept(ar_logits: np.ndarray, cand: np.ndarray, a: Sequence[int]) -> list:
    """Edit ``ar_logits`` in place so the greedy prefix match of ``cand`` stops
    after exactly a[b] tokens: candidate i < a[b] gets (row max + 1), and
    candidate a[b] (if a[b] < k) gets (row min - 1).  Returns the list of edits
    (b, row, token, old value) so a caller can undo them."""
    B, k = cand.shape
    edits = []
    for b in range(B):
        ab = int(a[b])
        for i in range(ab):
            t = int(cand[b, i])
            edits.append((b, i, t, float(ar_logits[b, i, t])))
            ar_logits[b, i, t] = ar_logits[b, i].max() + np.float32(1.0)
        if ab < k:
            t = int(cand[b, ab])
            edits.append((b, ab, t, float(ar_logits[b, ab, t])))
            ar_logits[b, ab, t] = ar_logits[b, ab].min() - np.float32(1.0)
    return edits


def verify_inputs(B: int, k: int, V: int, seed: int, step: int = 0, config_id: int = 0,
                  accept: str = "uniform", with_drafts: bool = True) -> dict:
    """ar_logits/draft_logits N(0,1) float32, cand uniform ids in [0, V).

    accept: "uniform"/"geometric" plant that accept length (returned as
    ``planted``); "boost" adds +4 to the candidate's logit at probability 0.7
    per candidate (lengths then vary by chance); "none" leaves logits as drawn."""
    ar = _normal(generator(seed, config_id, step, _T_AR), (B, k + 1, V))
    dr = _normal(generator(seed, config_id, step, _T_DRAFT), (B, k, k, V)) if with_drafts else None
    cand = generator(seed, config_id, step, _T_CAND).integers(0, V, size=(B, k)).astype(np.int32)
    planted = None
    if accept in ("uniform", "geometric"):
        planted = accept_lengths(accept, B, k, seed, step, config_id)
        plant_accept(ar, cand, planted)
    elif accept == "boost":
        coin = generator(seed, config_id, step, _T_BOOST).random(size=(B, k)) < 0.7
        for b in range(B):
            for i in range(k):
                if coin[b, i]:
                    ar[b, i, cand[b, i]] += np.float32(4.0)
    elif accept != "none":
        raise ValueError(accept)
    return {"ar_logits": ar, "draft_logits": dr, "cand": cand, "planted": planted}


def sample_inputs(B: int, k: int, V: int, seed: int, step: int = 0, config_id: int = 0,
                  carried: bool = True, masked: float = 0.0, shift=(-3.0, 1.0)) -> dict:
    """Inputs of stochastic verification: ar/q/draft logits N(0,1) float32 and
    candidate ids uniform in [0, V).  Each candidate's proposal logit gets a
    boost U(2, 5) and its AR logit that boost plus a shift U(shift), by
    default U(-3, 1), so the probability of keeping it ranges from small to
    certain.

    carried: q row 0 is a copy of ar row 0 (the carried AR row, the usual
    case); otherwise it is drawn like the others.  masked: fraction of the
    logits of every row set to -inf (a filtered vocabulary); a candidate's
    proposal logit is never masked, its AR logit may be."""
    ar = _normal(generator(seed, config_id, step, _T_AR), (B, k + 1, V))
    q = _normal(generator(seed, config_id, step, _T_QLOG), (B, k, V))
    dr = _normal(generator(seed, config_id, step, _T_DRAFT), (B, k, k, V)) if k > 1 else None
    cand = generator(seed, config_id, step, _T_CAND).integers(0, V, size=(B, k)).astype(np.int32)
    boost = generator(seed, config_id, step, _T_QBOOST).uniform(2.0, 5.0, size=(B, k)).astype(np.float32)
    shift = generator(seed, config_id, step, _T_SHIFT).uniform(shift[0], shift[1], size=(B, k)).astype(np.float32)
    if masked > 0:
        g = generator(seed, config_id, step, _T_MASK)
        for t in (ar, q) + ((dr,) if dr is not None else ()):
            t[g.random(size=t.shape) < masked] = -np.inf
        for t in (ar, q) + ((dr,) if dr is not None else ()):  # every row keeps a finite entry
            t[..., 0] = np.where(np.isfinite(t[..., 0]), t[..., 0], np.float32(0.0))
    bi = np.arange(B)[:, None]
    ii = np.arange(k)[None, :]
    q[bi, ii, cand] = np.where(np.isfinite(q[bi, ii, cand]), q[bi, ii, cand], np.float32(0.0)) + boost
    ar[bi, ii, cand] = ar[bi, ii, cand] + boost + shift
    if carried:
        q[:, 0] = ar[:, 0]
    return {"ar_logits": ar, "q_logits": q, "draft_logits": dr, "cand": cand}


# ----------------------------------------------------------------------------- tiny decoder
@dataclasses.dataclass(frozen=True)
class TinyConfig:
    """Tiny random-init decoder: 2 layers, d_model 256, 4 heads x 64, SwiGLU 1024,
    vocab 1024 (+1 MASK embedding row), RMSNorm (unit gain, eps 1e-6), RoPE base
    10000 (rotate-half), untied embedding / LM head, no biases."""
    n_layers: int = 2
    d_model: int = 256
    n_heads: int = 4
    head_dim: int = 64
    d_ff: int = 1024
    vocab: int = 1024
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    prompt_len: int = 64
    n_new: int = 64
    k: int = 4
    S_max: int = 256

    @property
    def mask_token(self) -> int:
        return self.vocab


def tiny_weights(cfg: TinyConfig = TinyConfig(), seed: int = 0) -> dict:
    """All weights N(0, 0.02), drawn as float32 (exactly representable in
    float32 and float64).  Linear weights are stored [in][out]."""
    g = generator(seed, 1, 0, _T_TINY_W)

    def w(*shape):
        return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(0.02)).astype(np.float32)

    d, f = cfg.d_model, cfg.d_ff
    out = {"emb": w(cfg.vocab + 1, d), "lm_head": w(d, cfg.vocab)}
    for l in range(cfg.n_layers):
        for name, shp in (("wq", (d, d)), ("wk", (d, d)), ("wv", (d, d)), ("wo", (d, d)),
                          ("w_gate", (d, f)), ("w_up", (d, f)), ("w_down", (f, d))):
            out[f"l{l}.{name}"] = w(*shp)
    return out


def tiny_prompt(cfg: TinyConfig = TinyConfig(), seed: int = 0) -> np.ndarray:
    return generator(seed, 1, 0, _T_PROMPT).integers(0, cfg.vocab, size=cfg.prompt_len).astype(np.int64)


def corrupt_drafts(truth: Sequence[int], vocab: int, p: float, seed: int, step: int) -> list:
    """Injected drafts: each token of ``truth`` is replaced by a uniform random
    id with probability p (drives accept lengths across 1..k)."""
    g = generator(seed, 1, step, _T_INJECT)
    out = []
    for t in truth:
        out.append(int(g.integers(0, vocab)) if g.random() < p else int(t))
    return out


# ----------------------------------------------------------------------------- device-side draws
def step_rows_device(shape: AttnShape, seed: int, step: int, device, config_id: int = 0) -> dict:
    """q, k_step, v_step for one step drawn directly on the GPU with torch's
    seeded Philox generator (bf16, rounded from float32 draws); used by the
    long serving loop, where host-side draws of every step would dominate.
    Callers hand host copies of these same tensors to the oracle."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([seed, config_id, step, 99]).generate_state(1)[0]))
    s = shape
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32

    def draw(shp, scale=1.0):
        x = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x = x * scale
        return x.to(dt)

    return {"q": draw((s.B, s.R, s.Hq, s.D)),
            "k_step": draw((s.B, s.R, s.Hkv, s.D), s.k_prescale),
            "v_step": draw((s.B, s.R, s.Hkv, s.D))}
