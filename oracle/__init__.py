"""CPU oracle for the TiDAR decode-step hot path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  It shares
no code with the HIP path (``diffusion_drafted_self_amd``): neither imports
the other.  Both take their inputs from ``workloads`` (seeded random draws
only).

Everything here is plain, slow and float64: an explicitly materialised mask
matrix, dense softmax attention, Python loops for verification and a NumPy
slice copy for the cache commit.  Each function cites the passage of the pages
it follows.  The pages cited are:

* "TiDAR : l'hybride de NVIDIA qui rédige par diffusion et parle de manière
  autorégressive" (nodesdaily.com, French) -- the mechanism: its paragraphs on
  the three zones, on drafting for every outcome and on masking.
* "TiDAR: Think in Diffusion, Talk in Autoregression" (mauroscia.it, Italian)
  -- sections "2. Single Forward Pass & Structured Attention Mask" and
  "KV Cache".
* "論文の概要: TiDAR: Think in Diffusion, Talk in Autoregression"
  (fugumt.com) -- the paper's English abstract.
* "TiDAR：Nvidia 的擴散＋自回歸混合架構——把閒置的 GPU 算力換成推論加速"
  (engineer-news.pages.dev) -- sections on the causal-mask training trick and
  on AR-exact sampling.

Parity status of each function (what pins it) is stated in its docstring; the
draft-slot conventions (slot positions, the MASK embedding, the a = 0
fallback) are readings of silent passages and are "parity unpinned" beyond the
invariants the tests check.
"""
from .step_attention import step_mask_ref, attention_ref, attention_split_ref, causal_attention_ref
from .verify import argmax_first, verify_ref
from .verify_sample import verify_sample_ref, philox4x32_10
from .commit import commit_ref
from .paged import gather_paged, paged_attention_ref, commit_paged_ref
from .train_mask import train_mask_ref, train_attention_ref
from .lmhead import lmhead_verify_ref
from .tiny_decoder import TinyDecoder, ar_greedy, tidar_greedy

__all__ = ["step_mask_ref", "attention_ref", "attention_split_ref", "causal_attention_ref",
           "argmax_first", "verify_ref", "verify_sample_ref", "philox4x32_10", "commit_ref", "gather_paged", "paged_attention_ref", "commit_paged_ref",
           "train_mask_ref", "train_attention_ref", "lmhead_verify_ref",
           "TinyDecoder", "ar_greedy", "tidar_greedy"]
