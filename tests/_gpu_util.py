"""Helpers of the GPU tests: host <-> device copies and the attention tolerance."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

DEV = torch.device("cuda:0")

# bf16 inputs with f32 accumulation: max-abs 2e-2 and mean-rel 5e-3, where
# mean-rel = sum|O - O_ref| / sum|O_ref|.  f32 inputs: max-abs 1e-5.
TOL = {"bf16": {"max_abs": 2e-2, "mean_rel": 5e-3, "lse": 1e-2},
       "f32": {"max_abs": 1e-5, "mean_rel": 1e-5, "lse": 1e-5}}


def to_dev(x: np.ndarray, bf16: bool = False) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if bf16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a device tensor (bf16 -> uint16, f32 -> uint32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def attn_to_dev(d: dict, dtype: str) -> dict:
    return {n: to_dev(a, dtype == "bf16" and n != "lens") for n, a in d.items()}


def attn_f32(d: dict, dtype: str) -> dict:
    return {n: (W.to_f32(a, dtype) if n != "lens" else a) for n, a in d.items()}


def check_attention(got_out, got_lse, ref_out, ref_lse, dtype, pairs=None, what=""):
    """Compare (out, lse) with the oracle; returns (max_abs, mean_rel)."""
    tol = TOL[dtype]
    out = got_out.float().cpu().numpy()
    lse = got_lse.cpu().numpy()
    if pairs is not None:
        sel_o = np.stack([out[b, :, h] for b, h in pairs])
        ref_o = np.stack([ref_out[b, :, h] for b, h in pairs])
        sel_l = np.stack([lse[b, h] for b, h in pairs])
        ref_l = np.stack([ref_lse[b, h] for b, h in pairs])
    else:
        sel_o, ref_o, sel_l, ref_l = out, ref_out, lse, ref_lse
    assert np.isfinite(sel_o).all(), f"{what}: non-finite outputs"
    err = np.abs(sel_o - ref_o)
    max_abs = float(err.max())
    mean_rel = float(err.sum() / max(np.abs(ref_o).sum(), 1e-30))
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    assert mean_rel <= tol["mean_rel"], f"{what}: mean-rel {mean_rel:.3e} > {tol['mean_rel']}"
    lse_err = float(np.abs(sel_l - ref_l).max())
    assert lse_err <= tol["lse"], f"{what}: lse err {lse_err:.3e}"
    return max_abs, mean_rel
