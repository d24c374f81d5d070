"""TiDAR decode-step hot path on MI355X (gfx950): thin Python binding.

The calls of ``include/tidar.h`` -- ``step_attention``,
``step_attention_paged``, ``train_attention``, ``verify_greedy``,
``lmhead_verify_greedy``, ``verify_sample``, ``kv_commit``,
``kv_commit_paged`` and ``verify_commit_greedy[_paged]`` -- under the same names, taking torch tensors that
live on the GPU.  This module only checks shapes and dtypes,
marshals pointers and the current HIP stream, and allocates outputs /
workspace with torch when the caller does not pass them.  Every step of the
computation runs in the HIP kernels of ``libtidar.so``; there is no other
implementation, and every call fails loudly (ImportError) when the library has not
been built (``python -m diffusion_drafted_self_amd.build``).

Tensor layouts (row-major, contiguous):
  q [B][R][Hq][D], k_step/v_step [B][R][Hkv][D],
  k_cache [B][Hkv][S_max][D], v_cache [B][Hkv][S_max/64][D][64] (values in
  pages of 64 positions, each page transposed),
  paged caches: k_pool [n_pages][Hkv][64][D], v_pool [n_pages][Hkv][D][64],
  block_table [B][max_pages] int32 (position p of sequence b is row p % 64 of
  page block_table[b][p // 64]),
  lens [B] int32, ar_logits [B][k+1][V] f32, q_logits [B][k][V] f32,
  draft_logits [B][k][k][V] f32, cand [B][k] int32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtidar.so")
LIB_CHECKED_PATH = os.path.join(_HERE, "libtidar_checked.so")  # device-side bounds tests

TIDAR_OK, TIDAR_EINVAL, TIDAR_EUNSUPPORTED, TIDAR_EWORKSPACE, TIDAR_ELAUNCH = 0, -1, -2, -3, -4
TIDAR_BF16, TIDAR_F32 = 0, 1

# every symbol include/tidar.h declares, with its ctypes signature
_c_int, _c_size, _p, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
SIGNATURES = {
    "tidar_strerror": (ctypes.c_char_p, [_c_int]),
    "tidar_abi_version": (_c_int, []),
    "tidar_step_attention_workspace": (_c_int, [_c_int] * 10 + [ctypes.POINTER(_c_size)]),
    "tidar_step_attention_plan": (_c_int, [_c_int] * 10 + [ctypes.POINTER(_c_int)]),
    "tidar_step_attention": (_c_int, [_c_int] * 9 + [_f, _c_int] + [_p] * 9 + [_c_size, _p]),
    "tidar_verify_workspace": (_c_int, [_c_int] * 3 + [ctypes.POINTER(_c_size)]),
    "tidar_verify_greedy": (_c_int, [_c_int] * 3 + [_p] * 6 + [_c_size, _p]),
    "tidar_verify_sample_workspace": (_c_int, [_c_int] * 3 + [ctypes.POINTER(_c_size)]),
    "tidar_verify_sample": (_c_int, [_c_int] * 3 + [_f] + [_p] * 4 + [ctypes.c_uint64, ctypes.c_uint32]
                            + [_p] * 3 + [_c_size, _p]),
    "tidar_kv_commit": (_c_int, [_c_int] * 7 + [_p] * 7 + [_p]),
    "tidar_step_attention_paged": (_c_int, [_c_int] * 10 + [_f, _c_int] + [_p] * 10 + [_c_size, _p]),
    "tidar_kv_commit_paged": (_c_int, [_c_int] * 8 + [_p] * 8 + [_p]),
    "tidar_train_attention": (_c_int, [_c_int] * 7 + [_f] + [_p] * 6),
    "tidar_lmhead_verify_workspace": (_c_int, [_c_int] * 4 + [ctypes.POINTER(_c_size)]),
    "tidar_lmhead_verify_greedy": (_c_int, [_c_int] * 4 + [_p] * 7 + [_c_size, _p]),
    "tidar_lmhead_packed_bytes": (_c_int, [_c_int] * 2 + [ctypes.POINTER(_c_size)]),
    "tidar_lmhead_pack": (_c_int, [_c_int] * 2 + [_p] * 3),
    "tidar_lmhead_verify_greedy_packed": (_c_int, [_c_int] * 4 + [_p] * 7 + [_c_size, _p]),
    "tidar_verify_commit_state_bytes": (_c_int, [_c_int] * 2 + [ctypes.POINTER(_c_size)]),
    "tidar_verify_commit_greedy": (_c_int, [_c_int] * 8 + [_p] * 12 + [_c_size, _p]),
    "tidar_verify_commit_greedy_paged": (_c_int, [_c_int] * 9 + [_p] * 13 + [_c_size, _p]),
    "tidar_verify_commit_greedy_noalloc": (_c_int, [_c_int] * 8 + [_p] * 11 + [_p]),
    "tidar_launch_shapes": (_c_int, [_c_int] * 7 + [ctypes.POINTER(_c_int)]),
    "tidar_read_probe": (_c_int, [_p, _c_size, _p, _p]),
    "tidar_mfma_probe": (_c_int, [_c_int, _c_int, _c_int, _p, _p]),
    "tidar_check_enabled": (_c_int, []),
    "tidar_check_read": (_c_int, [ctypes.POINTER(ctypes.c_uint32), _c_int]),
}


class TidarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {strerror(status)}")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m diffusion_drafted_self_amd.build` "
                          "(the TiDAR path has no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.tidar_abi_version() != 1:
        raise ImportError(f"{os.path.basename(path)} ABI version mismatch; rebuild it")
    return lib


_LIB = None
_LOADED = {}


def lib() -> ctypes.CDLL:
    """The library the calls of this module go through: libtidar.so (loaded
    on first use; raises ImportError if it has not been built), or the
    checked build inside ``checked_library()`` -- or throughout, when the
    environment sets TIDAR_LIBRARY=checked (a debugging run)."""
    global _LIB
    if _LIB is None:
        path = LIB_CHECKED_PATH if os.environ.get("TIDAR_LIBRARY") == "checked" else LIB_PATH
        if path not in _LOADED:
            _LOADED[path] = _load(path)
        _LIB = _LOADED[path]
    return _LIB


class checked_library:
    """Context manager: inside it every call of this module goes through
    libtidar_checked.so, the build with device-side bounds tests.  On entry
    the checked library's records are cleared; ``check_read()`` returns the
    first failed test."""

    def __enter__(self):
        global _LIB
        self._prev = lib()
        chk = _LOADED.get(LIB_CHECKED_PATH)
        if chk is None:
            chk = _LOADED[LIB_CHECKED_PATH] = _load(LIB_CHECKED_PATH)
        if chk.tidar_check_enabled() != 1:
            raise ImportError(f"{LIB_CHECKED_PATH} is not a checked build")
        _LIB = chk
        check_read(clear=True)
        return self

    def __exit__(self, *exc):
        global _LIB
        _LIB = self._prev
        return False


class library:
    """Context manager: inside it every call of this module goes through the
    library file at ``path``, another build of these sources with the same
    ABI version (e.g. to time two builds against each other in one process:
    ``bench.py --compare``)."""

    def __init__(self, path: str):
        self.path = os.path.abspath(path)

    def __enter__(self):
        global _LIB
        self._prev = lib()
        h = _LOADED.get(self.path)
        if h is None:
            h = _LOADED[self.path] = _load(self.path)
        if h.tidar_abi_version() != self._prev.tidar_abi_version():
            raise ImportError(f"{self.path} has ABI version {h.tidar_abi_version()}, "
                              f"this binding {self._prev.tidar_abi_version()}")
        _LIB = h
        return self

    def __exit__(self, *exc):
        global _LIB
        _LIB = self._prev
        return False


def check_read(clear: bool = True):
    """(code, workgroup, thread, value) of the first failed bounds test the
    current library recorded on the current device, code 0 if none (always 0
    in the release library); ``clear`` resets the records.  Synchronises the
    device in the checked build."""
    rec = (ctypes.c_uint32 * 4)()
    _check("tidar_check_read", lib().tidar_check_read(rec, 1 if clear else 0))
    code, block, thread, value = (int(x) for x in rec)
    return code, block, thread, ctypes.c_int32(value).value


CHECK_CODES = {0: "none", 1: "lens", 2: "page", 3: "key_tile", 4: "row", 5: "chunk", 6: "group", 7: "accept",
               8: "token", 9: "capacity", 10: "state"}


def strerror(status: int) -> str:
    return lib().tidar_strerror(status).decode()


def _check(fn: str, status: int):
    if status != TIDAR_OK:
        raise TidarError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TIDAR_BF16
    if t.dtype == torch.float32:
        return TIDAR_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(nbytes: int, device, given):
    if given is not None:
        _need(given, "workspace", torch.uint8, 1, device)
        return given
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


VALUE_PAGE = 64


def _check_caches(k_cache, v_cache, B, Hkv, S_max, D):
    if S_max % VALUE_PAGE:
        raise ValueError(f"cache capacity {S_max} must be a multiple of {VALUE_PAGE}")
    if tuple(k_cache.shape) != (B, Hkv, S_max, D):
        raise ValueError("k_cache must be [B][Hkv][S_max][D]")
    if tuple(v_cache.shape) != (B, Hkv, S_max // VALUE_PAGE, D, VALUE_PAGE):
        raise ValueError("v_cache must be [B][Hkv][S_max/64][D][64]")


# ------------------------------------------------------------------------ attention
def step_attention_workspace_bytes(dtype_code: int, B: int, Hq: int, Hkv: int, D: int, S_max: int,
                                   max_len: int, k: int, n_groups: int, kv_chunk: int = 0) -> int:
    n = _c_size(0)
    _check("tidar_step_attention_workspace",
           lib().tidar_step_attention_workspace(dtype_code, B, Hq, Hkv, D, S_max, max_len, k, n_groups,
                                               kv_chunk, ctypes.byref(n)))
    return n.value


PLAN_KERNELS = {0: "four_wave", 1: "eight_wave", 2: "f32"}


def step_attention_plan(dtype_code: int, B: int, Hq: int, Hkv: int, D: int, S_max: int, max_len: int, k: int,
                        n_groups: int, kv_chunk: int = 0) -> dict:
    """The launch plan of tidar_step_attention for these arguments (host only)."""
    arr = (_c_int * 6)()
    _check("tidar_step_attention_plan",
           lib().tidar_step_attention_plan(dtype_code, B, Hq, Hkv, D, S_max, max_len, k, n_groups, kv_chunk, arr))
    return {"kernel": PLAN_KERNELS[arr[0]], "tiles_per_wave": arr[1], "shared_tiles": arr[2],
            "row_blocks": arr[3], "chunk": arr[4], "chunks": arr[5]}


def step_attention(q, k_step, v_step, k_cache, v_cache, lens, k: int, n_groups: int, sm_scale: float,
                   max_len: int = None, out=None, lse=None, want_lse: bool = True, workspace=None,
                   kv_chunk: int = 0):
    """Structured-mask attention of one TiDAR step.  Returns (out, lse).

    ``max_len`` is the host-side upper bound on ``lens`` (reading it from the
    device costs a synchronisation when omitted)."""
    _need(q, "q", ndim=4)
    dev = q.device
    dt = q.dtype
    B, R, Hq, D = q.shape
    _need(k_step, "k_step", dt, 4, dev)
    _need(v_step, "v_step", dt, 4, dev)
    _need(k_cache, "k_cache", dt, 4, dev)
    _need(v_cache, "v_cache", dt, 5, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    Hkv = k_step.shape[2]
    S_max = k_cache.shape[2]
    if R != k + n_groups * k:
        raise ValueError(f"q has {R} step rows, expected k + n_groups*k = {k + n_groups * k}")
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    _check_caches(k_cache, v_cache, B, Hkv, S_max, D)
    if lens.shape[0] != B:
        raise ValueError("lens must be [B]")
    if max_len is None:
        max_len = int(lens.max().item()) if B > 0 else 0
    code = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", dt, 4, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, R), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, R):
            raise ValueError("lse must be [B][Hq][R]")
    nbytes = step_attention_workspace_bytes(code, B, Hq, Hkv, D, S_max, max_len, k, n_groups, kv_chunk)
    ws = _workspace(nbytes, dev, workspace)
    _check("tidar_step_attention",
           lib().tidar_step_attention(code, B, Hq, Hkv, D, S_max, int(max_len), k, n_groups, float(sm_scale),
                                     int(kv_chunk), _ptr(q), _ptr(k_step), _ptr(v_step), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(lens), _ptr(out), _ptr(lse), _ptr(ws),
                                     ws.numel(), _stream()))
    return out, lse


def step_attention_paged(q, k_step, v_step, k_pool, v_pool, block_table, lens, k: int, n_groups: int,
                         sm_scale: float, max_len: int = None, out=None, lse=None, want_lse: bool = True,
                         workspace=None, kv_chunk: int = 0):
    """Structured-mask attention of one TiDAR step over paged caches (bf16).
    Returns (out, lse)."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, R, Hq, D = q.shape
    _need(k_step, "k_step", torch.bfloat16, 4, dev)
    _need(v_step, "v_step", torch.bfloat16, 4, dev)
    _need(k_pool, "k_pool", torch.bfloat16, 4, dev)
    _need(v_pool, "v_pool", torch.bfloat16, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    Hkv = k_step.shape[2]
    n_pages = k_pool.shape[0]
    max_pages = block_table.shape[1]
    if R != k + n_groups * k:
        raise ValueError(f"q has {R} step rows, expected k + n_groups*k = {k + n_groups * k}")
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    if tuple(k_pool.shape) != (n_pages, Hkv, VALUE_PAGE, D) or tuple(v_pool.shape) != (n_pages, Hkv, D, VALUE_PAGE):
        raise ValueError("k_pool must be [n_pages][Hkv][64][D] and v_pool [n_pages][Hkv][D][64]")
    if block_table.shape[0] != B or lens.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages] and lens [B]")
    if max_len is None:
        max_len = int(lens.max().item()) if B > 0 else 0
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, R), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, R):
            raise ValueError("lse must be [B][Hq][R]")
    nbytes = step_attention_workspace_bytes(TIDAR_BF16, B, Hq, Hkv, D, max_pages * VALUE_PAGE, max_len, k,
                                            n_groups, kv_chunk)
    ws = _workspace(nbytes, dev, workspace)
    _check("tidar_step_attention_paged",
           lib().tidar_step_attention_paged(TIDAR_BF16, B, Hq, Hkv, D, max_pages, n_pages, int(max_len), k,
                                           n_groups, float(sm_scale), int(kv_chunk), _ptr(q), _ptr(k_step),
                                           _ptr(v_step), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                           _ptr(lens), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream()))
    return out, lse


def train_attention(q, k, v, N: int, block: int, sm_scale: float, out=None, lse=None, want_lse: bool = True):
    """Attention over the duplicated training sequence (bf16): clean half
    causal, masked half in blocks of ``block`` that see the clean prefix
    before them and themselves.  q [B][2N][Hq][D], k [B][Hkv][2N][D],
    v [B][Hkv][2N/64][D][64].  Returns (out, lse)."""
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, T, Hq, D = q.shape
    _need(k, "k", torch.bfloat16, 4, dev)
    _need(v, "v", torch.bfloat16, 5, dev)
    Hkv = k.shape[1]
    if T != 2 * N or tuple(k.shape) != (B, Hkv, T, D) or tuple(v.shape) != (B, Hkv, T // VALUE_PAGE, D, VALUE_PAGE):
        raise ValueError("expected q [B][2N][Hq][D], k [B][Hkv][2N][D], v [B][Hkv][2N/64][D][64]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 4, dev)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    elif lse is not None:
        _need(lse, "lse", torch.float32, 3, dev)
    _check("tidar_train_attention",
           lib().tidar_train_attention(TIDAR_BF16, B, Hq, Hkv, D, int(N), int(block), float(sm_scale), _ptr(q),
                                      _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream()))
    return out, lse


# ------------------------------------------------------------------------ verify
def verify_workspace_bytes(B: int, k: int, V: int) -> int:
    n = _c_size(0)
    _check("tidar_verify_workspace", lib().tidar_verify_workspace(B, k, V, ctypes.byref(n)))
    return n.value


def verify_greedy(ar_logits, draft_logits, cand, accept_len=None, next_cand=None, workspace=None):
    """Greedy verification of the carried candidates.  Returns (accept_len, next_cand)."""
    _need(ar_logits, "ar_logits", torch.float32, 3)
    dev = ar_logits.device
    B, k1, V = ar_logits.shape
    k = k1 - 1
    _need(cand, "cand", torch.int32, 2, dev)
    if tuple(cand.shape) != (B, k):
        raise ValueError("cand must be [B][k]")
    if k > 1 or draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, 4, dev)
        if tuple(draft_logits.shape) != (B, k, k, V):
            raise ValueError("draft_logits must be [B][k][k][V]")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        _need(accept_len, "accept_len", torch.int32, 1, dev)
    if next_cand is None:
        next_cand = torch.empty((B, k), dtype=torch.int32, device=dev)
    else:
        _need(next_cand, "next_cand", torch.int32, 2, dev)
    ws = _workspace(verify_workspace_bytes(B, k, V), dev, workspace)
    _check("tidar_verify_greedy",
           lib().tidar_verify_greedy(B, k, V, _ptr(ar_logits), _ptr(draft_logits), _ptr(cand), _ptr(accept_len),
                                    _ptr(next_cand), _ptr(ws), ws.numel(), _stream()))
    return accept_len, next_cand


def lmhead_verify_workspace_bytes(B: int, k: int, V: int, d_model: int) -> int:
    n = _c_size(0)
    _check("tidar_lmhead_verify_workspace", lib().tidar_lmhead_verify_workspace(B, k, V, d_model, ctypes.byref(n)))
    return n.value


def _lmhead_outputs(h_ar, h_draft, cand, d, accept_len, next_cand):
    """Checks the hidden rows and candidates; returns (B, k, accept_len, next_cand)."""
    dev = h_ar.device
    B, k1, _ = h_ar.shape
    k = k1 - 1
    _need(cand, "cand", torch.int32, 2, dev)
    if tuple(cand.shape) != (B, k):
        raise ValueError("cand must be [B][k]")
    if k > 1 or h_draft is not None:
        _need(h_draft, "h_draft", torch.bfloat16, 4, dev)
        if tuple(h_draft.shape) != (B, k, k, d):
            raise ValueError("h_draft must be [B][k][k][d_model]")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        _need(accept_len, "accept_len", torch.int32, 1, dev)
    if next_cand is None:
        next_cand = torch.empty((B, k), dtype=torch.int32, device=dev)
    else:
        _need(next_cand, "next_cand", torch.int32, 2, dev)
    return B, k, accept_len, next_cand


def lmhead_verify_greedy(h_ar, h_draft, w, cand, accept_len=None, next_cand=None, workspace=None):
    """LM head (logits = h . W^T, never stored) fused with greedy
    verification.  h_ar [B][k+1][d], h_draft [B][k][k][d], w [V][d], all
    bf16.  Returns (accept_len, next_cand)."""
    _need(h_ar, "h_ar", torch.bfloat16, 3)
    dev = h_ar.device
    d = h_ar.shape[2]
    _need(w, "w", torch.bfloat16, 2, dev)
    V = w.shape[0]
    if w.shape[1] != d:
        raise ValueError("w must be [V][d_model]")
    B, k, accept_len, next_cand = _lmhead_outputs(h_ar, h_draft, cand, d, accept_len, next_cand)
    ws = _workspace(lmhead_verify_workspace_bytes(B, k, V, d), dev, workspace)
    _check("tidar_lmhead_verify_greedy",
           lib().tidar_lmhead_verify_greedy(B, k, V, d, _ptr(h_ar), _ptr(h_draft), _ptr(w), _ptr(cand),
                                           _ptr(accept_len), _ptr(next_cand), _ptr(ws), ws.numel(), _stream()))
    return accept_len, next_cand


def lmhead_packed_bytes(V: int, d_model: int) -> int:
    n = _c_size(0)
    _check("tidar_lmhead_packed_bytes", lib().tidar_lmhead_packed_bytes(V, d_model, ctypes.byref(n)))
    return n.value


def lmhead_pack(w, out=None):
    """The packed layout of the LM head w [V][d] bf16 (tiles of 256 rows by
    64 columns, each one contiguous 32 KB block), as a flat bf16 tensor."""
    _need(w, "w", torch.bfloat16, 2)
    V, d = w.shape
    n = lmhead_packed_bytes(V, d) // 2
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=w.device)
    else:
        _need(out, "out", torch.bfloat16, 1, w.device)
        if out.numel() < n:
            raise ValueError(f"out holds {out.numel()} elements; the packed head needs {n}")
    _check("tidar_lmhead_pack", lib().tidar_lmhead_pack(V, d, _ptr(w), _ptr(out), _stream()))
    return out


def lmhead_verify_greedy_packed(h_ar, h_draft, w_packed, V: int, cand, accept_len=None, next_cand=None,
                                workspace=None):
    """lmhead_verify_greedy with the head given as lmhead_pack(w) for a w
    of V rows.  Returns (accept_len, next_cand)."""
    _need(h_ar, "h_ar", torch.bfloat16, 3)
    dev = h_ar.device
    d = h_ar.shape[2]
    _need(w_packed, "w_packed", torch.bfloat16, 1, dev)
    if w_packed.numel() * 2 < lmhead_packed_bytes(V, d):
        raise ValueError("w_packed is smaller than the packed head of V rows")
    B, k, accept_len, next_cand = _lmhead_outputs(h_ar, h_draft, cand, d, accept_len, next_cand)
    ws = _workspace(lmhead_verify_workspace_bytes(B, k, V, d), dev, workspace)
    _check("tidar_lmhead_verify_greedy_packed",
           lib().tidar_lmhead_verify_greedy_packed(B, k, V, d, _ptr(h_ar), _ptr(h_draft), _ptr(w_packed),
                                                  _ptr(cand), _ptr(accept_len), _ptr(next_cand), _ptr(ws),
                                                  ws.numel(), _stream()))
    return accept_len, next_cand


def verify_sample_workspace_bytes(B: int, k: int, V: int) -> int:
    n = _c_size(0)
    _check("tidar_verify_sample_workspace", lib().tidar_verify_sample_workspace(B, k, V, ctypes.byref(n)))
    return n.value


def verify_sample(ar_logits, q_logits, draft_logits, cand, temperature: float, seed: int, step: int,
                  accept_len=None, next_cand=None, workspace=None):
    """Stochastic verification at temperature > 0 with the Philox stream of
    (seed, step).  Returns (accept_len, next_cand)."""
    _need(ar_logits, "ar_logits", torch.float32, 3)
    dev = ar_logits.device
    B, k1, V = ar_logits.shape
    k = k1 - 1
    _need(q_logits, "q_logits", torch.float32, 3, dev)
    if tuple(q_logits.shape) != (B, k, V):
        raise ValueError("q_logits must be [B][k][V]")
    _need(cand, "cand", torch.int32, 2, dev)
    if tuple(cand.shape) != (B, k):
        raise ValueError("cand must be [B][k]")
    if k > 1 or draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, 4, dev)
        if tuple(draft_logits.shape) != (B, k, k, V):
            raise ValueError("draft_logits must be [B][k][k][V]")
    if not 0 <= int(seed) < 1 << 64 or not 0 <= int(step) < 1 << 32:
        raise ValueError("seed must fit 64 bits and step 32 bits")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        _need(accept_len, "accept_len", torch.int32, 1, dev)
    if next_cand is None:
        next_cand = torch.empty((B, k), dtype=torch.int32, device=dev)
    else:
        _need(next_cand, "next_cand", torch.int32, 2, dev)
    ws = _workspace(verify_sample_workspace_bytes(B, k, V), dev, workspace)
    _check("tidar_verify_sample",
           lib().tidar_verify_sample(B, k, V, float(temperature), _ptr(ar_logits), _ptr(q_logits),
                                    _ptr(draft_logits), _ptr(cand), int(seed), int(step), _ptr(accept_len),
                                    _ptr(next_cand), _ptr(ws), ws.numel(), _stream()))
    return accept_len, next_cand


# ------------------------------------------------------------------------ commit
def kv_commit(k_cache, v_cache, lens, k_step, v_step, accept_len, k: int, err_flags=None):
    """Append the accepted candidate rows to the caches in place and advance
    ``lens``.  Returns ``err_flags`` (or None when not requested)."""
    _need(k_cache, "k_cache", ndim=4)
    dev, dt = k_cache.device, k_cache.dtype
    B, Hkv, S_max, D = k_cache.shape
    _need(v_cache, "v_cache", dt, 5, dev)
    _need(k_step, "k_step", dt, 4, dev)
    _need(v_step, "v_step", dt, 4, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    _need(accept_len, "accept_len", torch.int32, 1, dev)
    R = k_step.shape[1]
    _check_caches(k_cache, v_cache, B, Hkv, S_max, D)
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    if err_flags is not None:
        _need(err_flags, "err_flags", torch.int32, 1, dev)
    _check("tidar_kv_commit",
           lib().tidar_kv_commit(_dtype_code(k_cache), B, Hkv, D, S_max, R, k, _ptr(k_cache), _ptr(v_cache),
                                _ptr(lens), _ptr(k_step), _ptr(v_step), _ptr(accept_len), _ptr(err_flags),
                                _stream()))
    return err_flags


def kv_commit_paged(k_pool, v_pool, block_table, lens, k_step, v_step, accept_len, k: int, err_flags=None):
    """Append the accepted candidate rows into their pages in place and
    advance ``lens``.  Returns ``err_flags`` (or None when not requested)."""
    _need(k_pool, "k_pool", ndim=4)
    dev, dt = k_pool.device, k_pool.dtype
    n_pages, Hkv, _, D = k_pool.shape
    _need(v_pool, "v_pool", dt, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(k_step, "k_step", dt, 4, dev)
    _need(v_step, "v_step", dt, 4, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    _need(accept_len, "accept_len", torch.int32, 1, dev)
    B, R = k_step.shape[0], k_step.shape[1]
    max_pages = block_table.shape[1]
    if tuple(k_pool.shape) != (n_pages, Hkv, VALUE_PAGE, D) or tuple(v_pool.shape) != (n_pages, Hkv, D, VALUE_PAGE):
        raise ValueError("k_pool must be [n_pages][Hkv][64][D] and v_pool [n_pages][Hkv][D][64]")
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    if err_flags is not None:
        _need(err_flags, "err_flags", torch.int32, 1, dev)
    _check("tidar_kv_commit_paged",
           lib().tidar_kv_commit_paged(_dtype_code(k_pool), B, Hkv, D, max_pages, n_pages, R, k, _ptr(k_pool),
                                      _ptr(v_pool), _ptr(block_table), _ptr(lens), _ptr(k_step), _ptr(v_step),
                                      _ptr(accept_len), _ptr(err_flags), _stream()))
    return err_flags


# ------------------------------------------------------------------------ fused verify + commit
def verify_commit_state_bytes(B: int, k: int) -> int:
    n = _c_size(0)
    _check("tidar_verify_commit_state_bytes", lib().tidar_verify_commit_state_bytes(B, k, ctypes.byref(n)))
    return n.value


def verify_commit_state(B: int, k: int, device) -> torch.Tensor:
    """A zeroed state buffer for the fused calls (every call leaves it zeroed,
    so one buffer serves a whole decode loop on one stream)."""
    return torch.zeros(max(verify_commit_state_bytes(B, k), 256), dtype=torch.uint8, device=device)


def _verify_commit_common(ar_logits, draft_logits, cand, accept_len, next_cand, err_flags, state, dev, B, k):
    _need(ar_logits, "ar_logits", torch.float32, 3, dev)
    if tuple(ar_logits.shape[:2]) != (B, k + 1):
        raise ValueError("ar_logits must be [B][k+1][V]")
    V = ar_logits.shape[2]
    _need(cand, "cand", torch.int32, 2, dev)
    if tuple(cand.shape) != (B, k):
        raise ValueError("cand must be [B][k]")
    if k > 1 or draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, 4, dev)
        if tuple(draft_logits.shape) != (B, k, k, V):
            raise ValueError("draft_logits must be [B][k][k][V]")
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    else:
        _need(accept_len, "accept_len", torch.int32, 1, dev)
    if next_cand is None:
        next_cand = torch.empty((B, k), dtype=torch.int32, device=dev)
    else:
        _need(next_cand, "next_cand", torch.int32, 2, dev)
    if err_flags is not None:
        _need(err_flags, "err_flags", torch.int32, 1, dev)
    if state is None:
        state = verify_commit_state(B, k, dev)
    else:
        _need(state, "state", torch.uint8, 1, dev)
    return V, accept_len, next_cand, state


def verify_commit_greedy(ar_logits, draft_logits, cand, k_cache, v_cache, lens, k_step, v_step, accept_len=None,
                         next_cand=None, err_flags=None, state=None):
    """Greedy verification and the KV commit in one call (the results of
    verify_greedy followed by kv_commit).  ``state`` must be a zeroed buffer
    (verify_commit_state) or None.  Returns (accept_len, next_cand)."""
    _need(k_cache, "k_cache", ndim=4)
    dev, dt = k_cache.device, k_cache.dtype
    B, Hkv, S_max, D = k_cache.shape
    _need(v_cache, "v_cache", dt, 5, dev)
    _need(k_step, "k_step", dt, 4, dev)
    _need(v_step, "v_step", dt, 4, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    R = k_step.shape[1]
    _check_caches(k_cache, v_cache, B, Hkv, S_max, D)
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    k = cand.shape[1]
    V, accept_len, next_cand, state = _verify_commit_common(ar_logits, draft_logits, cand, accept_len, next_cand,
                                                            err_flags, state, dev, B, k)
    _check("tidar_verify_commit_greedy",
           lib().tidar_verify_commit_greedy(_dtype_code(k_cache), B, Hkv, D, S_max, R, k, V, _ptr(ar_logits),
                                           _ptr(draft_logits), _ptr(cand), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
                                           _ptr(k_step), _ptr(v_step), _ptr(accept_len), _ptr(next_cand),
                                           _ptr(err_flags), _ptr(state), state.numel(), _stream()))
    return accept_len, next_cand


def verify_commit_greedy_noalloc(ar_logits, draft_logits, cand, k_cache, v_cache, lens, k_step, v_step,
                                 accept_len, next_cand, err_flags=None):
    """verify_commit_greedy with the library's own per-GPU state: nothing is
    allocated, so the outputs must be given.  Calls that may overlap on one
    GPU race.  Returns (accept_len, next_cand)."""
    _need(k_cache, "k_cache", ndim=4)
    dev, dt = k_cache.device, k_cache.dtype
    B, Hkv, S_max, D = k_cache.shape
    _need(v_cache, "v_cache", dt, 5, dev)
    _need(k_step, "k_step", dt, 4, dev)
    _need(v_step, "v_step", dt, 4, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    R = k_step.shape[1]
    _check_caches(k_cache, v_cache, B, Hkv, S_max, D)
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    k = cand.shape[1]
    if accept_len is None or next_cand is None:
        raise ValueError("accept_len and next_cand must be given (this call allocates nothing)")
    _need(ar_logits, "ar_logits", torch.float32, 3, dev)
    if tuple(ar_logits.shape[:2]) != (B, k + 1):
        raise ValueError("ar_logits must be [B][k+1][V]")
    V = ar_logits.shape[2]
    _need(cand, "cand", torch.int32, 2, dev)
    if cand.shape[0] != B:
        raise ValueError("cand must be [B][k]")
    if k > 1 or draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.float32, 4, dev)
        if tuple(draft_logits.shape) != (B, k, k, V):
            raise ValueError("draft_logits must be [B][k][k][V]")
    _need(accept_len, "accept_len", torch.int32, 1, dev)
    _need(next_cand, "next_cand", torch.int32, 2, dev)
    if err_flags is not None:
        _need(err_flags, "err_flags", torch.int32, 1, dev)
    _check("tidar_verify_commit_greedy_noalloc",
           lib().tidar_verify_commit_greedy_noalloc(_dtype_code(k_cache), B, Hkv, D, S_max, R, k, V,
                                                   _ptr(ar_logits), _ptr(draft_logits), _ptr(cand), _ptr(k_cache),
                                                   _ptr(v_cache), _ptr(lens), _ptr(k_step), _ptr(v_step),
                                                   _ptr(accept_len), _ptr(next_cand), _ptr(err_flags), _stream()))
    return accept_len, next_cand


def verify_commit_greedy_paged(ar_logits, draft_logits, cand, k_pool, v_pool, block_table, lens, k_step, v_step,
                               accept_len=None, next_cand=None, err_flags=None, state=None):
    """verify_commit_greedy into a paged cache (the pools and block table of
    step_attention_paged).  Returns (accept_len, next_cand)."""
    _need(k_pool, "k_pool", ndim=4)
    dev, dt = k_pool.device, k_pool.dtype
    n_pages, Hkv, _, D = k_pool.shape
    _need(v_pool, "v_pool", dt, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(k_step, "k_step", dt, 4, dev)
    _need(v_step, "v_step", dt, 4, dev)
    _need(lens, "lens", torch.int32, 1, dev)
    B, R = k_step.shape[0], k_step.shape[1]
    max_pages = block_table.shape[1]
    if tuple(k_pool.shape) != (n_pages, Hkv, VALUE_PAGE, D) or tuple(v_pool.shape) != (n_pages, Hkv, D, VALUE_PAGE):
        raise ValueError("k_pool must be [n_pages][Hkv][64][D] and v_pool [n_pages][Hkv][D][64]")
    if tuple(k_step.shape) != (B, R, Hkv, D) or tuple(v_step.shape) != (B, R, Hkv, D):
        raise ValueError("k_step/v_step must be [B][R][Hkv][D]")
    if block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages]")
    k = cand.shape[1]
    V, accept_len, next_cand, state = _verify_commit_common(ar_logits, draft_logits, cand, accept_len, next_cand,
                                                            err_flags, state, dev, B, k)
    _check("tidar_verify_commit_greedy_paged",
           lib().tidar_verify_commit_greedy_paged(_dtype_code(k_pool), B, Hkv, D, max_pages, n_pages, R, k, V,
                                                 _ptr(ar_logits), _ptr(draft_logits), _ptr(cand), _ptr(k_pool),
                                                 _ptr(v_pool), _ptr(block_table), _ptr(lens), _ptr(k_step),
                                                 _ptr(v_step), _ptr(accept_len), _ptr(next_cand), _ptr(err_flags),
                                                 _ptr(state), state.numel(), _stream()))
    return accept_len, next_cand


READ_PROBE_BLOCKS = 16384  # TIDAR_READ_PROBE_BLOCKS


def read_probe(buf, sink=None):
    """Read every byte of the contiguous device tensor ``buf`` once (the
    library's streaming-read helper, for achievable-bandwidth figures).
    Returns the int32 ``sink`` of READ_PROBE_BLOCKS words, whose XOR is the
    XOR of all 32-bit words of ``buf``."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(READ_PROBE_BLOCKS, dtype=torch.int32, device=buf.device)
    _need(sink, "sink", torch.int32, 1, buf.device)
    if sink.numel() < READ_PROBE_BLOCKS:
        raise ValueError(f"sink must hold {READ_PROBE_BLOCKS} words")
    _check("tidar_read_probe", lib().tidar_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream()))
    return sink


MFMA_PROBE_BLOCKS = 256  # TIDAR_MFMA_PROBE_BLOCKS


def mfma_probe(waves_per_simd: int, lds_reads: bool, iters: int, device="cuda"):
    """Shader-clock cycles of ``iters`` rounds of eight independent bf16
    16x16x32 MFMAs per wave (operands from LDS when ``lds_reads``), one
    int64 per wave of MFMA_PROBE_BLOCKS workgroups of 4 * waves_per_simd
    waves (tidar_mfma_probe); enqueued on the current stream."""
    cycles = torch.zeros(MFMA_PROBE_BLOCKS * 4 * waves_per_simd, dtype=torch.int64, device=device)
    _check("tidar_mfma_probe", lib().tidar_mfma_probe(int(waves_per_simd), 1 if lds_reads else 0, int(iters),
                                                      _ptr(cycles), _stream()))
    return cycles


__all__ = ["step_attention", "step_attention_workspace_bytes", "verify_greedy", "verify_workspace_bytes",
           "verify_sample", "verify_sample_workspace_bytes", "kv_commit",
           "step_attention_paged", "kv_commit_paged", "train_attention",
           "lmhead_verify_greedy", "lmhead_verify_workspace_bytes", "lmhead_pack", "lmhead_packed_bytes",
           "lmhead_verify_greedy_packed", "strerror", "lib", "TidarError", "LIB_PATH", "SIGNATURES",
           "read_probe", "READ_PROBE_BLOCKS", "mfma_probe", "MFMA_PROBE_BLOCKS", "checked_library", "library", "check_read", "CHECK_CODES", "LIB_CHECKED_PATH"]
