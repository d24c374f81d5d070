"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects invalid calls on the host before anything is enqueued
(so these calls never touch a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def T():
    import diffusion_drafted_self_amd as tidar
    if not os.path.exists(tidar.LIB_PATH):
        from diffusion_drafted_self_amd.build import build
        build()
    tidar.lib()
    return tidar


def _declared():
    text = open(os.path.join(ROOT, "include", "tidar.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tidar_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(T):
    names = _declared()
    assert set(names) == set(T.SIGNATURES), names
    raw = ctypes.CDLL(T.LIB_PATH)
    for n in names:
        assert getattr(raw, n) is not None


def _prototypes():
    """(name, parameter count) of every prototype the header declares."""
    text = open(os.path.join(ROOT, "include", "tidar.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"\b(tidar_\w+)\s*\(([^)]*)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_signatures_match_the_header(T):
    protos = _prototypes()
    assert set(protos) == set(T.SIGNATURES)
    for name, (_, args) in T.SIGNATURES.items():
        assert len(args) == protos[name], f"{name}: binding has {len(args)} arguments, header {protos[name]}"


def test_checked_build_exports_the_same_calls(T):
    """libtidar_checked.so (device-side bounds tests) exports every declared
    call and says it is the checked build; the release library says it is
    not and returns an empty record without touching a device."""
    if not os.path.exists(T.LIB_CHECKED_PATH):
        from diffusion_drafted_self_amd.build import build
        build()
    raw = ctypes.CDLL(T.LIB_CHECKED_PATH)
    for n in _declared():
        assert getattr(raw, n) is not None
    chk, rel = T._load(T.LIB_CHECKED_PATH), T._load(T.LIB_PATH)
    assert chk.tidar_check_enabled() == 1 and rel.tidar_check_enabled() == 0
    assert chk.tidar_abi_version() == rel.tidar_abi_version()
    rec = (ctypes.c_uint32 * 4)(1, 2, 3, 4)
    assert rel.tidar_check_read(rec, 1) == T.TIDAR_OK and list(rec) == [0, 0, 0, 0]
    assert chk.tidar_check_read(None, 0) == T.TIDAR_EINVAL  # refused before any device call
    assert rel.tidar_check_read(None, 0) == T.TIDAR_EINVAL
    # host validation is the same code in both
    n = ctypes.c_size_t(0)
    for lib in (chk, rel):
        assert lib.tidar_step_attention_workspace(0, 2, 6, 4, 128, 256, 100, 4, 4, 0, ctypes.byref(n)) == T.TIDAR_EINVAL


def test_check_codes_match_the_header(T):
    text = open(os.path.join(ROOT, "include", "tidar.h")).read()
    codes = {int(v): name.lower() for name, v in re.findall(r"\bTIDAR_CHECK_(\w+)\s*=\s*(\d+)", text)}
    assert codes == T.CHECK_CODES


def test_mfma_probe_validation(T):
    """tidar_mfma_probe refuses other wave counts, round counts and a null
    record pointer before anything is enqueued (host checks only)."""
    L = T.lib()
    good = ctypes.c_void_p(256)  # an aligned stand-in address; never dereferenced on a refusal
    assert L.tidar_mfma_probe(3, 0, 16, good, None) == T.TIDAR_EINVAL
    assert L.tidar_mfma_probe(0, 0, 16, good, None) == T.TIDAR_EINVAL
    assert L.tidar_mfma_probe(1, 2, 16, good, None) == T.TIDAR_EINVAL
    assert L.tidar_mfma_probe(1, 0, 0, good, None) == T.TIDAR_EINVAL
    assert L.tidar_mfma_probe(1, 0, (1 << 20) + 1, good, None) == T.TIDAR_EINVAL
    assert L.tidar_mfma_probe(1, 0, 16, None, None) == T.TIDAR_EINVAL
    assert L.tidar_mfma_probe(1, 0, 16, ctypes.c_void_p(260), None) == T.TIDAR_EINVAL


def test_library_switch(T):
    """tidar.library(path) routes the module's calls through another build of
    the same ABI (bench.py --compare times builds against each other that
    way) and restores the previous library on exit; a missing file raises."""
    before = T.lib()
    with T.library(T.LIB_CHECKED_PATH):
        assert T.lib() is not before
        assert T.lib().tidar_check_enabled() == 1
    assert T.lib() is before
    with pytest.raises(ImportError):
        with T.library(T.LIB_PATH + ".missing"):
            pass
    assert T.lib() is before


def test_strerror_and_version(T):
    assert T.lib().tidar_abi_version() == 1
    for code in (0, -1, -2, -3, -4, 7):
        assert T.strerror(code)


def _ws(T, *args):
    n = ctypes.c_size_t(0)
    st = T.lib().tidar_step_attention_workspace(*args, ctypes.byref(n))
    return st, n.value


def test_attention_workspace_validation(T):
    ok = (0, 16, 32, 8, 128, 4160, 4096, 8, 8, 0)
    assert _ws(T, *ok)[0] == 0
    bad = {
        "dtype": ((7,) + ok[1:], -2), "head dim": (ok[:4] + (96,) + ok[5:], -2),
        "S_max % 64": (ok[:5] + (4104,) + ok[6:], -1),
        "k too large": (ok[:7] + (17, 17, 0), -2), "k zero": (ok[:7] + (0, 0, 0), -1),
        "n_groups": (ok[:8] + (3, 0), -1), "S_max % 8": (ok[:5] + (4161,) + ok[6:], -1),
        "max_len > S_max": (ok[:6] + (4168,) + ok[7:], -1), "kv_chunk % 64": (ok[:9] + (100,), -1),
        "f32 chunk": ((1,) + ok[1:9] + (2048,), -1), "Hq % Hkv": (ok[:2] + (30,) + ok[3:], -1),
        "B < 0": ((0, -1) + ok[2:], -1),
    }
    for name, (args, want) in bad.items():
        assert _ws(T, *args)[0] == want, name


def test_attention_workspace_size(T):
    # B*Hkv*n_split*M partial rows of D f32 plus (max, sum), each rounded to 256 B
    B, Hq, Hkv, D, S, L, k, chunk = 3, 8, 2, 128, 1024, 1000, 4, 192
    R, M = k + k * k, (k + k * k) * 4
    n_split = -(-(L + R) // chunk)
    rows = B * Hkv * n_split * M
    want = -(-rows * D * 4 // 256) * 256 + -(-rows * 8 // 256) * 256
    assert _ws(T, 0, B, Hq, Hkv, D, S, L, k, k, chunk) == (0, want)
    assert _ws(T, 0, 0, Hq, Hkv, D, S, L, k, k, 0)[1] == 0


def test_attention_call_rejects_before_launch(T):
    f = T.lib().tidar_step_attention
    p = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: every call below fails validation
    # this shape splits its keys, so it needs a workspace: 16 bytes is rejected before any launch
    st, need = _ws(T, 0, 2, 8, 2, 128, 4096, 4000, 4, 4, 0)
    assert st == 0 and need > 16
    args = [0, 2, 8, 2, 128, 4096, 4000, 4, 4, 0.1, 0] + [p] * 6 + [p, None, p, 1 << 30, None]
    bad_ws = list(args); bad_ws[20] = 16
    assert f(*bad_ws) == -3
    bad_scale = list(args); bad_scale[9] = 0.0
    assert f(*bad_scale) == -1
    bad_ptr = list(args); bad_ptr[11] = ctypes.c_void_p(0x100004)
    assert f(*bad_ptr) == -1
    null_ptr = list(args); null_ptr[12] = None
    assert f(*null_ptr) == -1
    empty = [0, 0, 8, 2, 128, 256, 0, 4, 4, 0.1, 0] + [None] * 9 + [0, None]
    assert f(*empty) == 0


def test_verify_validation_and_size(T):
    n = ctypes.c_size_t(0)
    L = T.lib()
    assert L.tidar_verify_workspace(16, 8, 128256, ctypes.byref(n)) == 0
    chunks = -(-128256 // 4096)
    want = sum(-(-x // 256) * 256 for x in (16 * 9 * chunks * 8, 16 * 7 * chunks * 8, 16 * 4))
    assert n.value == want
    assert L.tidar_verify_workspace(16, 17, 100, ctypes.byref(n)) == -2
    assert L.tidar_verify_workspace(16, 0, 100, ctypes.byref(n)) == -1
    assert L.tidar_verify_workspace(16, 4, 0, ctypes.byref(n)) == -1
    p = ctypes.c_void_p(0x100000)
    assert L.tidar_verify_greedy(2, 4, 100, p, p, p, p, p, p, 8, None) == -3
    assert L.tidar_verify_greedy(2, 4, 100, p, None, p, p, p, p, 1 << 20, None) == -1


def test_commit_validation(T):
    L = T.lib()
    p = ctypes.c_void_p(0x100000)
    assert L.tidar_kv_commit(0, 2, 8, 96, 64, 72, 8, p, p, p, p, p, p, None, None) == -2
    assert L.tidar_kv_commit(0, 2, 8, 128, 64, 4, 8, p, p, p, p, p, p, None, None) == -1
    assert L.tidar_kv_commit(0, 2, 8, 128, 60, 72, 8, p, p, p, p, p, p, None, None) == -1
    assert L.tidar_kv_commit(0, 2, 8, 128, 64, 72, 8, p, None, p, p, p, p, None, None) == -1
    assert L.tidar_kv_commit(0, 0, 8, 128, 64, 72, 8, None, None, None, None, None, None, None, None) == 0
    # k above 16: more accepted rows than the two 64-position pages the paged
    # commit resolves could hold; refused by both forms even where k <= R
    assert L.tidar_kv_commit(0, 2, 8, 128, 4096, 400, 17, p, p, p, p, p, p, None, None) == -2
    assert L.tidar_kv_commit_paged(0, 2, 8, 128, 64, 100, 400, 17, p, p, p, p, p, p, p, None, None) == -2


def test_verify_commit_noalloc_refuses_before_enqueueing(T):
    """The allocation-free fused verify + commit checks everything on the host
    first: a refused call returns its own code, never the launch error a
    first enqueue (the clearing kernel) would give on a machine without a GPU."""
    L = T.lib()
    p = ctypes.c_void_p(0x100000)
    odd = ctypes.c_void_p(0x100002)

    def call(dtype=0, B=16, Hkv=8, D=128, S_max=4224, R=72, k=8, V=128256, ptrs=None):
        pp = ptrs or [p] * 11
        return L.tidar_verify_commit_greedy_noalloc(dtype, B, Hkv, D, S_max, R, k, V, *pp, None)

    assert call(dtype=7) == -2                              # dtype
    assert call(D=96) == -2                                 # head dim
    assert call(k=17) == -2                                 # k above 16
    assert call(S_max=4200) == -1                           # not a multiple of the 64-position page
    assert call(R=4) == -1                                  # fewer step rows than candidates
    assert call(ptrs=[odd] + [p] * 10) == -1                # misaligned logits
    assert call(ptrs=[p] * 10 + [odd]) == -1                # misaligned err_flags
    assert call(B=1024, k=16, V=64) == -3                   # a state beyond the 2 MiB array
    assert call(B=0) == 0                                   # nothing to do, nothing enqueued


def test_verify_sample_validation_and_size(T):
    n = ctypes.c_size_t(0)
    L = T.lib()
    assert L.tidar_verify_sample_workspace(16, 8, 128256, ctypes.byref(n)) == 0
    chunks = -(-128256 // 4096)
    # (max, sum) per chunk of 2k rows, (Mp, Zp, Mq, Zq) per sequence, draws per chunk of k rows, fallback draws
    want = sum(-(-x // 256) * 256 for x in (16 * 16 * chunks * 8, 16 * 16, 16 * 8 * chunks * 8, 16 * chunks * 8))
    assert n.value == want
    assert L.tidar_verify_sample_workspace(16, 17, 100, ctypes.byref(n)) == -2
    assert L.tidar_verify_sample_workspace(16, 0, 100, ctypes.byref(n)) == -1
    assert L.tidar_verify_sample_workspace(4096, 16, 100, ctypes.byref(n)) == -2  # 2*B*k workgroup rows
    p = ctypes.c_void_p(0x100000)
    f = L.tidar_verify_sample
    args = [2, 4, 100, 0.8, p, p, p, p, 1, 0, p, p, p, 1 << 20, None]
    small_ws = list(args); small_ws[13] = 8
    assert f(*small_ws) == -3
    for T_bad in (0.0, -1.0, float("inf"), float("nan")):
        bad_t = list(args); bad_t[3] = T_bad
        assert f(*bad_t) == -1, T_bad
    no_q = list(args); no_q[5] = None
    assert f(*no_q) == -1
    no_draft = list(args); no_draft[6] = None
    assert f(*no_draft) == -1
    empty = [0, 4, 100, 0.8] + [None] * 4 + [1, 0] + [None] * 3 + [0, None]
    assert f(*empty) == 0


def test_paged_validation(T):
    L = T.lib()
    p = ctypes.c_void_p(0x100000)
    f = L.tidar_step_attention_paged
    #       dtype B  Hq Hkv D   max_pages n_pages max_len k  ng  scale kv_chunk
    args = [0, 2, 8, 2, 128, 64, 200, 4000, 4, 4, 0.1, 0] + [p] * 7 + [p, None, p, 1 << 30, None]
    f32 = list(args); f32[0] = 1
    assert f(*f32) == -2  # paged pools: bf16 only
    no_pages = list(args); no_pages[6] = 0
    assert f(*no_pages) == -1
    too_long = list(args); too_long[7] = 64 * 64 + 1  # max_len above 64 * max_pages
    assert f(*too_long) == -1
    no_table = list(args); no_table[17] = None
    assert f(*no_table) == -1
    small_ws = list(args); small_ws[22] = 16
    assert f(*small_ws) == -3
    c = L.tidar_kv_commit_paged
    cargs = [0, 2, 8, 128, 64, 200, 72, 8] + [p] * 8 + [None, None]
    bad_table = list(cargs); bad_table[10] = ctypes.c_void_p(0x100002)
    assert c(*bad_table) == -1
    no_pool = list(cargs); no_pool[8] = None
    assert c(*no_pool) == -1
    zero_pages = list(cargs); zero_pages[5] = 0
    assert c(*zero_pages) == -1
    assert c(*([0, 0, 8, 128, 64, 200, 72, 8] + [None] * 10)) == 0


def test_train_attention_validation(T):
    f = T.lib().tidar_train_attention
    p = ctypes.c_void_p(0x100000)
    ok = [0, 2, 8, 2, 128, 128, 8, 0.1, p, p, p, p, p, None]
    bad = {
        "f32": ([1] + ok[1:], -2), "head dim": (ok[:4] + [96] + ok[5:], -2),
        "N % 64": (ok[:5] + [100] + ok[6:], -1), "N < 64": (ok[:5] + [0] + ok[6:], -1),
        "block 0": (ok[:6] + [0] + ok[7:], -1), "block > N": (ok[:6] + [129] + ok[7:], -1),
        "scale": (ok[:7] + [0.0] + ok[8:], -1), "Hq % Hkv": (ok[:2] + [7] + ok[3:], -1),
        "unaligned q": (ok[:8] + [ctypes.c_void_p(0x100008)] + ok[9:], -1),
    }
    for name, (args, want) in bad.items():
        assert f(*args) == want, name
    assert f(*([0, 0, 8, 2, 128, 128, 8, 0.1] + [None] * 6)) == 0


def test_lmhead_validation_and_size(T):
    L = T.lib()
    n = ctypes.c_size_t(0)
    assert L.tidar_lmhead_verify_workspace(16, 8, 128256, 4096, ctypes.byref(n)) == 0
    chunks = -(-128256 // 256)
    want = sum(-(-x // 256) * 256 for x in (16 * 9 * chunks * 8, 16 * 7 * chunks * 8, 16 * 4))
    assert n.value == want
    assert L.tidar_lmhead_verify_workspace(16, 8, 128256, 100, ctypes.byref(n)) == -1   # d % 64
    assert L.tidar_lmhead_verify_workspace(16, 17, 1000, 64, ctypes.byref(n)) == -2     # k
    # a head past 32-bit byte offsets: the packed form takes it, the row-major one does not
    assert L.tidar_lmhead_verify_workspace(1, 1, 600000, 4096, ctypes.byref(n)) == 0
    p = ctypes.c_void_p(0x100000)
    for f in (L.tidar_lmhead_verify_greedy, L.tidar_lmhead_verify_greedy_packed):
        assert f(2, 4, 1000, 64, p, p, p, p, p, p, p, 8, None) == -3
        assert f(2, 4, 1000, 64, p, None, p, p, p, p, p, 1 << 20, None) == -1
        assert f(0, 4, 1000, 64, None, None, None, None, None, None, None, 0, None) == 0
    assert L.tidar_lmhead_verify_greedy(1, 1, 600000, 4096, p, p, p, p, p, p, p, 1 << 30, None) == -2
    # k = 1: the AR pass addresses B*(k+1)*d*2 bytes of hidden rows, twice the
    # draft rows' B*k*k*d*2; the 32-bit offset bound takes the larger
    assert L.tidar_lmhead_verify_workspace(200000, 1, 1000, 4096, ctypes.byref(n)) == 0   # 3.3e9 B
    assert L.tidar_lmhead_verify_workspace(300000, 1, 1000, 4096, ctypes.byref(n)) == -2  # 4.9e9 B
    assert L.tidar_lmhead_verify_greedy_packed(1, 1, 600000, 4096, p, p, p, p, p, p, p, 8, None) == -3


def test_lmhead_pack_validation_and_size(T):
    L = T.lib()
    n = ctypes.c_size_t(0)
    assert L.tidar_lmhead_packed_bytes(1000, 64, ctypes.byref(n)) == 0
    assert n.value == 4 * 256 * 64 * 2            # V rounded up to whole 256-row chunks
    assert L.tidar_lmhead_packed_bytes(128256, 4096, ctypes.byref(n)) == 0
    assert n.value == 128256 * 4096 * 2           # 128256 = 501 chunks exactly
    assert L.tidar_lmhead_packed_bytes(0, 64, ctypes.byref(n)) == -1
    assert L.tidar_lmhead_packed_bytes(1000, 100, ctypes.byref(n)) == -1
    assert L.tidar_lmhead_packed_bytes(1000, 64, None) == -1
    p = ctypes.c_void_p(0x100000)
    f = L.tidar_lmhead_pack
    assert f(1000, 100, p, p, None) == -1          # d % 64
    assert f(0, 64, p, p, None) == -1
    assert f(1000, 64, ctypes.c_void_p(0x100004), p, None) == -1   # misaligned w
    assert f(1000, 64, p, None, None) == -1


def test_read_probe_validation(T):
    f = T.lib().tidar_read_probe
    buf = (ctypes.c_uint8 * 64)()
    base = ctypes.addressof(buf)
    a16 = base + (-base) % 16  # a 16-byte aligned host address inside buf (never dereferenced)
    sink = (ctypes.c_uint32 * 4)()
    assert f(None, 16, sink, None) == -1
    assert f(a16, 16, None, None) == -1
    assert f(a16 + 4, 16, sink, None) == -1   # misaligned source
    assert f(a16, 24, sink, None) == -1       # not a multiple of 16
    assert f(a16, 0, sink, None) == 0         # nothing to read: nothing enqueued


@pytest.mark.parametrize("path", [0, 1, 2])
def test_launch_shapes_fit_the_hardware(T, path):
    """Every launch of the verify and commit paths, for every k the library
    accepts, has a workgroup of 64..1024 threads (a multiple of 64) and a grid
    within the hardware's limits; the selection and finalisation workgroups
    cover every row of their sequence.  A 17-wave selection workgroup (k = 16
    with one wave per AR row) once failed to launch and left the draft group
    unwritten; this catches that class of mistake on the CPU."""
    L = T.lib()
    shapes = (ctypes.c_int * 12)()
    for k in range(1, 17):
        for B in (1, 16, 65535 // (k + 1)):
            for V in (64, 4097, 128256, 151936):
                n = L.tidar_launch_shapes(path, B, k, V, 8, 128, 0, shapes)
                assert n >= 1, (path, k, B, V, n)
                for i in range(n):
                    gx, gy, block = shapes[3 * i], shapes[3 * i + 1], shapes[3 * i + 2]
                    assert 64 <= block <= 1024 and block % 64 == 0, (path, k, B, i, block)
                    assert 1 <= gx <= 0x7FFFFFFF and 1 <= gy <= 65535, (path, k, B, i, gx, gy)
                if path == 0:
                    assert n == (2 if k == 1 else 4)
                    assert shapes[0] * 4096 >= V and shapes[1] == B * (k + 1)   # every AR logit chunk
                    # one selection workgroup per sequence; its waves loop over the k+1 rows
                    assert shapes[3] == B and shapes[5] == 64 * min(k + 1, 16)
                    if k > 1:
                        assert shapes[7] == B * (k - 1)
                if path == 2:
                    assert n == 2 and shapes[1] == B * (k + 1) and shapes[4] == B * max(k - 1, 1)
                    assert shapes[0] * 4096 >= V  # every AR logit chunk
                    if k > 1:
                        assert shapes[3] * 8192 >= V  # every draft logit span
                    assert shapes[5] >= 64  # the finalising wave
    # beyond k = 16 every path refuses
    for path in (0, 1, 2):
        assert L.tidar_launch_shapes(path, 4, 17, 1000, 8, 128, 0, shapes) == -2
    assert L.tidar_launch_shapes(3, 4, 4, 1000, 8, 128, 0, shapes) == -1
