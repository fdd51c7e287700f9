"""libkla.so loads, exports every entry point include/kla.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: every
call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")
# KLA_TEST_LIB: the host-only sanitizer build of the C-ABI layer
# (tests/sanitize/build.py); the default is the in-tree library.
LIB = os.environ.get("KLA_TEST_LIB") or os.path.join(ROOT, "delta_rule_linear_amd", "libkla.so")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from delta_rule_linear_amd import build
        build.build()
    L = ctypes.CDLL(LIB)
    L.kla_fwd_chunked.restype = ctypes.c_int
    L.kla_fwd_chunked.argtypes = [ctypes.c_void_p] * 6 + [
        ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.kla_decode_step.restype = ctypes.c_int
    L.kla_decode_step.argtypes = [ctypes.c_void_p] * 7 + [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int, ctypes.c_void_p]
    L.kla_fwd_chunked_ex.restype = ctypes.c_int
    L.kla_fwd_chunked_ex.argtypes = (L.kla_fwd_chunked.argtypes[:14] + [ctypes.c_int]
                                     + L.kla_fwd_chunked.argtypes[14:])
    L.kla_fwd_chunked_split.restype = ctypes.c_int
    L.kla_fwd_chunked_split.argtypes = (L.kla_fwd_chunked.argtypes[:14] + [ctypes.c_int, ctypes.c_int32]
                                        + L.kla_fwd_chunked.argtypes[14:])
    L.kla_fwd_chunked_split_workspace_size.restype = ctypes.c_size_t
    L.kla_fwd_chunked_split_workspace_size.argtypes = [ctypes.c_int32] * 5
    L.kla_decode_step_ex.restype = ctypes.c_int
    L.kla_decode_step_ex.argtypes = L.kla_decode_step.argtypes[:13] + [ctypes.c_int, ctypes.c_void_p]
    L.kla_fwd_chunked_kda.restype = ctypes.c_int
    L.kla_fwd_chunked_kda.argtypes = L.kla_fwd_chunked_ex.argtypes
    L.kla_decode_step_kda.restype = ctypes.c_int
    L.kla_decode_step_kda.argtypes = L.kla_decode_step_ex.argtypes
    L.kla_ccq_state_floats.restype = ctypes.c_size_t
    L.kla_ccq_state_floats.argtypes = [ctypes.c_int32]
    L.kla_fwd_chunked_ccq_workspace_size.restype = ctypes.c_size_t
    L.kla_fwd_chunked_ccq_workspace_size.argtypes = [ctypes.c_int64] + [ctypes.c_int32] * 3 + [ctypes.c_int]
    L.kla_decode_step_ccq_workspace_size.restype = ctypes.c_size_t
    L.kla_decode_step_ccq_workspace_size.argtypes = [ctypes.c_int32] * 3
    V, F = ctypes.c_void_p, ctypes.c_float
    L.kla_fwd_chunked_ccq.restype = ctypes.c_int
    L.kla_fwd_chunked_ccq.argtypes = [V] * 7 + [ctypes.c_int32, ctypes.c_int64] + [ctypes.c_int32] * 4 + [
        F, ctypes.c_int, ctypes.c_int] + [V] * 6 + [ctypes.c_size_t, V]
    L.kla_decode_step_ccq.restype = ctypes.c_int
    L.kla_decode_step_ccq.argtypes = [V] * 9 + [ctypes.c_int32] * 4 + [F, ctypes.c_int, ctypes.c_int, V,
                                                                        ctypes.c_size_t, V]
    L.kla_status_string.restype = ctypes.c_char_p
    L.kla_status_string.argtypes = [ctypes.c_int]
    L.kla_version.restype = ctypes.c_char_p
    L.kla_bwd_chunked_workspace_size.restype = ctypes.c_size_t
    L.kla_bwd_chunked_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64] + [ctypes.c_int32] * 4
    L.kla_bwd_chunked.restype = ctypes.c_int
    L.kla_bwd_chunked.argtypes = [V] * 6 + [ctypes.c_int32, ctypes.c_int64] + [ctypes.c_int32] * 4 + [
        F, ctypes.c_int, ctypes.c_int] + [V] * 9 + [V, ctypes.c_size_t, V]
    L.kla_fwd_chunked_workspace_size.restype = ctypes.c_size_t
    L.kla_fwd_chunked_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int64] + [ctypes.c_int32] * 4
    return L


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["kla_fwd_chunked", "kla_fwd_chunked_ex",
                                           "kla_fwd_chunked_split", "kla_fwd_chunked_kda",
                                           "kla_fwd_chunked_split_noalloc",
                                           "kla_decode_step_kda", "kla_ccq_state_floats",
                                           "kla_fwd_chunked_ccq", "kla_fwd_chunked_ccq_workspace_size",
                                           "kla_decode_step_ccq", "kla_decode_step_ccq_workspace_size",
                                           "kla_fwd_chunked_split_workspace_size",
                                           "kla_fwd_chunked_workspace_size", "kla_decode_step",
                                           "kla_decode_step_ex", "kla_status_string",
                                           "kla_version", "kla_bwd_chunked",
                                           "kla_bwd_chunked_workspace_size"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR, 7):
        s = lib.kla_status_string(code)
        assert s and len(s) > 0
    assert b"gfx950" in lib.kla_version()


# Fake, never-dereferenced device addresses (validation fails before use).
BASE = 1 << 40
MB = 1 << 20


def fwd_args(**over):
    a = dict(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, alpha=BASE + 192 * MB,
             eta=BASE + 200 * MB, cu=None, n_seqs=2, tok=128, H=2, dk=64, dv=64, chunk=64,
             eps=1e-6, dtype=1, s0=None, o=BASE + 256 * MB, s1=None, ws=None, wsb=0, stream=None)
    a.update(over)
    return [a[x] for x in ("q", "k", "v", "alpha", "eta", "cu", "n_seqs", "tok", "H", "dk", "dv",
                           "chunk", "eps", "dtype", "s0", "o", "s1", "ws", "wsb", "stream")]


@pytest.mark.parametrize("over,code", [
    (dict(n_seqs=0), INVALID),
    (dict(H=0), INVALID),
    (dict(tok=-1), INVALID),
    (dict(tok=129), INVALID),          # dense batch not divisible by n_seqs
    (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(q=None), INVALID),
    (dict(o=None), INVALID),
    (dict(eta=None), INVALID),         # alpha may be NULL (no decay), eta may not
    (dict(q=BASE + 2), INVALID),       # misaligned
    (dict(o=BASE + 256 * MB + 4), INVALID),
    (dict(o=BASE + 8), INVALID),       # o overlaps q
    (dict(s0=BASE + 300 * MB, s1=BASE + 300 * MB + 16), INVALID),  # partial state overlap
    (dict(s1=BASE + 64 * MB), INVALID),  # final state overlaps k
    (dict(dk=96, dv=96), UNSUPPORTED),
    (dict(dk=64, dv=128), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED),
    (dict(dtype=5), UNSUPPORTED),
])
def test_fwd_rejects(lib, over, code):
    assert lib.kla_fwd_chunked(*fwd_args(**over)) == code


@pytest.mark.parametrize("mode", [2, -1, 7])
def test_fwd_ex_rejects_unknown_beta_mode(lib, mode):
    a = fwd_args()
    assert lib.kla_fwd_chunked_ex(*a[:14], mode, *a[14:]) == INVALID


def test_fwd_ex_checks_like_fwd(lib):
    for over, code in ((dict(n_seqs=0), INVALID), (dict(eta=None), INVALID),
                       (dict(dk=96, dv=96), UNSUPPORTED), (dict(o=BASE + 8), INVALID)):
        a = fwd_args(**over)
        assert lib.kla_fwd_chunked_ex(*a[:14], 1, *a[14:]) == code


def test_split_workspace_query(lib):
    # maps (A, B) for P-1 segments and start states for P: (3P - 2) fp32 d x d per (seq, head)
    assert lib.kla_fwd_chunked_split_workspace_size(2, 16, 128, 128, 3) == 2 * 16 * 128 * 128 * 4 * 7
    assert lib.kla_fwd_chunked_split_workspace_size(2, 16, 64, 64, 2) == 2 * 16 * 64 * 64 * 4 * 4
    assert lib.kla_fwd_chunked_split_workspace_size(2, 16, 128, 128, 1) == 0
    assert lib.kla_fwd_chunked_split_workspace_size(2, 16, 96, 96, 3) == 0


def split_call(lib, n_splits, **over):
    a = fwd_args(**over)
    return lib.kla_fwd_chunked_split(*a[:14], 0, n_splits, *a[14:])


NOALLOC_MAX = 32 * MB


def noalloc_call(lib, n_splits, **over):
    a = fwd_args(**over)
    # the workspace arguments (a[17], a[18]) are not part of this entry point
    return lib.kla_fwd_chunked_split_noalloc(*a[:14], 0, n_splits, a[14], a[15], a[16], a[19])


def test_noalloc_header_limit_matches():
    text = open(HEADER).read()
    m = re.search(r"#define KLA_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * MB == NOALLOC_MAX


def test_noalloc_split_rejects_on_the_host(lib):
    """Validation and the scratch limit come before any HIP call."""
    L = lib
    L.kla_fwd_chunked_split_noalloc.restype = ctypes.c_int
    L.kla_fwd_chunked_split_noalloc.argtypes = (L.kla_fwd_chunked.argtypes[:14]
                                                + [ctypes.c_int, ctypes.c_int32]
                                                + [ctypes.c_void_p] * 4)
    assert noalloc_call(lib, 0) == INVALID                    # n_splits < 1
    assert noalloc_call(lib, 1025) == INVALID                 # n_splits too large
    assert noalloc_call(lib, 2, n_seqs=0) == INVALID
    assert noalloc_call(lib, 2, q=BASE + 2) == INVALID        # misaligned
    assert noalloc_call(lib, 2, o=BASE + 8) == INVALID        # o overlaps q
    assert noalloc_call(lib, 2, dk=96, dv=96) == UNSUPPORTED
    # (3P - 2) d x d fp32 per (sequence, head) must fit the 32 MiB array:
    # 2 sequences x 16 heads at d = 128 allow P <= 6
    big = dict(n_seqs=2, H=16, dk=128, dv=128, tok=2 * 64,
               o=BASE + 4096 * MB, eta=BASE + 3072 * MB, alpha=BASE + 3200 * MB)
    assert lib.kla_fwd_chunked_split_workspace_size(2, 16, 128, 128, 7) > NOALLOC_MAX
    assert lib.kla_fwd_chunked_split_workspace_size(2, 16, 128, 128, 6) <= NOALLOC_MAX
    assert noalloc_call(lib, 7, **big) == WORKSPACE


def test_split_rejects(lib):
    ws = BASE + 512 * MB
    need = 2 * 2 * 64 * 64 * 4 * 4   # fwd_args: n_seqs=2, H=2, d=64; P=2
    assert split_call(lib, 0) == INVALID                         # n_splits < 1
    assert split_call(lib, 1025) == INVALID                      # n_splits too large
    assert split_call(lib, 2) == WORKSPACE                       # no workspace
    assert split_call(lib, 2, ws=ws, wsb=need - 1) == WORKSPACE  # short workspace
    assert split_call(lib, 2, ws=ws + 8, wsb=need) == INVALID    # misaligned
    assert split_call(lib, 2, ws=BASE + 256 * MB, wsb=need) == INVALID  # overlaps o
    assert split_call(lib, 2, ws=BASE, wsb=need) == INVALID      # overlaps q
    assert split_call(lib, 2, ws=ws, wsb=need, n_seqs=0) == INVALID
    assert split_call(lib, 2, ws=ws, wsb=need, dk=96, dv=96) == UNSUPPORTED


@pytest.mark.parametrize("over,code", [
    (dict(alpha=None), INVALID),                 # the per-channel rates are required
    (dict(alpha=BASE + 192 * MB + 4), INVALID),  # misaligned rates
    (dict(o=BASE + 192 * MB + 1024), INVALID),   # o inside the [tok, H, dk] rates
    (dict(n_seqs=0), INVALID),
    (dict(eta=None), INVALID),
    (dict(dk=96, dv=96), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED),
])
def test_fwd_kda_rejects(lib, over, code):
    a = fwd_args(**over)
    assert lib.kla_fwd_chunked_kda(*a[:14], 0, *a[14:]) == code


def test_fwd_kda_rejects_unknown_beta_mode(lib):
    a = fwd_args()
    assert lib.kla_fwd_chunked_kda(*a[:14], 5, *a[14:]) == INVALID


def test_ccq_sizes(lib):
    assert lib.kla_ccq_state_floats(128) == 128 * 128 + 128 + 4
    th = 100 * 2
    r = lambda x: (x + 255) // 256 * 256
    assert lib.kla_fwd_chunked_ccq_workspace_size(100, 2, 64, 64, 1) == 2 * r(th * 64 * 2) + r(th * 64 * 4)
    assert lib.kla_fwd_chunked_ccq_workspace_size(100, 2, 64, 64, 0) == r(th * 64 * 4)
    assert lib.kla_fwd_chunked_ccq_workspace_size(0, 2, 64, 64, 1) == 0
    assert lib.kla_decode_step_ccq_workspace_size(4, 2, 128) == r(4 * 2 * 128 * 4)


def ccq_args(**over):
    # fwd_args layout plus lambda, ccq_in/ccq_out and a workspace large enough
    a = dict(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, alpha=BASE + 192 * MB,
             eta=BASE + 200 * MB, lam=BASE + 208 * MB, cu=None, n_seqs=2, tok=128, H=2, dk=64,
             dv=64, chunk=64, eps=1e-6, dtype=1, beta=0, s0=None, c0=None, o=BASE + 256 * MB,
             s1=None, c1=None, ws=BASE + 512 * MB, wsb=1 << 24, stream=None)
    a.update(over)
    return [a[x] for x in ("q", "k", "v", "alpha", "eta", "lam", "cu", "n_seqs", "tok", "H", "dk",
                           "dv", "chunk", "eps", "dtype", "beta", "s0", "c0", "o", "s1", "c1", "ws",
                           "wsb", "stream")]


@pytest.mark.parametrize("over,code", [
    (dict(lam=None), INVALID),                  # the gate is required
    (dict(wsb=0), WORKSPACE),
    (dict(ws=BASE + 512 * MB + 8), INVALID),     # misaligned workspace
    (dict(ws=BASE), INVALID),                   # workspace overlaps q
    (dict(c1=BASE + 256 * MB + 64), INVALID),   # end sums overlap o
    (dict(c0=BASE + 300 * MB, c1=BASE + 300 * MB), INVALID),  # end sums alias the start sums
    (dict(c1=BASE + 300 * MB + 4), INVALID),    # misaligned end sums
    (dict(beta=3), INVALID),
    (dict(dk=96, dv=96), UNSUPPORTED),
    (dict(n_seqs=0), INVALID),
])
def test_fwd_ccq_rejects(lib, over, code):
    assert lib.kla_fwd_chunked_ccq(*ccq_args(**over)) == code


def dccq_args(**over):
    a = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, eta=BASE + 4 * MB,
             lam=BASE + 5 * MB, state=BASE + 8 * MB, cs=BASE + 16 * MB, o=BASE + 64 * MB, N=4, H=2,
             dk=128, dv=128, eps=1e-6, dtype=1, beta=0, ws=BASE + 128 * MB, wsb=1 << 20,
             stream=None)
    a.update(over)
    return [a[x] for x in ("q", "k", "v", "alpha", "eta", "lam", "state", "cs", "o", "N", "H",
                           "dk", "dv", "eps", "dtype", "beta", "ws", "wsb", "stream")]


@pytest.mark.parametrize("over,code", [
    (dict(lam=None), INVALID),
    (dict(cs=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(wsb=16), WORKSPACE),
    (dict(cs=BASE + 8 * MB + 1024), INVALID),   # sums overlap the state
    (dict(o=BASE + 16 * MB + 64), INVALID),     # o inside the sums
    (dict(dk=32, dv=32), UNSUPPORTED),
])
def test_decode_ccq_rejects(lib, over, code):
    assert lib.kla_decode_step_ccq(*dccq_args(**over)) == code


def test_workspace_query(lib):
    # the longest-first order of 2 .. 1024 packed sequences: one int32 each, 256-byte rounded
    assert lib.kla_fwd_chunked_workspace_size(8, 16384, 16, 128, 128, 64) == 256
    assert lib.kla_fwd_chunked_workspace_size(64, 282233, 16, 128, 128, 64) == 256
    assert lib.kla_fwd_chunked_workspace_size(65, 1000, 16, 128, 128, 64) == 512
    assert lib.kla_fwd_chunked_workspace_size(1024, 1000, 16, 128, 128, 64) == 4096
    assert lib.kla_fwd_chunked_workspace_size(1, 1000, 16, 128, 128, 64) == 0
    assert lib.kla_fwd_chunked_workspace_size(1025, 100000, 16, 128, 128, 64) == 0


def test_packed_needs_the_order_workspace(lib):
    cu = BASE + 500 * MB
    ws = BASE + 600 * MB
    a = fwd_args(cu=cu)
    assert lib.kla_fwd_chunked(*a) == WORKSPACE                    # none given
    a = fwd_args(cu=cu, ws=ws, wsb=255)
    assert lib.kla_fwd_chunked(*a) == WORKSPACE                    # short
    a = fwd_args(cu=cu, ws=ws + 4, wsb=256)
    assert lib.kla_fwd_chunked(*a) == INVALID                      # misaligned
    a = fwd_args(cu=cu, ws=BASE + 256 * MB, wsb=256)
    assert lib.kla_fwd_chunked(*a) == INVALID                      # overlaps o
    a = fwd_args(cu=cu, ws=cu, wsb=256)
    assert lib.kla_fwd_chunked(*a) == INVALID                      # overlaps cu_seqlens


def dec_args(**over):
    a = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, eta=BASE + 4 * MB,
             state=BASE + 8 * MB, o=BASE + 64 * MB, N=4, H=2, dk=128, dv=128, eps=1e-6, dtype=1,
             stream=None)
    a.update(over)
    return [a[x] for x in ("q", "k", "v", "alpha", "eta", "state", "o", "N", "H", "dk", "dv",
                           "eps", "dtype", "stream")]


@pytest.mark.parametrize("over,code", [
    (dict(N=0), INVALID),
    (dict(state=None), INVALID),
    (dict(o=BASE + 8 * MB + 64), INVALID),   # o inside state
    (dict(state=BASE + 4), INVALID),         # misaligned
    (dict(state=BASE + 2 * MB), INVALID),    # state overlaps v
    (dict(eps=-0.5), INVALID),
    (dict(dk=32, dv=32), UNSUPPORTED),
    (dict(dtype=3), UNSUPPORTED),
])
def test_decode_rejects(lib, over, code):
    assert lib.kla_decode_step(*dec_args(**over)) == code
    a = dec_args(**over)
    assert lib.kla_decode_step_ex(*a[:13], 1, a[13]) == code


@pytest.mark.parametrize("over,code", [
    (dict(alpha=None), INVALID),
    (dict(alpha=BASE + 3 * MB + 8), INVALID),
    (dict(o=BASE + 3 * MB + 2048), INVALID),  # o inside the [N, H, dk] rates
    (dict(N=0), INVALID),
    (dict(dk=32, dv=32), UNSUPPORTED),
])
def test_decode_kda_rejects(lib, over, code):
    a = dec_args(**over)
    assert lib.kla_decode_step_kda(*a[:13], 0, a[13]) == code


@pytest.mark.parametrize("mode", [2, -3])
def test_decode_ex_rejects_unknown_beta_mode(lib, mode):
    a = dec_args()
    assert lib.kla_decode_step_ex(*a[:13], mode, a[13]) == INVALID


def test_binding_names_match_the_abi():
    import delta_rule_linear_amd as pkg
    for name in ("kla_fwd_chunked", "kla_decode_step", "kla_fwd_chunked_ex", "kla_decode_step_ex",
                 "kla_fwd_chunked_split", "kla_fwd_chunked_kda", "kla_decode_step_kda",
                 "kla_fwd_chunked_ccq", "kla_decode_step_ccq", "kla_ccq_state_floats",
                 "kla_fwd_chunked_workspace_size",
                 "kla_fwd_chunked_split_workspace_size", "kla_status_string", "kla_version"):
        assert callable(getattr(pkg, name))


def test_bwd_workspace_query(lib):
    # chunk-start states (tok/64 + n_seqs slots), 8 column slices of dq and dk,
    # their dbeta and decay sums, |k|^2 and the final states (each section
    # rounded up to 64 floats)
    n, tok, H, d = 8, 16384, 16, 128
    up = lambda x: (x + 63) // 64 * 64
    want = (up((tok // 64 + n) * H * d * d) + 2 * up(8 * tok * H * d) + 2 * up(8 * tok * H)
            + up(tok * H) + up(n * H * d * d)) * 4
    assert lib.kla_bwd_chunked_workspace_size(n, tok, H, d, d, 64) == want
    assert lib.kla_bwd_chunked_workspace_size(n, tok, H, 96, 96, 64) == 0
    assert lib.kla_bwd_chunked_workspace_size(n, tok, H, d, d, 32) == 0
    assert lib.kla_bwd_chunked_workspace_size(0, tok, H, d, d, 64) == 0


def bwd_args(lib, **over):
    a = dict(q=BASE, k=BASE + 64 * MB, v=BASE + 128 * MB, alpha=BASE + 192 * MB,
             eta=BASE + 200 * MB, cu=None, n_seqs=2, tok=128, H=2, dk=64, dv=64, chunk=64,
             eps=1e-6, dtype=1, beta=0, s0=None, do=BASE + 256 * MB, dfin=None,
             dq=BASE + 320 * MB, dkk=BASE + 384 * MB, dvv=BASE + 448 * MB, da=BASE + 512 * MB,
             de=BASE + 520 * MB, ds0=None, ws=BASE + 1024 * MB, wsb=None, stream=None)
    a.update(over)
    if a["wsb"] is None:
        a["wsb"] = lib.kla_bwd_chunked_workspace_size(2, 128, 2, 64, 64, 64)
    return [a[x] for x in ("q", "k", "v", "alpha", "eta", "cu", "n_seqs", "tok", "H", "dk", "dv",
                           "chunk", "eps", "dtype", "beta", "s0", "do", "dfin", "dq", "dkk", "dvv",
                           "da", "de", "ds0", "ws", "wsb", "stream")]


@pytest.mark.parametrize("over,code", [
    (dict(n_seqs=0), INVALID),
    (dict(tok=129), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(beta=2), INVALID),
    (dict(do=None), INVALID),
    (dict(dq=None), INVALID),
    (dict(de=None), INVALID),
    (dict(da=None), INVALID),           # alpha given: its gradient is required
    (dict(ws=None), INVALID),
    (dict(wsb=1024), WORKSPACE),
    (dict(dq=BASE + 8), INVALID),       # output overlaps q
    (dict(dkk=BASE + 320 * MB + 64), INVALID),  # dk overlaps dq
    (dict(ds0=BASE + 256 * MB), INVALID),       # initial-state gradient overlaps d_o
    (dict(ws=BASE + 448 * MB), INVALID),        # workspace overlaps dv
    (dict(dvv=BASE + 448 * MB + 4), INVALID),   # misaligned
    (dict(dk=96, dv=96), UNSUPPORTED),
    (dict(chunk=32), UNSUPPORTED),
    (dict(dtype=5), UNSUPPORTED),
])
def test_bwd_rejects(lib, over, code):
    assert lib.kla_bwd_chunked(*bwd_args(lib, **over)) == code


def test_bwd_no_alpha_needs_no_alpha_gradient(lib):
    # without a decay gate the alpha gradient pointer is ignored; a wrong dk
    # size still fails, so validation ran to the end without launching
    assert lib.kla_bwd_chunked(*bwd_args(lib, alpha=None, da=None, dk=96, dv=96)) == UNSUPPORTED
