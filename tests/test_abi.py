"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects invalid arguments on the host before any GPU
call (fake, never-dereferenced pointer values are used)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]
LIB = os.path.join(ROOT, "int4_output_head_amd", "libint4vh.so")

OK, EINVAL, EALIGN, EWORKSPACE, EHIP, EUNSUPPORTED = 0, -1, -2, -3, -4, -5


def declared_functions():
    """Every function declared by the public headers (comments stripped)."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w ]*?[\s*]+(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from int4_output_head_amd.build import build_library
        build_library()
    L = ctypes.CDLL(LIB)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.verify_lm_head_int4.argtypes = [P, P, P, P, i32, i32, i32, P, P, P, P, P, sz, P]
    L.verify_lm_head_int4_batch.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    L.verify_lm_head_int4_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.verify_lm_head_int4_workspace_bytes.restype = sz
    L.verify_lm_head_int4_sampled_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.verify_lm_head_int4_sampled_workspace_bytes.restype = sz
    L.verify_lm_head_int4_workspace_init.argtypes = [P, sz, P]
    L.verify_lm_head_int4_check_weights.argtypes = [P, i32, i32, P, P]
    L.verify_lm_head_int4_status_string.argtypes = [i32]
    L.verify_lm_head_int4_status_string.restype = ctypes.c_char_p
    L.verify_lm_head_int4_last_error.restype = ctypes.c_char_p
    return L


def test_header_declares_expected_api():
    names = declared_functions()
    for n in ("verify_lm_head_int4", "verify_lm_head_int4_batch", "verify_lm_head_int4_batch_timed",
              "verify_lm_head_int4_workspace_bytes", "verify_lm_head_int4_workspace_init",
              "verify_lm_head_int4_check_weights", "verify_lm_head_int4_status_string",
              "verify_lm_head_int4_last_error", "verify_lm_head_int4_mapped",
              "verify_lm_head_int4_check_vocab_map", "verify_lm_head_int4_sampled",
              "verify_lm_head_int4_sampled_timed", "verify_lm_head_int4_sampled_workspace_bytes",
              "context_copy_propose", "context_copy_propose_timed",
              "requant_lm_head_int4_amax",
              "requant_lm_head_int4_scales", "requant_lm_head_int4_pack",
              "requant_lm_head_int4_pack_timed", "requant_lm_head_int4",
              "verify_lm_head_int4_batch_noalloc", "int4vh_stream_read"):
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (OK, EINVAL, EALIGN, EWORKSPACE, EHIP, EUNSUPPORTED):
        s = lib.verify_lm_head_int4_status_string(st)
        assert s and s != b"unknown status"
    assert lib.verify_lm_head_int4_status_string(12345) == b"unknown status"
    assert lib.verify_lm_head_int4_last_error() == b""


def test_workspace_bytes(lib):
    n = lib.verify_lm_head_int4_workspace_bytes(1, 16, 151936, 5120)
    assert n > 0 and n % 256 == 0
    assert lib.verify_lm_head_int4_workspace_bytes(1, 0, 10, 64) == 0
    assert lib.verify_lm_head_int4_workspace_bytes(1, 17, 10, 64) == 0
    assert lib.verify_lm_head_int4_workspace_bytes(1, 4, 0, 64) == 0
    assert lib.verify_lm_head_int4_workspace_bytes(1, 4, 10, 48) == 0


def test_sampled_workspace_bytes(lib):
    g = lib.verify_lm_head_int4_workspace_bytes
    f = lib.verify_lm_head_int4_sampled_workspace_bytes
    # up to 64 rows the sampled epilogue rides on the weight stream: same workspace
    for R, T in ((1, 16), (4, 16), (3, 7)):
        assert f(R, T, 151936, 5120) == g(R, T, 151936, 5120) > 0
    # above, the call's logits, then its rows' best keys per vocabulary tile
    # of 128, follow the batch area
    for R, T, V in ((5, 13, 100), (64, 4, 151936), (256, 16, 8192), (9, 8, 300001)):
        base = g(R, T, V, 5120)
        assert base > 0
        lg_end = (base + 255) // 256 * 256 + R * T * V * 4
        assert f(R, T, V, 5120) == (lg_end + 255) // 256 * 256 + R * T * ((V + 127) // 128) * 8
    assert f(1, 0, 10, 64) == 0
    assert f(257, 16, 10, 64) == 0                    # more than 4096 rows
    assert f(1, 4, 10, 48) == 0


A = 0x10000          # a fake, 256-byte aligned "device pointer" (never dereferenced)
WS = 1 << 20


def call(lib, hidden=A, w=A, s=A, d=A, T=4, V=100, H=256, lmax=A, amax=A, nacc=A, lout=None,
         ws=A, ws_bytes=WS):
    P = ctypes.c_void_p
    return lib.verify_lm_head_int4(P(hidden), P(w), P(s), P(d), T, V, H, P(lmax), P(amax),
                                   P(nacc), P(lout), P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), EINVAL), (dict(T=17), EINVAL), (dict(V=0), EINVAL), (dict(H=16), EINVAL),
    (dict(H=48), EINVAL), (dict(H=8224), EUNSUPPORTED), (dict(hidden=0), EINVAL),
    (dict(w=0), EINVAL), (dict(s=0), EINVAL), (dict(d=0), EINVAL), (dict(lmax=0), EINVAL),
    (dict(amax=0), EINVAL), (dict(nacc=0), EINVAL), (dict(ws=0), EINVAL),
    (dict(hidden=A + 8), EALIGN), (dict(w=A + 4), EALIGN), (dict(s=A + 2), EALIGN),
    (dict(lmax=A + 4), EALIGN), (dict(lout=A + 8), EALIGN), (dict(ws=A + 16), EALIGN),
    (dict(d=A + 2), EALIGN), (dict(ws_bytes=100), EWORKSPACE),
    (dict(V=1 << 30, H=4096), EUNSUPPORTED),
])
def test_verify_rejects_invalid_arguments(lib, kw, status):
    assert call(lib, **kw) == status


def test_draft_may_be_null_only_for_T1(lib):
    assert call(lib, d=0, T=2) == EINVAL
    assert call(lib, d=0, T=1, ws=A + 16) == EALIGN   # passes the draft check, fails later


def test_batch_rejects_invalid(lib):
    """Every call here fails host validation, so nothing is launched on the
    fake pointers."""
    P = ctypes.c_void_p
    f = lib.verify_lm_head_int4_batch

    def bcall(R, T, V=10, H=64, ws_bytes=WS, d=A):
        return f(P(A), P(A), P(A), P(d), R, T, V, H, P(A), P(A), P(A), None, P(A), ws_bytes, None)

    assert bcall(0, 4) == EINVAL
    assert bcall(4097, 1) == EINVAL           # more than 4096 rows
    assert bcall(257, 16) == EINVAL
    assert bcall(-3, 4) == EINVAL
    assert bcall(64, 17) == EINVAL
    assert bcall(64, 4, d=0) == EINVAL        # drafts required for T > 1
    need = lib.verify_lm_head_int4_workspace_bytes(64, 4, 151936, 5120)
    assert bcall(64, 4, 151936, 5120, ws_bytes=need - 256) == EWORKSPACE
    assert bcall(64, 4, 151936, 5120, ws_bytes=need, d=A + 2) == EALIGN


def test_batch_workspace_bytes(lib):
    wb = lib.verify_lm_head_int4_workspace_bytes
    assert wb(4097, 1, 10, 64) == 0 and wb(257, 16, 10, 64) == 0
    small = wb(1, 16, 151936, 5120)
    # up to 16 rows: the single-block layout; 17-64 rows: one activation
    # fragment area per group of 16 rows (the weight-stream kernels); beyond:
    # activation fragments of 128-row tiles, 3 bytes per row and (padded)
    # channel (the matrix-core batch kernels)
    assert wb(4, 4, 151936, 5120) == small
    big = wb(64, 4, 151936, 5120)
    assert big > small and big % 256 == 0
    assert wb(256, 16, 10, 64) > 0
    per_tile = (wb(384, 1, 10, 5120) - wb(256, 1, 10, 5120))
    assert per_tile == 128 * 5120 * 3
    assert wb(65, 1, 10, 5120) == wb(128, 1, 10, 5120)
    assert wb(129, 1, 10, 5120) == wb(256, 1, 10, 5120)
    assert wb(17, 1, 10, 5120) == wb(32, 1, 10, 5120)
    group = wb(48, 1, 10, 5120) - wb(32, 1, 10, 5120)
    assert group > 0 and group % 256 == 0
    assert wb(64, 1, 10, 5120) - wb(17, 1, 10, 5120) == 2 * group


def test_workspace_init_and_check_weights_validation(lib):
    P = ctypes.c_void_p
    assert lib.verify_lm_head_int4_workspace_init(None, WS, None) == EINVAL
    assert lib.verify_lm_head_int4_workspace_init(P(A + 64), WS, None) == EALIGN
    assert lib.verify_lm_head_int4_workspace_init(P(A), 16, None) == EWORKSPACE
    assert lib.verify_lm_head_int4_check_weights(None, 10, 64, P(A), None) == EINVAL
    assert lib.verify_lm_head_int4_check_weights(P(A), 10, 48, P(A), None) == EINVAL
    assert lib.verify_lm_head_int4_check_weights(P(A + 8), 10, 64, P(A), None) == EALIGN


def test_requant_rejects_invalid_arguments(lib):
    """Host validation of the requantisation entry points (fake pointers,
    nothing launched)."""
    P, i32 = ctypes.c_void_p, ctypes.c_int
    am = lib.requant_lm_head_int4_amax
    am.argtypes = [P, i32, i32, i32, P, i32, P]
    sc = lib.requant_lm_head_int4_scales
    sc.argtypes = [P, i32, P, P]
    pk = lib.requant_lm_head_int4_pack
    pk.argtypes = [P, i32, i32, i32, P, P, P]
    rq = lib.requant_lm_head_int4
    rq.argtypes = [P, i32, i32, i32, P, i32, i32, P, P, P, P]
    a = P(A)
    assert am(None, 0, 4, 64, a, 0, None) == EINVAL
    assert am(a, 2, 4, 64, a, 0, None) == EINVAL          # unknown dtype
    assert am(a, 0, 0, 64, a, 0, None) == EINVAL
    assert am(a, 0, 4, 48, a, 0, None) == EINVAL
    assert am(a, 1, 4, 64, None, 0, None) == EINVAL
    assert am(P(A + 8), 0, 4, 64, a, 0, None) == EALIGN
    assert am(a, 0, 4, 64, P(A + 2), 0, None) == EALIGN
    assert am(a, 0, 1 << 30, 4096, a, 0, None) == EUNSUPPORTED
    assert sc(None, 64, a, None) == EINVAL
    assert sc(a, 16, a, None) == EINVAL
    assert sc(a, 64, P(A + 2), None) == EALIGN
    assert pk(a, 0, 0, 64, a, a, None) == EINVAL
    assert pk(a, 3, 10, 64, a, a, None) == EINVAL
    assert pk(a, 0, 10, 40, a, a, None) == EINVAL
    assert pk(a, 0, 10, 64, None, a, None) == EINVAL
    assert pk(a, 0, 10, 64, a, None, None) == EINVAL
    assert pk(P(A + 2), 0, 10, 64, a, a, None) == EALIGN
    assert pk(a, 0, 10, 64, a, P(A + 8), None) == EALIGN
    assert pk(a, 0, 1 << 28, 8192, a, a, None) == EUNSUPPORTED
    assert rq(a, 0, 10, 64, a, 0, 0, a, a, a, None) == EINVAL
    assert rq(a, 0, 10, 64, a, 5, 4, a, a, a, None) == EINVAL
    assert rq(a, 0, 10, 64, a, 0, 4, a, P(A + 2), a, None) == EALIGN
    assert rq(a, 0, 1 << 28, 8192, a, 0, 4, a, a, a, None) == EUNSUPPORTED


def test_sampled_rejects_invalid_arguments(lib):
    P, i32 = ctypes.c_void_p, ctypes.c_int
    f = lib.verify_lm_head_int4_sampled
    f.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, ctypes.c_float, P, P, P, P, P, P, P, P,
                  ctypes.c_size_t, P]
    a = P(A)

    def scall(R=1, T=4, V=100, H=256, k=8, tau=1.0, dprob=A, unif=A, pdr=A, tids=A, tlog=A, lse=A,
              ws_bytes=WS):
        return f(a, a, a, a, P(dprob), P(unif), R, T, V, H, k, tau, a, a, P(tids), P(tlog), P(lse),
                 P(pdr), a, a, ws_bytes, None)

    assert scall(k=-1) == EINVAL
    assert scall(k=0, tids=0, tlog=0, ws_bytes=100) == EWORKSPACE   # k = 0 needs no top-k buffers
    assert scall(lse=A + 2) == EALIGN
    assert scall(k=17) == EINVAL
    assert scall(k=8, V=7) == EINVAL                  # k > V
    assert scall(tau=0.0) == EINVAL
    assert scall(tau=-1.0) == EINVAL
    assert scall(tau=float("nan")) == EINVAL
    assert scall(tau=float("inf")) == EINVAL
    assert scall(dprob=0) == EINVAL
    assert scall(unif=0) == EINVAL
    assert scall(pdr=0) == EINVAL
    assert scall(tids=0) == EINVAL
    assert scall(tlog=A + 2) == EALIGN
    # more than 64 rows: the batch path, whose workspace also holds the logits
    assert scall(R=5, T=13, ws_bytes=lib.verify_lm_head_int4_workspace_bytes(5, 13, 100, 256)) == EWORKSPACE
    assert scall(R=5, T=13, ws_bytes=lib.verify_lm_head_int4_sampled_workspace_bytes(5, 13, 100, 256) - 1) \
        == EWORKSPACE
    assert scall(R=257, T=16) == EINVAL               # more than 4096 rows
    assert scall(R=1, T=17) == EINVAL
    assert scall(ws_bytes=100) == EWORKSPACE


def test_context_copy_rejects_invalid_arguments(lib):
    P, i32 = ctypes.c_void_p, ctypes.c_int
    f = lib.context_copy_propose
    f.argtypes = [P, P, i32, P, i32, i32, i32, P, P, P, P, P]
    a = P(A)

    def ccall(R=2, n_max=16, n_min=2, n_out=8, pr=A, off=A, keys=A, tok=A):
        return f(P(pr), P(off), R, P(keys), n_max, n_min, n_out, P(tok), a, a, a, None)

    assert ccall(R=0) == EINVAL
    assert ccall(n_max=0) == EINVAL
    assert ccall(n_max=65) == EINVAL
    assert ccall(n_min=0) == EINVAL
    assert ccall(n_min=17) == EINVAL
    assert ccall(n_out=0) == EINVAL
    assert ccall(n_out=65) == EINVAL
    assert ccall(pr=0) == EINVAL
    assert ccall(tok=0) == EINVAL
    assert ccall(off=A + 4) == EALIGN
    assert ccall(keys=A + 2) == EALIGN
