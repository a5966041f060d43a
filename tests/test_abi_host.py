"""The C ABI on a host without a GPU: the library loads, exports every symbol
include/moga.h declares, sizes workspaces, and rejects bad arguments on the
host before launching anything (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moga.h")
LIB = os.path.join(ROOT, "sparse_attention_long_router_amd", "libmoga.so")

OK, ENULL, ESHAPE, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4, -5
FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._load_build_script().build(verbose=False)
    from sparse_attention_long_router_amd import _lib
    return _lib.LIB


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moga_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) == 22, names
    for n in names:
        assert hasattr(lib, n), n
    from sparse_attention_long_router_amd import _lib
    assert sorted(_lib.SIGNATURES) == names


def test_strerror_and_version(lib):
    for code in (OK, ENULL, ESHAPE, EUNSUP, EWS, EHIP):
        assert lib.moga_strerror(code)
    assert lib.moga_strerror(-99) == b"unknown status"
    assert lib.moga_version() >= 100


def test_binding_matches_library_version():
    """The binding refuses a library built from other sources (a stale build)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    api = open(os.path.join(root, "sparse_attention_long_router_amd", "csrc", "api.hip")).read()
    src_version = int(re.search(r"moga_version\(void\) \{ return (\d+); \}", api).group(1))
    from sparse_attention_long_router_amd import _lib
    assert _lib.EXPECTED_VERSION == src_version
    assert _lib.LIB.moga_version() == src_version


def test_workspace_sizes(lib):
    ws = lib.moga_workspace_bytes
    assert ws(0, 1000, 4, 2, 64) == 0                      # route needs none
    assert ws(3, 1000, 4, 2, 64) == 0 and ws(4, 1000, 4, 2, 64) == 0
    n = ws(1, 190320, 16, 12, 128)
    nblk = -(-190320 // 1024)
    assert n >= 2 * 16 * nblk * 4 and n % 256 == 0
    assert ws(2, 190320, 16, 12, 128) >= (64 + 65) * 4
    assert ws(1, 0, 16, 12, 128) == 0 and ws(1, 10, 65, 1, 64) == 0 and ws(1, 10, 0, 1, 64) == 0


def test_route_argument_errors(lib):
    r = lib.moga_route
    assert r(None, FAKE, None, 10, 64, 4, FAKE, FAKE, None, 0, None) == ENULL
    assert r(FAKE, FAKE, None, 10, 64, 4, None, FAKE, None, 0, None) == ENULL
    assert r(FAKE, FAKE, None, 0, 64, 4, FAKE, FAKE, None, 0, None) == ESHAPE
    assert r(FAKE, FAKE, None, 1 << 31, 64, 4, FAKE, FAKE, None, 0, None) == ESHAPE
    assert r(FAKE, FAKE, None, 10, 64, 0, FAKE, FAKE, None, 0, None) == ESHAPE
    assert r(FAKE, FAKE, None, 10, 64, 65, FAKE, FAKE, None, 0, None) == EUNSUP
    assert r(FAKE, FAKE, None, 10, 48, 4, FAKE, FAKE, None, 0, None) == EUNSUP


def test_permute_argument_errors(lib):
    p = lib.moga_permute
    good_ws = lib.moga_workspace_bytes(1, 100, 4, 2, 128)
    args = dict(g=FAKE, Q=FAKE, K=FAKE, V=FAKE, N=100, H=2, D=128, M=4, Qp=FAKE, Kp=FAKE, Vp=FAKE,
                perm=FAKE, cu=FAKE, mx=FAKE, ws=FAKE, nb=good_ws)

    def call(**kw):
        a = dict(args, **kw)
        return p(a["g"], a["Q"], a["K"], a["V"], a["N"], a["H"], a["D"], a["M"], a["Qp"], a["Kp"], a["Vp"],
                 a["perm"], a["cu"], a["mx"], a["ws"], a["nb"], None)

    assert call(g=None) == ENULL
    assert call(cu=None) == ENULL
    assert call(Kp=None) == ENULL                    # some but not all row tensors
    assert call(N=0) == ESHAPE
    assert call(M=0) == ESHAPE
    assert call(M=65) == EUNSUP
    assert call(D=96) == EUNSUP
    assert call(H=0) == ESHAPE
    assert call(H=128, D=128) == EUNSUP              # H*D > 8192
    assert call(ws=None) == EWS
    assert call(nb=good_ws - 1) == EWS


def test_attention_argument_errors(lib):
    a = lib.moga_group_attention
    nb = lib.moga_workspace_bytes(2, 100, 4, 2, 128)
    assert a(None, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, FAKE, FAKE, nb, None) == ENULL
    assert a(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, None, FAKE, nb, None) == ENULL
    assert a(FAKE, FAKE, FAKE, FAKE, 0, 2, 128, 4, 0.0, FAKE, FAKE, nb, None) == ESHAPE
    assert a(FAKE, FAKE, FAKE, FAKE, 100, 2, 80, 4, 0.0, FAKE, FAKE, nb, None) == EUNSUP
    assert a(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 70, 0.0, FAKE, FAKE, nb, None) == EUNSUP
    assert a(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, FAKE, None, nb, None) == EWS
    assert a(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, FAKE, FAKE, nb - 1, None) == EWS


def test_fused_attention_argument_errors(lib):
    a = lib.moga_group_attention_unpermute
    nb = lib.moga_workspace_bytes(2, 100, 4, 2, 128)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, 0.0, FAKE, FAKE, nb, None]
    assert a(*args[:4], None, *args[5:]) == ENULL          # perm
    assert a(*args[:5], None, *args[6:]) == ENULL          # gate
    assert a(*args[:6], 0, *args[7:]) == ESHAPE            # N
    assert a(*args[:8], 48, *args[9:]) == EUNSUP           # D
    assert a(*args[:13], None, *args[14:]) == EWS
    assert a(*args[:14], nb - 1, None) == EWS


def test_transposed_v_argument_errors(lib):
    p = lib.moga_permute_vt
    nbp = lib.moga_workspace_bytes(1, 100, 4, 2, 128)
    pargs = [FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, nbp, None]
    assert p(None, *pargs[1:]) == ENULL                    # group_id
    assert p(*pargs[:3], None, *pargs[4:]) == ENULL        # V
    assert p(*pargs[:1], None, *pargs[2:]) == ENULL        # Q without Qp
    assert p(*pargs[:8], None, *pargs[9:]) == ENULL        # Qp without Q
    assert p(*pargs[:10], None, *pargs[11:]) == ENULL      # Vt
    assert p(*pargs[:4], 0, *pargs[5:]) == ESHAPE          # N
    assert p(*pargs[:6], 96, *pargs[7:]) == EUNSUP         # D
    assert p(*pargs[:4], (1 << 23) - 127, *pargs[5:]) == EUNSUP  # beyond the V^T offset range
    assert p(*pargs[:14], None, *pargs[15:]) == EWS
    assert p(*pargs[:15], nbp - 1, None) == EWS
    a = lib.moga_group_attention_unpermute_vt
    nb = lib.moga_workspace_bytes(2, 100, 4, 2, 128)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, 0.0, FAKE, FAKE, nb, None]
    assert a(*args[:2], None, *args[3:]) == ENULL          # Vt
    assert a(*args[:5], None, *args[6:]) == ENULL          # gate
    assert a(*args[:6], 0, *args[7:]) == ESHAPE            # N
    assert a(*args[:8], 48, *args[9:]) == EUNSUP           # D
    assert a(*args[:6], (1 << 23) - 127, *args[7:]) == EUNSUP
    assert a(*args[:13], None, *args[14:]) == EWS
    assert a(*args[:14], nb - 1, None) == EWS


def test_transposed_v_direct_q_argument_errors(lib):
    a = lib.moga_group_attention_unpermute_vtq
    nb = lib.moga_workspace_bytes(2, 100, 4, 2, 128)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, 0.0, FAKE, FAKE, nb, None]
    assert a(None, *args[1:]) == ENULL                     # Q
    assert a(*args[:4], None, *args[5:]) == ENULL          # perm
    assert a(*args[:12], None, *args[13:]) == ENULL        # O
    assert a(*args[:6], 0, *args[7:]) == ESHAPE            # N
    assert a(*args[:9], 65, *args[10:]) == EUNSUP          # M > 64
    assert a(*args[:8], 48, *args[9:]) == EUNSUP           # D
    assert a(*args[:6], (1 << 23) - 127, *args[7:]) == EUNSUP
    assert a(*args[:13], None, *args[14:]) == EWS
    assert a(*args[:14], nb - 1, None) == EWS


def test_gather_on_load_attention_argument_errors(lib):
    a = lib.moga_group_attention_fused
    nb = lib.moga_workspace_bytes(2, 100, 4, 2, 128)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, 0.0, FAKE, FAKE, nb, None]
    assert a(None, *args[1:]) == ENULL                     # Q
    assert a(*args[:4], None, *args[5:]) == ENULL          # perm
    assert a(*args[:5], None, *args[6:]) == ENULL          # gate
    assert a(*args[:12], None, *args[13:]) == ENULL        # O
    assert a(*args[:6], 0, *args[7:]) == ESHAPE            # N
    assert a(*args[:9], 65, *args[10:]) == EUNSUP          # M > 64
    assert a(*args[:8], 48, *args[9:]) == EUNSUP           # D
    assert a(*args[:13], None, *args[14:]) == EWS
    assert a(*args[:14], nb - 1, None) == EWS


def test_balance_argument_errors(lib):
    b = lib.moga_balance_stats
    nb = lib.moga_workspace_bytes(5, 5000, 8, 1, 64)
    assert nb >= 2 * 8 * 5 * 4
    assert b(None, FAKE, 5000, 8, 0.1, FAKE, FAKE, FAKE, FAKE, nb, None) == ENULL
    assert b(FAKE, FAKE, 5000, 8, 0.1, FAKE, FAKE, None, FAKE, nb, None) == ENULL
    assert b(FAKE, FAKE, 0, 8, 0.1, FAKE, FAKE, FAKE, FAKE, nb, None) == ESHAPE
    assert b(FAKE, FAKE, 5000, 65, 0.1, FAKE, FAKE, FAKE, FAKE, nb, None) == EUNSUP
    assert b(FAKE, FAKE, 5000, 8, 0.1, FAKE, FAKE, FAKE, FAKE, nb - 1, None) == EWS


def test_unpermute_argument_errors(lib):
    u = lib.moga_unpermute
    assert u(None, FAKE, FAKE, 10, 2, 64, 0.0, FAKE, None) == ENULL
    assert u(FAKE, FAKE, None, 10, 2, 64, 0.0, FAKE, None) == ENULL
    assert u(FAKE, FAKE, FAKE, -1, 2, 64, 0.0, FAKE, None) == ESHAPE
    assert u(FAKE, FAKE, FAKE, 10, 2, 32, 0.0, FAKE, None) == EUNSUP


def test_permute_noalloc_argument_errors(lib):
    """Argument and size errors come back before any device call (no GPU here)."""
    p = lib.moga_permute_vt_noalloc
    args = dict(g=FAKE, Q=None, K=FAKE, V=FAKE, N=100, H=2, D=128, M=4, Qp=None, Kp=FAKE, Vt=FAKE,
                perm=FAKE, cu=FAKE, mx=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return p(a["g"], a["Q"], a["K"], a["V"], a["N"], a["H"], a["D"], a["M"], a["Qp"], a["Kp"], a["Vt"],
                 a["perm"], a["cu"], a["mx"], None)

    assert call(g=None) == ENULL
    assert call(Q=FAKE) == ENULL                     # Q without Qp
    assert call(N=0) == ESHAPE
    assert call(M=65) == EUNSUP
    assert call(D=96) == EUNSUP
    assert call(N=(1 << 23)) == EUNSUP               # beyond the transposed-V layout
    # the fixed 1 MiB sort scratch: 8 * M * ceil(N / 1024) bytes at most
    assert call(N=(1 << 21) + 1024, M=64) == EWS
    assert call(N=(1 << 22), M=33) == EWS


def test_stga_argument_errors(lib):
    s = lib.moga_stga_attention
    assert s(None, FAKE, FAKE, 6, 30, 52, 3, 30, 26, 2, 128, 0.0, 1.0, 0.0, FAKE, None, 0, None) == ENULL
    assert s(FAKE, FAKE, FAKE, 6, 30, 52, 4, 30, 26, 2, 128, 0.0, 1.0, 0.0, FAKE, None, 0, None) == ESHAPE  # 4 !| 6
    assert s(FAKE, FAKE, FAKE, 6, 30, 52, 3, 7, 26, 2, 128, 0.0, 1.0, 0.0, FAKE, None, 0, None) == ESHAPE   # 7 !| 30
    assert s(FAKE, FAKE, FAKE, 6, 30, 52, 3, 30, 25, 2, 128, 0.0, 1.0, 0.0, FAKE, None, 0, None) == ESHAPE  # 25 !| 52
    assert s(FAKE, FAKE, FAKE, 0, 30, 52, 1, 30, 26, 2, 128, 0.0, 1.0, 0.0, FAKE, None, 0, None) == ESHAPE
    assert s(FAKE, FAKE, FAKE, 6, 30, 52, 3, 30, 26, 2, 100, 0.0, 1.0, 0.0, FAKE, None, 0, None) == EUNSUP
    assert s(FAKE, FAKE, FAKE, 2048, 1024, 1024, 2048, 1024, 1024, 1, 64, 0.0, 1.0, 0.0, FAKE, None, 0, None) == ESHAPE


def test_stga_shot_workspace_and_argument_errors(lib):
    w = lib.moga_stga_shot_workspace_bytes
    assert w(372, 10, 3) >= 256 + 16 * (124 + 10)
    assert w(0, 1, 3) == 0 and w(10, 0, 3) == 0 and w(10, 1, 0) == 0
    s = lib.moga_stga_shot_attention
    need = w(6, 2, 3)
    args = lambda **kw: [kw.get("Q", FAKE), FAKE, FAKE, kw.get("T", 6), 30, 52, kw.get("ss", FAKE),  # noqa: E731
                         kw.get("n", 2), 3, 30, kw.get("tw", 26), 1, 2, kw.get("D", 128), 0.0, 1.0, 0.0, FAKE,
                         kw.get("ws", FAKE), kw.get("wsb", need), None]
    assert s(*args(Q=None)) == ENULL
    assert s(*args(ss=None)) == ENULL
    assert s(*args(tw=25)) == ESHAPE            # 25 does not divide 52
    assert s(*args(n=0)) == ESHAPE
    assert s(*args(n=7)) == ESHAPE              # more shots than frames
    assert s(*args(D=100)) == EUNSUP
    aug = args()
    aug[11] = -1
    assert s(*aug) == ESHAPE                    # negative augmentation
    assert s(*args(ws=None)) == EWS
    assert s(*args(wsb=need - 1)) == EWS


def test_backward_workspace_and_argument_errors(lib):
    ws = lib.moga_workspace_bytes
    assert ws(7, 1000, 4, 2, 128) >= 2 * (64 + 65) * 4
    n = ws(6, 190320, 16, 1, 1536)
    assert n >= 190320 * 16 * 4 + 186 * 16 * 1536 * 4 and n % 256 == 0
    assert ws(6, 1000, 4, 1, 0) == 0
    t = lib.moga_group_attention_train
    nb = ws(2, 100, 4, 2, 128)
    assert t(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, FAKE, None, FAKE, nb, None) == ENULL   # lse
    assert t(FAKE, FAKE, FAKE, FAKE, 100, 2, 96, 4, 0.0, FAKE, FAKE, FAKE, nb, None) == EUNSUP
    assert t(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, 4, 0.0, FAKE, FAKE, FAKE, nb - 1, None) == EWS
    u = lib.moga_unpermute_backward
    assert u(FAKE, FAKE, FAKE, FAKE, 100, 2, 128, FAKE, FAKE, None, None) == ENULL
    assert u(FAKE, FAKE, FAKE, FAKE, 0, 2, 128, FAKE, FAKE, FAKE, None) == ESHAPE
    assert u(FAKE, FAKE, FAKE, FAKE, 100, 2, 32, FAKE, FAKE, FAKE, None) == EUNSUP
    b = lib.moga_group_attention_backward
    nbb = ws(7, 100, 4, 2, 128)
    args = [FAKE] * 8 + [100, 2, 128, 4, 0.0, FAKE, FAKE, FAKE, FAKE, nbb, None]
    assert b(*args[:4], None, *args[5:]) == ENULL            # lse
    assert b(*args[:8], 0, *args[9:]) == ESHAPE
    assert b(*args[:11], 65, *args[12:]) == EUNSUP
    assert b(*args[:17], nbb - 1, None) == EWS
    # the staged-dS workspace: 4 KB + H * sum_g ceil(n/32) * (that rounded up to even) * 2 KB
    sb = lib.moga_attention_backward_staged_bytes
    cu = (ctypes.c_int32 * 6)(0, 1, 1, 33, 100, 357)  # sizes 1, 0, 32, 67, 257 -> blocks 1, 0, 1, 3, 9
    assert sb(cu, 5, 3) == 4096 + 3 * (1 * 2 + 0 + 1 * 2 + 3 * 4 + 9 * 10) * 2048
    assert sb(None, 5, 3) == 0 and sb(cu, 0, 3) == 0 and sb(cu, 65, 3) == 0 and sb(cu, 5, 0) == 0
    bad = (ctypes.c_int32 * 3)(0, 10, 5)  # a negative group size
    assert sb(bad, 2, 1) == 0
    huge = (ctypes.c_int32 * 2)(0, (1 << 24) + 64)  # above 2^24 tokens in one group
    assert sb(huge, 1, 1) == 0
    ok = (ctypes.c_int32 * 2)(0, 1 << 24)
    assert sb(ok, 1, 1) == 4096 + (1 << 19) * (1 << 19) * 2048
    r = lib.moga_route_backward
    nr = ws(6, 100, 4, 1, 128)
    assert r(FAKE, FAKE, None, FAKE, None, 100, 128, 4, FAKE, FAKE, None, FAKE, nr, None, 0, None) == ENULL   # dgate
    assert r(FAKE, FAKE, None, FAKE, FAKE, 100, 100, 4, FAKE, FAKE, None, FAKE, nr, None, 0, None) == EUNSUP  # d % 32
    assert r(FAKE, FAKE, None, FAKE, FAKE, 100, 128, 4, FAKE, FAKE, None, FAKE, nr - 1, None, 0, None) == EWS
