"""The two-call sketch (logra_sketch_project + logra_sketch_accumulate_p) at
the C ABI on the CPU: sizes, and every invalid argument rejected with a status
code before any HIP call (stand-in addresses that are never dereferenced)."""
import ctypes

import pytest

from rank_gradient_sketching_amd import _lib

OK, EINVAL, EWS = _lib.OK, _lib.EINVAL, _lib.EWORKSPACE
P = 0x100000          # a 256-byte-aligned stand-in address
MIS = P + 2


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_sizes_add_up_to_the_one_call_workspace(L):
    for T, d, k, r in ((8192, 4096, 4096, 64), (1000, 300, 520, 16), (77, 1030, 264, 256),
                       (1, 8, 8, 1), (16384, 1536, 8960, 256)):
        dd = (ctypes.c_int64 * 1)(d)
        p = L.logra_sketch_p_bytes(T, r)
        g = L.logra_sketch_project_ws_bytes(k, r)
        a = L.logra_sketch_accumulate_p_ws_bytes(T, r, 1, dd)
        rp = next(x for x in (16, 32, 64, 128, 256) if r <= x)
        assert p == 2 * rp * (-(-T // 32) * 32) * 2          # hi and lo, tokens padded to 32
        assert g == max(rp, 32) * (-(-k // 256) * 256) * 2    # the bf16 Gaussian basis
        rnd = lambda x: -(-x // 256) * 256
        assert rnd(p) + rnd(a) + rnd(g) == L.logra_sketch_ws_bytes(T, d, k, r)
    # the shared form sums the partial tiles of every output's d groups
    d3 = (ctypes.c_int64 * 3)(1536, 256, 256)
    assert L.logra_sketch_accumulate_p_ws_bytes(16384, 64, 3, d3) > \
        L.logra_sketch_accumulate_p_ws_bytes(16384, 64, 1, d3)
    # a P for T = 0 still has one (empty) step
    assert L.logra_sketch_p_bytes(0, 4) == 2 * 16 * 32 * 2


@pytest.mark.parametrize("args", [(8192, 0), (8192, 257), (-1, 4), (1 << 31, 4)])
def test_p_bytes_invalid(L, args):
    assert L.logra_sketch_p_bytes(*args) == 0


def test_ws_queries_invalid(L):
    assert L.logra_sketch_project_ws_bytes(0, 4) == 0
    assert L.logra_sketch_project_ws_bytes(256, 0) == 0
    assert L.logra_sketch_project_ws_bytes(1 << 31, 4) == 0
    d = (ctypes.c_int64 * 2)(256, 0)
    assert L.logra_sketch_accumulate_p_ws_bytes(128, 4, 2, d) == 0
    assert L.logra_sketch_accumulate_p_ws_bytes(128, 4, 0, d) == 0
    assert L.logra_sketch_accumulate_p_ws_bytes(128, 4, 5, d) == 0
    assert L.logra_sketch_accumulate_p_ws_bytes(128, 4, 1, None) == 0


def _project(L, **kw):
    a = dict(X=P, ldx=256, T=128, k=256, r=4, seed=1, stream=0, kind=0, P=P, p_bytes=1 << 30,
             ws=P, ws_bytes=1 << 30, s=None)
    a.update(kw)
    return L.logra_sketch_project(a["X"], a["ldx"], a["T"], a["k"], a["r"], a["seed"],
                                  a["stream"], a["kind"], a["P"], a["p_bytes"], a["ws"],
                                  a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), EINVAL), (dict(X=MIS), EINVAL), (dict(ldx=255), EINVAL), (dict(ldx=260), EINVAL),
    (dict(k=0), EINVAL), (dict(k=1 << 31), EINVAL), (dict(r=0), EINVAL), (dict(r=257), EINVAL),
    (dict(kind=2), EINVAL), (dict(T=-1), EINVAL), (dict(T=1 << 31), EINVAL),
    (dict(P=None), EINVAL), (dict(P=P + 8), EINVAL), (dict(p_bytes=2 * 16 * 128 * 2 - 1), EINVAL),
    # the Gaussian basis needs the scratch; the sign basis does not look at it
    (dict(kind=1, ws=None), EWS), (dict(kind=1, ws_bytes=16), EWS), (dict(kind=1, ws=P + 16), EWS),
])
def test_project_rejects(L, kw, status):
    assert _project(L, **kw) == status


def test_project_T0_is_noop(L):
    assert _project(L, T=0, X=None, P=None, ws=None, ws_bytes=0) == OK
    assert _project(L, T=0, r=0) == EINVAL


def _acc(L, n_out=2, **kw):
    a = dict(P=P, p_bytes=1 << 30, T=128, r=4, flags=0, dY=[P] * n_out, ldd=[256] * n_out,
             d=[256] * n_out, S=[P + 4096 * (o + 1) for o in range(n_out)], ws=P,
             ws_bytes=1 << 30, s=None)
    a.update(kw)
    n = kw.get("n_out_arg", n_out)
    arr = lambda t, xs: None if xs is None else (t * max(1, len(xs)))(*xs)
    return L.logra_sketch_accumulate_p(
        a["P"], a["p_bytes"], a["T"], a["r"], a["flags"], n, arr(ctypes.c_void_p, a["dY"]),
        arr(ctypes.c_int64, a["ldd"]), arr(ctypes.c_int64, a["d"]), arr(ctypes.c_void_p, a["S"]),
        a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(n_out_arg=0), EINVAL), (dict(n_out_arg=5), EINVAL), (dict(dY=None), EINVAL),
    (dict(ldd=None), EINVAL), (dict(d=None), EINVAL), (dict(S=None), EINVAL),
    (dict(P=None), EINVAL), (dict(P=P + 8), EINVAL), (dict(p_bytes=2 * 16 * 128 * 2 - 1), EINVAL),
    (dict(dY=[P, None]), EINVAL), (dict(S=[P, None]), EINVAL), (dict(S=[P, P]), EINVAL),
    (dict(d=[256, 0]), EINVAL), (dict(d=[256, 1 << 31]), EINVAL), (dict(ldd=[256, 100]), EINVAL),
    (dict(ldd=[256, 1 << 26]), EINVAL), (dict(dY=[P, MIS]), EINVAL), (dict(S=[P, P + 2]), EINVAL),
    (dict(r=0), EINVAL), (dict(r=257), EINVAL), (dict(T=-1), EINVAL), (dict(T=1 << 31), EINVAL),
    (dict(ws=None), EWS), (dict(ws_bytes=16), EWS), (dict(ws=P + 16), EWS),
    (dict(flags=8), EINVAL), (dict(flags=3), EINVAL), (dict(flags=7), EINVAL),
    (dict(flags=4, T=0), EINVAL), (dict(flags=2, T=0), EINVAL),
    (dict(flags=1, T=0, S=[P, None]), EINVAL), (dict(flags=1, T=0, S=[P, P]), EINVAL),
])
def test_accumulate_p_rejects(L, kw, status):
    assert _acc(L, **kw) == status


def test_accumulate_p_T0_is_noop(L):
    assert _acc(L, T=0, P=None, dY=[None, None], S=[None, None], ws=None, ws_bytes=0) == OK
    assert _acc(L, T=0, r=0) == EINVAL
