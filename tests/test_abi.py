"""The C ABI boundary on the CPU: the library loads without a GPU, exports every
function include/logra.h declares, and rejects invalid arguments with status
codes before any HIP call (so these paths need no device).
"""
import ctypes
import subprocess

import pytest

from rank_gradient_sketching_amd import _lib

OK, EINVAL, EWS = _lib.OK, _lib.EINVAL, _lib.EWORKSPACE
P = 0x100000          # a 256-byte-aligned stand-in address; never dereferenced
MIS = P + 2           # misaligned by 2 bytes


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    declared = _lib.header_symbols()
    assert len(declared) == 23
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert L.logra_abi_version() == 1
    for st in (0, -1, -2, -3, 7):
        assert isinstance(_lib.status_str(st), str) and _lib.status_str(st)


def test_workspace_queries(L):
    assert L.logra_sketch_ws_bytes(8192, 4096, 4096, 64) > 2 * 8192 * 64 * 2
    assert L.logra_sketch_ws_bytes(8192, 4096, 4096, 0) == 0
    assert L.logra_sketch_ws_bytes(8192, 4096, 4096, 257) == 0
    assert L.logra_sketch_ws_bytes(8192, 0, 4096, 64) == 0
    assert L.logra_sketch_ws_bytes(-1, 16, 16, 4) == 0
    assert L.logra_kl_ws_bytes(65536, 152064) >= 65536 * 4
    assert L.logra_kl_ws_bytes(0, 10) == 0
    # the workspace grows with T and shrinks to a floor at T = 0
    assert L.logra_sketch_ws_bytes(16384, 256, 256, 4) > L.logra_sketch_ws_bytes(128, 256, 256, 4)


def _sketch(L, **kw):
    a = dict(X=P, ldx=256, dY=P, ldd=256, T=128, d=256, k=256, r=4, seed=1234, stream=0,
             kind=0, flags=0, S=P, ws=P, ws_bytes=1 << 30, s=None)
    a.update(kw)
    return L.logra_sketch_accumulate(a["X"], a["ldx"], a["dY"], a["ldd"], a["T"], a["d"],
                                     a["k"], a["r"], a["seed"], a["stream"], a["kind"],
                                     a["flags"], a["S"], a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), EINVAL), (dict(dY=None), EINVAL), (dict(S=None), EINVAL),
    (dict(r=0), EINVAL), (dict(r=257), EINVAL), (dict(r=-3), EINVAL),
    (dict(d=0), EINVAL), (dict(k=0), EINVAL), (dict(T=-1), EINVAL),
    (dict(ldx=255), EINVAL), (dict(ldx=260), EINVAL), (dict(ldd=100), EINVAL),
    (dict(kind=2), EINVAL), (dict(kind=-1), EINVAL),
    (dict(X=MIS), EINVAL), (dict(dY=MIS), EINVAL), (dict(S=P + 1), EINVAL),
    (dict(d=1 << 31), EINVAL), (dict(T=1 << 31), EINVAL), (dict(ldd=1 << 26), EINVAL),
    (dict(ws=None), EWS), (dict(ws_bytes=16), EWS), (dict(ws=P + 16), EWS),
    (dict(flags=8), EINVAL), (dict(flags=-1), EINVAL),
    # deferred chains: a deferring call takes no overwrite flag, and every
    # call of a chain has tokens
    (dict(flags=3), EINVAL), (dict(flags=7), EINVAL), (dict(flags=4, T=0), EINVAL),
    (dict(flags=6, T=0), EINVAL), (dict(flags=5, T=0), EINVAL),
    (dict(flags=1, S=None), EINVAL),
    # the zero fill of an empty first microbatch still needs a valid S
    (dict(flags=1, T=0, S=None), EINVAL), (dict(flags=1, T=0, S=P + 2), EINVAL),
    (dict(flags=2, T=0), EINVAL),
])
def test_sketch_rejects(L, kw, status):
    assert _sketch(L, **kw) == status


def test_sketch_T0_is_noop_without_touching_pointers(L):
    assert _sketch(L, T=0, X=None, dY=None, S=None, ws=None, ws_bytes=0) == 0
    assert _sketch(L, T=0, r=0) == EINVAL      # sizes are still checked


def _merge(L, **kw):
    a = dict(W=P, ldw=256, S=P, d=256, k=256, r=4, seed=1, stream=0, kind=0,
             alpha=1.0, eta=1e-3, s=None)
    a.update(kw)
    return L.logra_merge(a["W"], a["ldw"], a["S"], a["d"], a["k"], a["r"], a["seed"],
                         a["stream"], a["kind"], a["alpha"], a["eta"], a["s"])


@pytest.mark.parametrize("kw", [
    dict(W=None), dict(S=None), dict(r=0), dict(r=300), dict(d=0), dict(k=-5),
    dict(ldw=200), dict(ldw=257), dict(kind=3), dict(W=MIS), dict(S=P + 2),
    dict(alpha=float("nan")), dict(eta=float("inf")), dict(alpha=-float("inf")),
])
def test_merge_rejects(L, kw):
    assert _merge(L, **kw) == EINVAL


def _kl(L, **kw):
    a = dict(zc=P, zp=P, n=64, V=1000, ld=1000, tau=1.0, delta=2e-4, amax=4.0,
             out=P, kl=None, ws=P, ws_bytes=1 << 20, s=None)
    a.update(kw)
    return L.logra_predicted_kl(a["zc"], a["zp"], a["n"], a["V"], a["ld"], a["tau"],
                                a["delta"], a["amax"], a["out"], a["kl"], a["ws"],
                                a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(zc=None), EINVAL), (dict(zp=None), EINVAL), (dict(out=None), EINVAL),
    (dict(n=0), EINVAL), (dict(V=0), EINVAL), (dict(ld=999), EINVAL), (dict(ld=1004), EINVAL),
    (dict(tau=0.0), EINVAL), (dict(tau=-1.0), EINVAL), (dict(tau=float("nan")), EINVAL),
    (dict(delta=0.0), EINVAL), (dict(delta=float("inf")), EINVAL),
    (dict(amax=-1.0), EINVAL), (dict(amax=float("nan")), EINVAL),
    (dict(zc=MIS), EINVAL), (dict(out=P + 1), EINVAL), (dict(kl=P + 2), EINVAL),
    (dict(ws=None), EWS), (dict(ws_bytes=8), EWS), (dict(ws=P + 64), EWS),
])
def test_kl_rejects(L, kw, status):
    assert _kl(L, **kw) == status


@pytest.mark.parametrize("kw", [dict(A=None), dict(r=0), dict(r=512), dict(k=0), dict(kind=5),
                                dict(A=P + 2)])
def test_regen_rejects(L, kw):
    a = dict(seed=1, stream=0, kind=0, r=4, k=256, A=P, s=None)
    a.update(kw)
    assert L.logra_regen_A(a["seed"], a["stream"], a["kind"], a["r"], a["k"], a["A"], a["s"]) == EINVAL


def test_binding_refuses_cpu_tensors():
    import torch
    import rank_gradient_sketching_amd as lg
    X = torch.zeros(8, 8, dtype=torch.bfloat16)
    S = torch.zeros(8, 4)
    with pytest.raises(ValueError, match="GPU"):
        lg.sketch_accumulate(X, X, S, seed=1)
    with pytest.raises(ValueError, match="GPU"):
        lg.merge(X, S, seed=1)


def _sweep(L, **kw):
    import ctypes
    al = kw.pop("alphas", [0.5, 1.0])
    a = dict(z=P, delta=P, n_tok=16, vocab=1000, ld=1000, n_alpha=len(al or [0.0]), tau=1.0,
             weight=None,
             kl_mean=P, kl_tok=None, ws=P, ws_bytes=1 << 20, s=None)
    a.update(kw)
    c_al = None if al is None else (ctypes.c_float * max(1, len(al)))(*al)
    return L.logra_predicted_kl_sweep(a["z"], a["delta"], a["n_tok"], a["vocab"], a["ld"], c_al,
                                      a["n_alpha"], a["tau"], a["weight"], a["kl_mean"],
                                      a["kl_tok"], a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), EINVAL), (dict(delta=None), EINVAL), (dict(kl_mean=None), EINVAL),
    (dict(alphas=None), EINVAL), (dict(n_alpha=0), EINVAL), (dict(n_alpha=9), EINVAL),
    (dict(alphas=[float("nan")]), EINVAL), (dict(alphas=[1.0, float("inf")]), EINVAL),
    (dict(tau=0.0), EINVAL), (dict(tau=float("nan")), EINVAL), (dict(n_tok=0), EINVAL),
    (dict(vocab=0), EINVAL), (dict(ld=999), EINVAL), (dict(ld=1004), EINVAL),
    (dict(z=MIS), EINVAL), (dict(weight=P + 2), EINVAL), (dict(kl_tok=P + 1), EINVAL),
    (dict(kl_mean=P + 3), EINVAL),
    (dict(ws=None), EWS), (dict(ws_bytes=64), EWS), (dict(ws=P + 16), EWS),
])
def test_kl_sweep_rejects(L, kw, status):
    assert _sweep(L, **kw) == status


def test_kl_sweep_ws_bytes(L):
    assert L.logra_kl_sweep_ws_bytes(65536, 4) >= 65536 * 4 * 4
    assert L.logra_kl_sweep_ws_bytes(10, 0) == 0
    assert L.logra_kl_sweep_ws_bytes(10, 9) == 0
    assert L.logra_kl_sweep_ws_bytes(0, 2) == 0


def test_kl_budget_schedule():
    from rank_gradient_sketching_amd import kl_budget_schedule as sched
    assert sched(0, 300) == 2e-4
    assert sched(299, 300) == 2e-5
    assert sched(5000, 300) == 2e-5
    vals = [sched(s, 300) for s in range(300)]
    assert all(a > b for a, b in zip(vals, vals[1:]))
    assert abs(sched(149.5, 300) - 1.1e-4) < 1e-12


def _shared(L, n_out=2, **kw):
    import ctypes
    a = dict(X=P, ldx=256, T=128, k=256, r=4, seed=1, stream=0, kind=0, flags=0,
             dY=[P] * n_out, ldd=[256] * n_out, d=[256] * n_out,
             S=[P + 4096 * (o + 1) for o in range(n_out)], ws=P, ws_bytes=1 << 30, s=None)
    a.update(kw)
    n = kw.get("n_out_arg", n_out)
    arr = lambda t, xs: None if xs is None else (t * max(1, len(xs)))(*xs)
    return L.logra_sketch_accumulate_shared(
        a["X"], a["ldx"], a["T"], a["k"], a["r"], a["seed"], a["stream"], a["kind"], a["flags"], n,
        arr(ctypes.c_void_p, a["dY"]), arr(ctypes.c_int64, a["ldd"]), arr(ctypes.c_int64, a["d"]),
        arr(ctypes.c_void_p, a["S"]), a["ws"], a["ws_bytes"], a["s"])


@pytest.mark.parametrize("kw,status", [
    (dict(n_out_arg=0), EINVAL), (dict(n_out_arg=5), EINVAL), (dict(dY=None), EINVAL),
    (dict(ldd=None), EINVAL), (dict(d=None), EINVAL), (dict(S=None), EINVAL),
    (dict(X=None), EINVAL), (dict(dY=[P, None]), EINVAL), (dict(S=[P, None]), EINVAL),
    (dict(S=[P, P]), EINVAL),                                  # one accumulator per output
    (dict(d=[256, 0]), EINVAL), (dict(ldd=[256, 100]), EINVAL), (dict(ldd=[256, 1 << 26]), EINVAL),
    (dict(dY=[P, MIS]), EINVAL), (dict(S=[P, P + 2]), EINVAL), (dict(ldx=255), EINVAL),
    (dict(r=0), EINVAL), (dict(kind=5), EINVAL),
    (dict(ws=None), EWS), (dict(ws_bytes=16), EWS),
    (dict(flags=8), EINVAL), (dict(flags=3), EINVAL), (dict(flags=4, T=0), EINVAL),
    (dict(flags=1, T=0, S=[P, None]), EINVAL),
    (dict(flags=1, T=0, S=[P, P]), EINVAL),
])
def test_sketch_shared_rejects(L, kw, status):
    assert _shared(L, **kw) == status


def test_sketch_shared_T0_and_sizes(L):
    import ctypes
    assert _shared(L, T=0, X=None, dY=[None, None], S=[None, None], ws=None, ws_bytes=0) == 0
    d3 = (ctypes.c_int64 * 3)(1536, 256, 256)
    shared = L.logra_sketch_shared_ws_bytes(16384, 1536, 64, 3, d3)
    assert shared >= 2 * 64 * 16384 * 2                       # at least the P buffer
    d1 = (ctypes.c_int64 * 1)(1536)
    assert L.logra_sketch_shared_ws_bytes(16384, 1536, 64, 1, d1) == \
        L.logra_sketch_ws_bytes(16384, 1536, 1536, 64)
    assert L.logra_sketch_shared_ws_bytes(16384, 1536, 64, 0, d3) == 0
    assert L.logra_sketch_shared_ws_bytes(16384, 1536, 64, 5, d3) == 0
    assert L.logra_sketch_shared_ws_bytes(16384, 1536, 64, 3, None) == 0


def _update(L, **kw):
    n4 = 64 * 16 * 4                       # bytes of one d x r array below
    a = dict(rule=2, S=P, m=P + n4, v=P + 2 * n4, U=P + 3 * n4, d=64, r=16, b1=0.9, b2=0.999,
             eps=1e-8, step=1, s=None)
    a.update(kw)
    return L.logra_sketch_update(a["rule"], a["S"], a["m"], a["v"], a["U"], a["d"], a["r"],
                                 a["b1"], a["b2"], a["eps"], a["step"], a["s"])


N4 = 64 * 16 * 4


@pytest.mark.parametrize("kw", [
    dict(rule=3), dict(rule=-1), dict(S=None), dict(U=None), dict(rule=1, m=None), dict(v=None),
    dict(d=0), dict(r=0), dict(r=300), dict(S=P + 2), dict(U=P + 3 * N4 + 2), dict(m=P + N4 + 1),
    dict(b1=1.0), dict(b1=-0.1), dict(b1=float("nan")), dict(b2=1.0), dict(b2=float("inf")),
    dict(eps=-1e-8), dict(eps=float("inf")), dict(step=0), dict(step=-3),
    dict(rule=1, m=P),                     # momentum state aliasing S
    dict(U=P + 2 * N4),                    # U aliasing Adam's v
    dict(U=P + N4),                        # U aliasing Adam's m
    dict(U=P + 4),                         # U partially overlapping S
    dict(v=P + N4 + 64),                   # v partially overlapping m
    dict(rule=0, U=P + 16),                # SGD: U partially overlapping S
])
def test_sketch_update_rejects(L, kw):
    assert _update(L, **kw) == EINVAL


def test_sketch_update_ignores_unused_state_arguments(L):
    # SGD and momentum never look at v (nor SGD at m), so their validity does not
    # depend on them; a valid call then fails only at the launch (no GPU here).
    import torch
    if torch.cuda.is_available():
        pytest.skip("a valid call would launch on placeholder pointers")
    st = _update(L, rule=0, m=None, v=None, b1=7.0, b2=-1.0, eps=-1.0, step=0)
    assert st != EINVAL
    st = _update(L, rule=1, v=None, b2=9.0, eps=float("nan"), step=0)
    assert st != EINVAL


def test_kernel_choice_setter(L):
    for which in (0, 1):
        for mode in (-1, 0, 1):
            assert L.logra_set_kernel_choice(which, mode) == OK
        # mode 2 (128-token tiles) exists for the projection tile only
        assert L.logra_set_kernel_choice(which, 2) == (OK if which == 0 else EINVAL)
        assert L.logra_set_kernel_choice(which, 3) == EINVAL
        assert L.logra_set_kernel_choice(which, -2) == EINVAL
    assert L.logra_set_kernel_choice(2, 0) == EINVAL
    for which in (0, 1):
        assert L.logra_set_kernel_choice(which, -1) == OK
    # the wide accumulate choice changes the workspace plan at r > 64 only
    base = L.logra_sketch_ws_bytes(8192, 4096, 4096, 256)
    L.logra_set_kernel_choice(1, 1)
    wide = L.logra_sketch_ws_bytes(8192, 4096, 4096, 256)
    small_r = L.logra_sketch_ws_bytes(8192, 4096, 4096, 64)
    L.logra_set_kernel_choice(1, -1)
    assert L.logra_sketch_ws_bytes(8192, 4096, 4096, 256) == base
    assert L.logra_sketch_ws_bytes(8192, 4096, 4096, 64) == small_r
    assert wide != base


def test_sketch_noalloc_rejects_before_any_hip_call(L):
    f = L.logra_sketch_accumulate_noalloc
    ok = dict(X=P, ldx=4096, dY=P, ldd=4096, T=8192, d=4096, k=4096, r=64, seed=1, stream=0,
              kind=0, flags=0, S=P, s=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["X"], a["ldx"], a["dY"], a["ldd"], a["T"], a["d"], a["k"], a["r"], a["seed"],
                 a["stream"], a["kind"], a["flags"], a["S"], a["s"])
    assert call(X=0) == EINVAL
    assert call(dY=MIS) == EINVAL
    assert call(S=0) == EINVAL
    assert call(r=0) == EINVAL
    assert call(kind=2) == EINVAL
    assert call(flags=8) == EINVAL
    assert call(ldd=4095) == EINVAL
    # no deferred chains in the shared scratch
    for fl in (2, 4, 6, 5):
        assert call(flags=fl) == EINVAL
    # the r = 256 layers need more than the 32 MiB of library scratch
    assert L.logra_sketch_ws_bytes(32768, 3584, 18944, 256) > 32 << 20
    assert call(T=32768, d=3584, k=18944, r=256, ldx=18944, ldd=3584) == EWS
    assert call(T=16384, d=5120, k=25600, r=256, ldx=25600, ldd=5120) == EWS
    # T = 0 without the overwrite flag: nothing to do
    assert call(T=0, X=0, dY=0) == OK


def _groups(spec):
    """ctypes logra_sketch_group array; spec: [dict(X, ldx, k, seed, stream,
    outs=[(dY, ldd, d, S)], n_out=len(outs))]."""
    arr = (_lib.SketchGroup * max(1, len(spec)))()
    for g, q in enumerate(spec):
        outs = q.get("outs", [])
        arr[g].X, arr[g].ldx, arr[g].k = q.get("X", P), q.get("ldx", 256), q.get("k", 256)
        arr[g].seed, arr[g].stream = q.get("seed", 1), q.get("stream", 0)
        arr[g].n_out = q.get("n_out", len(outs))
        for o, (dY, ldd, d, S) in enumerate(outs):
            arr[g].dY[o], arr[g].ldd[o], arr[g].d[o], arr[g].S[o] = dY, ldd, d, S
    return arr


def _layer_spec(n_groups=3, per=2, d=256, r=4):
    """n_groups groups of `per` outputs with disjoint S (d x r floats each)."""
    nb = d * r * 4
    return [dict(outs=[(P, 256, d, P + nb * (g * per + o + 1)) for o in range(per)])
            for g in range(n_groups)]


def _layer(L, spec, T=128, r=4, kind=0, flags=0, ws=P, ws_bytes=1 << 30, n_groups=None):
    arr = _groups(spec)
    n = len(spec) if n_groups is None else n_groups
    return L.logra_sketch_accumulate_layer(T, r, kind, flags, n, arr, ws, ws_bytes, None)


def _mut(spec, g, **kw):
    spec = [dict(q) for q in spec]
    spec[g].update(kw)
    return spec


def _layer_reject_cases():
    base = _layer_spec()
    nb = 256 * 4 * 4
    cases = [
        (dict(n_groups=0), EINVAL), (dict(n_groups=5), EINVAL), (dict(r=0), EINVAL),
        (dict(r=257), EINVAL), (dict(kind=2), EINVAL), (dict(flags=8), EINVAL),
        (dict(flags=3), EINVAL), (dict(flags=2, T=0), EINVAL), (dict(T=-1), EINVAL),
        (dict(ws=None), EWS), (dict(ws_bytes=256), EWS), (dict(ws=P + 128), EWS),
        (dict(spec=_mut(base, 1, X=None)), EINVAL), (dict(spec=_mut(base, 1, X=MIS)), EINVAL),
        (dict(spec=_mut(base, 2, ldx=100)), EINVAL), (dict(spec=_mut(base, 0, k=0)), EINVAL),
        (dict(spec=_mut(base, 1, n_out=0)), EINVAL), (dict(spec=_mut(base, 1, n_out=5)), EINVAL),
        (dict(spec=_mut(base, 2, outs=[(None, 256, 256, P + 100 * nb), (P, 256, 256, P + 101 * nb)])),
         EINVAL),
        (dict(spec=_mut(base, 2, outs=[(P, 255, 256, P + 100 * nb), (P, 256, 256, P + 101 * nb)])),
         EINVAL),
        (dict(spec=_mut(base, 2, outs=[(P, 256, 0, P + 100 * nb), (P, 256, 256, P + 101 * nb)])),
         EINVAL),
        # S of group 2 overlapping S of group 0, wholly and in part
        (dict(spec=_mut(base, 2, outs=[(P, 256, 256, P + nb), (P, 256, 256, P + 101 * nb)])), EINVAL),
        (dict(spec=_mut(base, 2, outs=[(P, 256, 256, P + nb + 512), (P, 256, 256, P + 101 * nb)])),
         EINVAL),
        # nine outputs in all
        (dict(spec=_layer_spec(n_groups=3, per=3)), EINVAL),
        (dict(spec=_mut(base, 0, outs=[(P, 256, 256, None), (P, 256, 256, P + 2 * nb)])), EINVAL),
    ]
    return cases


@pytest.mark.parametrize("kw,status", _layer_reject_cases())
def test_sketch_layer_rejects(L, kw, status):
    kw = dict(kw)
    spec = kw.pop("spec", _layer_spec())
    assert _layer(L, spec, **kw) == status


def test_sketch_layer_T0_and_sizes(L):
    # T == 0 without the overwrite flag: no pointer is inspected
    spec = [dict(X=None, outs=[(None, 0, 256, None)]), dict(X=None, outs=[(None, 0, 64, None)] * 2)]
    assert _layer(L, spec, T=0, ws=None, ws_bytes=0) == OK
    # one group equals the shared query; the sizes grow with the groups
    groups = [(1536, [1536, 256, 256]), (1536, [1536]), (1536, [8960, 8960]), (8960, [1536])]

    def q(gs, T=16384, r=64):
        arr = (_lib.SketchGroup * len(gs))()
        for g, (k, ds) in enumerate(gs):
            arr[g].k, arr[g].n_out = k, len(ds)
            for o, d in enumerate(ds[:_lib.MAX_SHARED]):
                arr[g].d[o] = d
        return L.logra_sketch_layer_ws_bytes(T, r, len(gs), arr)

    d3 = (ctypes.c_int64 * 3)(1536, 256, 256)
    assert q(groups[:1]) == L.logra_sketch_shared_ws_bytes(16384, 1536, 64, 3, d3)
    full = q(groups)
    assert full >= 4 * 2 * 64 * 16384 * 2                 # four P buffers at least
    assert q(groups, T=0) > 0 and q(groups, r=0) == 0 and q(groups, T=-5) == 0
    assert q([(1536, [])]) == 0 and q([(1536, [64] * 5)]) == 0
    assert q(groups + [(256, [64])]) == 0                  # five groups
    assert q([(256, [64] * 4), (256, [64] * 4), (256, [64])]) == 0   # nine outputs
    assert L.logra_sketch_layer_ws_bytes(16384, 64, 2, None) == 0


def _merge_many(L, items, r=4, kind=0, alpha=1.0, eta=1.0, n=None):
    arr = (_lib.MergeItem * max(1, len(items)))()
    for i, (W, ldw, S, d, k) in enumerate(items):
        arr[i].W, arr[i].ldw, arr[i].S, arr[i].d, arr[i].k = W, ldw, S, d, k
        arr[i].seed, arr[i].stream = 1, 0
    return L.logra_merge_many(len(items) if n is None else n, arr, r, kind, alpha, eta, None)


# three weights of 64 x 256 bf16 (32 KiB each) and their S (64 x 4 floats)
W_NB, S_NB = 64 * 256 * 2, 64 * 4 * 4
GOOD = [(P + i * W_NB, 256, P + 8 * W_NB + i * S_NB, 64, 256) for i in range(3)]


@pytest.mark.parametrize("kw", [
    dict(n=0), dict(n=9), dict(r=0), dict(r=257), dict(kind=3), dict(alpha=float("nan")),
    dict(eta=float("inf")),
    dict(items=[GOOD[0], (None, 256, P + 9 * W_NB, 64, 256)]),
    dict(items=[GOOD[0], (P + W_NB, 256, None, 64, 256)]),
    dict(items=[GOOD[0], (P + W_NB + 8, 256, P + 9 * W_NB, 64, 256)]),     # W misaligned
    dict(items=[GOOD[0], (P + W_NB, 256, P + 9 * W_NB + 2, 64, 256)]),     # S misaligned
    dict(items=[GOOD[0], (P + W_NB, 250, P + 9 * W_NB, 64, 256)]),         # ldw < k
    dict(items=[GOOD[0], (P + W_NB, 256, P + 9 * W_NB, 0, 256)]),
    dict(items=[GOOD[0], (P + W_NB, 256, P + 9 * W_NB, 64, 0)]),
    dict(items=[GOOD[0], (P + W_NB // 2, 256, P + 9 * W_NB, 64, 256)]),    # W overlaps W
    dict(items=[GOOD[0], (P + W_NB, 256, P + 16, 64, 256)]),               # S inside a W
    dict(items=[GOOD[0], GOOD[0]]),
])
def test_merge_many_rejects(L, kw):
    kw = dict(kw)
    items = kw.pop("items", GOOD)
    assert _merge_many(L, items, **kw) == EINVAL
