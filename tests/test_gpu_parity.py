"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bars: A bit-exact for the sign basis (the Gaussian basis: >= 99.9 % of entries
equal, the rest within one bf16 ulp, since fp64 and fp32 transcendentals may
round differently); S and the merged-W delta within 2e-3 relative Frobenius
error; q(D) within 1e-3 relative error.  Beside each Frobenius bound an
elementwise one (tests/parity_bars.py), so that a single wrong entry cannot
hide in the norm.  Shapes span several tiles and ragged tails; every input is
seeded.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import bf16 as obf16
from oracle import kl as okl
from oracle import merge as omerge
from oracle import projection as oproj
from oracle import sketch as osketch
from rank_gradient_sketching_amd import synth

pytestmark = pytest.mark.gpu

from parity_bars import (Q_TOL, S_TOL, W_ELEM, W_TOL, max_rel, rel_fro, s_elem_bar,  # noqa: E402
                         w_elem_bar, w_excess)


@pytest.fixture(scope="module")
def lg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_gradient_sketching_amd as m
    return m


def say(*a):
    print(*a, flush=True)








def padded_bf16(t, ld):
    """Copy of a 2-D bf16 tensor on the GPU with row stride ld (>= cols)."""
    rows, cols = t.shape
    buf = torch.full((rows, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, :cols] = t.cuda()
    return buf[:, :cols]


# ------------------------------------------------------------------ regen_A

@pytest.mark.parametrize("seed,stream,r,k", [
    (1234, 0, 4, 256), (1234, 0, 64, 4096), (7, 3, 1, 1), (99, 1, 3, 257),
    (2 ** 64 - 1, 2 ** 63, 100, 1000), (1261, 0, 256, 1536), (5, 2, 17, 4099),
])
def test_regen_sign_bit_exact(lg, seed, stream, r, k):
    say("regen sign", seed, stream, r, k)
    A = lg.regen_A(seed, stream, 0, r, k).cpu().numpy()
    ref = oproj.projection(seed, stream, 0, r, k).astype(np.float32)
    np.testing.assert_array_equal(A.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("seed,stream,r,k", [(1234, 0, 64, 4096), (3, 1, 7, 1001), (1261, 2, 256, 1536)])
def test_regen_gaussian_within_one_ulp(lg, seed, stream, r, k):
    say("regen gauss", seed, stream, r, k)
    A = lg.regen_A(seed, stream, 1, r, k).cpu().numpy().astype(np.float64)
    ref = oproj.projection(seed, stream, 1, r, k)
    np.testing.assert_array_equal(obf16.round_f64(A), A)      # GPU values are bf16
    bits_g = obf16.f64_to_bits(A).astype(np.int32)
    bits_o = obf16.f64_to_bits(ref).astype(np.int32)
    same = bits_g == bits_o
    assert same.mean() >= 0.999, same.mean()
    assert np.abs(bits_g - bits_o).max() <= 1


# ------------------------------------------------------------------ sketch

SKETCH_CASES = [
    # T, d, k, r, kind, n_mb
    (128, 256, 256, 4, 0, 2),       # the d = k = 256, r = 4 layer
    (1000, 300, 520, 16, 0, 2),     # ragged T, d, k
    (77, 1030, 264, 64, 0, 1),
    (300, 200, 700, 100, 0, 2),     # r not a power of two, rank padding
    (64, 128, 512, 256, 0, 1),      # maximum rank
    (33, 17, 9, 3, 0, 3),           # tiny ragged everything
    (1, 8, 8, 1, 0, 1),             # single token, rank one
    (2048, 512, 1024, 32, 0, 2),    # several work-groups along T (split path)
    (4096, 1536, 256, 64, 0, 1),    # narrow k, many splits
    (200, 300, 520, 16, 1, 2),      # Gaussian basis
    (129, 256, 1000, 256, 1, 1),
    # many d groups along with several splits
    (4096, 1024, 1024, 64, 0, 2),   # 8 d groups x 8 splits
    (3000, 4096, 512, 16, 0, 1),    # 32 d groups, 5 splits, ragged T
    (1000, 4000, 256, 64, 0, 1),    # ragged d (masked columns), 2 splits
    (1024, 4224, 256, 32, 0, 1),    # 33 d groups
    (2048, 1024, 768, 64, 1, 1),    # Gaussian basis
]


def _sketch_case(lg, T, d, k, r, kind, n_mb, seed=1234, stream=0, ld_pad=0):
    mbs = [(synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=d),
            synth.host_normal_bf16((T, d), synth.DY_ID, mb=mb, salt=d)) for mb in range(n_mb)]
    S0 = synth.host_normal_f32((d, r), synth.S_ID, salt=T)
    S = S0.clone().cuda()
    ws = lg.sketch_workspace(T, d, k, r)
    for X, dY in mbs:
        ldx = -(-k // 8) * 8 + ld_pad
        ldd = -(-d // 8) * 8 + ld_pad
        lg.sketch_accumulate(padded_bf16(X, ldx), padded_bf16(dY, ldd), S, seed, stream, kind, ws=ws)
    torch.cuda.synchronize()
    A = oproj.projection(seed, stream, kind, r, k)
    ref = osketch.accumulate(S0.numpy().astype(np.float64),
                             [(synth.bf16_to_f64(X), synth.bf16_to_f64(dY)) for X, dY in mbs], A)
    delta_ref = ref - S0.numpy().astype(np.float64)
    delta_gpu = S.cpu().numpy().astype(np.float64) - S0.numpy().astype(np.float64)
    elem = max_rel(delta_gpu, delta_ref)
    assert elem < s_elem_bar(kind), ("elementwise", elem)
    return S, rel_fro(delta_gpu, delta_ref), rel_fro(S.cpu().numpy(), ref)


@pytest.mark.parametrize("T,d,k,r,kind,n_mb", SKETCH_CASES)
def test_sketch_matches_oracle(lg, T, d, k, r, kind, n_mb):
    say("sketch", T, d, k, r, kind, n_mb)
    _, err_delta, err_total = _sketch_case(lg, T, d, k, r, kind, n_mb)
    assert err_delta < S_TOL, err_delta
    assert err_total < S_TOL, err_total


# Every projection kernel on each case (logra_set_kernel_choice with
# LOGRA_CHOICE_PROJECT_TILE: 0 = the 32-token kernel, 1 = the 64-token tile,
# 2 = the 128-token tile where r > 64, else the 64-token one), ragged and
# whole tiles alike.
PROJECTION_CASES = [
    # T, d, k, r, kind, n_mb
    (77, 1030, 264, 64, 0, 1),      # 3 steps: the last tile's second block is empty
    (300, 200, 700, 100, 0, 2),     # padded rank, ragged k
    (64, 128, 512, 256, 0, 1),      # one whole tile, maximum rank
    (129, 256, 1000, 256, 1, 1),    # Gaussian basis, ragged
    (1056, 384, 1280, 128, 0, 1),   # odd step count, five chunks over four lanes
    (640, 256, 2304, 256, 0, 1),    # whole tiles and chunks (unmasked), nine chunks
    (1024, 512, 4096, 64, 0, 1),    # unmasked, one 32-row block per wave
    (2048, 1024, 768, 64, 1, 1),    # Gaussian basis, unmasked tiles
    (200, 300, 520, 200, 0, 2),     # 128-token tiles: ragged T (second tile partly past T), k, r
    (256, 128, 1536, 128, 1, 1),    # 128-token tiles, Gaussian, one 32-row block per wave
]


def _fuzz_shapes(n, seed, budget=1.5e8):
    """Seeded random small shapes: any rank 1..256 (the padded-rank edges
    and off-power-of-two values weighted up), ragged T, d and k, both bases,
    one or two microbatches; the oracle's work T (k + d) r stays under
    `budget` multiply-adds."""
    rng = np.random.default_rng(seed)
    ranks = [1, 2, 3, 5, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 127, 128, 129, 200,
             255, 256]
    out = []
    while len(out) < n:
        T = int(rng.integers(1, 3001))
        d = int(rng.integers(1, 2200))
        k = int(rng.integers(1, 1400))
        r = int(rng.choice(ranks)) if rng.random() < 0.7 else int(rng.integers(1, 257))
        if T * (k + d) * r > budget:
            continue
        out.append((T, d, k, r, int(rng.integers(0, 2)), int(rng.integers(1, 3))))
    return out


FUZZ_SKETCH = _fuzz_shapes(16, 2027)


@pytest.mark.parametrize("T,d,k,r,kind,n_mb", FUZZ_SKETCH)
def test_sketch_fuzz_small_shapes(lg, T, d, k, r, kind, n_mb):
    say("sketch fuzz", T, d, k, r, kind, n_mb)
    _, err, _ = _sketch_case(lg, T, d, k, r, kind, n_mb, seed=77 + T, stream=d % 3)
    assert err < S_TOL, err


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("T,d,k,r,kind,n_mb", PROJECTION_CASES)
def test_sketch_both_projection_kernels(lg, mode, T, d, k, r, kind, n_mb):
    say("sketch projection kernel", mode, T, d, k, r, kind, n_mb)
    with lg.kernel_choice(lg.CHOICE_PROJECT_TILE, mode):
        _, err_delta, err_total = _sketch_case(lg, T, d, k, r, kind, n_mb)
    assert err_delta < S_TOL, err_delta
    assert err_total < S_TOL, err_total


# Both accumulate kernels at r = 128 and 256 (LOGRA_CHOICE_ACC_WIDE: 0 = the
# kernel whose waves split r and T, 1 = the work-group-wide tile of 2 or 4 d
# groups, which by default serves only T >= 16384).
WIDE_CASES = [
    # T, d, k, r, kind, n_mb
    (77, 1030, 264, 256, 0, 1),     # ragged T and d, nine d groups (the last work-group half empty)
    (256, 384, 256, 256, 0, 2),     # three d groups: a work-group with a group past d
    (512, 512, 512, 256, 0, 1),     # whole tiles (unmasked)
    (2048, 1024, 512, 128, 0, 1),   # r = 128: four d groups per work-group, several splits
    (1000, 640, 300, 100, 0, 2),    # padded rank, five d groups over two work-groups
    (129, 256, 1000, 256, 1, 1),    # Gaussian basis
    (4096, 256, 256, 256, 0, 1),    # many splits of one work-group column
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,d,k,r,kind,n_mb", WIDE_CASES)
def test_sketch_both_accumulate_kernels(lg, mode, T, d, k, r, kind, n_mb):
    say("sketch accumulate kernel", mode, T, d, k, r, kind, n_mb)
    with lg.kernel_choice(lg.CHOICE_ACC_WIDE, mode):
        _, err_delta, err_total = _sketch_case(lg, T, d, k, r, kind, n_mb)
    assert err_delta < S_TOL, err_delta
    assert err_total < S_TOL, err_total


SHARED_CASES = [
    # T, k, ds (outputs sharing X), r, kind
    (512, 256, (256, 64, 64), 64, 0),          # q/k/v-shaped
    (1000, 520, (300, 1030), 16, 0),           # gate/up-shaped, ragged
    (77, 264, (17, 256, 129, 8), 4, 0),        # four outputs, tiny and ragged
    (2048, 512, (512, 128), 100, 0),           # split path, padded rank
    (129, 1000, (256, 100), 256, 1),           # Gaussian basis, maximum rank
]


SHARED_WIDE_CASES = [
    # outputs with odd and even d-group counts, so work-groups of the wide
    # accumulate kernel stop at each output's last group
    (512, 256, (256, 64, 136), 256, 0),      # 2, 1, 2 groups at 2 per work-group
    (300, 520, (300, 1030), 128, 0),         # 3 and 9 groups at 4 per work-group, ragged T
    (129, 1000, (256, 100, 384, 17), 256, 1),
]


@pytest.mark.parametrize("T,k,ds,r,kind", SHARED_WIDE_CASES)
def test_sketch_shared_wide_accumulate(lg, T, k, ds, r, kind):
    with lg.kernel_choice(lg.CHOICE_ACC_WIDE, 1):
        test_sketch_shared_matches_oracle_and_single_calls(lg, T, k, ds, r, kind)


@pytest.mark.parametrize("T,k,ds,r,kind", SHARED_CASES)
def test_sketch_shared_matches_oracle_and_single_calls(lg, T, k, ds, r, kind):
    say("sketch shared", T, k, ds, r, kind)
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=k)
    dYs = [synth.host_normal_bf16((T, d), synth.DY_ID, mb=o, salt=d) for o, d in enumerate(ds)]
    S0 = [synth.host_normal_f32((d, r), synth.S_ID, mb=o, salt=T) for o, d in enumerate(ds)]
    ldx = -(-k // 8) * 8
    Xg = padded_bf16(X, ldx)
    dYg = [padded_bf16(dY, -(-dY.shape[1] // 8) * 8 + 8) for dY in dYs]
    Ss = [s0.clone().cuda() for s0 in S0]
    lg.sketch_accumulate_shared(Xg, dYg, Ss, 1234, 0, kind)
    singles = [s0.clone().cuda() for s0 in S0]
    for dY, S in zip(dYg, singles):
        lg.sketch_accumulate(Xg, dY, S, 1234, 0, kind)
    torch.cuda.synchronize()
    A = oproj.projection(1234, 0, kind, r, k)
    Xf = synth.bf16_to_f64(X)
    for o in range(len(ds)):
        ref = osketch.accumulate(S0[o].numpy().astype(np.float64),
                                 [(Xf, synth.bf16_to_f64(dYs[o]))], A)
        base = S0[o].numpy().astype(np.float64)
        got = Ss[o].cpu().numpy().astype(np.float64)
        assert rel_fro(got - base, ref - base) < S_TOL, o
        assert max_rel(got - base, ref - base) < s_elem_bar(kind), o
        one = singles[o].cpu().numpy().astype(np.float64)
        assert rel_fro(got - base, one - base) < 1e-5, o


def test_sketch_shared_one_output_is_the_single_call_bitwise(lg):
    say("sketch shared n_out = 1")
    T, d, k, r = 2048, 384, 512, 64
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=5).cuda()
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=5).cuda()
    a = torch.zeros(d, r, device="cuda")
    b = torch.zeros(d, r, device="cuda")
    lg.sketch_accumulate(X, dY, a, 99)
    lg.sketch_accumulate_shared(X, [dY], [b], 99)
    assert torch.equal(a, b)


OVERWRITE_CASES = [
    # T, d, k, r, kind: one split (S written by the accumulate kernel), several
    # splits (S written by the finalize kernel), a rank that is not a multiple
    # of four (scalar finalize stores), the Gaussian basis at maximum rank
    (128, 256, 256, 4, 0),
    (2048, 512, 1024, 64, 0),
    (2048, 300, 520, 3, 0),
    (1000, 1536, 512, 256, 1),
]


@pytest.mark.parametrize("T,d,k,r,kind", OVERWRITE_CASES)
def test_sketch_overwrite_is_zero_then_add(lg, T, d, k, r, kind):
    say("sketch overwrite", T, d, k, r, kind)
    mbs = [(padded_bf16(synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=d), -(-k // 8) * 8),
            padded_bf16(synth.host_normal_bf16((T, d), synth.DY_ID, mb=mb, salt=d), -(-d // 8) * 8))
           for mb in range(2)]
    ref = torch.zeros(d, r, device="cuda")
    got = torch.full((d, r), float("nan"), device="cuda")
    for mb, (X, dY) in enumerate(mbs):
        lg.sketch_accumulate(X, dY, ref, 1234, 0, kind)
        lg.sketch_accumulate(X, dY, got, 1234, 0, kind, overwrite=mb == 0)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), mb
    # overwriting again discards everything accumulated so far
    lg.sketch_accumulate(mbs[1][0], mbs[1][1], got, 1234, 0, kind, overwrite=True)
    one = torch.zeros(d, r, device="cuda")
    lg.sketch_accumulate(mbs[1][0], mbs[1][1], one, 1234, 0, kind)
    torch.cuda.synchronize()
    assert torch.equal(got, one)


def test_sketch_overwrite_empty_microbatch_zeroes_S(lg):
    say("sketch overwrite T = 0")
    for d, r in ((256, 4), (300, 3), (1, 1), (4097, 256)):
        S = torch.full((d, r), float("nan"), device="cuda")
        X = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
        dY = torch.zeros(0, d, dtype=torch.bfloat16, device="cuda")
        lg.sketch_accumulate(X, dY, S, 1234, overwrite=True)
        torch.cuda.synchronize()
        assert torch.count_nonzero(S).item() == 0 and not torch.isnan(S).any()
    # an empty microbatch without the flag leaves S as it is
    S = torch.full((64, 8), 3.0, device="cuda")
    lg.sketch_accumulate(torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"),
                         torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"), S, 1234)
    torch.cuda.synchronize()
    assert torch.all(S == 3.0)


def test_sketch_shared_overwrite(lg):
    say("sketch shared overwrite")
    T, k, ds, r = 512, 256, (256, 64, 136), 64
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=3).cuda()
    dYs = [synth.host_normal_bf16((T, d), synth.DY_ID, mb=o, salt=d).cuda() for o, d in enumerate(ds)]
    ref = [torch.zeros(d, r, device="cuda") for d in ds]
    got = [torch.full((d, r), float("nan"), device="cuda") for d in ds]
    lg.sketch_accumulate_shared(X, dYs, ref, 1234)
    lg.sketch_accumulate_shared(X, dYs, got, 1234, overwrite=True)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    empty = [torch.full((d, r), float("nan"), device="cuda") for d in ds]
    lg.sketch_accumulate_shared(X[:0], [dY[:0] for dY in dYs], empty, 1234, overwrite=True)
    torch.cuda.synchronize()
    for e in empty:
        assert torch.count_nonzero(e).item() == 0 and not torch.isnan(e).any()


DEFER_CASES = [
    # T, d, k, r, kind, n_mb, accumulate kernel at r > 64 (None: automatic)
    (2048, 512, 1024, 64, 0, 4, None),    # several splits
    (128, 256, 256, 4, 0, 3, None),       # a single split (deferred through the partial tile)
    (1000, 300, 520, 16, 1, 2, None),     # Gaussian basis, ragged
    (8192, 4096, 512, 64, 0, 4, None),    # the headline's split plan (8 x 32) on a narrow k
    (512, 384, 256, 256, 0, 3, 1),        # work-group-wide accumulate kernel
    (512, 384, 256, 256, 0, 2, 0),        # the other kernel at r = 256
]


@pytest.mark.parametrize("T,d,k,r,kind,n_mb,wide", DEFER_CASES)
def test_sketch_deferred_chain(lg, T, d, k, r, kind, n_mb, wide):
    # DEFER, DEFER|PENDING, ..., PENDING (+ OVERWRITE): S written once, at the end
    say("sketch deferred chain", T, d, k, r, kind, n_mb, wide)
    mbs = [(padded_bf16(synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=d + 3), -(-k // 8) * 8),
            padded_bf16(synth.host_normal_bf16((T, d), synth.DY_ID, mb=mb, salt=d + 3), -(-d // 8) * 8))
           for mb in range(n_mb)]
    S0 = synth.host_normal_f32((d, r), synth.S_ID, salt=T + 3)
    ctx = lg.kernel_choice(lg.CHOICE_ACC_WIDE, wide) if wide is not None else None
    if ctx:
        ctx.__enter__()
    try:
        ws = lg.sketch_workspace(T, d, k, r)
        for overwrite in (False, True):
            S = S0.clone().cuda()
            plain = S0.clone().cuda()
            for mb, (X, dY) in enumerate(mbs):
                last = mb == n_mb - 1
                lg.sketch_accumulate(X, dY, S, 1234, 1, kind, ws=ws, defer=not last, pending=mb > 0,
                                     overwrite=overwrite and last)
                if not last:
                    torch.cuda.synchronize()
                    assert torch.equal(S.cpu(), S0), "a deferring call touched S"
                lg.sketch_accumulate(X, dY, plain, 1234, 1, kind, overwrite=overwrite and mb == 0)
            torch.cuda.synchronize()
            A = oproj.projection(1234, 1, kind, r, k)
            base = np.zeros((d, r)) if overwrite else S0.numpy().astype(np.float64)
            ref = osketch.accumulate(base, [(synth.bf16_to_f64(X), synth.bf16_to_f64(dY))
                                            for X, dY in mbs], A)
            got = S.cpu().numpy().astype(np.float64)
            assert rel_fro(got - base, ref - base) < S_TOL
            assert max_rel(got - base, ref - base) < s_elem_bar(kind)
            # the same sums as the call-by-call chain, up to fp32 summation order
            assert rel_fro(got, plain.cpu().numpy()) < 1e-5
        # deterministic: the same chain again gives the same bits
        again = S0.clone().cuda()
        for mb, (X, dY) in enumerate(mbs):
            last = mb == n_mb - 1
            lg.sketch_accumulate(X, dY, again, 1234, 1, kind, ws=ws, defer=not last, pending=mb > 0,
                                 overwrite=last)
        torch.cuda.synchronize()
        assert torch.equal(again, S)
    finally:
        if ctx:
            ctx.__exit__(None, None, None)


def test_sketch_shared_deferred_chain(lg):
    say("sketch shared deferred chain")
    T, k, ds, r = 1024, 512, (512, 128, 136), 64
    X = [synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=9).cuda() for mb in range(3)]
    dYs = [[synth.host_normal_bf16((T, dd), synth.DY_ID, mb=mb * 10 + o, salt=9).cuda()
            for o, dd in enumerate(ds)] for mb in range(3)]
    S = [torch.full((dd, r), float("nan"), device="cuda") for dd in ds]
    ws = torch.empty(lg.sketch_shared_ws_bytes(T, k, r, ds), dtype=torch.uint8, device="cuda")
    for mb in range(3):
        last = mb == 2
        lg.sketch_accumulate_shared(X[mb], dYs[mb], S, 77, 0, 0, ws=ws, defer=not last,
                                    pending=mb > 0, overwrite=last)
    torch.cuda.synchronize()
    A = oproj.projection(77, 0, 0, r, k)
    for o, dd in enumerate(ds):
        ref = osketch.accumulate(np.zeros((dd, r)), [(synth.bf16_to_f64(X[mb]),
                                                       synth.bf16_to_f64(dYs[mb][o])) for mb in range(3)], A)
        got = S[o].cpu().numpy().astype(np.float64)
        assert rel_fro(got, ref) < S_TOL, o
        assert max_rel(got, ref) < s_elem_bar(0), o


@pytest.mark.parametrize("T,d,k,r", [(2048, 1536, 256, 64), (3000, 4096, 512, 16), (4096, 1536, 256, 64),
                                     (1000, 4000, 256, 64)])
def test_sketch_overflow_stays_infinite(lg, T, d, k, r):
    # One token of dY near the bf16 maximum in the last split: that split's
    # partial overflows to +-inf, which must reach S as inf (never NaN) whatever
    # the split count.
    say("sketch overflow", T, d, k, r)
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=11)
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=11)
    col = d // 3
    dY[T - 1, col] = 3.0e38
    S = torch.zeros(d, r, device="cuda")
    lg.sketch_accumulate(padded_bf16(X, -(-k // 8) * 8), padded_bf16(dY, -(-d // 8) * 8), S, 1234)
    torch.cuda.synchronize()
    got = S.cpu()
    assert not torch.isnan(got).any()
    assert torch.isinf(got[col]).sum().item() > r // 2
    others = torch.cat([got[:col], got[col + 1:]])
    assert torch.isfinite(others).all()


def test_sketch_padded_strides(lg):
    say("sketch padded strides")
    _, e1, _ = _sketch_case(lg, 300, 100, 120, 16, 0, 2, ld_pad=24)
    assert e1 < S_TOL


def test_sketch_deterministic(lg):
    say("sketch determinism")
    T, d, k, r = 4096, 1024, 1024, 64
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=77).cuda()
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=77).cuda()
    outs = []
    for _ in range(3):
        S = torch.zeros(d, r, device="cuda")
        lg.sketch_accumulate(X, dY, S, 1234)
        outs.append(S.cpu().numpy().view(np.uint32).copy())
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_binding_refuses_host_and_strided_buffers(lg):
    # a workspace or P that is not one contiguous block of device memory is
    # refused before anything reaches the library (a host address would
    # reach the kernels)
    say("binding buffer checks")
    T, d, k, r = 64, 128, 256, 16
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=3).cuda()
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=3).cuda()
    S = torch.zeros(d, r, device="cuda")
    n = lg.sketch_ws_bytes(T, d, k, r)
    for ws in (torch.empty(n, dtype=torch.uint8),                        # host memory
               torch.empty(2 * n, dtype=torch.uint8, device="cuda")[::2]):  # strided
        with pytest.raises(ValueError):
            lg.sketch_accumulate(X, dY, S, 1, ws=ws)
    with pytest.raises(ValueError):
        lg.sketch_project(X, 1, r, P=torch.empty(2 * lg.sketch_p_bytes(T, r), dtype=torch.uint8,
                                                 device="cuda")[::2])
    z = synth.host_normal_bf16((4, 512), synth.Z_ID, salt=3).cuda()
    with pytest.raises(ValueError):
        lg.predicted_kl(z, z, 1.0, 2e-4, 4.0, ws=torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(ValueError):
        lg.predicted_kl_sweep(z, z, [1.0], 1.0, ws=torch.empty(4096, dtype=torch.uint8))
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0          # nothing ran


def test_sketch_zero_tokens_is_noop(lg):
    S = torch.ones(16, 4, device="cuda")
    X = torch.empty(0, 32, dtype=torch.bfloat16, device="cuda")
    dY = torch.empty(0, 16, dtype=torch.bfloat16, device="cuda")
    lg.sketch_accumulate(X, dY, S, 1)
    assert torch.equal(S, torch.ones(16, 4, device="cuda"))


def test_sketch_linear_across_calls_and_resume(lg):
    say("sketch linearity")
    T, d, k, r = 512, 384, 640, 32
    X = synth.host_normal_bf16((2 * T, k), synth.X_ID, salt=5).cuda()
    dY = synth.host_normal_bf16((2 * T, d), synth.DY_ID, salt=5).cuda()
    S_two = torch.zeros(d, r, device="cuda")
    lg.sketch_accumulate(X[:T], dY[:T], S_two, 42)
    # checkpoint S to the host and back between the microbatches
    S_two = S_two.cpu().clone().cuda()
    lg.sketch_accumulate(X[T:], dY[T:], S_two, 42)
    S_one = torch.zeros(d, r, device="cuda")
    lg.sketch_accumulate(X, dY, S_one, 42)
    assert rel_fro(S_two.cpu().numpy(), S_one.cpu().numpy()) < 1e-5


# ------------------------------------------------------------------ merge

MERGE_CASES = [
    # d, k, r, kind, alpha, eta
    (256, 256, 4, 0, 1.0, 1e-3),
    (4096, 4096, 64, 0, 1.0, 2e-4),
    (300, 520, 16, 0, 0.4, 1e-3),
    (1030, 264, 100, 0, 2.0, 5e-4),
    (17, 9, 3, 0, 1.0, 1e-2),
    (1, 8, 1, 0, 1.0, 1e-2),
    (512, 1000, 256, 0, 0.5, 1e-3),
    (300, 520, 16, 1, 1.0, 1e-3),
    (256, 1000, 256, 1, 1.0, 1e-3),
    # whole row blocks and 64-column passes, short last column block
    (512, 832, 64, 0, 1.0, 1e-3),
    (256, 1344, 256, 0, 1.0, 1e-3),
    (512, 1536, 128, 0, 0.5, 1e-3),
    (256, 1280, 256, 1, 1.0, 1e-3),
    # 128-row blocks of the small-rank sign basis, 256-row blocks of 16-row
    # waves for the small-rank Gaussian basis
    (384, 576, 32, 0, 1.0, 1e-3),
    (128, 256, 16, 0, 1.0, 1e-3),
    (200, 300, 64, 0, 1.0, 1e-3),
    (512, 768, 64, 1, 1.0, 1e-3),
    (640, 512, 64, 1, 0.5, 1e-3),
    # whole tiles with a rank that is not a multiple of 32 (unmasked kernel,
    # K tail cleared in the S loads)
    (384, 1024, 24, 0, 1.0, 1e-3),
    (512, 768, 100, 0, 1.0, 1e-3),
    (256, 512, 200, 1, 1.0, 1e-3),
    (128, 64, 1, 0, 1.0, 1e-2),
]


def _merge_case(lg, d, k, r, kind, alpha, eta, seed=1234, stream=0, ld_pad=0):
    W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=k)
    # S of realistic scale for the step: the sketch of a few hundred tokens
    S = synth.host_normal_f32((d, r), synth.S_ID, salt=d, sigma=15.0)
    ldw = -(-k // 8) * 8 + ld_pad
    W = padded_bf16(W0, ldw)
    lg.merge(W, S.cuda(), seed, stream, kind, alpha, eta)
    torch.cuda.synchronize()
    A = oproj.projection(seed, stream, kind, r, k)
    Wb = synth.bf16_bits(W0)
    ref_delta = omerge.merged_delta(Wb, S.numpy().astype(np.float64), A, alpha, eta)
    got = synth.bf16_to_f64(W) - synth.bf16_to_f64(W0)
    ex = w_excess(synth.bf16_bits(W), omerge.merge_bits(Wb, S.numpy().astype(np.float64), A,
                                                          alpha, eta), ref_delta)
    assert ex <= w_elem_bar(kind), ("elementwise", ex)
    return W, rel_fro(got, ref_delta)


@pytest.mark.parametrize("d,k,r,kind,alpha,eta", MERGE_CASES)
def test_merge_matches_oracle(lg, d, k, r, kind, alpha, eta):
    say("merge", d, k, r, kind, alpha, eta)
    _, err = _merge_case(lg, d, k, r, kind, alpha, eta)
    assert err < W_TOL, err


FUZZ_MERGE = [(d, k, r, kind) for (_, d, k, r, kind, _) in _fuzz_shapes(12, 2028, budget=1e12)]


@pytest.mark.parametrize("d,k,r,kind", FUZZ_MERGE)
def test_merge_fuzz_small_shapes(lg, d, k, r, kind):
    say("merge fuzz", d, k, r, kind)
    _, err = _merge_case(lg, d, k, r, kind, 1.0, 1e-3, seed=91 + d, stream=k % 3)
    assert err < W_TOL, err


def test_merge_padded_stride_keeps_padding(lg):
    say("merge padded stride")
    d, k, r = 70, 100, 8
    W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=3)
    buf = torch.full((d, 112), 7.0, dtype=torch.bfloat16, device="cuda")
    buf[:, :k] = W0.cuda()
    S = synth.host_normal_f32((d, r), synth.S_ID, salt=3).cuda()
    lg.merge(buf[:, :k], S, 9, 0, 0, 1.0, 1e-3)
    assert torch.all(buf[:, k:] == 7.0)
    A = oproj.projection(9, 0, 0, r, k)
    ref = omerge.merged_delta(synth.bf16_bits(W0), S.cpu().numpy().astype(np.float64), A, 1.0, 1e-3)
    assert rel_fro(synth.bf16_to_f64(buf[:, :k]) - synth.bf16_to_f64(W0), ref) < W_TOL
    ref_bits = omerge.merge_bits(synth.bf16_bits(W0), S.cpu().numpy().astype(np.float64), A, 1.0,
                                 1e-3)
    assert w_excess(synth.bf16_bits(buf[:, :k]), ref_bits, ref) <= W_ELEM


@pytest.mark.parametrize("d,k,r,kind", [(512, 768, 64, 0), (300, 1000, 17, 0), (256, 512, 128, 1),
                                        (4096, 4096, 64, 0)])
def test_merge_S_four_bytes_off_alignment(lg, d, k, r, kind):
    # The ABI asks S for 4-byte alignment only: an S that starts 4 bytes into a
    # 256-byte-aligned buffer must give the same weights as an aligned copy.
    say("merge misaligned S", d, k, r, kind)
    W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=d + 1).cuda()
    S_host = synth.host_normal_f32((d, r), synth.S_ID, salt=d + 1, sigma=15.0)
    buf = torch.empty(d * r + 4, device="cuda")
    S_off = buf[1:1 + d * r].view(d, r)
    assert S_off.data_ptr() % 16 == 4
    S_off.copy_(S_host.cuda())
    S_al = S_host.cuda()
    W_a = lg.merge(W0.clone(), S_al, 31, 1, kind, 1.0, 1e-3)
    W_b = lg.merge(W0.clone(), S_off, 31, 1, kind, 1.0, 1e-3)
    torch.cuda.synchronize()
    assert torch.equal(W_a.view(torch.int16), W_b.view(torch.int16))
    A = oproj.projection(31, 1, kind, r, k)
    Sh = S_host.numpy().astype(np.float64)
    ref_bits = omerge.merge_bits(synth.bf16_bits(W0), Sh, A, 1.0, 1e-3)
    ref = omerge.merged_delta(synth.bf16_bits(W0), Sh, A, 1.0, 1e-3)
    assert rel_fro(synth.bf16_to_f64(W_b) - synth.bf16_to_f64(W0), ref) < W_TOL
    assert w_excess(synth.bf16_bits(W_b), ref_bits, ref) <= w_elem_bar(kind)


def test_merge_zero_step_is_bitwise_noop(lg):
    W0 = synth.host_normal_bf16((300, 520), synth.W_ID, salt=8).cuda()
    W = W0.clone()
    S = synth.host_normal_f32((300, 16), synth.S_ID, salt=8).cuda()
    lg.merge(W, S, 5, 0, 0, 0.0, 1e-3)
    assert torch.equal(W.view(torch.int16), W0.view(torch.int16))


def test_rollout_apply_matches_trainer_merge(lg):
    """The rollout side receives alpha*eta*U and the seed and applies the same
    merge; passing the scaled factor with alpha = eta = 1 gives the same W."""
    say("rollout apply")
    d, k, r = 512, 768, 64
    W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=11).cuda()
    S = synth.host_normal_f32((d, r), synth.S_ID, salt=11, sigma=15.0).cuda()
    alpha, eta = 0.5, 2e-4
    W_train = lg.merge(W0.clone(), S, 77, 0, 0, alpha, eta)
    U_sent = S * np.float32(np.float32(alpha) * np.float32(eta))
    W_roll = lg.merge(W0.clone(), U_sent, 77, 0, 0, 1.0, 1.0)
    diff = (W_train.float() - W_roll.float()).abs().max().item()
    ulp = (W0.float().abs().max() * 2 ** -7).item()
    assert diff <= ulp
    # and the rollout's weights against the oracle's merge of the received factor
    A = oproj.projection(77, 0, 0, r, k)
    W0b = synth.bf16_bits(W0)
    U = U_sent.cpu().numpy().astype(np.float64)
    ref = omerge.merged_delta(W0b, U, A, 1.0, 1.0)
    got = synth.bf16_to_f64(W_roll) - synth.bf16_to_f64(W0)
    assert rel_fro(got, ref) < W_TOL
    assert w_excess(synth.bf16_bits(W_roll), omerge.merge_bits(W0b, U, A, 1.0, 1.0), ref) <= W_ELEM


# ------------------------------------------------------------------ predicted KL

KL_CASES = [
    # n, V, tau, sigma_dir
    (64, 1000, 1.0, 0.05),
    (7, 152064, 1.0, 0.05),
    (3, 1001, 0.7, 0.05),
    (5, 2, 1.0, 0.5),
    (9, 4099, 1.3, 0.3),      # large steps: exercises the exp fallback for |d| > 1/2
    (300, 32000, 1.0, 0.01),
]


@pytest.mark.parametrize("n,V,tau,sig", KL_CASES)
def test_predicted_kl_matches_oracle(lg, n, V, tau, sig):
    say("kl", n, V, tau, sig)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V)
    dirn = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V, sigma=sig)
    zp = synth.proposal_logits(z, dirn, 1.0)
    ld = -(-V // 8) * 8
    zc_g, zp_g = padded_bf16(z, ld), padded_bf16(zp, ld)
    kl_tok = torch.empty(n, device="cuda")
    out = lg.predicted_kl(zc_g, zp_g, tau, 2e-4, 4.0, kl_tok=kl_tok)
    out_ws = lg.predicted_kl(zc_g, zp_g, tau, 2e-4, 4.0)
    torch.cuda.synchronize()
    ref_rows = okl.kl_rows(synth.bf16_to_f64(z), synth.bf16_to_f64(zp), tau)
    q_ref = float(ref_rows.mean())
    q, alpha = out.cpu().numpy().astype(np.float64)
    assert abs(q / q_ref - 1) < Q_TOL, (q, q_ref)
    np.testing.assert_allclose(kl_tok.cpu().numpy(), ref_rows, rtol=1e-3, atol=1e-9)
    assert abs(alpha - okl.step_size(q_ref, 2e-4, 4.0)) <= 1e-3 * okl.step_size(q_ref, 2e-4, 4.0)
    assert torch.equal(out, out_ws)


@pytest.mark.parametrize("n,V,offset", [(6, 152064, 0.75), (6, 152064, -3.0), (16, 4099, 2.0),
                                        (3, 40, -1.5)])
def test_predicted_kl_with_a_row_offset(lg, n, V, offset):
    # proposed logits = current + a per-row constant + a small spread: the KL
    # ignores the constant; the kernels take each row relative to a reference
    # difference so the constant does not cancel in fp32
    say("kl offset", n, V, offset)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 7)
    noise = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 7, sigma=0.01)
    shift = torch.linspace(-0.5, 0.5, n).view(n, 1) + offset     # a different constant per row
    zp = (z.float() + shift + noise.float()).to(torch.bfloat16)
    ld = -(-V // 8) * 8
    kl_tok = torch.empty(n, device="cuda")
    out = lg.predicted_kl(padded_bf16(z, ld), padded_bf16(zp, ld), 1.0, 2e-4, 4.0, kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref_rows = okl.kl_rows(synth.bf16_to_f64(z), synth.bf16_to_f64(zp), 1.0)
    np.testing.assert_allclose(kl_tok.cpu().numpy(), ref_rows, rtol=1e-3, atol=1e-9)
    assert abs(out[0].item() / ref_rows.mean() - 1) < Q_TOL


@pytest.mark.parametrize("n,V,offset,alphas", [(6, 152064, 0.75, [0.25, 0.5, 1.0, 2.0]),
                                               (8, 4099, -3.0, [1.0, -0.5, 4.0])])
def test_predicted_kl_sweep_with_a_direction_offset(lg, n, V, offset, alphas):
    say("kl sweep offset", n, V, offset, alphas)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 9)
    base = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 9, sigma=0.01)
    dirn = (base.float() + offset + torch.linspace(0, 1, n).view(n, 1)).to(torch.bfloat16)
    m = len(alphas)
    kl_tok = torch.empty(m, n, device="cuda")
    ld = -(-V // 8) * 8
    out = lg.predicted_kl_sweep(padded_bf16(z, ld), padded_bf16(dirn, ld), alphas, 1.0,
                                kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref_rows = okl.kl_sweep_rows(synth.bf16_to_f64(z), synth.bf16_to_f64(dirn), alphas, 1.0)
    np.testing.assert_allclose(kl_tok.cpu().numpy(), ref_rows, rtol=1e-3, atol=1e-9)
    got = out.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, ref_rows.mean(axis=1), rtol=Q_TOL)


def test_kl_controller_edges(lg):
    say("kl controller edges")
    z = synth.host_normal_bf16((4, 512), synth.Z_ID, salt=1).cuda()
    out = lg.predicted_kl(z, z, 1.0, 2e-4, 3.0)           # q = 0 -> alpha_max
    q, a = out.cpu().tolist()
    assert q == 0.0 and a == 3.0
    # q = 4 delta -> alpha = 1/2: choose the budget from the measured q
    dirn = synth.host_normal_bf16((4, 512), synth.DIR_ID, salt=1, sigma=0.1).cuda()
    zp = synth.proposal_logits(z, dirn, 1.0)
    q = lg.predicted_kl(z, zp, 1.0, 1.0, 10.0)[0].item()
    a = lg.predicted_kl(z, zp, 1.0, q / 4, 10.0)[1].item()
    assert abs(a - 0.5) < 1e-6
    # NaN logits give a NaN alpha
    zn = z.clone()
    zn[0, 0] = float("nan")
    q, a = lg.predicted_kl(zn, zp, 1.0, 2e-4, 4.0).cpu().tolist()
    assert np.isnan(q) and np.isnan(a)


@pytest.mark.parametrize("n,V,offset", [(6, 152064, 0.75), (6, 152064, -3.0), (16, 4099, 2.0)])
def test_predicted_kl_offset_missed_by_the_row_reference(lg, n, V, offset):
    # the proposal carries a per-row offset everywhere except on the row's
    # first 64 tokens, where the reference is taken: the one-pass result is a
    # small difference of large terms, and the row is read again about the
    # p-weighted mean of z' - z.  Bar 1e-4 (ten times below the parity bar)
    say("kl offset past the reference", n, V, offset)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 11)
    noise = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 11, sigma=0.01)
    shift = torch.linspace(-0.25, 0.25, n).view(n, 1) + offset
    shift = shift.expand(n, V).clone()
    shift[:, :64] = 0.0
    zp = (z.float() + shift + noise.float()).to(torch.bfloat16)
    ld = -(-V // 8) * 8
    kl_tok = torch.empty(n, device="cuda")
    out = lg.predicted_kl(padded_bf16(z, ld), padded_bf16(zp, ld), 1.0, 2e-4, 4.0, kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref_rows = okl.kl_rows(synth.bf16_to_f64(z), synth.bf16_to_f64(zp), 1.0)
    np.testing.assert_allclose(kl_tok.cpu().numpy(), ref_rows, rtol=1e-4, atol=1e-9)
    assert abs(out[0].item() / ref_rows.mean() - 1) < Q_TOL


@pytest.mark.parametrize("n,V", [(12, 4099), (6, 152064)])
def test_predicted_kl_masked_vocabulary(lg, n, V):
    # logits of -inf: tokens of probability zero.  Rows 0 .. n-5 masked at the
    # same tokens in z and z' (row 0 at its whole first 64, where the row
    # reference is taken; row 1 at its first three), row n-4 in z only
    # (p = 0, p' > 0), row n-3 unmasked, row n-2 with one token of p > 0 and
    # p' = 0 (KL +inf), row n-1 masked everywhere (NaN)
    say("kl masked", n, V)
    rng = np.random.default_rng(V + n)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 3)
    dirn = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 3, sigma=0.05)
    zp = synth.proposal_logits(z, dirn, 1.0)
    mask = torch.from_numpy(rng.random((n, V)) < 0.1)
    mask[0, :64] = True
    mask[1, :3] = True
    mask[n - 3:] = False
    ninf = float("-inf")
    zm, zpm = z.clone(), zp.clone()
    zm[: n - 3][mask[: n - 3]] = ninf
    zpm[: n - 4][mask[: n - 4]] = ninf
    zpm[n - 2, 5] = ninf
    zm[n - 1] = ninf
    zpm[n - 1] = ninf
    ld = -(-V // 8) * 8
    z_g, zp_g = padded_bf16(zm, ld), padded_bf16(zpm, ld)
    kl_tok = torch.empty(n, device="cuda")
    out = lg.predicted_kl(z_g, zp_g, 1.0, 2e-4, 4.0, kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref = okl.kl_rows(synth.bf16_to_f64(zm), synth.bf16_to_f64(zpm), 1.0)
    got = kl_tok.cpu().numpy().astype(np.float64)
    assert np.isinf(ref[n - 2]) and np.isnan(ref[n - 1])
    assert got[n - 2] == np.inf, got[n - 2]
    assert np.isnan(got[n - 1]), got[n - 1]
    np.testing.assert_allclose(got[: n - 2], ref[: n - 2], rtol=1e-3, atol=1e-9)
    assert np.isnan(out.cpu().numpy()).all()          # the NaN row reaches q and alpha
    # the finite rows alone: q and alpha against the oracle
    out_f = lg.predicted_kl(z_g[: n - 2], zp_g[: n - 2], 1.0, 2e-4, 4.0)
    q, alpha = out_f.cpu().numpy().astype(np.float64)
    q_ref = float(ref[: n - 2].mean())
    assert abs(q / q_ref - 1) < Q_TOL, (q, q_ref)
    assert abs(alpha / okl.step_size(q_ref, 2e-4, 4.0) - 1) < 1e-3
    # with the +inf row: q = +inf and the controller takes no step
    q, alpha = lg.predicted_kl(z_g[: n - 1], zp_g[: n - 1], 1.0, 2e-4, 4.0).cpu().tolist()
    assert q == float("inf") and alpha == 0.0


# ------------------------------------------------------- predicted-KL sweep

SWEEP_CASES = [
    # n, V, tau, sigma_dir, multipliers, weighted
    (64, 1000, 1.0, 0.05, [0.25, 0.5, 1.0, 2.0], False),
    (7, 152064, 1.0, 0.05, [0.25, 0.5, 1.0, 2.0], True),
    (3, 1001, 0.7, 0.05, [1.0], False),
    (5, 2, 1.0, 0.5, [-1.0, 0.5, 3.0], False),
    # |amax * delta / tau| > 1 for about a quarter of the elements: the exact path
    (9, 4099, 1.3, 0.3, [0.5, 1.0, 2.0, 4.0, -2.0], True),
    (300, 32000, 1.0, 0.01, [0.0, 0.1, 1.0, 2.0, 3.0, 4.0, 6.0, 8.0], True),
]


@pytest.mark.parametrize("n,V,tau,sig,alphas,weighted", SWEEP_CASES)
def test_predicted_kl_sweep_matches_oracle(lg, n, V, tau, sig, alphas, weighted):
    say("kl sweep", n, V, tau, sig, alphas, weighted)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V)
    dirn = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V, sigma=sig)
    ld = -(-V // 8) * 8
    z_g, d_g = padded_bf16(z, ld), padded_bf16(dirn, ld)
    w = None
    if weighted:
        rng = np.random.default_rng(n * 131 + V)
        w = rng.uniform(0.0, 2.0, n)
        w[rng.uniform(size=n) < 0.3] = 0.0          # a token mask
        w[0] = 1.0
    w_g = None if w is None else torch.tensor(w, dtype=torch.float32, device="cuda")
    m = len(alphas)
    kl_tok = torch.empty(m, n, device="cuda")
    out = lg.predicted_kl_sweep(z_g, d_g, alphas, tau, weight=w_g, kl_tok=kl_tok)
    out_ws = lg.predicted_kl_sweep(z_g, d_g, alphas, tau, weight=w_g)
    torch.cuda.synchronize()
    zf, df = synth.bf16_to_f64(z), synth.bf16_to_f64(dirn)
    ref_rows = okl.kl_sweep_rows(zf, df, alphas, tau)
    ref = okl.predicted_kl_sweep(zf, df, alphas, tau, None if w is None else np.float32(w))
    got_rows = kl_tok.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_rows, ref_rows, rtol=1e-3, atol=1e-9)
    got = out.cpu().numpy().astype(np.float64)
    for i, a in enumerate(alphas):
        if a == 0.0:
            assert got[i] == 0.0 and np.all(got_rows[i] == 0.0)
        else:
            assert abs(got[i] / ref[i] - 1) < Q_TOL, (a, got[i], ref[i])
    assert torch.equal(out, out_ws)


def test_kl_sweep_alpha_squared_law_and_edges(lg):
    say("kl sweep alpha^2 law")
    n, V = 16, 32768
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=77)
    dirn = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=77, sigma=0.05)
    z_g, d_g = z.cuda(), dirn.cuda()
    alphas = np.array([0.25, 0.5, 1.0, 2.0])
    kl = lg.predicted_kl_sweep(z_g, d_g, alphas, 1.0).cpu().numpy().astype(np.float64)
    ratios = kl / alphas ** 2
    assert ratios.max() / ratios.min() - 1 < 3e-3
    # the rounded-proposal entry point on the same direction does not keep the law
    zp = synth.proposal_logits(z, dirn, 0.25).cuda()
    q_rounded = lg.predicted_kl(z_g, zp, 1.0, 2e-4, 4.0)[0].item()
    assert abs(q_rounded / 0.25 ** 2 / ratios[2] - 1) > 0.05
    # zero weights everywhere: NaN means; a shift of every row: zero KL
    zero_w = torch.zeros(n, device="cuda")
    assert torch.isnan(lg.predicted_kl_sweep(z_g, d_g, [1.0, 2.0], 1.0, weight=zero_w)).all()
    shift = torch.full((n, V), 0.75, dtype=torch.bfloat16, device="cuda")
    flat = lg.predicted_kl_sweep(z_g, shift, [1.0, 4.0], 1.0).cpu().numpy()
    assert np.all(np.abs(flat) < 1e-6)


@pytest.mark.parametrize("n,V,offset,spread", [(6, 152064, 0.45, 0.025), (8, 4099, -0.35, 0.01),
                                               (4, 32000, 3.0, 0.05)])
def test_predicted_kl_sweep_offset_missed_by_the_direction_reference(lg, n, V, offset, spread):
    # the direction carries an offset everywhere except on the row's first 64
    # tokens, where the reference is taken (at alpha = 2 the first two cases
    # put max|alpha| |delta| near the series bound with a narrow spread, the
    # third puts it far past it): the row is read again about the p-weighted
    # mean of the direction.  Bar 1e-4 (ten times below the parity bar)
    say("kl sweep offset past the reference", n, V, offset, spread)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 13)
    base = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 13, sigma=spread)
    off = torch.full((n, V), offset) + torch.linspace(0, 0.05, n).view(n, 1)
    off[:, :64] = 0.0
    dirn = (base.float() + off).to(torch.bfloat16)
    alphas = [0.25, 0.5, 1.0, 2.0]
    ld = -(-V // 8) * 8
    kl_tok = torch.empty(len(alphas), n, device="cuda")
    out = lg.predicted_kl_sweep(padded_bf16(z, ld), padded_bf16(dirn, ld), alphas, 1.0,
                                kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref_rows = okl.kl_sweep_rows(synth.bf16_to_f64(z), synth.bf16_to_f64(dirn), alphas, 1.0)
    np.testing.assert_allclose(kl_tok.cpu().numpy(), ref_rows, rtol=1e-4, atol=1e-9)
    np.testing.assert_allclose(out.cpu().numpy(), ref_rows.mean(axis=1), rtol=Q_TOL)


@pytest.mark.parametrize("V", [1, 3, 65])
def test_kl_masked_tiny_vocabularies(lg, V):
    # vocabularies shorter than the reference window, with masked tokens
    # (each row keeps at least one): both entry points against the oracle
    n = 16
    say("kl masked tiny", V)
    rng = np.random.default_rng(V + 101)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 17)
    dirn = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 17, sigma=0.3)
    zp = synth.proposal_logits(z, dirn, 1.0)
    mask = torch.from_numpy(rng.random((n, V)) < 0.3)
    for t in range(n):
        mask[t, t % V] = False          # every row keeps a token
    ninf = torch.tensor(float("-inf"), dtype=torch.bfloat16)
    zm = torch.where(mask, ninf, z)
    zpm = torch.where(mask, ninf, zp)
    dm = torch.where(mask, torch.tensor(float("nan"), dtype=torch.bfloat16), dirn)
    ld = -(-V // 8) * 8
    kl_tok = torch.empty(n, device="cuda")
    lg.predicted_kl(padded_bf16(zm, ld), padded_bf16(zpm, ld), 1.0, 2e-4, 4.0, kl_tok=kl_tok)
    sw_tok = torch.empty(2, n, device="cuda")
    lg.predicted_kl_sweep(padded_bf16(zm, ld), padded_bf16(dm, ld), [0.5, 2.0], 1.0, kl_tok=sw_tok)
    torch.cuda.synchronize()
    ref = okl.kl_rows(synth.bf16_to_f64(zm), synth.bf16_to_f64(zpm), 1.0)
    ref_sw = okl.kl_sweep_rows(synth.bf16_to_f64(zm), synth.bf16_to_f64(dm), [0.5, 2.0], 1.0)
    np.testing.assert_allclose(kl_tok.cpu().numpy(), ref, rtol=1e-3, atol=1e-9)
    np.testing.assert_allclose(sw_tok.cpu().numpy(), ref_sw, rtol=1e-3, atol=1e-9)


@pytest.mark.parametrize("n,V", [(8, 4099), (4, 152064)])
def test_predicted_kl_sweep_masked_vocabulary(lg, n, V):
    # masked tokens (z = -inf) stay masked in every proposal whatever their
    # direction entry (NaN, +-inf or finite here); row 0 masked at its whole
    # first 64 (the direction reference), row n-1 unmasked, row n-2 masked
    # everywhere (NaN at every multiplier)
    say("kl sweep masked", n, V)
    rng = np.random.default_rng(V * 3 + n)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=V + 5)
    dirn = synth.host_normal_bf16((n, V), synth.DIR_ID, salt=V + 5, sigma=0.05)
    mask = torch.from_numpy(rng.random((n, V)) < 0.1)
    mask[0, :64] = True
    mask[n - 1] = False
    mask[n - 2] = True
    junk = torch.from_numpy(rng.choice([np.nan, np.inf, -np.inf, 3.0], (n, V))).to(torch.bfloat16)
    zm = torch.where(mask, torch.tensor(float("-inf"), dtype=torch.bfloat16), z)
    dm = torch.where(mask, junk, dirn)
    alphas = [0.25, 1.0, -2.0]
    ld = -(-V // 8) * 8
    z_g, d_g = padded_bf16(zm, ld), padded_bf16(dm, ld)
    kl_tok = torch.empty(len(alphas), n, device="cuda")
    lg.predicted_kl_sweep(z_g, d_g, alphas, 1.0, kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref = okl.kl_sweep_rows(synth.bf16_to_f64(zm), synth.bf16_to_f64(dm), alphas, 1.0)
    got = kl_tok.cpu().numpy().astype(np.float64)
    assert np.isnan(ref[:, n - 2]).all() and np.isnan(got[:, n - 2]).all()
    keep = [t for t in range(n) if t != n - 2]
    np.testing.assert_allclose(got[:, keep], ref[:, keep], rtol=1e-3, atol=1e-9)
    # the means over the rows with a distribution
    means = lg.predicted_kl_sweep(padded_bf16(zm[keep], ld), padded_bf16(dm[keep], ld), alphas,
                                  1.0).cpu().numpy()
    np.testing.assert_allclose(means, ref[:, keep].mean(axis=1), rtol=Q_TOL)
    # the same through a token mask: the fully masked row has weight zero and
    # is left out (its NaN does not reach the mean)
    w = np.ones(n)
    w[n - 2] = 0.0
    w[1] = 0.5
    means_w = lg.predicted_kl_sweep(z_g, d_g, alphas, 1.0,
                                    weight=torch.tensor(w, dtype=torch.float32, device="cuda"))
    ref_w = okl.predicted_kl_sweep(synth.bf16_to_f64(zm), synth.bf16_to_f64(dm), alphas, 1.0, w)
    assert np.isfinite(ref_w).all()
    np.testing.assert_allclose(means_w.cpu().numpy(), ref_w, rtol=Q_TOL)


def test_rollout_payload_apply_is_bitwise_the_trainer_merge(lg):
    """[LoGRA] Sync: the rollout side rebuilds A from the seed and applies the
    received factor; with (U, alpha, eta, seed) in the payload it runs the same
    merge and its weights equal the trainer's bit for bit."""
    say("rollout payload")
    from rank_gradient_sketching_amd import sync
    for kind, (d, k, r) in ((0, (512, 768, 64)), (1, (300, 1000, 17))):
        W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=d).cuda()
        S = synth.host_normal_f32((d, r), synth.S_ID, salt=d, sigma=15.0).cuda()
        W_train = lg.merge(W0.clone(), S, 4321, 3, kind, 0.75, 2e-4)
        payload = sync.pack_update(S, 4321, 3, kind, 0.75, 2e-4, k)
        W_roll = sync.apply_update(W0.clone(), payload)
        assert torch.equal(W_train, W_roll)
        # the rollout rebuilds A from the seed in the payload: its weights
        # against the oracle's merge with the oracle's A for that seed
        A = oproj.projection(4321, 3, kind, r, k)
        W0b = synth.bf16_bits(W0)
        Sh = S.cpu().numpy().astype(np.float64)
        ref = omerge.merged_delta(W0b, Sh, A, 0.75, 2e-4)
        got = synth.bf16_to_f64(W_roll) - synth.bf16_to_f64(W0)
        assert rel_fro(got, ref) < W_TOL, kind
        assert w_excess(synth.bf16_bits(W_roll), omerge.merge_bits(W0b, Sh, A, 0.75, 2e-4),
                        ref) <= w_elem_bar(kind)
