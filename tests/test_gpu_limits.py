"""Parity at the size limits of the C ABI: row strides past 2^31 elements,
the largest dY row stride the sketch accepts, and very long T, k and d.

Each case checks the kernels' index arithmetic where a 32-bit product would
wrap: X, W and the logits with a row stride of 2^31 + 8 elements (a row offset
past 4 GiB from the second row on), dY at the sketch's stride limit
(2^26 - 8 elements, read through 32-bit buffer offsets that span 32 rows), a
million tokens (32769 steps, hundreds of splits), a million input columns
(4097 chunks of 256) and a quarter-million output rows (2049 d groups).  The
row padding is filled with NaN, which must neither leak into the results nor
be written.  Bars as in the other parity tests.  The largest case allocates
~17 GB of device memory (288 GB on the part).
"""
import numpy as np
import pytest
import torch

from oracle import kl as okl
from oracle import merge as omerge
from oracle import projection as oproj
from oracle import sketch as osketch
from rank_gradient_sketching_amd import synth

from parity_bars import (Q_TOL, S_TOL, W_TOL, max_rel, rel_fro, s_elem_bar,  # noqa: E402
                         w_elem_bar, w_excess)

pytestmark = pytest.mark.gpu

BIG_LD = (1 << 31) + 8          # row stride past 2^31 elements
DY_LD_MAX = (1 << 26) - 8       # the sketch's largest dY row stride


@pytest.fixture(scope="module")
def lg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_gradient_sketching_amd as m
    return m


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(*a):
    print(*a, flush=True)


def strided(host, ld):
    """GPU copy of a 2-D bf16 host tensor with row stride ld, the padding NaN."""
    rows, cols = host.shape
    buf = torch.full((rows, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, :cols] = host.cuda()
    return buf[:, :cols]


def _sketch_vs_oracle(lg, X_dev, dY_dev, X, dY, r, kind=0, seed=1234, stream=0):
    d = dY.shape[1]
    S0 = synth.host_normal_f32((d, r), synth.S_ID, salt=X.shape[0])
    S = S0.clone().cuda()
    lg.sketch_accumulate(X_dev, dY_dev, S, seed, stream, kind)
    torch.cuda.synchronize()
    A = oproj.projection(seed, stream, kind, r, X.shape[1])
    base = S0.numpy().astype(np.float64)
    ref = osketch.accumulate(base, [(synth.bf16_to_f64(X), synth.bf16_to_f64(dY))], A) - base
    got = S.cpu().numpy().astype(np.float64) - base
    e, m = rel_fro(got, ref), max_rel(got, ref)
    say(f"  S rel fro {e:.2e}, largest entry {m:.2e}")
    assert e < S_TOL, e
    assert m < s_elem_bar(kind), m


@pytest.mark.parametrize("r,tile", [(64, 0), (256, 1)])
def test_sketch_x_row_stride_past_2_31(lg, r, tile):
    T, d, k = 3, 264, 520
    say("sketch, ldx = 2^31 + 8", T, d, k, r, "tile" if tile else "32-token")
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=11)
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=11)
    X_dev = strided(X, BIG_LD)
    with lg.kernel_choice(lg.CHOICE_PROJECT_TILE, tile):
        _sketch_vs_oracle(lg, X_dev, dY.cuda(), X, dY, r)


def test_sketch_dy_row_stride_at_limit(lg):
    T, d, k, r = 40, 264, 520, 64
    say("sketch, ldd = 2^26 - 8", T, d, k, r)
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=12)
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=12)
    _sketch_vs_oracle(lg, X.cuda(), strided(dY, DY_LD_MAX), X, dY, r)


@pytest.mark.parametrize("T,d,k,r", [
    ((1 << 20) + 5, 256, 256, 16),     # a million tokens: 32769 steps
    (100, 64, (1 << 20) + 8, 64),      # a million input columns: 4097 chunks
    (64, (1 << 18) + 8, 256, 4),       # a quarter-million output rows: 2049 d groups
])
def test_sketch_long_dimensions(lg, T, d, k, r):
    say("sketch, long dimension", T, d, k, r)
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=13)
    dY = synth.host_normal_bf16((T, d), synth.DY_ID, salt=13)
    _sketch_vs_oracle(lg, X.cuda(), dY.cuda(), X, dY, r)


@pytest.mark.parametrize("r", [64, 256])
def test_merge_row_stride_past_2_31(lg, r):
    d, k, alpha, eta = 3, 300, 1.0, 2e-4
    say("merge, ldw = 2^31 + 8", d, k, r)
    W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=14)
    S = synth.host_normal_f32((d, r), synth.S_ID, salt=14, sigma=15.0)
    W = strided(W0, BIG_LD)
    lg.merge(W, S.cuda(), 1234, 0, 0, alpha, eta)
    torch.cuda.synchronize()
    A = oproj.projection(1234, 0, 0, r, k)
    Wb = synth.bf16_bits(W0)
    S64 = S.numpy().astype(np.float64)
    ref = omerge.merged_delta(Wb, S64, A, alpha, eta)
    got = synth.bf16_to_f64(W) - synth.bf16_to_f64(W0)
    e = rel_fro(got, ref)
    ex = w_excess(synth.bf16_bits(W), omerge.merge_bits(Wb, S64, A, alpha, eta), ref)
    say(f"  W delta rel fro {e:.2e}, elementwise excess {ex:.2e}")
    assert e < W_TOL, e
    assert ex <= w_elem_bar(0), ex
    # the padding after each row is not written
    pad = W.as_strided((d, 64), (BIG_LD, 1), W.storage_offset() + k)
    assert torch.isnan(pad.float()).all()


def test_kl_row_stride_past_2_31(lg):
    n, V = 2, 1000
    say("predicted KL, ld = 2^31 + 8", n, V)
    z = synth.host_normal_bf16((n, V), synth.Z_ID, salt=15)
    zp = synth.proposal_logits(z, synth.host_normal_bf16((n, V), synth.DIR_ID, salt=15), 1.0)
    kl_tok = torch.empty(n, device="cuda")
    qa = lg.predicted_kl(strided(z, BIG_LD), strided(zp, BIG_LD), 1.0, 2e-4, 4.0, kl_tok=kl_tok)
    torch.cuda.synchronize()
    ref_rows = okl.kl_rows(synth.bf16_to_f64(z), synth.bf16_to_f64(zp), 1.0)
    q_ref = okl.predicted_kl(synth.bf16_to_f64(z), synth.bf16_to_f64(zp), 1.0)
    rows_err = np.abs(kl_tok.cpu().numpy() / ref_rows - 1).max()
    q_err = abs(qa[0].item() / q_ref - 1)
    say(f"  row rel err {rows_err:.2e}, q rel err {q_err:.2e}")
    assert rows_err < Q_TOL and q_err < Q_TOL
