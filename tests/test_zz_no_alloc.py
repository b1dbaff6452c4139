"""logra_sketch_accumulate_noalloc through the C ABI against the workspace entry point.

The entry point that allocates nothing runs the same kernels as
logra_sketch_accumulate with the library's own per-GPU scratch in place of
the caller's workspace, so its S must equal the workspace entry point's bit
for bit.  Two calls in a row (the second on a smaller input, which finds the
first call's contents in the shared scratch), the overwrite flag, an empty
microbatch, and a size past the scratch limit (refused with
LOGRA_EWORKSPACE, nothing enqueued).
"""
import numpy as np
import pytest
import torch

from oracle import projection as oproj
from oracle import sketch as osketch
from rank_gradient_sketching_amd import _lib, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_gradient_sketching_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def noalloc(X, dY, S, seed, stream=0, kind=0, flags=0):
    T, k = X.shape
    d = dY.shape[1]
    return _lib.lib().logra_sketch_accumulate_noalloc(
        X.data_ptr(), X.stride(0), dY.data_ptr(), dY.stride(0), T, d, k, S.shape[1], seed,
        stream, kind, flags, S.data_ptr(), _stream())


def _padded(t):
    """GPU copy with the row stride rounded up to a multiple of 8 (NaN padding)."""
    rows, cols = t.shape
    buf = torch.full((rows, -(-cols // 8) * 8), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, :cols] = t.cuda()
    return buf[:, :cols]


def _inputs(T, d, k, salt):
    X = _padded(synth.host_normal_bf16((T, k), synth.X_ID, salt=salt))
    dY = _padded(synth.host_normal_bf16((T, d), synth.DY_ID, salt=salt))
    return X, dY


# (T, d, k, r, kind, flags): the larger call first, then a smaller one
CALLS = [
    (8192, 4096, 4096, 64, 0, 1),   # the d = k = 4096, r = 64 microbatch, overwrite (10.5 MiB)
    (1000, 300, 520, 16, 0, 0),     # ragged and small, accumulate onto S0
    (3000, 1536, 1536, 64, 1, 0),   # Gaussian basis (its bf16 basis also lives in the scratch)
    (77, 1030, 264, 100, 0, 0),     # padded rank, ragged everything
]


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3), (0, 3)])
def test_noalloc_equals_workspace_entry_point_two_calls(lg, first, second):
    for ci in (first, second):
        T, d, k, r, kind, flags = CALLS[ci]
        say("noalloc", dict(T=T, d=d, k=k, r=r, kind=kind, flags=flags))
        assert lg.sketch_ws_bytes(T, d, k, r) <= 32 << 20
        X, dY = _inputs(T, d, k, salt=ci)
        S0 = synth.host_normal_f32((d, r), synth.S_ID, salt=ci).cuda()
        S_ref = S0.clone()
        S_got = S0.clone()
        lg.sketch_accumulate(X, dY, S_ref, 4321, 2, kind, overwrite=bool(flags & 1))
        st = noalloc(X, dY, S_got, 4321, 2, kind, flags)
        assert st == 0, _lib.status_str(st)
        torch.cuda.synchronize()
        assert torch.equal(S_got.view(torch.int32), S_ref.view(torch.int32)), ci
        # and the oracle's value, to the parity bar (2e-3 relative Frobenius)
        if T * (d + k) * r < 3e9:
            A = oproj.projection(4321, 2, kind, r, k)
            base = 0.0 if flags & 1 else S0.cpu().numpy().astype(np.float64)
            ref = osketch.sketch_input_first(synth.bf16_to_f64(X), synth.bf16_to_f64(dY), A)
            got = S_got.cpu().numpy().astype(np.float64) - base
            err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
            assert err < 2e-3, err


def test_noalloc_empty_and_refused(lg):
    say("noalloc edges")
    d, r = 300, 8
    S = torch.full((d, r), float("nan"), device="cuda")
    X = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros(0, d, dtype=torch.bfloat16, device="cuda")
    assert noalloc(X, dY, S, 1, flags=1) == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(S).item() == 0
    # past the scratch limit: refused before anything is enqueued, S untouched
    T, d, k, r = 32768, 3584, 18944, 256
    assert _lib.lib().logra_sketch_ws_bytes(T, d, k, r) > _lib.lib().logra_sketch_ws_bytes(1, 1, 1, 1)
    S = torch.full((d, r), 5.0, device="cuda")
    X = torch.zeros(T, k, dtype=torch.bfloat16, device="cuda")
    dY = torch.zeros(T, d, dtype=torch.bfloat16, device="cuda")
    st = noalloc(X, dY, S, 1)
    assert st == _lib.EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(S == 5.0)
