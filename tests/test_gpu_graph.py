"""Whole optimizer steps captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

No entry point of the library allocates, synchronises or records a memset
(fills are kernels), so a step - a deferred chain of sketch calls over the
microbatches, the merge, the predicted-KL controller - can be captured once
and replayed.  Each replay is checked bit for bit against the same step run
eagerly, with eager work between the replays (W restored, S filled with NaN,
an unrelated sketch call through the same workspace, a host synchronisation),
so that a replay that depended on state left by capture or by the previous
replay would show.  The entry point that allocates nothing is captured the
same way: it is the one meant for callers that capture.
"""
import pytest
import torch

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


def _bits(t):
    return t.contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).clone()


def _noalloc(X, dY, S, seed, stream, kind, flags):
    T, k = X.shape
    d = dY.shape[1]
    st = _lib.lib().logra_sketch_accumulate_noalloc(
        X.data_ptr(), X.stride(0), dY.data_ptr(), dY.stride(0), T, d, k, S.shape[1], seed,
        stream, kind, flags, S.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "logra_sketch_accumulate_noalloc")


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("T,d,k,r,kind,n_mb", [(2048, 1024, 1536, 64, 0, 4),
                                               (1000, 520, 776, 16, 1, 3),
                                               (4096, 4096, 4096, 64, 0, 2)])
def test_step_graph_replays_equal_eager(lg, entry, T, d, k, r, kind, n_mb):
    say("graph step", entry, T, d, k, r, kind, n_mb)
    seed, stream, alpha, eta = 1234, 3, 1.0, 2e-4
    Xs = [synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=d).cuda() for mb in range(n_mb)]
    dYs = [synth.host_normal_bf16((T, d), synth.DY_ID, mb=mb, salt=d).cuda() for mb in range(n_mb)]
    W0 = synth.host_normal_bf16((d, k), synth.W_ID, salt=d).cuda()
    z = synth.host_normal_bf16((64, 4000), synth.Z_ID, salt=d).cuda()
    zp = synth.proposal_logits(z.cpu(), synth.host_normal_bf16((64, 4000), synth.DIR_ID, salt=d),
                               1.0).cuda()
    ws = lg.sketch_workspace(T, d, k, r)
    kl_ws = torch.empty(max(lg.kl_ws_bytes(64, 4000), 256), dtype=torch.uint8, device="cuda")

    def step(S, W, qa):
        # the microbatches' sketches (with a workspace: one deferred chain, the
        # last call writes S; without: the first call overwrites S), then the
        # merge and the controller
        for mb in range(n_mb):
            last = mb == n_mb - 1
            if entry == "workspace":
                lg.sketch_accumulate(Xs[mb], dYs[mb], S, seed, stream, kind, ws=ws,
                                     defer=not last, pending=mb > 0, overwrite=last)
            else:
                # (no deferred chains here: the library's scratch is shared)
                _noalloc(Xs[mb], dYs[mb], S, seed, stream, kind,
                         lg.SKETCH_OVERWRITE if mb == 0 else 0)
        lg.merge(W, S, seed, stream, kind, alpha, eta)
        lg.predicted_kl(z, zp, 1.0, 2e-4, 4.0, out=qa, ws=kl_ws)

    # eager reference
    S_e = torch.full((d, r), float("nan"), device="cuda")
    W_e = W0.clone()
    qa_e = torch.empty(2, device="cuda")
    step(S_e, W_e, qa_e)
    torch.cuda.synchronize()
    ref = (_bits(S_e), _bits(W_e), _bits(qa_e))

    # capture (after a warm-up on a side stream, as torch asks)
    S_g = torch.full((d, r), float("nan"), device="cuda")
    W_g = W0.clone()
    qa_g = torch.empty(2, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(S_g, W_g, qa_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(S_g, W_g, qa_g)
    torch.cuda.synchronize()

    S_other = torch.zeros(d, r, device="cuda")
    for rep in range(4):
        # eager work between replays: restore W, poison S, use the workspace
        W_g.copy_(W0)
        S_g.fill_(float("nan"))
        qa_g.fill_(float("nan"))
        if entry == "workspace":
            lg.sketch_accumulate(Xs[-1], dYs[0], S_other, 7, 0, 0, ws=ws, overwrite=True)
        else:
            _noalloc(Xs[-1], dYs[0], S_other, 7, 0, 0, lg.SKETCH_OVERWRITE)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (_bits(S_g), _bits(W_g), _bits(qa_g))
        for name, a, b in zip(("S", "W", "q/alpha"), got, ref):
            assert torch.equal(a, b), (rep, name)
    del g
