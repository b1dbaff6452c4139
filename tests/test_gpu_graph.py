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


@pytest.mark.parametrize("r,kind", [(64, 0), (16, 1)])
def test_layer_step_graph_replays_equal_eager(lg, r, kind):
    """A decoder layer's step (q/k/v, o, gate/up, down: four input groups,
    seven outputs) as one deferred chain of layer calls and one grouped merge."""
    say("graph layer step", r, kind)
    T, n_mb, h, kv, mlp = 1040, 2, 384, 64, 1000
    shapes = {"q": (h, h), "k": (kv, h), "v": (kv, h), "o": (h, h), "gate": (mlp, h),
              "up": (mlp, h), "down": (h, mlp)}          # (d, k) per projection
    groups_of = [("qkv", ["q", "k", "v"], h), ("o", ["o"], h), ("gu", ["gate", "up"], h),
                 ("down", ["down"], mlp)]
    seed, stream = 77, 2
    X = {(g, mb): synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=len(g) * 7 + k).cuda()
         for g, _, k in groups_of for mb in range(n_mb)}
    dY = {(p, mb): synth.host_normal_bf16((T, shapes[p][0]), synth.DY_ID, mb=mb,
                                          salt=shapes[p][0] + len(p)).cuda()
          for p in shapes for mb in range(n_mb)}
    W0 = {p: synth.host_normal_bf16(shapes[p], synth.W_ID, salt=len(p)).cuda() for p in shapes}
    spec = [(X[(g, 0)], [dY[(p, 0)] for p in ps], [None] * len(ps), seed + i, stream)
            for i, (g, ps, _) in enumerate(groups_of)]
    ws = lg.sketch_layer_workspace(T, r, [(x.shape[1], [t.shape[1] for t in dys])
                                          for x, dys, _, _, _ in spec])

    def step(S, W):
        for mb in range(n_mb):
            last = mb == n_mb - 1
            groups = [(X[(g, mb)], [dY[(p, mb)] for p in ps], [S[p] for p in ps], seed + i, stream)
                      for i, (g, ps, _) in enumerate(groups_of)]
            lg.sketch_accumulate_layer(groups, kind, ws=ws, defer=not last, pending=mb > 0,
                                       overwrite=last)
        items = [(W[p], S[p], seed + i, stream) for i, (g, ps, _) in enumerate(groups_of)
                 for p in ps]
        lg.merge_many(items, kind, 1.0, 2e-4)

    def fresh():
        return ({p: torch.full((shapes[p][0], r), float("nan"), device="cuda") for p in shapes},
                {p: W0[p].clone() for p in shapes})

    S_e, W_e = fresh()
    step(S_e, W_e)
    torch.cuda.synchronize()
    ref = {p: (_bits(S_e[p]), _bits(W_e[p])) for p in shapes}

    S_g, W_g = fresh()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(S_g, W_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(S_g, W_g)
    torch.cuda.synchronize()
    for rep in range(3):
        for p in shapes:
            W_g[p].copy_(W0[p])
            S_g[p].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for p in shapes:
            assert torch.equal(_bits(S_g[p]), ref[p][0]), (rep, p, "S")
            assert torch.equal(_bits(W_g[p]), ref[p][1]), (rep, p, "W")
    del g
