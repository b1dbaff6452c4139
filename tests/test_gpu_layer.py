"""Parity of the layer-set entry points (through the C ABI) with the oracle.

logra_sketch_accumulate_layer sketches up to four input groups (each an input
X shared by up to four outputs) in one projection and one accumulate launch;
every output is checked against the fp64 oracle, the input-first sketch of
its own group (bars of tests/parity_bars.py), and against the per-group
shared call (the same arithmetic up to fp32 summation order).  Deferred
chains and both kernel choices run through the layer call too.
logra_merge_many merges up to eight weights in one launch and must equal,
bit for bit, one logra_merge per weight (the same tiles and arithmetic).
Shapes: decoder-layer-like group structures (q/k/v, o, gate/up, down) at
sizes the oracle finishes in seconds, with ragged T, k and d.
"""
import numpy as np
import pytest
import torch

from oracle import merge as omerge
from oracle import projection as oproj
from oracle import sketch as osketch
from rank_gradient_sketching_amd import synth

pytestmark = pytest.mark.gpu

from parity_bars import (S_TOL, W_TOL, max_rel, rel_fro, s_elem_bar, w_elem_bar,  # noqa: E402
                         w_excess)


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


def _pad8(n):
    return -(-n // 8) * 8


def _make_layer(T, spec, r, salt, n_mb=1):
    """Host inputs of a layer set: spec = [(k, [d, ...], seed, stream)]; per
    microbatch one X per group and one dY per output, and one S0 per output."""
    mbs = []
    for mb in range(n_mb):
        Xs, dYs = [], []
        for g, (k, ds, _, _) in enumerate(spec):
            Xs.append(synth.host_normal_bf16((T, k), synth.X_ID, mb=mb, salt=salt + 16 * g))
            dYs.append([synth.host_normal_bf16((T, d), synth.DY_ID, mb=mb, salt=salt + 16 * g + o)
                        for o, d in enumerate(ds)])
        mbs.append((Xs, dYs))
    S0 = [[synth.host_normal_f32((d, r), synth.S_ID, mb=o, salt=salt + g) for o, d in enumerate(ds)]
          for g, (_, ds, _, _) in enumerate(spec)]
    return mbs, S0


def _device_groups(spec, Xs, dYs, Ss):
    groups = []
    for g, (k, ds, seed, stream) in enumerate(spec):
        X = padded_bf16(Xs[g], _pad8(k))
        dY = [padded_bf16(y, _pad8(y.shape[1]) + 8) for y in dYs[g]]
        groups.append((X, dY, Ss[g], seed, stream))
    return groups


def _oracle_layer(spec, mbs, S0, kind, r):
    """Per output: S0 + the input-first sketch of every microbatch."""
    ref = []
    for g, (k, ds, seed, stream) in enumerate(spec):
        A = oproj.projection(seed, stream, kind, r, k)
        row = []
        for o in range(len(ds)):
            pairs = [(synth.bf16_to_f64(Xs[g]), synth.bf16_to_f64(dYs[g][o])) for Xs, dYs in mbs]
            row.append(osketch.accumulate(S0[g][o].numpy().astype(np.float64), pairs, A))
        ref.append(row)
    return ref


def _check(got, ref, S0, kind, what):
    for g in range(len(ref)):
        for o in range(len(ref[g])):
            base = S0[g][o].numpy().astype(np.float64)
            x = got[g][o].cpu().numpy().astype(np.float64)
            err, elem = rel_fro(x - base, ref[g][o] - base), max_rel(x - base, ref[g][o] - base)
            assert err < S_TOL and elem < s_elem_bar(kind), (what, g, o, err, elem)


# (T, groups [(k, [d...], seed, stream)], r, kind).  The first is a decoder
# layer's structure: q/k/v on one input, o, gate/up on one input, down.
LAYER_CASES = [
    (1000, [(320, [200, 40, 40], 1234, 0), (320, [136], 1234, 0), (320, [500, 500], 1234, 0),
            (1000, [77], 1234, 0)], 64, 0),
    (1000, [(320, [200, 40, 40], 1234, 0), (320, [136], 1234, 0), (320, [500, 500], 1234, 0),
            (1000, [77], 1234, 0)], 64, 1),
    (2048, [(512, [256, 128], 7, 0), (768, [300], 8, 3)], 4, 0),
    (4096, [(256, [384, 64, 64], 11, 0), (1024, [256], 12, 1), (256, [640, 640], 11, 0)], 16, 0),
    (777, [(300, [129, 33], 5, 2), (520, [1000], 6, 2), (264, [17], 9, 0), (1500, [250, 250, 8, 300], 10, 1)],
     3, 0),
    (3000, [(512, [256, 256], 21, 0), (1536, [384], 22, 0)], 128, 0),
    (1024, [(300, [520, 64], 31, 0), (700, [200], 32, 0), (256, [96], 33, 1)], 256, 1),
    (16384, [(256, [128, 64, 64], 41, 0), (256, [128], 41, 0), (256, [384, 384], 41, 0),
             (768, [128], 41, 0)], 64, 0),
]


@pytest.mark.parametrize("T,spec,r,kind", LAYER_CASES)
def test_sketch_layer_matches_oracle_and_shared_calls(lg, T, spec, r, kind):
    say("sketch layer", T, spec, r, kind)
    salt = 97 * len(spec) + r
    mbs, S0 = _make_layer(T, spec, r, salt)
    Xs, dYs = mbs[0]
    Ss = [[s.clone().cuda() for s in row] for row in S0]
    groups = _device_groups(spec, Xs, dYs, Ss)
    lg.sketch_accumulate_layer(groups, kind)
    shared = [[s.clone().cuda() for s in row] for row in S0]
    for g, (X, dY, _, seed, stream) in enumerate(groups):
        lg.sketch_accumulate_shared(X, dY, shared[g], seed, stream, kind)
    torch.cuda.synchronize()
    ref = _oracle_layer(spec, mbs, S0, kind, r)
    _check(Ss, ref, S0, kind, "layer")
    for g in range(len(spec)):
        for o in range(len(spec[g][1])):
            base = S0[g][o].numpy().astype(np.float64)
            a = Ss[g][o].cpu().numpy().astype(np.float64)
            b = shared[g][o].cpu().numpy().astype(np.float64)
            assert rel_fro(a - base, b - base) < 1e-5, (g, o)


@pytest.mark.parametrize("project_tile", [0, 1, 2])
@pytest.mark.parametrize("acc_wide", [0, 1])
def test_sketch_layer_both_kernel_choices(lg, project_tile, acc_wide):
    """The group table through project_kernel and both forms of
    project_tile_kernel (64 and 128 tokens), the per-output P through
    accumulate_kernel and accumulate_wide_kernel."""
    T, r, kind = 2080, 128, 0
    spec = [(520, [300, 136], 3, 0), (256, [64], 4, 1), (1024, [520], 5, 0)]
    say("sketch layer kernel choice", project_tile, acc_wide)
    mbs, S0 = _make_layer(T, spec, r, 555)
    Ss = [[s.clone().cuda() for s in row] for row in S0]
    groups = _device_groups(spec, mbs[0][0], mbs[0][1], Ss)
    with lg.kernel_choice(lg.CHOICE_PROJECT_TILE, project_tile), \
            lg.kernel_choice(lg.CHOICE_ACC_WIDE, acc_wide):
        lg.sketch_accumulate_layer(groups, kind)
        torch.cuda.synchronize()
    _check(Ss, _oracle_layer(spec, mbs, S0, kind, r), S0, kind, "choice")


@pytest.mark.parametrize("r,kind", [(64, 0), (256, 1), (16, 0)])
def test_sketch_layer_deferred_chain(lg, r, kind):
    """Three microbatches: DEFER, DEFER | PENDING, PENDING | OVERWRITE on S
    full of NaN: S = the sum of the three sketches."""
    T = 1056
    spec = [(320, [200, 40, 40], 1234, 0), (320, [136], 1234, 0), (1000, [77], 1234, 0)]
    say("sketch layer deferred chain", r, kind)
    mbs, S0 = _make_layer(T, spec, r, 777, n_mb=3)
    zeros = [[torch.zeros_like(s) for s in row] for row in S0]
    Ss = [[torch.full_like(s, float("nan")).cuda() for s in row] for row in S0]
    ws = lg.sketch_layer_workspace(T, r, [(k, ds) for k, ds, _, _ in spec])
    for mb, (Xs, dYs) in enumerate(mbs):
        last = mb == len(mbs) - 1
        groups = _device_groups(spec, Xs, dYs, Ss)
        lg.sketch_accumulate_layer(groups, kind, ws=ws, defer=not last, pending=mb > 0,
                                   overwrite=last)
    torch.cuda.synchronize()
    _check(Ss, _oracle_layer(spec, mbs, zeros, kind, r), zeros, kind, "chain")


def test_sketch_layer_one_group_is_the_shared_call_bitwise(lg):
    T, k, ds, r = 2048, 512, [384, 128], 64
    X = synth.host_normal_bf16((T, k), synth.X_ID, salt=6).cuda()
    dY = [synth.host_normal_bf16((T, d), synth.DY_ID, salt=6 + o).cuda() for o, d in enumerate(ds)]
    a = [torch.zeros(d, r, device="cuda") for d in ds]
    b = [torch.zeros(d, r, device="cuda") for d in ds]
    lg.sketch_accumulate_shared(X, dY, a, 99, 2)
    lg.sketch_accumulate_layer([(X, dY, b, 99, 2)])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_sketch_layer_overwrite_empty_microbatch_zeroes_every_S(lg):
    r = 16
    spec = [(256, [64, 32], 1, 0), (512, [128], 2, 0)]
    Ss = [[torch.full((d, r), 5.0, device="cuda") for d in ds] for _, ds, _, _ in spec]
    groups = [(torch.empty(0, k, dtype=torch.bfloat16, device="cuda"),
               [torch.empty(0, d, dtype=torch.bfloat16, device="cuda") for d in ds], Ss[g], seed,
               stream) for g, (k, ds, seed, stream) in enumerate(spec)]
    lg.sketch_accumulate_layer(groups, overwrite=True)
    torch.cuda.synchronize()
    for row in Ss:
        for s in row:
            assert torch.count_nonzero(s).item() == 0


# (weights [(d, k, seed, stream)], r, kind)
MERGE_MANY_CASES = [
    ([(1536, 1536, 1234, 0), (256, 1536, 1234, 0), (256, 1536, 1234, 0), (1536, 1536, 1234, 0),
      (1000, 1536, 1234, 0), (1000, 1536, 1234, 0), (1536, 1000, 1234, 0)], 64, 0),
    ([(300, 520, 5, 1), (129, 264, 6, 0), (64, 4100, 7, 2)], 3, 0),
    ([(512, 768, 8, 0), (300, 1000, 9, 1)], 64, 1),
    ([(256, 512, 10, 0), (520, 300, 11, 0), (128, 256, 12, 3)], 256, 0),
    ([(384, 640, 13, 0), (200, 256, 14, 0)], 128, 1),
    ([(1, 1, 15, 0)], 1, 0),
]


@pytest.mark.parametrize("items,r,kind", MERGE_MANY_CASES)
def test_merge_many_is_single_merges_bitwise_and_matches_oracle(lg, items, r, kind):
    say("merge many", items, r, kind)
    alpha, eta = 0.75, 3e-3
    W0 = [synth.host_normal_bf16((d, k), synth.W_ID, salt=7 * i + d) for i, (d, k, _, _) in
          enumerate(items)]
    S = [synth.host_normal_f32((d, r), synth.S_ID, mb=i, salt=k, sigma=0.5) for i, (d, k, _, _) in
         enumerate(items)]
    Wm = [padded_bf16(w, _pad8(w.shape[1]) + (8 if i % 2 else 0)) for i, w in enumerate(W0)]
    Ws = [padded_bf16(w, _pad8(w.shape[1])) for w in W0]
    Sd = [s.cuda() for s in S]
    lg.merge_many([(Wm[i], Sd[i], seed, stream) for i, (_, _, seed, stream) in enumerate(items)],
                  kind, alpha, eta)
    for i, (_, _, seed, stream) in enumerate(items):
        lg.merge(Ws[i], Sd[i], seed, stream, kind, alpha, eta)
    torch.cuda.synchronize()
    for i, (d, k, seed, stream) in enumerate(items):
        a, b = synth.bf16_bits(Wm[i]), synth.bf16_bits(Ws[i])
        assert np.array_equal(a, b), i
        A = oproj.projection(seed, stream, kind, r, k)
        W0b = synth.bf16_bits(W0[i])
        Sf = S[i].numpy().astype(np.float64)
        delta_ref = omerge.merged_delta(W0b, Sf, A, alpha, eta)
        delta_got = synth.bf16_to_f64(Wm[i]) - synth.bf16_to_f64(W0[i])
        assert rel_fro(delta_got, delta_ref) < W_TOL, i
        assert w_excess(a, omerge.merge_bits(W0b, Sf, A, alpha, eta), delta_ref) <= w_elem_bar(kind), i
