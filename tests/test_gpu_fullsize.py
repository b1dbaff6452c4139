"""Parity at the full sizes of every workload, whole or on sampled outputs.

The d = k = 4096, r = 64 layer (four microbatches of T = 8192) is checked
whole, in the call sequence the benchmark times (the first microbatch with
the overwrite flag on an S full of NaN): all of S and all of the merged W.
The predicted KL over 65536 rows x 152064 vocabulary (the controller
workload, row offsets past 2^31 elements) is checked on sampled rows that
include the first and the last, together with q = the fp64 mean of the
per-row values and the controller's alpha; the sweep over the workload's
four multipliers likewise.  The larger layer shapes run at their full token
counts in the launch configuration the library picks for them, and the
oracle computes a sample of the outputs exactly:
  sketch  every d row of S for eight r columns j (column j of S depends only
          on row j of A), summed over token chunks (the sketch is linear in
          the tokens, a pinned property);
  merge   eight whole rows of W after the merge of the GPU's S.
Bars as everywhere: 2e-3 relative Frobenius error on S and on the merged-W
delta (whole or sampled), with the elementwise bars of tests/parity_bars.py
beside them, and each KL row within 1e-3.  Shapes: one wide layer (d = 5120,
k = 25600, r = 256, T = 16384); the largest projections of the 7B-shaped
layer set (r = 256, T = 32768); 1.5B-shaped projections at r = 4, 16, 64
and 256 with the fixed, per-step-refreshed and Gaussian bases.
"""
import numpy as np
import pytest
import torch

from oracle import bf16 as obf16
from oracle import merge as omerge
from oracle import projection as oproj
from oracle import sketch as osketch
from rank_gradient_sketching_amd import synth

pytestmark = pytest.mark.gpu

from parity_bars import (S_ELEM, S_TOL, W_ELEM, W_TOL, max_rel, rel_fro, s_elem_bar,  # noqa: E402
                         w_elem_bar, w_excess)

CHUNK = 2048


@pytest.fixture(scope="module")
def lg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_gradient_sketching_amd as m
    return m


def say(*a):
    print(*a, flush=True)








def test_fullsize_headline_layer_whole(lg):
    """d = k = 4096, r = 64, four microbatches of T = 8192, fixed sign basis
    from seed 1234, alpha eta = 2e-4: whole S and whole merged W."""
    cfg = synth.WORKLOADS["layer_d4096_r64"]
    d, k, r, T, n_mb = cfg["d"], cfg["k"], cfg["r"], cfg["T"], cfg["n_mb"]
    say("full size headline layer", dict(d=d, k=k, r=r, T=T, n_mb=n_mb))
    A = oproj.projection(cfg["seed"], cfg["stream"], cfg["kind"], r, k)
    S = torch.full((d, r), float("nan"), device="cuda")
    ws = lg.sketch_workspace(T, d, k, r)
    ref = np.zeros((d, r))
    for mb in range(n_mb):
        X = synth.device_normal_bf16((T, k), synth.X_ID, "layer_d4096_r64", mb)
        dY = synth.device_normal_bf16((T, d), synth.DY_ID, "layer_d4096_r64", mb)
        lg.sketch_accumulate(X, dY, S, cfg["seed"], cfg["stream"], cfg["kind"], ws=ws,
                             overwrite=mb == 0)
        ref += osketch.sketch_input_first(synth.bf16_to_f64(X), synth.bf16_to_f64(dY), A)
        del X, dY
    torch.cuda.synchronize()
    got = S.cpu().numpy().astype(np.float64)
    err, elem = rel_fro(got, ref), max_rel(got, ref)
    say("   S rel err", err, "max entry err", elem)
    assert err < S_TOL and elem < S_ELEM, (err, elem)
    W0 = synth.device_normal_bf16((d, k), synth.W_ID, "layer_d4096_r64")
    W = W0.clone()
    lg.merge(W, S, cfg["seed"], cfg["stream"], cfg["kind"], cfg["alpha"], cfg["eta"])
    torch.cuda.synchronize()
    W0b = synth.bf16_bits(W0)
    delta_ref = omerge.merged_delta(W0b, got, A, cfg["alpha"], cfg["eta"])
    delta_got = synth.bf16_to_f64(W) - synth.bf16_to_f64(W0)
    werr = rel_fro(delta_got, delta_ref)
    ex = w_excess(synth.bf16_bits(W), omerge.merge_bits(W0b, got, A, cfg["alpha"], cfg["eta"]),
                  delta_ref)
    say("   W delta rel err", werr, "elementwise excess", ex)
    assert werr < W_TOL and ex <= W_ELEM, (werr, ex)


def test_fullsize_predicted_kl_and_sweep(lg):
    """64 responses x 1024 tokens x vocabulary 152064: z ~ N(0, 3^2), proposal
    z + Delta (Delta ~ N(0, 0.05^2)) rounded to bf16, tau 1, budget 2e-4,
    alpha_max 4; the sweep over alpha in {0.25, 0.5, 1, 2} on (z, Delta)."""
    from oracle import kl as okl
    cfg = synth.WORKLOADS["kl_vocab152064"]
    n, V = cfg["n_resp"] * cfg["resp_len"], cfg["vocab"]
    say("full size predicted KL", n, V)
    z = synth.device_normal_bf16((n, V), synth.Z_ID, "kl_vocab152064")
    dirn = synth.device_normal_bf16((n, V), synth.DIR_ID, "kl_vocab152064")
    zp = synth.proposal_logits(z, dirn, 1.0)
    # the last rows start past 2^31 elements
    assert (n - 1) * V > 2 ** 31
    rows = np.unique(np.concatenate([[0, 1, n // 2, 14122, n - 2, n - 1],
                                     np.linspace(0, n - 1, 10).round()]).astype(np.int64))
    kl_tok = torch.empty(n, device="cuda")
    out = lg.predicted_kl(z, zp, cfg["tau"], cfg["kl_budget"], cfg["alpha_max"], kl_tok=kl_tok)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).cuda()
    ref = okl.kl_rows(synth.bf16_to_f64(z[idx]), synth.bf16_to_f64(zp[idx]), cfg["tau"])
    got = kl_tok[idx].cpu().numpy().astype(np.float64)
    say("   sampled rows", rows.tolist(), "max rel err", float(np.max(np.abs(got / ref - 1))))
    np.testing.assert_allclose(got, ref, rtol=1e-3, atol=1e-9)
    q, alpha = out.cpu().numpy().astype(np.float64)
    q_mean = float(kl_tok.double().mean().item())
    assert abs(q / q_mean - 1) < 1e-6, (q, q_mean)
    a_ref = okl.step_size(q_mean, cfg["kl_budget"], cfg["alpha_max"])
    assert abs(alpha / a_ref - 1) < 1e-6, (alpha, a_ref)
    del zp
    torch.cuda.empty_cache()
    alphas = list(cfg["alphas"])
    sw_tok = torch.empty(len(alphas), n, device="cuda")
    sw = lg.predicted_kl_sweep(z, dirn, alphas, cfg["tau"], kl_tok=sw_tok)
    torch.cuda.synchronize()
    ref_sw = okl.kl_sweep_rows(synth.bf16_to_f64(z[idx]), synth.bf16_to_f64(dirn[idx]), alphas,
                               cfg["tau"])
    got_sw = sw_tok[:, idx].cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got_sw, ref_sw, rtol=1e-3, atol=1e-9)
    means = sw_tok.double().mean(dim=1).cpu().numpy()
    np.testing.assert_allclose(sw.cpu().numpy().astype(np.float64), means, rtol=1e-6)
    del z, dirn, sw_tok, kl_tok
    torch.cuda.empty_cache()


CASES = [
    # label, workload, T, d, k, r, kind, stream, n_mb, seed, merge
    ("wide layer", "kl_vocab152064", 16384, 5120, 25600, 256, 0, 0, 1, 1234, True),
    ("7B down", "qwen7b_layers", 32768, 3584, 18944, 256, 0, 0, 1, 1234 + 27, True),
    ("7B gate", "qwen7b_layers", 32768, 18944, 3584, 256, 0, 0, 1, 1234 + 5, False),
    ("1.5B q r4", "qwen1p5b_layers", 16384, 1536, 1536, 4, 0, 0, 2, 1234, False),
    ("1.5B k r16", "qwen1p5b_layers", 16384, 256, 1536, 16, 0, 0, 2, 1234 + 1, False),
    ("1.5B up r64 refreshed", "qwen1p5b_layers", 16384, 8960, 1536, 64, 0, 2, 2, 1234 + 2, True),
    ("1.5B down r256 Gaussian", "qwen1p5b_layers", 16384, 1536, 8960, 256, 1, 0, 2, 1234 + 3, False),
]


@pytest.mark.parametrize("label,wl,T,d,k,r,kind,stream,n_mb,seed,do_merge", CASES,
                         ids=[c[0] for c in CASES])
def test_fullsize_sketch_and_merge_sampled(lg, label, wl, T, d, k, r, kind, stream, n_mb, seed,
                                           do_merge):
    say("full size", label, dict(T=T, d=d, k=k, r=r, kind=kind, stream=stream, n_mb=n_mb))
    salt = d * 31 + k
    S0 = synth.host_normal_f32((d, r), synth.S_ID, salt=salt, sigma=0.5)
    S = S0.clone().cuda()
    ws = lg.sketch_workspace(T, d, k, r)
    A = oproj.projection(seed, stream, kind, r, k)
    J = np.unique(np.linspace(0, r - 1, min(r, 8)).round().astype(int))
    ref = np.zeros((d, len(J)))
    for mb in range(n_mb):
        X = synth.device_normal_bf16((T, k), synth.X_ID, wl, mb=mb, salt=salt)
        dY = synth.device_normal_bf16((T, d), synth.DY_ID, wl, mb=mb, salt=salt)
        lg.sketch_accumulate(X, dY, S, seed, stream, kind, ws=ws)
        for t0 in range(0, T, CHUNK):
            Xc = X[t0:t0 + CHUNK].float().cpu().numpy()
            dYc = dY[t0:t0 + CHUNK].float().cpu().numpy()
            ref += osketch.sketch_input_first(Xc, dYc, A[J])
        del X, dY
    torch.cuda.synchronize()
    got = S.cpu().numpy().astype(np.float64)[:, J] - S0.numpy().astype(np.float64)[:, J]
    err, elem = rel_fro(got, ref), max_rel(got, ref)
    say("   sampled S columns", J.tolist(), "rel err", err, "max entry err", elem)
    assert err < S_TOL and elem < s_elem_bar(kind), (err, elem)
    if not do_merge:
        return
    W = synth.device_normal_bf16((d, k), synth.W_ID, wl, salt=salt)
    rows = np.unique(np.linspace(0, d - 1, 8).round().astype(int))
    W0 = synth.bf16_bits(W[torch.from_numpy(rows).cuda()])
    lg.merge(W, S, seed, stream, kind, 1.0, 2e-4)
    torch.cuda.synchronize()
    W1 = synth.bf16_bits(W[torch.from_numpy(rows).cuda()])
    Sr = S.cpu().numpy().astype(np.float64)[rows]
    delta_ref = omerge.merged_delta(W0, Sr, A, 1.0, 2e-4)
    delta_got = obf16.bits_to_f64(W1) - obf16.bits_to_f64(W0)
    werr = rel_fro(delta_got, delta_ref)
    ex = w_excess(W1, omerge.merge_bits(W0, Sr, A, 1.0, 2e-4), delta_ref)
    say("   sampled W rows", rows.tolist(), "rel err", werr, "elementwise excess", ex)
    assert werr < W_TOL and ex <= w_elem_bar(kind), (werr, ex)
