"""Benchmark of the LoGRA hot path on one MI355X.

A step is one pass of the path over one batch of the d = k = 4096, r = 64
layer: four microbatches of T = 8192 tokens are sketched into S
(logra_sketch_accumulate, which regenerates the sign basis in registers, as
one deferred chain: the first three calls keep their contributions in the
workspace and the fourth writes S, so the split reduction runs once per step)
and the rank-64 update is merged into the bf16 weights (logra_merge,
alpha * eta = 2e-4).  Inputs are synthetic, seeded, generated on the GPU and
resident in HBM before the timed region; consecutive steps take two
different sets of four microbatches (1 GiB in all), so that no input is
re-read from the 256 MB Infinity Cache (with one set, a step's dY was partly
still there a step later: X is read non-temporally and does not displace it).

Printed: one JSON line.  `value` is tokens sketched and merged per second for
the whole step.  Extra objects report the sketch and merge bandwidth against
the 8 TB/s HBM peak, the roofline of the dominant entry point (its calls
run back to back after the timed steps, one event pair around the batch on
the library's stream), full-size parity against the CPU oracle,
the predicted-KL leg at 64 x 1024 rows x 152064 vocab, and the CPU oracle's
own throughput on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-kl] [--no-cpu]
"""
import argparse
import gc
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sketch-accumulate tokens/s + merge GB/s at d=k=4096,r=64; % of HBM peak"
WORKLOAD = "layer_d4096_r64"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sketch_bytes(T, d, k, r):
    """Algorithmic bytes of one sketch call: X and dY once, S read + write."""
    return 2 * T * (d + k) + 8 * d * r


def chain_bytes(T, d, k, r, n_mb):
    """Algorithmic bytes of a deferred chain of n_mb sketch calls that ends with
    the overwrite flag: X and dY of every microbatch once, S written once."""
    return n_mb * 2 * T * (d + k) + 4 * d * r


BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix cores


def sketch_mfma(T, d, k, r, us):
    """Matrix-core rate of one sketch call: algorithmic FLOP 2 T r (k + d) (the
    projection and the contraction), executed 2 T r (k + 2 d) (P enters the
    contraction as a hi/lo bf16 pair), over the call time."""
    alg = 2.0 * T * r * (k + d)
    exe = 2.0 * T * r * (k + 2 * d)
    t = us * 1e-6
    return dict(TFLOPs_algorithmic=alg / t / 1e12, TFLOPs_executed=exe / t / 1e12,
                frac_bf16_mfma_peak=exe / t / 1e12 / BF16_MFMA_PEAK_TFLOPS)


def merge_bytes(d, k, r):
    """Algorithmic bytes of one merge: W read + write, S read once."""
    return 4 * d * k + 4 * d * r


class Timer:
    """Pairs of events on the current stream around repeated launches."""

    def __init__(self):
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append([e, None])

    def stop(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[-1][1] = e

    def times_ms(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def run_layer(lg, synth, steps, warmup):
    cfg = synth.WORKLOADS[WORKLOAD]
    d, k, r, T, n_mb = cfg["d"], cfg["k"], cfg["r"], cfg["T"], cfg["n_mb"]
    seed, stream, kind, alpha, eta = cfg["seed"], cfg["stream"], cfg["kind"], cfg["alpha"], cfg["eta"]
    # Two sets of the step's microbatches, used by alternate steps: X is read
    # non-temporally and does not stay in the 256 MB Infinity Cache, so with
    # one set the 4 x 64 MiB of dY came back a step later partly from that
    # cache (measured: 155 us per step with one set, 166 us with two or
    # three); with two sets 448 MiB of other dY pass between two uses of a
    # buffer.  Every step still sketches n_mb microbatches of T tokens.
    n_sets = 2 * n_mb
    log(f"[bench] generating {WORKLOAD}: {n_mb} x T={T}, d=k={d}, r={r} ({n_sets} buffer sets)")
    Xs = [synth.device_normal_bf16((T, k), synth.X_ID, WORKLOAD, mb) for mb in range(n_sets)]
    dYs = [synth.device_normal_bf16((T, d), synth.DY_ID, WORKLOAD, mb) for mb in range(n_sets)]
    W0 = synth.device_normal_bf16((d, k), synth.W_ID, WORKLOAD)
    W = W0.clone()
    S = torch.zeros(d, r, device="cuda")
    ws = lg.sketch_workspace(T, d, k, r)
    torch.cuda.synchronize()

    # ---- full-size parity of one step against the CPU oracle (S starts as
    # NaN: the first microbatch overwrites it, as in the timed steps)
    log("[bench] parity step")
    S.fill_(float("nan"))

    def sketch_chain(half=0):
        # one deferred chain over a step's microbatches (buffer set `half`):
        # S written by the last call
        for mb in range(n_mb):
            last = mb == n_mb - 1
            X, dY = Xs[half * n_mb + mb], dYs[half * n_mb + mb]
            lg.sketch_accumulate(X, dY, S, seed, stream, kind, ws=ws, defer=not last,
                                 pending=mb > 0, overwrite=last)

    sketch_chain(0)
    lg.merge(W, S, seed, stream, kind, alpha, eta)
    torch.cuda.synchronize()
    parity = check_layer_parity(synth, Xs[:n_mb], dYs[:n_mb], W0, W, S, cfg)
    log(f"[bench] parity {parity}")

    # ---- timed steps: back to back, one event pair around all of them (an
    # event recorded between calls would sit inside the step); step i takes
    # buffer set i % 2
    def one_step(half):
        # the chain's last call stores S (overwrite): no separate zero fill
        sketch_chain(half)
        lg.merge(W, S, seed, stream, kind, alpha, eta)

    for i in range(warmup):
        one_step(i % 2)
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        one_step(i % 2)
    t1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3
    total_ms = t0.elapsed_time(t1)
    step_ms = total_ms / steps

    # the same steps captured once in a HIP graph and replayed (no entry point
    # allocates or records a memset, so the whole step captures): two steps
    # per graph, one on each buffer set; reported beside the eager figure,
    # which is `value`
    def two_steps():
        one_step(0)
        one_step(1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        two_steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        two_steps()
    graph_step_ms = _time_ms(graph.replay, max(steps // 10, 4)) / 2
    del graph

    # ---- average duration of each entry point: the same calls back to back
    # (sketches cycling over both buffer sets, merges over copies of W), one
    # event pair around each batch, outside the timed steps
    reps = max(steps, 20)

    def batch_us(fn, n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    # five batches each; the median batch mean is the figure, the minimum is
    # reported beside it
    sk_b = [batch_us(lambda i: lg.sketch_accumulate(Xs[i % n_sets], dYs[i % n_sets], S, seed,
                                                    stream, kind, ws=ws), reps * n_mb)
            for _ in range(5)]
    # whole deferred chains back to back, alternating buffer sets (per call:
    # the chain's time / n_mb)
    ch_b = [batch_us(lambda i: sketch_chain(i % 2), reps) / n_mb for _ in range(5)]
    # merges cycle over at least 16 copies of W, 512 MiB in all: twice the
    # 256 MB Infinity Cache, as inside a step (where W was last touched a
    # step earlier); one W repeated would be served from that cache
    n_w = max(16, -(-(512 << 20) // (2 * d * k)))
    Wc = [W.clone() for _ in range(n_w)]
    mg_b = [batch_us(lambda i: lg.merge(Wc[i % n_w], S, seed, stream, kind, alpha, eta),
                     max(reps, n_w)) for _ in range(5)]
    del Wc
    sk_us, mg_us = float(np.median(sk_b)), float(np.median(mg_b))
    ch_us = float(np.median(ch_b))
    sb = sketch_bytes(T, d, k, r)
    cb = chain_bytes(T, d, k, r, n_mb) / n_mb
    mb_ = merge_bytes(d, k, r)
    res = dict(
        cfg=cfg, total_ms=total_ms, step_ms=step_ms, wall_ms=wall_ms, graph_step_ms=graph_step_ms,
        tokens_per_step=T * n_mb,
        sketch=dict(us_per_call=sk_us, us_min=min(sk_b), bytes_per_call=sb,
                    GBps=sb / (sk_us * 1e-6) / 1e9,
                    tokens_per_s=T / (sk_us * 1e-6)),
        chain=dict(us_per_call=ch_us, us_min=min(ch_b), bytes_per_call=cb,
                   GBps=cb / (ch_us * 1e-6) / 1e9, tokens_per_s=T / (ch_us * 1e-6)),
        merge=dict(us_per_call=mg_us, us_min=min(mg_b), bytes_per_call=mb_,
                   GBps=mb_ / (mg_us * 1e-6) / 1e9),
        parity=parity)
    res["sketch"]["frac_hbm"] = res["sketch"]["GBps"] / HBM_PEAK_GBPS
    res["chain"]["frac_hbm"] = res["chain"]["GBps"] / HBM_PEAK_GBPS
    res["merge"]["frac_hbm"] = res["merge"]["GBps"] / HBM_PEAK_GBPS
    return res, (Xs[:n_mb], dYs[:n_mb], W0, cfg)


def check_layer_parity(synth, Xs, dYs, W0, W, S, cfg):
    from oracle import bf16 as obf16
    from oracle import merge as omerge
    from oracle import projection as oproj
    d, k, r = cfg["d"], cfg["k"], cfg["r"]
    A = oproj.projection(cfg["seed"], cfg["stream"], cfg["kind"], r, k)
    S_ref = np.zeros((d, r))
    for X, dY in zip(Xs, dYs):
        P = synth.bf16_to_f64(X) @ A.T
        S_ref += synth.bf16_to_f64(dY).T @ P
    S_got = S.cpu().numpy().astype(np.float64)
    s_err = float(np.linalg.norm(S_got - S_ref) / np.linalg.norm(S_ref))
    s_elem = float(np.abs(S_got - S_ref).max() / np.abs(S_ref).max())
    W0b = synth.bf16_bits(W0)
    ref_delta = omerge.merged_delta(W0b, S_got, A, cfg["alpha"], cfg["eta"])
    got_delta = synth.bf16_to_f64(W) - synth.bf16_to_f64(W0)
    w_err = float(np.linalg.norm(got_delta - ref_delta) / np.linalg.norm(ref_delta))

    # elementwise: each merged element within one bf16 spacing of the
    # oracle's, plus 1e-4 of the largest delta (where W - alpha eta S A
    # cancels to nearly zero, the fp32/fp64 difference of S A is what is left)
    a = synth.bf16_to_f64(W)
    b = obf16.bits_to_f64(omerge.merge_bits(W0b, S_got, A, cfg["alpha"], cfg["eta"]))
    m = np.maximum(np.abs(a), np.abs(b))
    spacing = np.where(m > 0, np.ldexp(1.0, np.frexp(m)[1] - 8), 0.0)
    w_elem = float(np.maximum(np.abs(a - b) - spacing, 0.0).max() / np.abs(ref_delta).max())
    return dict(S_rel_fro=s_err, S_max_entry_rel=s_elem, W_delta_rel_fro=w_err,
                W_entry_excess=w_elem, S_tol=2e-3, S_entry_tol=1e-4, W_tol=2e-3,
                W_entry_tol=1e-4,
                ok=bool(s_err < 2e-3 and s_elem < 1e-4 and w_err < 2e-3 and w_elem <= 1e-4))


def run_kl(lg, synth, reps=5):
    cfg = synth.WORKLOADS["kl_vocab152064"]
    n = cfg["n_resp"] * cfg["resp_len"]
    V = cfg["vocab"]
    log(f"[bench] generating KL logits {n} x {V}")
    z = synth.device_normal_bf16((n, V), synth.Z_ID, "kl_vocab152064")
    dirn = synth.device_normal_bf16((n, V), synth.DIR_ID, "kl_vocab152064")
    zp = synth.proposal_logits(z, dirn, 1.0)
    kl_tok = torch.empty(n, device="cuda")
    out = torch.empty(2, device="cuda")
    lg.predicted_kl(z, zp, cfg["tau"], cfg["kl_budget"], cfg["alpha_max"], out=out, kl_tok=kl_tok)
    torch.cuda.synchronize()
    tm = Timer()
    for _ in range(reps):
        tm.start()
        lg.predicted_kl(z, zp, cfg["tau"], cfg["kl_budget"], cfg["alpha_max"], out=out, kl_tok=kl_tok)
        tm.stop()
    torch.cuda.synchronize()
    ms = float(np.mean(tm.times_ms()))
    nbytes = 2 * 2 * n * V
    q, alpha = out.cpu().tolist()
    # sampled rows against the oracle, and q = mean of the per-row values
    from oracle import kl as okl
    rows = np.linspace(0, n - 1, 16).astype(np.int64)
    ref = okl.kl_rows(synth.bf16_to_f64(z[rows]), synth.bf16_to_f64(zp[rows]), cfg["tau"])
    got = kl_tok[rows].cpu().numpy().astype(np.float64)
    row_err = float(np.max(np.abs(got / ref - 1)))
    q_mean = float(kl_tok.double().mean().item())
    res = dict(rows=n, vocab=V, ms=ms, bytes=nbytes, GBps=nbytes / (ms * 1e-3) / 1e9,
               q=q, alpha=alpha, sampled_row_max_rel_err=row_err,
               q_vs_row_mean_rel=abs(q / q_mean - 1))
    res["frac_hbm"] = res["GBps"] / HBM_PEAK_GBPS
    del zp
    res["sweep"] = run_kl_sweep(lg, synth, cfg, z, dirn, rows, reps, ms)
    del z, dirn
    torch.cuda.empty_cache()
    return res


def run_kl_sweep(lg, synth, cfg, z, dirn, rows, reps, ms_single):
    """Direction-form sweep over the controller workload's multipliers: one
    pass over (z, delta) for all of them; sampled rows against the oracle."""
    alphas = list(cfg["alphas"])
    n = z.shape[0]
    out = torch.empty(len(alphas), device="cuda")
    kl_tok = torch.empty(len(alphas), n, device="cuda")
    lg.predicted_kl_sweep(z, dirn, alphas, cfg["tau"], out=out, kl_tok=kl_tok)
    torch.cuda.synchronize()
    tm = Timer()
    for _ in range(reps):
        tm.start()
        lg.predicted_kl_sweep(z, dirn, alphas, cfg["tau"], out=out, kl_tok=kl_tok)
        tm.stop()
    torch.cuda.synchronize()
    ms = float(np.mean(tm.times_ms()))
    nbytes = 2 * 2 * n * z.shape[1]
    from oracle import kl as okl
    ref = okl.kl_sweep_rows(synth.bf16_to_f64(z[rows]), synth.bf16_to_f64(dirn[rows]), alphas,
                            cfg["tau"])
    got = kl_tok[:, rows].cpu().numpy().astype(np.float64)
    kl = out.cpu().numpy().astype(np.float64)
    res = dict(alphas=alphas, ms=ms, bytes=nbytes, GBps=nbytes / (ms * 1e-3) / 1e9,
               kl=kl.tolist(), kl_over_alpha2=(kl / np.array(alphas) ** 2).tolist(),
               sampled_row_max_rel_err=float(np.max(np.abs(got / ref - 1))),
               speedup_vs_one_call_per_alpha=len(alphas) * ms_single / ms)
    res["frac_hbm"] = res["GBps"] / HBM_PEAK_GBPS
    return res


def run_layer_set(lg, synth, reps=10, r=64):
    """One decoder layer of the 1.5B-shaped layer set (hidden 1536, KV 256, MLP
    8960) at T = 16384, r = 64: the seven projections sketched with one call
    each, against q/k/v and gate/up sharing their input and A (four calls).
    Same inputs and accumulators; the two results are compared."""
    cfg = synth.QWEN1P5B
    T = cfg["T"]
    wl = "qwen1p5b_layers"
    proj = {n: (d, k) for n, d, k in cfg["projections"]}
    groups = [("attn", ["q", "k", "v"]), ("o", ["o"]), ("mlp", ["gate", "up"]), ("down", ["down"])]
    log(f"[bench] generating one 1.5B-shaped layer at T = {T}")
    X = {g: synth.device_normal_bf16((T, proj[names[0]][1]), synth.X_ID, wl, salt=gi)
         for gi, (g, names) in enumerate(groups)}
    dY = {n: synth.device_normal_bf16((T, proj[n][0]), synth.DY_ID, wl, salt=i)
          for i, n in enumerate(proj)}
    S_sep = {n: torch.zeros(proj[n][0], r, device="cuda") for n in proj}
    S_sh = {n: torch.zeros(proj[n][0], r, device="cuda") for n in proj}
    seed = 1234
    ws_sep = {n: lg.sketch_workspace(T, proj[n][0], proj[n][1], r) for n in proj}
    ws_sh = {}
    for g, names in groups:
        n_b = lg.sketch_shared_ws_bytes(T, proj[names[0]][1], r, [proj[n][0] for n in names])
        ws_sh[g] = torch.empty(max(n_b, 256), dtype=torch.uint8, device="cuda")

    def separate():
        for g, names in groups:
            for n in names:
                lg.sketch_accumulate(X[g], dY[n], S_sep[n], seed, ws=ws_sep[n])

    def shared():
        for g, names in groups:
            lg.sketch_accumulate_shared(X[g], [dY[n] for n in names], [S_sh[n] for n in names],
                                        seed, ws=ws_sh[g])

    S_ly = {n: torch.zeros(proj[n][0], r, device="cuda") for n in proj}
    ws_ly = lg.sketch_layer_workspace(T, r, [(proj[names[0]][1], [proj[n][0] for n in names])
                                             for _, names in groups])

    def layer():
        lg.sketch_accumulate_layer([(X[g], [dY[n] for n in names], [S_ly[n] for n in names], seed, 0)
                                    for g, names in groups], ws=ws_ly)

    separate()
    shared()
    layer()
    torch.cuda.synchronize()
    def rel_fro(a, b):
        a, b = a.astype(np.float64), b.astype(np.float64)
        return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))

    err = max(rel_fro(S_sh[n].cpu().numpy(), S_sep[n].cpu().numpy()) for n in proj)
    err_ly = max(rel_fro(S_ly[n].cpu().numpy(), S_sep[n].cpu().numpy()) for n in proj)
    times = {}
    for name, fn in (("separate", separate), ("shared", shared), ("layer", layer)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        times[name] = t0.elapsed_time(t1) / reps
    b_sep = sum(2 * T * (proj[n][0] + proj[n][1]) + 8 * proj[n][0] * r for n in proj)
    b_sh = sum(2 * T * proj[names[0]][1] for _, names in groups) + \
        sum(2 * T * proj[n][0] + 8 * proj[n][0] * r for n in proj)
    res = dict(workload="qwen1p5b_layers (one layer, 7 projections)", T=T, r=r,
               us_separate=times["separate"] * 1e3, us_shared=times["shared"] * 1e3,
               tokens_per_s_separate=T / (times["separate"] * 1e-3),
               tokens_per_s_shared=T / (times["shared"] * 1e-3),
               bytes_separate=b_sep, bytes_shared=b_sh,
               GBps_separate=b_sep / (times["separate"] * 1e-3) / 1e9,
               GBps_shared=b_sh / (times["shared"] * 1e-3) / 1e9,
               speedup=times["separate"] / times["shared"],
               shared_vs_separate_rel_fro=err,
               us_layer_call=times["layer"] * 1e3,
               GBps_layer_call=b_sh / (times["layer"] * 1e-3) / 1e9,
               speedup_layer_call=times["separate"] / times["layer"],
               layer_vs_separate_rel_fro=err_ly)
    del X, dY, ws_sep, ws_sh, ws_ly
    torch.cuda.empty_cache()
    return res


def _time_ms(fn, reps, batches=5):
    """Median over `batches` of the mean time of `reps` back-to-back calls, one
    event pair per batch: a host stall that lets the GPU run dry moves one
    batch, not the figure."""
    fn()
    torch.cuda.synchronize()
    per = []
    for _ in range(batches):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) / reps)
    return float(np.median(per))


def _layer_set_step(lg, synth, wl, cfg, r, kind, stream, n_mb, n_layers=2, fused=True):
    """n_layers distinct decoder layers of a layer-set workload (own buffers; A
    from seed 1234 + layer, as the workload states), one optimizer step each:
    every projection sketched over n_mb microbatches as one deferred chain
    (q/k/v and gate/up share their input), then merged.  fused: one layer call
    per microbatch (all four input groups in one projection and one accumulate
    launch) and one merge call for the seven weights; else one shared call per
    input group and one merge per weight.  The microbatches reuse one set of
    tensors per layer (each is either far above the Infinity Cache or evicted
    by the layer's other tensors before its next use).  Returns (fn,
    algorithmic bytes, algorithmic FLOPs, tokens) for the n_layers layers."""
    T = cfg["T"]
    proj = {n: (d, k) for n, d, k in cfg["projections"]}
    groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
    layers = []
    for layer in range(n_layers):
        X = [synth.device_normal_bf16((T, proj[g[0]][1]), synth.X_ID, wl, salt=16 * layer + gi)
             for gi, g in enumerate(groups)]
        dY = {n: synth.device_normal_bf16((T, proj[n][0]), synth.DY_ID, wl, salt=16 * layer + i)
              for i, n in enumerate(proj)}
        W = {n: synth.device_normal_bf16(proj[n], synth.W_ID, wl, salt=16 * layer + i)
             for i, n in enumerate(proj)}
        S = {n: torch.zeros(proj[n][0], r, device="cuda") for n in proj}
        if fused:
            ws = lg.sketch_layer_workspace(T, r, [(proj[g[0]][1], [proj[n][0] for n in g])
                                                  for g in groups])
        else:
            ws = []
            for g in groups:
                nb = lg.sketch_shared_ws_bytes(T, proj[g[0]][1], r, [proj[n][0] for n in g])
                ws.append(torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda"))
        layers.append((1234 + layer, X, dY, W, S, ws))

    def step():
        for seed, X, dY, W, S, ws in layers:
            # one deferred chain per layer (or per input group): the last
            # microbatch stores S
            for mb in range(n_mb):
                last = mb == n_mb - 1
                flags = dict(defer=not last, pending=mb > 0, overwrite=last)
                if fused:
                    lg.sketch_accumulate_layer(
                        [(X[gi], [dY[n] for n in g], [S[n] for n in g], seed, stream)
                         for gi, g in enumerate(groups)], kind, ws=ws, **flags)
                else:
                    for gi, g in enumerate(groups):
                        lg.sketch_accumulate_shared(X[gi], [dY[n] for n in g], [S[n] for n in g],
                                                    seed, stream, kind, ws=ws[gi], **flags)
            if fused:
                lg.merge_many([(W[n], S[n], seed, stream) for n in proj], kind, 1.0, 2e-4)
            else:
                for n in proj:
                    lg.merge(W[n], S[n], seed, stream, kind, 1.0, 2e-4)

    per_layer_bytes = n_mb * (sum(2 * T * proj[g[0]][1] for g in groups) +
                              sum(2 * T * proj[n][0] for n in proj)) + \
        sum(4 * proj[n][0] * r for n in proj) + sum(merge_bytes(proj[n][0], proj[n][1], r) for n in proj)
    # algorithmic FLOPs: projection 2 T k r per input group, contraction 2 T d r
    # per projection, merge 2 d k r per weight
    per_layer_flop = n_mb * 2.0 * T * r * (sum(proj[g[0]][1] for g in groups) +
                                           sum(proj[n][0] for n in proj)) + \
        sum(2.0 * proj[n][0] * proj[n][1] * r for n in proj)
    return step, n_layers * per_layer_bytes, n_layers * per_layer_flop, n_layers * n_mb * T


def _mfma_roofline(flop, ms):
    """Roofline object of an MFMA-bound workload: algorithmic FLOPs over time,
    against the dense bf16 matrix-core peak."""
    tf = flop / (ms * 1e-3) / 1e12
    return dict(bound="mfma", achieved=tf, peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                frac=tf / BF16_MFMA_PEAK_TFLOPS, flop_per_step=flop,
                note="algorithmic FLOPs (projection 2Tkr per input, contraction 2Tdr, merge 2dkr); "
                     "the kernels execute more (P and S enter the matrix cores as hi/lo pairs)")


def run_other_configs(lg, synth):
    """Throughput of the other workloads at one GPU: the d = k = 256 layer,
    decoder layers of the 1.5B-shaped set at each rank and basis, of the
    7B-shaped set at r = 256, and the wide layer (d = 5120, k = 25600,
    r = 256, T = 16384).  Each: one optimizer step (every microbatch sketched,
    then merged), algorithmic bytes / time; layer sets also as the time of a
    28-layer pass, extrapolated from two distinct layers; r = 256 also against
    the matrix-core peak."""
    out = {}

    def report(name, ms, nbytes, tokens, **extra):
        out[name] = dict(us_per_step=ms * 1e3, tokens_per_s=tokens / (ms * 1e-3),
                         GBps=nbytes / (ms * 1e-3) / 1e9,
                         frac_hbm=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, bytes=nbytes, **extra)
        log(f"[bench] {name}: {ms * 1e3:.1f} us/step, {out[name]['GBps']:.0f} GB/s")

    # d = k = 256, r = 4, two microbatches of T = 128 (latency bound)
    c = synth.WORKLOADS["layer_d256_r4"]
    d, k, r, T = c["d"], c["k"], c["r"], c["T"]
    Xs = [synth.device_normal_bf16((T, k), synth.X_ID, "layer_d256_r4", mb) for mb in range(2)]
    dYs = [synth.device_normal_bf16((T, d), synth.DY_ID, "layer_d256_r4", mb) for mb in range(2)]
    W = synth.device_normal_bf16((d, k), synth.W_ID, "layer_d256_r4")
    S = torch.zeros(d, r, device="cuda")
    ws = lg.sketch_workspace(T, d, k, r)

    def small():
        for mb, (X, dY) in enumerate(zip(Xs, dYs)):
            lg.sketch_accumulate(X, dY, S, 1234, ws=ws, overwrite=mb == 0)
        lg.merge(W, S, 1234, 0, 0, c["alpha"], c["eta"])
    ms_small = _time_ms(small, 50)
    # The same step captured once in a HIP graph and replayed: the kernel
    # launches no longer wait on this process's per-call host work.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        small()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        small()
    ms_graph = _time_ms(graph.replay, 50)
    report("layer_d256_r4", ms_small, 2 * sketch_bytes(T, d, k, r) + merge_bytes(d, k, r), 2 * T,
           us_per_step_graph=ms_graph * 1e3,
           graph_note="the step captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed")
    del graph

    n_layers = 2
    for wl, cfg, r, kind, stream, label, reps in (
            ("qwen1p5b_layers", synth.QWEN1P5B, 4, 0, 0, "qwen1p5b_layer_r4", 3),
            ("qwen1p5b_layers", synth.QWEN1P5B, 16, 0, 0, "qwen1p5b_layer_r16", 3),
            ("qwen1p5b_layers", synth.QWEN1P5B, 64, 0, 0, "qwen1p5b_layer_r64", 3),
            ("qwen1p5b_layers", synth.QWEN1P5B, 64, 0, 1, "qwen1p5b_layer_r64_refreshed", 3),
            ("qwen1p5b_layers", synth.QWEN1P5B, 64, 1, 0, "qwen1p5b_layer_r64_gaussian", 3),
            ("qwen1p5b_layers", synth.QWEN1P5B, 256, 0, 0, "qwen1p5b_layer_r256", 3),
            ("qwen7b_layers", synth.QWEN7B, 256, 0, 0, "qwen7b_layer_r256", 2)):
        fn, nbytes, flop, tokens = _layer_set_step(lg, synth, wl, cfg, r, kind, stream, cfg["n_mb"],
                                                   n_layers)
        ms = _time_ms(fn, reps) / n_layers
        extra = dict(pass_28_layers_ms=28 * ms,
                     pass_note=f"28 x the per-layer time of {n_layers} distinct layers stepped in turn",
                     layers_measured=n_layers,
                     launches="one layer sketch call per microbatch, one merge call for the 7 weights")
        if label == "qwen1p5b_layer_r64":
            del fn
            torch.cuda.empty_cache()
            fn_g = _layer_set_step(lg, synth, wl, cfg, r, kind, stream, cfg["n_mb"], n_layers,
                                   fused=False)[0]
            extra["us_per_step_per_group_calls"] = _time_ms(fn_g, reps) / n_layers * 1e3
            del fn_g
            torch.cuda.empty_cache()
            fn = None
        if r == 256:
            extra["roofline_mfma"] = _mfma_roofline(flop / n_layers, ms)
        report(label, ms, nbytes / n_layers, tokens / n_layers, **extra)
        del fn
        torch.cuda.empty_cache()

    wide = synth.WORKLOADS["kl_vocab152064"]["wide"]
    d, k, r, T = wide["d"], wide["k"], wide["r"], wide["T"]
    X = synth.device_normal_bf16((T, k), synth.X_ID, "kl_vocab152064")
    dY = synth.device_normal_bf16((T, d), synth.DY_ID, "kl_vocab152064")
    W = synth.device_normal_bf16((d, k), synth.W_ID, "kl_vocab152064")
    S = torch.zeros(d, r, device="cuda")
    ws = lg.sketch_workspace(T, d, k, r)
    sk_ms = _time_ms(lambda: lg.sketch_accumulate(X, dY, S, 1234, ws=ws), 5)
    mg_ms = _time_ms(lambda: lg.merge(W, S, 1234, 0, 0, 1.0, 2e-4), 5)
    flop = 2.0 * T * r * (k + d) + 2.0 * d * k * r
    report("wide_layer_d5120_k25600_r256", sk_ms + mg_ms, sketch_bytes(T, d, k, r) + merge_bytes(d, k, r),
           T, sketch_us=sk_ms * 1e3, sketch_GBps=sketch_bytes(T, d, k, r) / (sk_ms * 1e-3) / 1e9,
           merge_us=mg_ms * 1e3, merge_GBps=merge_bytes(d, k, r) / (mg_ms * 1e-3) / 1e9,
           sketch_mfma=sketch_mfma(T, d, k, r, sk_ms * 1e3),
           merge_TFLOPs_executed=4.0 * d * k * r / (mg_ms * 1e-3) / 1e12,
           roofline_mfma=_mfma_roofline(flop, sk_ms + mg_ms),
           roofline_mfma_sketch=_mfma_roofline(2.0 * T * r * (k + d), sk_ms))
    del X, dY, W
    torch.cuda.empty_cache()
    return out


def run_update(lg, synth, d=4096, r=64, reps=200):
    """The sketch-space Adam and momentum updates on the layer's d x r sketch
    (24 and 16 bytes per entry); the merge would then read U."""
    S = synth.host_normal_f32((d, r), synth.S_ID, sigma=15.0).cuda()
    m = torch.zeros(d, r, device="cuda")
    v = torch.zeros(d, r, device="cuda")
    U = torch.empty(d, r, device="cuda")
    res = {}
    for name, rule, nbytes in (("adam", lg.UPDATE_ADAM, 24), ("momentum", lg.UPDATE_MOMENTUM, 16)):
        for t in range(1, 4):
            lg.sketch_update(rule, S, U, m, v, step=t)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for t in range(reps):
            lg.sketch_update(rule, S, U, m, v, step=4 + t)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / reps * 1e3
        res[name] = dict(us_per_call=us, GBps=nbytes * d * r / (us * 1e-6) / 1e9)
    res["shape"] = [d, r]
    return res


PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "sketch_merge_d4096_r64_traffic.md")


def measured_traffic(kernels):
    """HBM bytes per call of the given kernels from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None when there is no summary or the kernel sources changed since."""
    from rank_gradient_sketching_amd import profiling
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    text = open(PROFILE_TRAFFIC).read()
    tag = "<!-- traffic-json: "
    if tag not in text:
        return None
    tr = json.loads(text.split(tag, 1)[1].split(" -->", 1)[0])
    if tr.get("source_hash") != profiling.kernel_source_hash():
        return None
    total = 0.0
    for want in kernels:
        hits = [v for k, v in tr["kernels"].items() if k.startswith(want)]
        if not hits or hits[0]["read_bytes"] is None or hits[0]["write_bytes"] is None:
            return None
        total += hits[0]["read_bytes"] + hits[0]["write_bytes"]
    return total


def run_copy_calibration():
    """The hand-written device copy (liblogra_calib.so: chunked work-groups,
    non-temporal 16-byte loads and stores) as the practical HBM ceiling:
    32 MiB -> 32 MiB rotating over 16 buffer pairs (the merge's own bytes: its W
    read and written once; 1 GiB in all, beyond the 256 MB Infinity Cache), and
    512 MiB -> 512 MiB.  Its hardware byte counters also calibrate the path's
    counters (profiling.py)."""
    import ctypes
    from rank_gradient_sketching_amd import build as _b
    lib = ctypes.CDLL(_b.CALIB_LIB)
    lib.logra_calib_copy.restype = ctypes.c_int
    lib.logra_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream

    def copy(dst, src):
        st = lib.logra_calib_copy(dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(),
                                  stream)
        if st != 0:
            raise RuntimeError(f"logra_calib_copy failed ({st})")

    out = {}
    for name, nbytes, n_pairs, reps in (("copy_32MiB", 32 << 20, 16, 64),
                                        ("copy_512MiB", 512 << 20, 1, 5)):
        src = [torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
               for _ in range(n_pairs)]
        dst = [torch.empty_like(x) for x in src]
        copy(dst[0], src[0])
        torch.cuda.synchronize()
        per = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(reps):
                copy(dst[i % n_pairs], src[i % n_pairs])
            b.record()
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) / reps)
        ms = float(np.median(per))
        out[name] = dict(bytes_read=nbytes, bytes_written=nbytes, us=ms * 1e3,
                         GBps=2 * nbytes / (ms * 1e-3) / 1e9,
                         frac_hbm=2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
        del src, dst
        torch.cuda.empty_cache()
    out["kernel"] = "logra_calib_copy (hand-written HIP, non-temporal, 32 KB per work-group)"
    return out


def run_read_calibration():
    """The hand-written read-only stream (liblogra_calib.so: each 16-byte vector
    loaded once, 32 KB per work-group, nothing written) as the practical ceiling
    of the sketch's two read passes: 64 MiB (one microbatch of X or dY)
    rotating over 8 buffers (512 MiB in all, twice the Infinity Cache), with
    plain and with non-temporal loads, and one 512 MiB pass."""
    import ctypes
    from rank_gradient_sketching_amd import build as _b
    lib = ctypes.CDLL(_b.CALIB_LIB)
    lib.logra_calib_read.restype = ctypes.c_int
    lib.logra_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(64, dtype=torch.uint8, device="cuda")

    def read(src, nt):
        st = lib.logra_calib_read(src.data_ptr(), src.numel() * src.element_size(), nt,
                                  sink.data_ptr(), stream)
        if st != 0:
            raise RuntimeError(f"logra_calib_read failed ({st})")

    out = {}
    for name, nbytes, n_buf, reps in (("read_64MiB", 64 << 20, 8, 64),
                                      ("read_512MiB", 512 << 20, 1, 5)):
        bufs = [torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
                for _ in range(n_buf)]
        for nt in (0, 1):
            read(bufs[0], nt)
            torch.cuda.synchronize()
            per = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for i in range(reps):
                    read(bufs[i % n_buf], nt)
                b.record()
                torch.cuda.synchronize()
                per.append(a.elapsed_time(b) / reps)
            ms = float(np.median(per))
            out[name + ("_nontemporal" if nt else "")] = dict(
                bytes_read=nbytes, us=ms * 1e3, GBps=nbytes / (ms * 1e-3) / 1e9,
                frac_hbm=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS)
        del bufs
        torch.cuda.empty_cache()
    out["kernel"] = "logra_calib_read (hand-written HIP, 32 KB per work-group, no stores)"
    return out


def cpu_baseline(synth, data, budget_s=12.0):
    """The oracle, as it stands, on this host's cores, over whole steps of the
    same workload (four microbatches + merge), until about budget_s seconds."""
    from oracle import merge as omerge
    from oracle import projection as oproj
    from oracle import sketch as osketch
    Xs, dYs, W0, cfg = data
    d, k, r, T = cfg["d"], cfg["k"], cfg["r"], cfg["T"]
    mbs = [(synth.bf16_to_f64(X), synth.bf16_to_f64(dY)) for X, dY in zip(Xs, dYs)]
    Wb = synth.bf16_bits(W0)
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    n_steps = 0
    t0 = time.perf_counter()
    while True:
        A = oproj.projection(cfg["seed"], cfg["stream"], cfg["kind"], r, k)
        S = osketch.accumulate(np.zeros((d, r)), mbs, A)
        omerge.merge_bits(Wb, S, A, cfg["alpha"], cfg["eta"])
        n_steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    tokens = n_steps * T * len(mbs)
    return dict(value=tokens / el, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{n_steps} whole step(s) of {WORKLOAD} (4 x T={T} input-first "
                       f"fp64 sketch + fp64 merge with one bf16 rounding), {el:.1f} s",
                host_cores_available=len(os.sched_getaffinity(0)))


def cpu_baseline_others(synth):
    """The oracle, as it stands, on bounded samples of the other workloads
    (each figure extrapolated linearly and said so): the d = k = 256 layer in
    full; one layer x one microbatch of the 1.5B-shaped set at r = 64 and of
    the 7B-shaped set at r = 256 (its first 4096 of 32768 tokens), scaled to
    a 28-layer pass; 1024 of the 65536 predicted-KL rows, scaled x 64."""
    from oracle import kl as okl
    from oracle import merge as omerge
    from oracle import projection as oproj
    from oracle import sketch as osketch
    out = {}
    # d = k = 256, r = 4: whole steps for about a second
    c = synth.WORKLOADS["layer_d256_r4"]
    d, k, r, T = c["d"], c["k"], c["r"], c["T"]
    mbs = [(synth.bf16_to_f64(synth.host_normal_bf16((T, k), synth.X_ID, "layer_d256_r4", mb)),
            synth.bf16_to_f64(synth.host_normal_bf16((T, d), synth.DY_ID, "layer_d256_r4", mb)))
           for mb in range(c["n_mb"])]
    Wb = synth.bf16_bits(synth.host_normal_bf16((d, k), synth.W_ID, "layer_d256_r4"))
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        A = oproj.projection(c["seed"], c["stream"], c["kind"], r, k)
        S = osketch.accumulate(np.zeros((d, r)), mbs, A)
        omerge.merge_bits(Wb, S, A, c["alpha"], c["eta"])
        n += 1
    el = time.perf_counter() - t0
    out["layer_d256_r4"] = dict(value=n * T * c["n_mb"] / el, unit="tokens/s",
                                sample=f"{n} whole steps (2 x T={T} + merge), {el:.1f} s")
    # one decoder layer: the sketch of one microbatch on sub-sampled tokens,
    # scaled by tokens and microbatches; the merge on 256 rows of every W (each
    # row of W depends only on its row of S), scaled by the rows
    for name, cfg, r, t_used in (("qwen1p5b_layers_r64", synth.QWEN1P5B, 64, 8192),
                                 ("qwen7b_layers_r256", synth.QWEN7B, 256, 4096)):
        T = cfg["T"]
        proj = {nm: (dd, kk) for nm, dd, kk in cfg["projections"]}
        groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
        rng = np.random.default_rng(7)
        t_sk = t_mg = 0.0
        for g in groups:
            kk = proj[g[0]][1]
            A = oproj.projection(1234, 0, 0, r, kk)
            X = rng.standard_normal((t_used, kk))
            for nm in g:
                dd = proj[nm][0]
                dY = rng.standard_normal((t_used, dd)) * 1e-2
                t0 = time.perf_counter()
                S = osketch.sketch_input_first(X, dY, A)
                t_sk += time.perf_counter() - t0
                rows = min(dd, 256)
                Wb = synth.bf16_bits(synth.host_normal_bf16((rows, kk), synth.W_ID, salt=1))
                t0 = time.perf_counter()
                omerge.merge_bits(Wb, S[:rows], A, 1.0, 2e-4)
                t_mg += (time.perf_counter() - t0) * dd / rows
        per_layer_step = t_sk * (T / t_used) * cfg["n_mb"] + t_mg
        tokens = T * cfg["n_mb"]
        out[name] = dict(value=tokens / per_layer_step, unit="tokens/s (per layer step)",
                         pass_28_layers_s=28 * per_layer_step,
                         sample=f"one decoder layer (7 projections, each sketched input-first on "
                                f"its own): sketch of {t_used} of {T} tokens in {t_sk:.2f} s, "
                                f"scaled x {T // t_used} tokens x {cfg['n_mb']} microbatches; "
                                f"merge of 256 rows per W, scaled to all rows ({t_mg:.1f} s); "
                                "the pass is 28 x that")
    # predicted KL: 512 of 65536 rows
    kc = synth.WORKLOADS["kl_vocab152064"]
    V = kc["vocab"]
    rows = 512
    z = synth.bf16_to_f64(synth.host_normal_bf16((rows, V), synth.Z_ID, "kl_vocab152064"))
    dz = synth.host_normal_bf16((rows, V), synth.DIR_ID, "kl_vocab152064")
    zp = synth.bf16_to_f64(synth.proposal_logits(synth.host_normal_bf16((rows, V), synth.Z_ID,
                                                                        "kl_vocab152064"), dz, 1.0))
    t0 = time.perf_counter()
    for r0 in range(0, rows, 128):
        okl.kl_rows(z[r0:r0 + 128], zp[r0:r0 + 128], kc["tau"])
    el = time.perf_counter() - t0
    n_all = kc["n_resp"] * kc["resp_len"]
    out["kl_vocab152064"] = dict(value=rows * V * 4 / el / 1e9, unit="GB/s",
                                 call_s=el * n_all / rows,
                                 sample=f"{rows} of {n_all} rows x {V} in {el:.1f} s, scaled x {n_all // rows}")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-kl", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-calib", action="store_true")
    ap.add_argument("--no-layerset", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this path has no multi-GPU leg "
              "(sharding is a design note only).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    import rank_gradient_sketching_amd as lg
    from rank_gradient_sketching_amd import synth

    # no cyclic garbage collection inside the timed regions (the bench makes
    # few objects; tensors are freed by reference count)
    gc.disable()
    layer, data = run_layer(lg, synth, args.steps, args.warmup)
    kl = None if args.no_kl else run_kl(lg, synth)
    layer_set = None if args.no_layerset else run_layer_set(lg, synth)
    update = run_update(lg, synth)
    others = None if args.no_configs else run_other_configs(lg, synth)
    calib = None if args.no_calib else run_copy_calibration()
    read_cal = None if args.no_calib else run_read_calibration()
    cpu = None if args.no_cpu else cpu_baseline(synth, data, args.cpu_budget)
    if cpu is not None:
        cpu["other_configs"] = cpu_baseline_others(synth)

    cfg = layer["cfg"]
    sk, mg = layer["sketch"], layer["merge"]
    tokens_per_s = layer["tokens_per_step"] / (layer["step_ms"] * 1e-3)
    # dominant entry point: the sketch call (4 per step); its kernels
    # (project, accumulate, finalize) run back to back on the library's stream
    sketch_kernels = ["project_kernel", "accumulate_kernel", "finalize_kernel"]
    roof = dict(kernel="logra_sketch_accumulate (project + accumulate + finalize kernels)",
                bound="hbm", achieved=sk["GBps"], peak=HBM_PEAK_GBPS, unit="GB/s",
                frac=sk["GBps"] / HBM_PEAK_GBPS, traffic=measured_traffic(sketch_kernels),
                bytes_per_launch=sk["bytes_per_call"], us_per_launch=sk["us_per_call"])
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": layer["step_ms"],
        "ms_per_step_graph": layer["graph_step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.01^2) output grads, N(0,0.02^2) weights)",
        "config": {"workload": WORKLOAD, "d": cfg["d"], "k": cfg["k"], "r": cfg["r"],
                   "tokens_per_microbatch": cfg["T"], "microbatches": cfg["n_mb"],
                   "global_batch": cfg["T"] * cfg["n_mb"], "seq_len": None,
                   "alpha_eta": cfg["alpha"] * cfg["eta"], "projection": "rademacher",
                   "buffer_sets": 2 * cfg["n_mb"], "parallelism": "single-gpu"},
        "sketch": {"tokens_per_s": sk["tokens_per_s"], "GBps": sk["GBps"],
                   "frac_hbm": sk["frac_hbm"], "us_per_call": sk["us_per_call"],
                   "us_per_call_min": sk["us_min"],
                   # against two passes of the hand-written read stream over one
                   # microbatch's X and dY (64 MiB each, plain loads)
                   "read_us_same_bytes": (2 * read_cal["read_64MiB"]["us"]) if read_cal else None,
                   "frac_of_read": ((2 * read_cal["read_64MiB"]["us"]) / sk["us_per_call"])
                   if read_cal else None,
                   "frac_of_read_in_chain": ((2 * read_cal["read_64MiB"]["us"]) /
                                             layer["chain"]["us_per_call"]) if read_cal else None,
                   **sketch_mfma(cfg["T"], cfg["d"], cfg["k"], cfg["r"], sk["us_per_call"]),
                   # inside the step's deferred chain (one split reduction per step)
                   "in_chain": {k_: layer["chain"][k_] for k_ in
                                ("us_per_call", "us_min", "GBps", "frac_hbm", "tokens_per_s",
                                 "bytes_per_call")}},
        "merge": {"GBps": mg["GBps"], "frac_hbm": mg["frac_hbm"], "us_per_call": mg["us_per_call"],
                  "us_per_call_min": mg["us_min"],
                  # against the hand-written copy of the same bytes (W read and written)
                  "copy_us_same_bytes": calib["copy_32MiB"]["us"] if calib else None,
                  "frac_of_copy": (calib["copy_32MiB"]["us"] / mg["us_per_call"]) if calib else None},
        "wall_ms_timed_steps": layer["wall_ms"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": layer["parity"],
        "kl": kl,
        "layer_set": layer_set,
        "sketch_update": update,
        "other_configs": others,
        "copy_calibration": calib,
        "read_calibration": read_cal,
    }
    print(json.dumps(out), flush=True)
    # a parity failure anywhere fails the run (after the line is printed)
    bad = []
    if not layer["parity"]["ok"]:
        bad.append("layer")
    if kl is not None:
        if not (kl["sampled_row_max_rel_err"] < 1e-3 and kl["q_vs_row_mean_rel"] < 1e-6):
            bad.append("predicted KL")
        if not kl["sweep"]["sampled_row_max_rel_err"] < 1e-3:
            bad.append("predicted-KL sweep")
    if layer_set is not None and not layer_set["shared_vs_separate_rel_fro"] < 1e-5:
        bad.append("shared sketch")
    if bad:
        log(f"[bench] PARITY FAILED: {', '.join(bad)}")
        sys.exit(1)


if __name__ == "__main__":
    main()
