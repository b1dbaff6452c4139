"""Seeded synthetic inputs for tests and the benchmark.

This module only draws random tensors; it holds none of the method's
arithmetic.  Host tensors come from NumPy's `default_rng` seeded with a tuple
(workload id, tensor id, microbatch), drawn in fp32 and rounded to bf16 by
torch (round to nearest even).  Device tensors for the large workloads come
from a seeded torch generator on the GPU, in row chunks so the fp32 staging
copy stays small.

Workloads (single-GPU shapes; sizes in elements):
  layer_d256_r4         d = k = 256, r = 4, 2 microbatches of T = 128
  layer_d4096_r64       d = k = 4096, r = 64, 4 microbatches of T = 8192
  qwen1p5b_layers       28 decoder layers of a 1.5B model, r in {4,16,64,256},
                        2 microbatches of T = 16384
  qwen7b_layers         28 decoder layers of a 7B model, r = 256,
                        4 microbatches of T = 32768
  kl_vocab152064        64 responses x 1024 tokens x vocab 152064 logits,
                        plus one wide layer d = 5120, k = 25600, r = 256,
                        T = 16384
Value distributions: X ~ N(0, 1), dY ~ N(0, 0.01^2), W ~ N(0, 0.02^2),
logits z ~ N(0, 3^2), proposal direction ~ N(0, 0.05^2).
"""
import numpy as np
import torch

X_ID, DY_ID, W_ID, Z_ID, DIR_ID, S_ID = 1, 2, 3, 4, 5, 6
SIGMA = {X_ID: 1.0, DY_ID: 1e-2, W_ID: 0.02, Z_ID: 3.0, DIR_ID: 0.05, S_ID: 1.0}

WORKLOAD_IDS = {"layer_d256_r4": 1, "layer_d4096_r64": 2, "qwen1p5b_layers": 3,
                "qwen7b_layers": 4, "kl_vocab152064": 5, "adhoc": 99}

WORKLOADS = {
    "layer_d256_r4": dict(d=256, k=256, r=4, T=128, n_mb=2, seed=1234, stream=0,
                          kind=0, alpha=1.0, eta=1e-3),
    "layer_d4096_r64": dict(d=4096, k=4096, r=64, T=8192, n_mb=4, seed=1234, stream=0,
                            kind=0, alpha=1.0, eta=2e-4),
    "kl_vocab152064": dict(n_resp=64, resp_len=1024, vocab=152064, tau=1.0,
                           kl_budget=2e-4, alpha_max=4.0, alphas=(0.25, 0.5, 1.0, 2.0),
                           wide=dict(d=5120, k=25600, r=256, T=16384)),
}


def layer_set(hidden, kv_dim, mlp):
    """(name, d_out, k_in) of the seven projections of one decoder layer."""
    return [("q", hidden, hidden), ("k", kv_dim, hidden), ("v", kv_dim, hidden),
            ("o", hidden, hidden), ("gate", mlp, hidden), ("up", mlp, hidden),
            ("down", hidden, mlp)]


QWEN1P5B = dict(layers=28, projections=layer_set(1536, 256, 8960), T=16384, n_mb=2)
QWEN7B = dict(layers=28, projections=layer_set(3584, 512, 18944), T=32768, n_mb=4)


def host_normal_bf16(shape, tensor_id, workload="adhoc", mb=0, sigma=None, salt=0):
    """CPU bf16 tensor of N(0, sigma^2) values, seeded by (workload, tensor, mb, salt)."""
    sig = SIGMA[tensor_id] if sigma is None else sigma
    rng = np.random.default_rng([WORKLOAD_IDS[workload], tensor_id, mb, salt])
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(sig)
    return torch.from_numpy(x).to(torch.bfloat16)


def host_normal_f32(shape, tensor_id, workload="adhoc", mb=0, sigma=None, salt=0):
    """CPU fp32 tensor of N(0, sigma^2) values (used for fp32 sketch states)."""
    sig = SIGMA[tensor_id] if sigma is None else sigma
    rng = np.random.default_rng([WORKLOAD_IDS[workload], tensor_id, mb, salt])
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(sig))


def device_normal_bf16(shape, tensor_id, workload="adhoc", mb=0, sigma=None, salt=0,
                       device="cuda", out=None, chunk_rows=4096):
    """Device bf16 tensor of N(0, sigma^2) values from a seeded torch generator."""
    sig = SIGMA[tensor_id] if sigma is None else sigma
    seed = (WORKLOAD_IDS[workload] * 1000003 + tensor_id * 10007 + mb * 101 + salt) & 0x7FFFFFFF
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        tmp = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                          dtype=torch.float32)
        flat[r0:r1].copy_(tmp.mul_(sig))
    return out


def proposal_logits(z, direction, alpha, chunk_rows=4096):
    """Proposed-model logits z + alpha * direction, formed in fp32, stored bf16.

    This stands in for the forward pass of the model after the proposed update
    (the logits the controller compares against the current ones).
    """
    out = torch.empty_like(z)
    for r0 in range(0, z.shape[0], chunk_rows):
        r1 = min(z.shape[0], r0 + chunk_rows)
        out[r0:r1] = (z[r0:r1].float() + alpha * direction[r0:r1].float()).to(torch.bfloat16)
    return out


def bf16_to_f64(t):
    """Exact float64 NumPy copy of a bf16 tensor (any device)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits(t):
    """uint16 bit patterns of a bf16 tensor (any device) as a NumPy array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
