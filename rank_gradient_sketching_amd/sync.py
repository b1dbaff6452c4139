"""Rollout-side sync payload: the merged update as (U, seed, metadata).

[LoGRA] Sync: at policy sync the rollout engine rebuilds A from the seed and
applies the received factor alpha * eta * U, so the transfer is O(d r)
numbers plus a seed and metadata instead of the d x k update; the same
compact representation serves accumulation, update and sync.

The payload carries U (= S in the plain SGD form) in fp32 together with the
separate alpha and eta, so the rollout side runs the very merge the trainer
ran (same kernel, same fp32 inputs) and its weights match bit for bit.
Layout (little-endian): a fixed header, then U as d x r fp32 rows.

    magic   4s   b"LGRA"
    version u32  1
    kind    i32  projection kind (0 sign basis, 1 Gaussian)
    r       i32
    d       i64
    k       i64
    seed    u64
    stream  u64
    alpha   f32
    eta     f32
    crc32   u32  of the U bytes
    nbytes  u64  of the U bytes (= 4 d r)
"""
import struct
import zlib

import numpy as np
import torch

from . import api

MAGIC = b"LGRA"
VERSION = 1
_HEADER = struct.Struct("<4sIiiqqQQffIQ")
HEADER_BYTES = _HEADER.size


def pack_update(U, seed, stream, kind, alpha, eta, k):
    """bytes of one layer's sync payload; U is the (d, r) fp32 factor (on any device)."""
    if U.dtype != torch.float32 or U.dim() != 2:
        raise ValueError("U must be a 2-D float32 tensor")
    d, r = U.shape
    body = U.detach().contiguous().cpu().numpy().tobytes()
    head = _HEADER.pack(MAGIC, VERSION, int(kind), int(r), int(d), int(k), int(seed) & (2**64 - 1),
                        int(stream) & (2**64 - 1), float(alpha), float(eta),
                        zlib.crc32(body) & 0xFFFFFFFF, len(body))
    return head + body


def unpack_update(payload, device="cuda"):
    """dict(U, seed, stream, kind, alpha, eta, d, k, r) from a payload; raises
    ValueError on a bad header, size or checksum."""
    if len(payload) < HEADER_BYTES:
        raise ValueError("payload shorter than its header")
    (magic, version, kind, r, d, k, seed, stream, alpha, eta, crc,
     nbytes) = _HEADER.unpack_from(payload, 0)
    if magic != MAGIC or version != VERSION:
        raise ValueError("not a LoGRA sync payload of a known version")
    if d < 1 or k < 1 or r < 1 or nbytes != 4 * d * r or len(payload) != HEADER_BYTES + nbytes:
        raise ValueError("payload sizes do not match its header")
    body = memoryview(payload)[HEADER_BYTES:]
    if zlib.crc32(body) & 0xFFFFFFFF != crc:
        raise ValueError("payload checksum mismatch")
    U = torch.from_numpy(np.frombuffer(body, dtype=np.float32).reshape(d, r).copy())
    return dict(U=U.to(device), seed=seed, stream=stream, kind=kind, alpha=alpha, eta=eta,
                d=d, k=k, r=r)


def apply_update(W, payload):
    """Rollout-side merge of a received payload into W (d x k bf16, in place)."""
    u = payload if isinstance(payload, dict) else unpack_update(payload, W.device)
    if tuple(W.shape) != (u["d"], u["k"]):
        raise ValueError(f"W is {tuple(W.shape)} but the payload is for ({u['d']}, {u['k']})")
    return api.merge(W, u["U"].to(W.device), u["seed"], u["stream"], u["kind"], u["alpha"],
                     u["eta"])
