"""Rollout sync payload (host side): layout, round trip, corruption checks.

[LoGRA] Sync: the rollout engine receives the factor and the seed and
rebuilds A itself, so the payload is O(d r) numbers plus metadata.
"""
import numpy as np
import pytest
import torch

from rank_gradient_sketching_amd import sync


def _payload(d=96, r=8, k=200, seed=2**64 - 3, stream=5, kind=1, alpha=0.375, eta=2e-4):
    U = torch.from_numpy(np.random.default_rng(3).standard_normal((d, r)).astype(np.float32))
    return U, sync.pack_update(U, seed, stream, kind, alpha, eta, k)


def test_round_trip_keeps_every_field_and_bit():
    U, p = _payload()
    u = sync.unpack_update(p, device="cpu")
    assert torch.equal(u["U"], U)
    assert (u["d"], u["k"], u["r"], u["kind"], u["stream"]) == (96, 200, 8, 1, 5)
    assert u["seed"] == 2**64 - 3
    assert u["alpha"] == np.float32(0.375) and u["eta"] == np.float32(2e-4)
    assert len(p) == sync.HEADER_BYTES + 4 * 96 * 8


def test_payload_is_o_dr_not_dk(golden):
    # the page's d = k = 4096, r = 64 layer: 1 MiB of factor instead of the d x k update
    d = k = 4096
    r = 64
    U = torch.zeros(d, r)
    p = sync.pack_update(U, 1234, 0, 0, 1.0, 2e-4, k)
    assert len(p) - sync.HEADER_BYTES == golden["accumulator"]["sketch_fp32_MiB"] * 2**20
    assert len(p) < 2 * d * k / 30          # vs a bf16 d x k update


@pytest.mark.parametrize("mutate", ["flip_body", "flip_magic", "truncate", "extend", "version"])
def test_corrupt_payloads_are_rejected(mutate):
    _, p = _payload()
    b = bytearray(p)
    if mutate == "flip_body":
        b[sync.HEADER_BYTES + 17] ^= 0x40
    elif mutate == "flip_magic":
        b[0] ^= 1
    elif mutate == "truncate":
        b = b[:-4]
    elif mutate == "extend":
        b += b"\0\0\0\0"
    else:
        b[4] = 9
    with pytest.raises(ValueError):
        sync.unpack_update(bytes(b), device="cpu")
