"""Pins for the oracle's bf16 rounding and Philox generator.

bf16: checked against torch's independent float32 -> bfloat16 conversion
(round to nearest even) and against hand-worked tie and double-rounding cases.
Philox4x64-10: checked against NumPy's independent `numpy.random.Philox`,
which implements the same published generator (Salmon et al., SC'11) and
advances its counter by one before each block, so NumPy at counter c equals
the oracle at counter c + 1.
"""
import numpy as np
import pytest
import torch

from oracle import bf16, philox


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-30, 30, 20000),
        rng.standard_normal(1000) * 1e-40,          # fp32 subnormals
        np.array([0.0, -0.0, 3e38, -3e38, 3.39e38, np.inf, -np.inf]),
    ]).astype(np.float32)
    ours = bf16.f64_to_bits(x.astype(np.float64))
    np.testing.assert_array_equal(ours, _torch_bf16_bits(x))


def test_bf16_ties_and_double_rounding():
    # spacing of bf16 at 1.0 is 2**-7
    assert bf16.round_f64(1.0 + 2.0 ** -8) == 1.0                  # tie -> even
    assert bf16.round_f64(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie -> even
    assert bf16.round_f64(-(1.0 + 2.0 ** -8)) == -1.0
    # just above a tie: one rounding from fp64 must go up; rounding through
    # fp32 first would land on the tie and then round down to 1.0
    assert bf16.round_f64(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert bf16.f64_to_bits(np.nan) == 0x7FC0
    assert bf16.f64_to_bits(1e39) == 0x7F80
    assert bf16.f64_to_bits(-0.0) == 0x8000


def test_bf16_decode_roundtrip_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.bits_to_f64(bits)
    finite = np.isfinite(vals)
    np.testing.assert_array_equal(bf16.f64_to_bits(vals[finite]), bits[finite])


@pytest.mark.parametrize("ctr,key", [
    ((1, 0, 0, 0), (0, 0)),
    ((6, 0, 0, 0), (123, 456)),
    ((6, 7, 9, 11), (1, 2)),
    ((0, 1, 0, 0), (2 ** 64 - 1, 2 ** 63)),     # NumPy counter wraps word 0
    ((17, 255, 0, 0), (1234, 0)),
    ((3, 63, 1, 0), (1234 + 27, 5)),
])
def test_philox_known_answers_against_numpy(ctr, key):
    c = ctr[0] + (ctr[1] << 64) + (ctr[2] << 128) + (ctr[3] << 192) - 1
    words = [(c >> (64 * i)) & (2 ** 64 - 1) for i in range(4)]
    ref = np.random.Philox(counter=np.array(words, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64)).random_raw(4)
    assert philox.philox4x64_10(ctr, key) == tuple(int(v) for v in ref)


def test_philox_vectorised_equals_scalar():
    rng = np.random.default_rng(3)
    n = 300
    ctr = rng.integers(0, 2 ** 63, size=(4, n), dtype=np.uint64) * np.uint64(2) \
        + rng.integers(0, 2, size=(4, n), dtype=np.uint64)
    for key in [(0, 0), (2 ** 64 - 1, 12345), (987654321, 2 ** 63 + 5)]:
        out = philox.philox4x64_10_np(*ctr, *key)
        for j in range(n):
            ref = philox.philox4x64_10(tuple(int(c[j]) for c in ctr), key)
            assert tuple(int(o[j]) for o in out) == ref
