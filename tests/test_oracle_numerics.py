"""Pins for the oracle's bfloat16 rounding: brute-force nearest representable
value, and torch's own float32 -> bfloat16 conversion as a library routine."""
import numpy as np
import torch

from oracle.numerics import round_bf16


def _all_bf16_neighbours(x):
    """Brute force: the bf16 values just below and just above |x| from the bit
    patterns of the format (the float32 patterns with a zero low half)."""
    f = np.float32(abs(x))
    u = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) & 0xFFFF0000
    cands = []
    for du in (-0x10000, 0, 0x10000, 0x20000):
        v = u + du
        if 0 <= v <= 0x7F800000:
            cands.append(float(np.array([v], dtype=np.uint32).view(np.float32)[0]))
    return cands


def _brute_round(x):
    if x == 0.0:
        return x
    best = None
    for c in _all_bf16_neighbours(x):
        c = np.copysign(c, x)
        d = abs(c - x)
        if best is None or d < best[0] or (d == best[0] and _mant_even(c) and not _mant_even(best[1])):
            best = (d, c)
    return best[1]


def _mant_even(v):
    u = int(np.array([abs(v)], dtype=np.float32).view(np.uint32)[0])
    return ((u >> 16) & 1) == 0


def test_round_bf16_matches_brute_force():
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000)),
        rng.uniform(-2, 2, 500),
    ])
    got = round_bf16(xs)
    for x, g in zip(xs, got):
        assert g == _brute_round(float(x)), (x, g)


def test_round_bf16_ties_to_even_and_edges():
    one = 1.0
    ulp = 2.0 ** -7
    # exact halfway points between 1 and 1+ulp rounds to even (1.0); next one up rounds up
    assert round_bf16(np.array([one + ulp / 2]))[0] == 1.0
    assert round_bf16(np.array([one + 3 * ulp / 2]))[0] == one + 2 * ulp
    # subnormal quantum 2^-133, overflow to inf, passthrough of non-finite
    tiny = 2.0 ** -133
    assert round_bf16(np.array([tiny * 0.75]))[0] == tiny
    assert round_bf16(np.array([tiny * 0.5]))[0] == 0.0
    big = float.fromhex("0x1.fep127")
    assert round_bf16(np.array([big]))[0] == big
    assert np.isinf(round_bf16(np.array([2.0 ** 128]))[0])
    r = round_bf16(np.array([np.inf, -np.inf, np.nan]))
    assert np.isinf(r[0]) and np.isinf(r[1]) and np.isnan(r[2])


def test_round_bf16_matches_torch_on_float32_inputs():
    # torch rounds float32 -> bfloat16 to nearest even; on float32 inputs a
    # single rounding from float64 must agree with it exactly.
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(200000) * 3).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), ref)
