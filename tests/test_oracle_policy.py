"""Pins for the oracle's mixed AR / self-speculation step and its mode choice
by concurrency: closed forms of the choice under constant, linear and affine
cost curves, the pages' qualitative claim (self-speculation at low
concurrency, AR at high), the structure of the optimum, and losslessness of
mixed steps against greedy AR."""
import numpy as np
import pytest

import seeded
from oracle import MODE_AR, MODE_SELFSPEC, OracleModel, OracleSession
from oracle.policy import choose_modes, forward_ms, step_rate, step_rows


# ------------------------------------------------------------------ cost curve
def test_forward_ms_is_piecewise_linear():
    rows = [1, 8, 64, 512]
    ms = [4.0, 4.1, 4.6, 15.0]
    for r, t in zip(rows, ms):
        assert forward_ms(rows, ms, r) == t
    # interior points: the library's piecewise-linear interpolation
    for r in (2, 5.5, 20, 63, 100, 511):
        assert forward_ms(rows, ms, r) == pytest.approx(float(np.interp(r, rows, ms)), rel=1e-15)
    assert forward_ms(rows, ms, 0) == 4.0                       # below the first point
    # beyond the last point: the line through the last two (slope 10.4/448 ms per row)
    assert forward_ms(rows, ms, 960) == pytest.approx(15.0 + 448 * 10.4 / 448, rel=1e-15)
    assert forward_ms([32], [5.0], 4096) == 5.0                # one point: constant
    with pytest.raises(ValueError):
        forward_ms([8, 8], [1.0, 2.0], 3)
    with pytest.raises(ValueError):
        forward_ms([1, 8], [1.0, 0.0], 3)


def test_step_rows_counts_both_forwards():
    # AR: pending rows, then one row; self-speculation: pending + k, then k
    assert step_rows([1, 1, 3], [False, True, False], 32) == (1 + 33 + 3, 1 + 32 + 1)
    assert step_rows([1] * 4, [True] * 4, 8) == (36, 32)


# -------------------------------------------------------------- closed forms
@pytest.mark.parametrize("seed", range(6))
def test_no_gain_no_selfspec(seed):
    """A round committing at most 2 tokens never beats two AR tokens on rows
    that are never fewer: with a non-decreasing curve every sequence is AR."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    e = rng.uniform(1.0, 2.0, n)
    rows = np.cumsum(rng.integers(1, 100, 5)).tolist()
    ms = np.cumsum(rng.uniform(0.0, 3.0, 5) + 0.01).tolist()
    assert choose_modes(rows, ms, e, int(rng.integers(1, 33))) == [MODE_AR] * n


@pytest.mark.parametrize("seed", range(6))
def test_flat_cost_takes_every_gain(seed):
    """With a constant curve the step time is fixed, so a sequence runs
    self-speculation exactly when its expected round beats 2 tokens."""
    rng = np.random.default_rng(10 + seed)
    n = int(rng.integers(1, 9))
    k = int(rng.integers(2, 33))
    e = rng.uniform(1.0, k + 1.0, n)
    got = choose_modes([1], [4.0], e, k)
    assert got == [MODE_SELFSPEC if x > 2.0 else MODE_AR for x in e]


@pytest.mark.parametrize("seed", range(6))
def test_cost_proportional_to_rows_is_always_ar(seed):
    """t = c * rows with one pending row each: AR gets 1 token per row, a
    self-speculation round at most (k+1)/(2k+1) < 1, so all AR."""
    rng = np.random.default_rng(20 + seed)
    n = int(rng.integers(1, 9))
    k = int(rng.integers(1, 33))
    c = float(rng.uniform(0.01, 1.0))
    e = rng.uniform(1.0, k + 1.0, n)
    assert choose_modes([1, 2], [c, 2 * c], e, k) == [MODE_AR] * n


@pytest.mark.parametrize("seed", range(10))
def test_single_sequence_affine_threshold(seed):
    """One sequence, t = a + b * rows, p pending rows: AR commits 2 tokens in
    2a + b(p + 1), a round e tokens in 2a + b(p + 2k); self-speculation wins
    exactly when e > 2 (2a + b(p + 2k)) / (2a + b(p + 1))."""
    rng = np.random.default_rng(30 + seed)
    a, b = float(rng.uniform(1, 8)), float(rng.uniform(0.001, 0.05))
    k, p = int(rng.integers(1, 33)), int(rng.integers(1, 4))
    grid = ([1, 4096], [a + b, a + 4096 * b])
    thr = 2 * (2 * a + b * (p + 2 * k)) / (2 * a + b * (p + 1))
    if thr < k + 1 - 1e-6:
        assert choose_modes(*grid, [min(k + 1.0, thr + 1e-6)], k, [p]) == [MODE_SELFSPEC]
    assert choose_modes(*grid, [max(1.0, thr - 1e-6)], k, [p]) == [MODE_AR]


def test_concurrency_claim_selfspec_low_ar_high():
    """The pages' deployment claim.  With t = a + b * rows, one more
    self-speculation sequence adds 2k - 1 rows for e - 2 more tokens; once n
    AR sequences already commit 2n tokens per 2a + 2bn, that only pays while
    (e - 2) / (b (2k - 1)) beats the step's rate.  a = 4, b = 0.2, k = 32,
    e = 7: self-speculation alone, AR once 16 sequences share the step."""
    rows, ms = [1, 4096], [4.2, 4.0 + 0.2 * 4096]
    assert choose_modes(rows, ms, [7.0], 32) == [MODE_SELFSPEC]
    assert choose_modes(rows, ms, [7.0] * 16, 32) == [MODE_AR] * 16
    # a device-like curve (weight streaming flat to 128 rows, then compute):
    # in the middle, a mixed batch beats both pure choices
    rows, ms = [1, 128, 4096], [4.0, 4.6, 80.0]
    got = choose_modes(rows, ms, [7.0] * 12, 32)
    assert 0 < got.count(MODE_SELFSPEC) < 12
    best = step_rate(rows, ms, [7.0] * 12, 32, [1] * 12, [m == MODE_SELFSPEC for m in got])
    assert best > step_rate(rows, ms, [7.0] * 12, 32, [1] * 12, [False] * 12)
    assert best > step_rate(rows, ms, [7.0] * 12, 32, [1] * 12, [True] * 12)


@pytest.mark.parametrize("seed", range(8))
def test_optimum_takes_the_best_acceptances(seed):
    """Rows depend only on how many sequences speculate, so the optimum's
    self-speculation set holds the largest expected rounds; its rate is the
    best over every subset."""
    rng = np.random.default_rng(50 + seed)
    n = int(rng.integers(2, 9))
    k = int(rng.integers(4, 33))
    rows = [1, 32, 256, 2048]
    ms = sorted(rng.uniform(1, 60, 4).tolist())
    e = rng.uniform(1.0, k + 1.0, n)
    got = choose_modes(rows, ms, e, k)
    spec = [m == MODE_SELFSPEC for m in got]
    if any(spec) and not all(spec):
        assert min(e[i] for i in range(n) if spec[i]) >= max(e[i] for i in range(n) if not spec[i])
    best = step_rate(rows, ms, e, k, [1] * n, spec)
    for mask in range(1 << n):
        other = [(mask >> i) & 1 == 1 for i in range(n)]
        assert step_rate(rows, ms, e, k, [1] * n, other) <= best


def test_choice_rejects_bad_input():
    with pytest.raises(ValueError):
        choose_modes([1], [1.0], [0.5], 8)            # a round commits at least one token
    with pytest.raises(ValueError):
        choose_modes([1], [1.0], [10.0], 8)           # and at most k + 1
    with pytest.raises(ValueError):
        choose_modes([1], [1.0], [2.0], 0)
    assert choose_modes([1], [1.0], [], 8) == []


# ------------------------------------------------------------------ mixed step
def test_mixed_steps_are_lossless_against_greedy_ar():
    """Any sequence of per-step modes commits the greedy AR continuation; an
    AR step commits two tokens in two forwards."""
    shape = seeded.TINY_SHARP
    m = OracleModel(shape, seeded.gen_weights(shape))
    prompt = seeded.prompt(16, shape.vocab)
    ar = OracleSession(m, 128)
    ar.prefill(prompt)
    want = ar.generate(MODE_AR, 40)
    s = OracleSession(m, 128)
    s.prefill(prompt)
    rng = np.random.default_rng(3)
    got = []
    while len(got) < 40:
        mode = MODE_AR if rng.random() < 0.5 else MODE_SELFSPEC
        before = s.forwards
        out = s.mixed_step(mode, 8)
        assert s.forwards - before == 2
        if mode == MODE_AR:
            assert len(out) == 2
        else:
            assert 1 <= len(out) <= 9
        got += out
    assert got[:40] == want
    with pytest.raises(ValueError):
        s.mixed_step(1, 8)
