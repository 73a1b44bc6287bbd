"""The library's mode choice by concurrency (tri_choose_modes, host code, no
device work) against the oracle's brute force over every subset."""
import os

import numpy as np
import pytest

from oracle import MODE_AR, MODE_SELFSPEC
from oracle.policy import choose_modes as oracle_choose, step_rate


@pytest.fixture(scope="module")
def tm():
    from self_speculative_lm_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from self_speculative_lm_amd.build import build
        build()
    import self_speculative_lm_amd as tm
    assert (tm.TRI_AR, tm.TRI_SELFSPEC) == (MODE_AR, MODE_SELFSPEC)
    return tm


@pytest.mark.parametrize("seed", range(40))
def test_choice_matches_brute_force(tm, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 11))
    k = int(rng.integers(1, 65))
    ng = int(rng.integers(1, 6))
    rows = np.sort(rng.choice(np.arange(1, 4097), ng, replace=False)).tolist()
    ms = np.sort(rng.uniform(0.5, 80.0, ng)).tolist()
    if seed % 4 == 0:                                  # a curve that is not monotone
        ms = rng.uniform(0.5, 80.0, ng).tolist()
    e = rng.uniform(1.0, k + 1.0, n)
    if seed % 5 == 0:
        e = np.round(e)                                # exact ties between sequences
    pend = rng.integers(1, 4, n) if seed % 3 == 0 else None
    got = tm.choose_modes(rows, ms, e, k, pend).tolist()
    want = oracle_choose(rows, ms, e.tolist(), k, None if pend is None else pend.tolist())
    p = [1] * n if pend is None else pend.tolist()
    r_got = step_rate(rows, ms, e, k, p, [m == MODE_SELFSPEC for m in got])
    r_want = step_rate(rows, ms, e, k, p, [m == MODE_SELFSPEC for m in want])
    # the optimum's rate is unique; the set is, up to exact ties of rate
    assert r_got == pytest.approx(r_want, rel=1e-12, abs=0)
    if abs(r_got - r_want) <= 1e-12 * r_want and got != want:
        assert sorted(e[[m == MODE_SELFSPEC for m in got]]) == sorted(e[[m == MODE_SELFSPEC for m in want]])
    assert set(got) <= {MODE_AR, MODE_SELFSPEC}


def test_choice_on_a_larger_batch_is_top_s(tm):
    """64 sequences (past the brute force): the choice is the s largest
    expected rounds for the best s, checked against every s."""
    rng = np.random.default_rng(7)
    e = rng.uniform(1.0, 33.0, 64)
    rows, ms = [1, 64, 512, 4096], [4.0, 4.3, 14.5, 95.0]
    got = tm.choose_modes(rows, ms, e, 32)
    spec = got == MODE_SELFSPEC
    s = int(spec.sum())
    order = np.argsort(-e, kind="stable")
    assert spec[order[:s]].all() and not spec[order[s:]].any()
    rates = []
    for t in range(65):
        sp = np.zeros(64, bool)
        sp[order[:t]] = True
        rates.append(step_rate(rows, ms, e, 32, [1] * 64, sp.tolist()))
    assert rates[s] == pytest.approx(max(rates), rel=1e-12)


def test_choice_validates(tm):
    with pytest.raises(tm.TriError):
        tm.choose_modes([1, 1], [1.0, 2.0], [3.0], 8)          # rows not increasing
    with pytest.raises(tm.TriError):
        tm.choose_modes([1], [0.0], [3.0], 8)                  # time not positive
    with pytest.raises(tm.TriError):
        tm.choose_modes([1], [1.0], [0.5], 8)                  # fewer than one token per round
    with pytest.raises(tm.TriError):
        tm.choose_modes([1], [1.0], [10.0], 8)                 # more than k + 1
    with pytest.raises(tm.TriError):
        tm.choose_modes([1], [1.0], [3.0], 65)                 # block outside [1, 64]
    with pytest.raises(tm.TriError):
        tm.choose_modes([1], [1.0], [3.0], 8, [0])             # no pending row
    assert tm.choose_modes([1], [1.0], [], 8).tolist() == []
