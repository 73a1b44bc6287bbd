"""Oracle of the concurrency-adaptive mode choice -- TEST INFRASTRUCTURE ONLY.

The pages' deployment rule: one checkpoint serves AR at high concurrency and
self-speculation at low concurrency ([Notes] table of the three modes in §2
and the engineering summary in §11; [Digest] Limitations: the advantage of
self-speculation shrinks at high concurrency, where AR is preferred;
[Abstract]: the model switches modes to keep throughput high across
concurrency levels).  The pages do not say how a server switches.

Reading R19 (the plainest one the rest supports):
* the choice is made per decode step and per sequence;
* a step is one round of two forwards over every stepped sequence: a
  self-speculation sequence runs its draft and verify forwards and commits
  1..k+1 tokens; an AR sequence commits one greedy token in each forward,
  2 tokens per step;
* the first forward carries each sequence's pending rows, plus k [MASK] rows
  for a self-speculation sequence; the second carries one row for an AR
  sequence and the k drafts for a self-speculation sequence;
* the cost of a forward is a measured curve t(rows);
* the choice maximises the step's expected committed tokens per millisecond,
  with each sequence's expected tokens per self-speculation round given
  (for example a running mean of its accepted lengths + 1).

Ties: the fewest self-speculation sequences, then the lowest indices.

This module writes the definition out by brute force over every subset of
the sequences (small batches only).
"""
from __future__ import annotations

import itertools
from typing import List, Optional, Sequence

MODE_AR, MODE_SELFSPEC = 0, 2


def forward_ms(grid_rows: Sequence[int], grid_ms: Sequence[float], rows: float) -> float:
    """Cost of one forward over `rows` rows from the measured points
    (grid_rows strictly increasing): linear between points, the first point's
    time below it, the line through the last two points beyond the last."""
    if len(grid_rows) != len(grid_ms) or not grid_rows:
        raise ValueError("cost grid")
    if any(b <= a for a, b in zip(grid_rows, grid_rows[1:])) or any(t <= 0 for t in grid_ms):
        raise ValueError("cost grid must have increasing rows and positive times")
    if rows <= grid_rows[0] or len(grid_rows) == 1:
        return float(grid_ms[0])
    for i in range(1, len(grid_rows)):
        if rows <= grid_rows[i] or i == len(grid_rows) - 1:
            r0, r1 = grid_rows[i - 1], grid_rows[i]
            t0, t1 = grid_ms[i - 1], grid_ms[i]
            return t0 + (t1 - t0) * (rows - r0) / (r1 - r0)
    raise AssertionError("unreachable")


def step_rows(pending: Sequence[int], spec: Sequence[bool], block: int):
    """Rows of the step's two forwards."""
    rows1 = sum(p + (block if s else 0) for p, s in zip(pending, spec))
    rows2 = sum(block if s else 1 for s in spec)
    return rows1, rows2


def step_rate(grid_rows, grid_ms, expected, block, pending, spec) -> float:
    """Expected committed tokens per millisecond of one step."""
    rows1, rows2 = step_rows(pending, spec, block)
    tokens = sum(e if s else 2.0 for e, s in zip(expected, spec))
    if rows1 == 0:
        return 0.0
    return tokens / (forward_ms(grid_rows, grid_ms, rows1) + forward_ms(grid_rows, grid_ms, rows2))


def choose_modes(grid_rows, grid_ms, expected: Sequence[float], block: int,
                 pending: Optional[Sequence[int]] = None) -> List[int]:
    """Per-sequence mode (MODE_AR or MODE_SELFSPEC) of the best step, by
    enumerating every subset of self-speculation sequences."""
    n = len(expected)
    if n > 16:
        raise ValueError("brute force is for small batches")
    if block < 1:
        raise ValueError("block")
    if any(not (1.0 <= e <= block + 1) for e in expected):
        raise ValueError("expected tokens per round must lie in [1, block + 1]")
    pending = [1] * n if pending is None else list(pending)
    if len(pending) != n or any(p < 1 for p in pending):
        raise ValueError("pending rows")
    best, best_key = None, None
    for size in range(n + 1):
        for idx in itertools.combinations(range(n), size):   # lexicographic: lowest indices first
            spec = [i in idx for i in range(n)]
            rate = step_rate(grid_rows, grid_ms, expected, block, pending, spec)
            if best is None or rate > best_key:
                best, best_key = spec, rate
    return [MODE_SELFSPEC if s else MODE_AR for s in best]
