"""Oracle sampling rules (test infrastructure only): greedy choice with
confidence, the diffusion threshold commit, and self-speculation acceptance."""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def vocab_reduce(logits_row) -> Tuple[int, float]:
    """Greedy token and its confidence for one row of logits.

    token = argmax, the lowest id winning exact ties (reading R7); confidence =
    the largest softmax probability = 1 / sum_j exp(l_j - max l) (reading R5,
    the top-1 confidence of [Notes §5.2]).  Temperature 0 throughout (R14).
    """
    l = np.asarray(logits_row, dtype=np.float64)
    m = l.max()
    tok = int(np.flatnonzero(l == m)[0])
    conf = 1.0 / np.exp(l - m).sum()
    return tok, float(conf)


def commit_set(conf: Sequence[float], eligible: Sequence[bool], threshold: float) -> list:
    """Block positions committed by one diffusion step.

    Commit every eligible (still masked) position whose confidence passes the
    threshold, strictly (``conf > threshold``) [Notes §5.2; Blog, FastDiffuser];
    if none passes, commit the single eligible position of highest confidence,
    the lowest position winning ties (reading R6: at least one per step).
    """
    conf = np.asarray(conf, dtype=np.float64)
    el = np.asarray(eligible, dtype=bool)
    if not el.any():
        return []
    s = [i for i in range(len(conf)) if el[i] and conf[i] > threshold]
    if s:
        return s
    best = None
    for i in range(len(conf)):
        if el[i] and (best is None or conf[i] > conf[best]):
            best = i
    return [best]


def accept_length(draft: Sequence[int], ar: Sequence[int]) -> int:
    """Self-speculation acceptance: the longest prefix of the drafts that
    matches the AR pathway's greedy tokens, stopping at the first mismatch
    [Notes §5.3; Digest, Method].  ``draft`` has k entries, ``ar`` k + 1; the
    round then commits ar[0..a], so 1..k+1 tokens."""
    k = len(draft)
    for i in range(k):
        if draft[i] != ar[i]:
            return i
    return k
