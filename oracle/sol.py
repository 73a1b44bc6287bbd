"""Oracle of the speed-of-light (SOL) analysis -- TEST INFRASTRUCTURE ONLY.

The pages estimate the headroom of diffusion mode ([Notes] §7; [Abstract];
[Digest] Key Contributions): serial denoising first gives the sequence the
model converges to, then one asks which positions could have been committed
in parallel while still reaching that same result (the pages report about
7.6 tokens per step at block 32 for the trained 8B model).

Reading R20 (the plainest one the rest supports):
* serial denoising = the diffusion block with one commit per forward: the
  most confident masked position (lowest position on ties), i.e. the
  threshold rule at threshold 1, which no confidence exceeds;
* the SOL pass restarts from the same state and, at every forward, commits
  every masked position whose greedy prediction already equals its target
  token; when none does it commits the next position of the serial order
  (with its target token), so every forward commits at least one and the
  pass ends with the target block;
* SOL tokens per forward = block / (SOL forwards); the serial pass takes
  block forwards.  The pages' lower "real" SOL TPF is not derived here.

Both passes run the pending tokens as clean rows in their first forward,
like a diffusion block.  The session ends as after the serial block (the
state tri-mode decoding at threshold 1 reaches), so blocks chain over a
generation; the SOL pass runs on a fork and is not counted in its forwards.
"""
from __future__ import annotations

import copy
from typing import List

from .model import Row
from .sampler import commit_set, vocab_reduce


def fork(sess):
    """A session sharing the model with its own tokens, cache and counters."""
    f = copy.copy(sess)
    f.cache = sess.cache.copy()
    f.tokens = list(sess.tokens)
    f.accepts = list(sess.accepts)
    f.records = []
    return f


def _block_rows(sess, y, first, block):
    L = sess.L
    clean = sess.clean_rows() if first else []
    return clean, clean + [Row(y[i], L + i, L + block) for i in range(block)]


def serial_denoise(sess, block: int):
    """One commit per forward from an all-[MASK] block.  Commits the block to
    ``sess`` and returns (target, serial order of the positions)."""
    mask = sess.model.shape.mask_id
    y: List[int] = [mask] * block
    done = [False] * block
    order: List[int] = []
    first = True
    while not all(done):
        clean, rows = _block_rows(sess, y, first, block)
        logits = sess.run(rows)
        if first:
            sess.kv_append(len(clean))
            first = False
        tok = [0] * block
        conf = [0.0] * block
        for i in range(block):
            if not done[i]:
                tok[i], conf[i] = vocab_reduce(logits[len(clean) + i])
        (i,) = commit_set(conf, [not d for d in done], 1.0)
        y[i] = tok[i]
        done[i] = True
        order.append(i)
    sess.tokens.extend(y)
    sess.rounds += 1
    return y, order


def sol_pass(sess, block: int, target: List[int], order: List[int]):
    """From the state before the block: each forward commits every masked
    position already predicting its target, else the next serial position.
    Returns (forwards, forward index at which each position was committed)."""
    mask = sess.model.shape.mask_id
    y: List[int] = [mask] * block
    done = [False] * block
    step = [-1] * block
    first, forwards = True, 0
    while not all(done):
        clean, rows = _block_rows(sess, y, first, block)
        logits = sess.run(rows)
        if first:
            sess.kv_append(len(clean))
            first = False
        s = [i for i in range(block)
             if not done[i] and vocab_reduce(logits[len(clean) + i])[0] == target[i]]
        if not s:
            s = [next(i for i in order if not done[i])]
        for i in s:
            y[i] = target[i]
            done[i] = True
            step[i] = forwards
        forwards += 1
    return forwards, step


def sol_block(sess, block: int) -> dict:
    """SOL analysis of the session's next block; advances ``sess`` by the
    serial block.  Returns the target, the serial order, the SOL forward of
    every position and the SOL forward count."""
    start = fork(sess)
    target, order = serial_denoise(sess, block)
    forwards, step = sol_pass(start, block, target, order)
    return {"target": target, "order": order, "step": step, "sol_forwards": forwards,
            "tokens_per_forward": block / forwards}
