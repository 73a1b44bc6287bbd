"""Oracle decode loop for the three modes (test infrastructure only).

State (reading R4): the committed tokens x[0..L) and a cache holding causal
K/V for positions [0, kv_len).  Tokens x[kv_len..L) are *pending*: committed
but not yet run through the model.  A forward's rows are the pending tokens as
clean causal rows, optionally followed by a block of rows at [L, L + nb).

* AR [Notes §5.1; Blog, "纯自回归 ar_mode=true"]: one forward over the pending
  rows; the greedy token of the last row is the next token.
* Diffusion [Notes §5.2; Blog, "扩散模式 FastDiffuser"]: a block of B [MASK]
  rows predicting their own positions (reading R2), re-run until every
  position is committed by the threshold rule (readings R5, R6, R8).
* Self-speculation [Notes §5.3; Digest, Method; Blog, "自推测 LinearSpec"]: a
  draft forward (pending rows + k [MASK] rows, LoRA on the mask rows only)
  gives the AR token g0 and k drafts; a causal verify forward over the drafts
  gives g1..gk; the longest matching prefix a is accepted and g0..ga committed
  (1..k+1 tokens), the K/V of the k - a rejected rows rolled back.

* Quadratic self-speculation ([Notes §8.1]; [Blog], performance highlights;
  reading R24): one forward per round verifies the drafts carried from the
  previous round and, for every possible accept length, drafts the next
  block: (k + 1) blocks of k + 1 [MASK] rows, so the forward has
  1 + k + (k + 1)^2 rows.

Every step counts its executed forwards; TPF = committed tokens / forwards,
the draft and verify forwards counted separately (reading R17).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from .model import KVCache, OracleModel, Row, forward
from .sampler import accept_length, commit_set, vocab_reduce

MODE_AR, MODE_DIFFUSION, MODE_SELFSPEC, MODE_QUADSPEC = 0, 1, 2, 3


@dataclasses.dataclass
class ForwardRecord:
    rows: List[Row]
    lora: bool
    logits: Optional[np.ndarray]


class OracleSession:
    def __init__(self, model: OracleModel, max_ctx: int, keep_logits: bool = False,
                 prefill_chunk: int = 64):
        self.model = model
        self.cache = KVCache(model.shape, max_ctx)
        self.tokens: List[int] = []
        self.kv_len = 0
        self.forwards = 0
        self.rounds = 0
        self.accepts: List[int] = []
        self.keep_logits = keep_logits
        self.prefill_chunk = prefill_chunk
        self.records: List[ForwardRecord] = []
        # quadratic self-speculation: drafts for positions L .. L+k-1 carried
        # from the previous round (None: the next round starts without drafts)
        self.qdrafts: Optional[List[int]] = None

    # -- basic pieces ---------------------------------------------------
    @property
    def L(self) -> int:
        return len(self.tokens)

    def run(self, rows: List[Row], lora: bool = False, count: bool = True) -> np.ndarray:
        logits = forward(self.model, self.cache, rows, lora_enabled=lora)
        if count:
            self.forwards += 1
        self.records.append(ForwardRecord(rows, lora, logits if self.keep_logits else None))
        return logits

    def clean_rows(self) -> List[Row]:
        """The pending tokens as clean causal rows (hi = pos + 1)."""
        return [Row(self.tokens[p], p, p + 1) for p in range(self.kv_len, self.L)]

    def prefill(self, prompt) -> None:
        """Run x[0..P-1) causally into the cache; x[P-1] stays pending (R15).
        Not counted as decode forwards."""
        self.qdrafts = None
        toks = [int(t) for t in prompt]
        if not toks:
            raise ValueError("empty prompt")
        self.tokens = toks
        self.kv_len = 0
        n = len(toks) - 1
        for s in range(0, n, self.prefill_chunk):
            e = min(n, s + self.prefill_chunk)
            self.run([Row(toks[p], p, p + 1) for p in range(s, e)], count=False)
        self.kv_len = n

    def kv_append(self, n: int) -> None:
        if self.kv_len + n > self.L:
            raise ValueError("append beyond committed tokens")
        self.kv_len += n

    def kv_rollback(self, n: int) -> None:
        if n < 0 or n > self.kv_len:
            raise ValueError("bad rollback")
        self.kv_len -= n
        self.qdrafts = None

    # -- the three modes -------------------------------------------------
    def ar_step(self) -> List[int]:
        self.qdrafts = None
        rows = self.clean_rows()
        logits = self.run(rows)
        g, _ = vocab_reduce(logits[-1])
        self.kv_append(len(rows))
        self.tokens.append(g)
        self.rounds += 1
        return [g]

    def diffusion_block(self, block: int, threshold: float) -> List[int]:
        self.qdrafts = None
        mask = self.model.shape.mask_id
        L = self.L
        y = [mask] * block
        done = [False] * block
        first = True
        while not all(done):
            clean = self.clean_rows() if first else []
            rows = clean + [Row(y[i], L + i, L + block) for i in range(block)]
            logits = self.run(rows)
            if first:
                self.kv_append(len(clean))
                first = False
            tok = [0] * block
            conf = [0.0] * block
            for i in range(block):
                if not done[i]:
                    tok[i], conf[i] = vocab_reduce(logits[len(clean) + i])
            for i in commit_set(conf, [not d for d in done], threshold):
                y[i] = tok[i]
                done[i] = True
        self.tokens.extend(y)
        self.rounds += 1
        return y

    def diffusion_block_scheduled(self, block: int, counts: List[int]) -> List[int]:
        """A diffusion block whose t-th forward commits the min(counts[t mod
        len(counts)], remaining) most confident masked positions (lowest
        position on ties), each with its greedy token.  A controlled stand-in
        for a trained sampler's commit rate (the pages report about 2.6x TPF
        for diffusion mode, [Blog] performance highlights): the forwards are
        those of the threshold rule, only the number committed is fixed."""
        if not counts or min(counts) < 1:
            raise ValueError("commit counts must be >= 1")
        self.qdrafts = None
        mask = self.model.shape.mask_id
        L = self.L
        y = [mask] * block
        done = [False] * block
        first, t = True, 0
        while not all(done):
            clean = self.clean_rows() if first else []
            rows = clean + [Row(y[i], L + i, L + block) for i in range(block)]
            logits = self.run(rows)
            if first:
                self.kv_append(len(clean))
                first = False
            cand = []
            for i in range(block):
                if not done[i]:
                    tok, conf = vocab_reduce(logits[len(clean) + i])
                    cand.append((-conf, i, tok))
            cand.sort()
            for _, i, tok in cand[: counts[t % len(counts)]]:
                y[i] = tok
                done[i] = True
            t += 1
        self.tokens.extend(y)
        self.rounds += 1
        return y

    def draft(self, k: int, lora: bool = False):
        """The draft forward: returns (g0, drafts) and appends the pending rows."""
        mask = self.model.shape.mask_id
        L = self.L
        clean = self.clean_rows()
        rows = clean + [Row(mask, L + i, L + k, lora=True) for i in range(k)]
        logits = self.run(rows, lora=lora)
        g0, _ = vocab_reduce(logits[len(clean) - 1])
        d = [vocab_reduce(logits[len(clean) + i])[0] for i in range(k)]
        self.kv_append(len(clean))
        return g0, d

    def verify(self, d: List[int]) -> List[int]:
        """The verify forward over the drafts as causal rows: returns g1..gk."""
        L = self.L
        rows = [Row(d[i], L + i, L + i + 1) for i in range(len(d))]
        logits = self.run(rows)
        return [vocab_reduce(logits[i])[0] for i in range(len(d))]

    def selfspec_round(self, k: int, lora: bool = False) -> List[int]:
        self.qdrafts = None
        g0, d = self.draft(k, lora)
        g = [g0] + self.verify(d)
        a = accept_length(d, g)
        L = self.L
        self.tokens.extend(g[: a + 1])
        self.kv_len = L + a          # append the k verify rows, roll back k - a
        self.rounds += 1
        self.accepts.append(a)
        return g[: a + 1]

    def quad_rows(self, k: int):
        """The rows of one quadratic round (reading R24): the clean rows (the
        pending tokens, then the carried drafts at L .. L+len(drafts)-1, hi =
        pos + 1) and, for b = 0 .. len(drafts), block b: k + 1 [MASK] rows at
        L+b .. L+b+k (LoRA rows) that see the clean stream [0, L+b) and each
        other."""
        mask = self.model.shape.mask_id
        L = self.L
        drafts = self.qdrafts or []
        clean = self.clean_rows() + [Row(t, L + i, L + i + 1) for i, t in enumerate(drafts)]
        blocks = [[Row(mask, L + b + j, L + b + k + 1, lora=True) for j in range(k + 1)]
                  for b in range(len(drafts) + 1)]
        return clean, blocks

    def quad_forward(self, clean: List[Row], blocks: List[List[Row]], lora: bool = False):
        """One forward over the rows of quad_rows: the clean rows run into the
        cache; each block runs on a copy of that cache, where its own K/V take
        positions L+b .. L+b+k, so a block sees [0, L+b) of the clean stream and
        itself, never the drafts past L+b or another block.  Returns the clean
        rows' logits and each block's logits; counts one forward."""
        logits = forward(self.model, self.cache, clean)
        blk = [forward(self.model, self.cache.copy(), rows, lora_enabled=lora) for rows in blocks]
        self.forwards += 1
        self.records.append(ForwardRecord(clean + [r for rows in blocks for r in rows], lora,
                                          np.concatenate([logits] + blk) if self.keep_logits else None))
        return logits, blk

    def quad_round(self, k: int, lora: bool = False) -> List[int]:
        """One round of quadratic self-speculation (reading R24).  The AR
        pathway verifies the carried drafts d_0..d_{n-1} (n = k, or 0 on the
        first round and after any other step): g_0 is the greedy token of the
        last pending row, g_{i+1} that of draft row i.  a = accept_length(d, g);
        g_0..g_a are committed (1..n+1 tokens); the K/V of the pending rows and
        of d_0..d_{a-1} stay, the rest is rolled back; g_a becomes the pending
        token.  The next drafts are block a's greedy tokens at L+a+1 .. L+a+k
        (its row at L+a, the position g_a now holds, is not used)."""
        if not 1 <= k <= 63:
            raise ValueError("quadratic self-speculation needs 1 <= k <= 63")
        L = self.L
        c = L - self.kv_len
        drafts = self.qdrafts or []
        clean, blocks = self.quad_rows(k)
        logits, blk = self.quad_forward(clean, blocks, lora)
        g = [vocab_reduce(logits[c - 1 + i])[0] for i in range(len(drafts) + 1)]
        a = accept_length(drafts, g)
        self.tokens.extend(g[: a + 1])
        self.kv_len = L + a
        self.qdrafts = [vocab_reduce(blk[a][1 + i])[0] for i in range(k)]
        self.rounds += 1
        self.accepts.append(a)
        return g[: a + 1]

    def mixed_step(self, mode: int, k: int, lora: bool = False) -> List[int]:
        """One step of a mixed batch (reading R19): two forwards, in which an
        AR sequence commits a greedy token in each and a self-speculation
        sequence runs one draft + verify round.  Sequences do not interact, so
        a mixed batch is each sequence taking its own step."""
        if mode == MODE_AR:
            return self.ar_step() + self.ar_step()
        if mode == MODE_SELFSPEC:
            return self.selfspec_round(k, lora)
        raise ValueError(f"mode {mode} cannot take part in a mixed step")

    def generate(self, mode: int, n_new: int, block: int = 32, threshold: float = 0.9,
                 lora: bool = False) -> List[int]:
        """Generate exactly ``n_new`` tokens (no EOS, overshoot truncated: R13)."""
        out: List[int] = []
        while len(out) < n_new:
            if mode == MODE_AR:
                out += self.ar_step()
            elif mode == MODE_DIFFUSION:
                out += self.diffusion_block(block, threshold)
            elif mode == MODE_SELFSPEC:
                out += self.selfspec_round(block, lora)
            elif mode == MODE_QUADSPEC:
                out += self.quad_round(block, lora)
            else:
                raise ValueError(f"bad mode {mode}")
        return out[:n_new]
