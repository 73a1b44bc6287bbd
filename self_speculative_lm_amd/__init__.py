"""Python binding of libtrimode.so: the MI355X tri-mode (AR / block diffusion /
self-speculation) decode step.

Argument marshalling only: every step of the decode path runs in the library's
HIP kernels.  PyTorch provides device memory and the stream.  There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import numpy as np

from ._lib import (TRI_AR, TRI_BF16, TRI_BF16_V16, TRI_DIFFUSION, TRI_F32, TRI_QUADSPEC, TRI_SELFSPEC, ModelDesc, SeqStats, TriError,  # noqa: F401
                   check, lib)

__all__ = ["Model", "Session", "block_causal_attn", "block_causal_attn_noalloc", "sample_commit", "verify_accept", "weight_names", "choose_modes",
           "TriError", "TRI_AR", "TRI_DIFFUSION", "TRI_SELFSPEC", "TRI_QUADSPEC", "TRI_F32", "TRI_BF16", "TRI_BF16_V16"]


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ip(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def weight_names(n_layers: int, lora_rank: int = 0) -> List[str]:
    """Names of the weight pointers in the order tri_model_create takes them."""
    names = ["embed"]
    for l in range(n_layers):
        p = f"layers.{l}."
        names += [p + s for s in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm", "ffn_norm")]
    names += ["final_norm", "lm_head"]
    if lora_rank > 0:
        for l in range(n_layers):
            names += [f"lora.{l}.a", f"lora.{l}.b"]
    return names


class Model:
    """tri_model: the weights are copied/repacked into a torch-allocated model
    buffer (kept here); the caller's weight tensors may be dropped afterwards."""

    def __init__(self, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, weights,
                 dtype: int = TRI_BF16, rope_base: float = 10000.0, rms_eps: float = 1e-6, lora_rank: int = 0,
                 stream=None):
        torch = _torch()
        names = weight_names(n_layers, lora_rank)
        if isinstance(weights, dict):
            weights = [weights[n] for n in names]
        weights = list(weights)
        self.desc = ModelDesc(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, rope_base, rms_eps,
                              dtype, lora_rank)
        n = ctypes.c_size_t()
        check(lib().tri_model_bytes(ctypes.byref(self.desc), ctypes.byref(n)))
        self.buffer = torch.empty(n.value + 256, dtype=torch.uint8, device=weights[0].device)
        off = (-self.buffer.data_ptr()) % 256
        arr = (ctypes.c_void_p * len(weights))(*[w.data_ptr() for w in weights])
        h = ctypes.c_void_p()
        check(lib().tri_model_create(ctypes.byref(self.desc), arr, len(weights), self.buffer.data_ptr() + off,
                                     n.value, _stream(stream), ctypes.byref(h)))
        self.handle = h
        self.vocab = vocab

    def close(self):
        if getattr(self, "handle", None):
            try:
                lib().tri_model_destroy(self.handle)
            except Exception:  # interpreter shutdown
                pass
            self.handle = None

    def __del__(self):
        self.close()


class Session:
    """tri_session with a torch-allocated device workspace."""

    def __init__(self, model: Model, max_batch: int, max_ctx: int, max_rows: int, device="cuda", stream=None):
        torch = _torch()
        self.model = model
        self.max_batch, self.max_ctx, self.max_rows = max_batch, max_ctx, max_rows
        n = ctypes.c_size_t()
        check(lib().tri_session_bytes(model.handle, max_batch, max_ctx, max_rows, ctypes.byref(n)))
        self.workspace = torch.empty(n.value + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        off = (-base) % 256
        self.stream = stream
        h = ctypes.c_void_p()
        check(lib().tri_session_create(model.handle, max_batch, max_ctx, max_rows, base + off, n.value,
                                       _stream(stream), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            try:
                lib().tri_session_destroy(self.handle)
            except Exception:  # interpreter shutdown
                pass
            self.handle = None

    def __del__(self):
        self.close()

    def prefill(self, seq: int, tokens) -> None:
        t = _i32(tokens)
        check(lib().tri_prefill(self.handle, seq, _ip(t), len(t)))

    def decode_step(self, mode: int, block: int = 1, threshold: float = 0.0):
        """Returns (tokens [max_batch][block+1] with -1 padding, stats list)."""
        out = np.full((self.max_batch, block + 1), -1, dtype=np.int32)
        st = (SeqStats * self.max_batch)()
        check(lib().tri_decode_step(self.handle, mode, block, float(threshold), _ip(out), st))
        return out, [(s.n_committed, s.n_forwards, s.accept_len, s.n_flags) for s in st]

    def decode_step_mixed(self, modes, block: int = 32):
        """One mixed step; modes[b] in {TRI_AR, TRI_SELFSPEC} or < 0 (not
        stepped).  Returns (tokens [max_batch][block+1] -1 padded, stats list)."""
        m = _i32(modes)
        if m.shape != (self.max_batch,):
            raise ValueError(f"modes must have {self.max_batch} entries")
        out = np.full((self.max_batch, block + 1), -1, dtype=np.int32)
        st = (SeqStats * self.max_batch)()
        check(lib().tri_decode_step_mixed(self.handle, _ip(m), block, _ip(out), st))
        return out, [(s.n_committed, s.n_forwards, s.accept_len, s.n_flags) for s in st]

    def sol_block(self, block: int = 32):
        """Speed-of-light analysis of every prefilled sequence's next block;
        the sequences advance by the serial block.  Returns a dict of arrays
        target, order, step ([max_batch][block]) and forwards ([max_batch]),
        -1 for sequences not prefilled."""
        tgt = np.full((self.max_batch, block), -1, dtype=np.int32)
        order, step = tgt.copy(), tgt.copy()
        fw = np.full(self.max_batch, -1, dtype=np.int32)
        check(lib().tri_sol_block(self.handle, block, _ip(tgt), _ip(order), _ip(step), _ip(fw)))
        return {"target": tgt, "order": order, "step": step, "forwards": fw}

    def set_lora(self, enabled: bool) -> None:
        check(lib().tri_set_lora(self.handle, int(bool(enabled))))

    def kv_append(self, seq: int, n: int) -> None:
        check(lib().kv_append(self.handle, seq, n))

    def kv_rollback(self, seq: int, n: int) -> None:
        check(lib().kv_rollback(self.handle, seq, n))

    def state(self, seq: int):
        """(committed tokens list, kv_len)."""
        L, kv = ctypes.c_int(), ctypes.c_int()
        check(lib().tri_get_state(self.handle, seq, ctypes.byref(L), ctypes.byref(kv), None, 0))
        toks = np.zeros(max(L.value, 1), dtype=np.int32)
        check(lib().tri_get_state(self.handle, seq, None, None, _ip(toks), L.value))
        return toks[: L.value].tolist(), kv.value

    def forward(self, seq, tok, pos, hi, lora=None, logits=None):
        """Teacher-forced forward over explicit rows; returns (tok, conf) numpy arrays."""
        seq, tok, pos, hi = _i32(seq), _i32(tok), _i32(pos), _i32(hi)
        lo = _i32(lora) if lora is not None else np.zeros_like(seq)
        n = len(seq)
        ot = np.zeros(n, dtype=np.int32)
        oc = np.zeros(n, dtype=np.float32)
        check(lib().tri_forward(self.handle, n, _ip(seq), _ip(tok), _ip(pos), _ip(hi), _ip(lo), _ptr(logits),
                                _ip(ot), oc.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
        return ot, oc

    def forward_bytes(self, rows_per_seq: int) -> float:
        b = ctypes.c_double()
        check(lib().tri_forward_bytes(self.handle, rows_per_seq, ctypes.byref(b)))
        return b.value

    def set_trace(self, enabled: bool) -> None:
        check(lib().tri_set_trace(self.handle, int(bool(enabled))))

    def trace(self) -> list:
        """Recorded forwards: list of dicts with rows and logits (or None)."""
        n = ctypes.c_int()
        check(lib().tri_trace_count(self.handle, ctypes.byref(n)))
        out = []
        for i in range(n.value):
            nr, hl = ctypes.c_int(), ctypes.c_int()
            check(lib().tri_trace_get(self.handle, i, ctypes.byref(nr), None, None, None, None, None, None, 0,
                                      ctypes.byref(hl)))
            r = nr.value
            a = {k: np.zeros(r, dtype=np.int32) for k in ("seq", "tok", "pos", "hi", "lora")}
            lg = np.zeros((r, self.model.vocab), dtype=np.float32) if hl.value else None
            check(lib().tri_trace_get(self.handle, i, ctypes.byref(nr), _ip(a["seq"]), _ip(a["tok"]), _ip(a["pos"]),
                                      _ip(a["hi"]), _ip(a["lora"]),
                                      lg.ctypes.data_as(ctypes.POINTER(ctypes.c_float)) if lg is not None else None,
                                      r, ctypes.byref(hl)))
            a["logits"] = lg
            out.append(a)
        return out

    def set_commit_schedule(self, seq: int, counts=None) -> None:
        """Diffusion forwards of `seq` commit counts[t % len] most confident
        positions (None or empty: the threshold rule again)."""
        if not counts:
            check(lib().tri_set_commit_schedule(self.handle, seq, None, 0))
            return
        c = _i32(counts)
        check(lib().tri_set_commit_schedule(self.handle, seq, _ip(c), len(c)))

    def set_draft_override(self, seq: int, ref=None, a_star: int = -1) -> None:
        if a_star < 0 or ref is None:
            check(lib().tri_set_draft_override(self.handle, seq, None, 0, -1))
            return
        r = _i32(ref)
        check(lib().tri_set_draft_override(self.handle, seq, _ip(r), len(r), int(a_star)))

    def profile(self, kernel_class: int) -> None:
        check(lib().tri_profile(self.handle, kernel_class))

    def profile_read(self):
        ms, n = ctypes.c_double(), ctypes.c_int()
        check(lib().tri_profile_read(self.handle, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value


def choose_modes(grid_rows, grid_ms, expected, block: int, pending=None) -> np.ndarray:
    """Per-sequence TRI_AR / TRI_SELFSPEC for one mixed step from a measured
    forward-cost curve (rows -> ms) and each sequence's expected tokens per
    self-speculation round (tri_choose_modes)."""
    gr = _i32(grid_rows)
    gm = np.ascontiguousarray(np.asarray(grid_ms, dtype=np.float64))
    e = np.ascontiguousarray(np.asarray(expected, dtype=np.float64))
    if gr.shape != gm.shape:
        raise ValueError("grid_rows and grid_ms differ in length")
    pd = None if pending is None else _i32(pending)
    if pd is not None and pd.shape != e.shape:
        raise ValueError("pending must match expected")
    out = np.zeros(len(e), dtype=np.int32)
    dp = ctypes.POINTER(ctypes.c_double)
    check(lib().tri_choose_modes(_ip(gr), gm.ctypes.data_as(dp), len(gr), len(e), e.ctypes.data_as(dp),
                                 None if pd is None else _ip(pd), block, _ip(out)))
    return out


# ----------------------------------------------------------- kernel-level calls
def block_causal_attn_ws_bytes(rows: int, hq: int, hd: int, max_hi: int, kv_split: int = 0) -> int:
    n = ctypes.c_size_t()
    check(lib().block_causal_attn_ws_bytes(rows, hq, hd, max_hi, kv_split, ctypes.byref(n)))
    return n.value


def block_causal_attn(q, k_cache, v_cache, seq_start, row_hi, out, scale: float, *, max_rows_per_seq: int,
                      max_hi: int, kv_split: int = 0, ws=None, dtype: Optional[int] = None, stream=None):
    """q [rows, hq, hd]; k_cache [n_seq, hkv, ctx, hd]; v_cache [n_seq, hkv, hd, ctx] (transposed);
    seq_start int32 [n_seq+1]; row_hi int32 [rows]; out like q.  Device tensors.  A float16 v_cache
    with bfloat16 q selects TRI_BF16_V16 (the session's fp16 form of the V cache)."""
    torch = _torch()
    rows, hq, hd = q.shape
    n_seq, hkv, ctx, _ = k_cache.shape
    if dtype is None:
        if q.dtype == torch.bfloat16:
            dtype = TRI_BF16_V16 if v_cache.dtype == torch.float16 else TRI_BF16
        else:
            dtype = TRI_F32
    need = block_causal_attn_ws_bytes(rows, hq, hd, max_hi, kv_split)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    check(lib().block_causal_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), n_seq, _ptr(seq_start), _ptr(row_hi), rows,
                                  max_rows_per_seq, max_hi, hq, hkv, hd, ctx, float(scale), dtype, kv_split,
                                  _ptr(out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def block_causal_attn_noalloc(q, k_cache, v_cache, seq_start, row_hi, out, scale: float, *, max_rows_per_seq: int,
                              max_hi: int, kv_split: int = 0, dtype: Optional[int] = None, stream=None):
    """block_causal_attn with the split partials in the library's static device
    scratch (no workspace; for callers that cannot allocate)."""
    torch = _torch()
    rows, hq, hd = q.shape
    n_seq, hkv, ctx, _ = k_cache.shape
    if dtype is None:
        if q.dtype == torch.bfloat16:
            dtype = TRI_BF16_V16 if v_cache.dtype == torch.float16 else TRI_BF16
        else:
            dtype = TRI_F32
    check(lib().block_causal_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), n_seq, _ptr(seq_start),
                                          _ptr(row_hi), rows, max_rows_per_seq, max_hi, hq, hkv, hd, ctx, float(scale),
                                          dtype, kv_split, _ptr(out), _stream(stream)))
    return out


def sample_commit_ws_bytes(rows: int, vocab: int) -> int:
    n = ctypes.c_size_t()
    check(lib().sample_commit_ws_bytes(rows, vocab, ctypes.byref(n)))
    return n.value


def sample_commit(logits, row_kind, block_start, threshold: float, out_tok, out_conf, out_commit, out_status,
                  ws=None, stream=None):
    """logits float32 [rows, vocab]; row_kind int32 [rows]; block_start int32 [n_blocks+1] or None."""
    torch = _torch()
    rows, vocab = logits.shape
    nb = 0 if block_start is None else block_start.numel() - 1
    if ws is None:
        ws = torch.empty(sample_commit_ws_bytes(rows, vocab), dtype=torch.uint8, device=logits.device)
    check(lib().sample_commit(_ptr(logits), rows, vocab, _ptr(row_kind), _ptr(block_start), nb, float(threshold),
                              _ptr(out_tok), _ptr(out_conf), _ptr(out_commit), _ptr(out_status), _ptr(ws),
                              ws.numel(), _stream(stream)))


def verify_accept(draft, ar_tok, accept_len, committed, kv_len=None, stream=None):
    """draft int32 [b, k]; ar_tok int32 [b, k+1]; accept_len [b]; committed [b, k+1]; kv_len [b] or None."""
    b, k = draft.shape
    check(lib().verify_accept(_ptr(draft), _ptr(ar_tok), b, k, _ptr(accept_len), _ptr(committed), _ptr(kv_len),
                              _stream(stream)))
