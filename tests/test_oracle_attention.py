"""Pins for the oracle's per-row-limit attention against the block-causal mask
written out densely from its definition (bidirectional inside a block, causal
across blocks, strictly causal clean prefix), and against torch's SDPA."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.model import attend


def block_ids(prefix_len, block_sizes):
    """Block id of every position: each clean prefix token is its own block
    (strictly causal clean stream), then the noisy blocks in order."""
    ids = list(range(prefix_len))
    nxt = prefix_len
    for b in block_sizes:
        ids += [nxt] * b
        nxt += 1
    return np.array(ids)


def dense_block_causal_mask(ids_q, ids_k):
    """allowed[i, j] iff key j's block is the query's block or an earlier one."""
    return ids_k[None, :] <= ids_q[:, None]


def brute_attention(q, K, V, allowed, group):
    """Masked softmax attention with -inf fill on the dense mask (float64)."""
    nq, hq, hd = q.shape
    out = np.zeros((nq, hq, hd))
    for i in range(nq):
        for h in range(hq):
            s = K[:, h // group, :] @ q[i, h] / np.sqrt(hd)
            s = np.where(allowed[i], s, -np.inf)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[i, h] = p @ V[:, h // group, :]
    return out


def limits_from_mask(allowed):
    """The per-row exclusive key limit hi: the mask of every row must be a prefix."""
    hi = allowed.sum(axis=1)
    for i, h in enumerate(hi):
        assert allowed[i, :h].all() and not allowed[i, h:].any()
    return hi


@pytest.mark.parametrize("prefix,blocks,hq,hkv,hd", [
    (5, [4], 4, 4, 8), (0, [6], 2, 1, 16), (9, [3, 5], 4, 2, 8), (3, [1, 1, 1], 6, 3, 4),
])
def test_attend_matches_dense_block_causal_mask(prefix, blocks, hq, hkv, hd):
    rng = np.random.default_rng(prefix * 7 + hq)
    ids = block_ids(prefix, blocks)
    n = len(ids)
    q = rng.standard_normal((n, hq, hd))
    K = rng.standard_normal((n, hkv, hd))
    V = rng.standard_normal((n, hkv, hd))
    allowed = dense_block_causal_mask(ids, ids)
    hi = limits_from_mask(allowed)
    ref = brute_attention(q, K, V, allowed, hq // hkv)
    got = np.stack([attend(q[i], K, V, int(hi[i]), hq // hkv) for i in range(n)])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_block_limits_are_clean_causal_and_block_end():
    # clean prefix rows: hi = pos + 1; rows of the last block: hi = block end
    ids = block_ids(7, [5])
    hi = limits_from_mask(dense_block_causal_mask(ids, ids))
    np.testing.assert_array_equal(hi[:7], np.arange(1, 8))
    np.testing.assert_array_equal(hi[7:], np.full(5, 12))


def test_block_size_one_is_causal():
    ids = block_ids(4, [1, 1, 1, 1])
    allowed = dense_block_causal_mask(ids, ids)
    np.testing.assert_array_equal(allowed, np.tril(np.ones((8, 8), dtype=bool)))


def test_attend_matches_torch_sdpa_with_gqa():
    rng = np.random.default_rng(3)
    prefix, B, hq, hkv, hd = 11, 6, 8, 2, 16
    ids = block_ids(prefix, [B])
    n = len(ids)
    q = rng.standard_normal((n, hq, hd))
    K = rng.standard_normal((n, hkv, hd))
    V = rng.standard_normal((n, hkv, hd))
    allowed = dense_block_causal_mask(ids, ids)
    hi = limits_from_mask(allowed)
    got = np.stack([attend(q[i], K, V, int(hi[i]), hq // hkv) for i in range(n)])
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1, hq, n, hd]
    tk = torch.from_numpy(K).permute(1, 0, 2)[None]
    tv = torch.from_numpy(V).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(allowed),
                                         enable_gqa=True)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
