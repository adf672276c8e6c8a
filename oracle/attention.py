"""Block-sparse self-attention, float64, written from its definition.

ScalingAttention, section 4.3.2: the CRM kernel is FlashAttention whose dense
KV-block iterator is replaced by a walk over the set bits of the query block's
row mask; inside every kept block the computation stays dense.  The result is
therefore plain softmax attention in which every key outside the kept blocks is
removed:

    for head h, query i (block u = i // B), kept keys K(i) = {j < N : bit(h,u,j//B)}
    s_ij = scale * <q_i, k_j>
    o_i  = sum_{j in K(i)} exp(s_ij - m_i) v_j / sum_{j in K(i)} exp(s_ij - m_i),
           m_i = max_{j in K(i)} s_ij
    o_i  = 0 when K(i) is empty.

Keys j >= N (padding of the last block) do not exist: they are excluded, not
treated as zero vectors.  The operation is full (non-causal) 3D self-attention
over the flattened (frame, height, width) tokens (ScalingAttention, sections 1
and 2.1).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .crm import unpack_rows


def block_output(q, k, v, keep_row, u, scale, block=64):
    """Output rows of query block ``u`` for one head.  q, k, v are [N, d] real
    arrays; keep_row is the boolean row of kept key blocks."""
    n = q.shape[0]
    rows = np.arange(u * block, min(n, (u + 1) * block))
    qs = np.asarray(q[rows], dtype=np.float64)
    kept = np.flatnonzero(keep_row)
    if kept.size == 0:
        return np.zeros((rows.size, v.shape[1]), np.float64)
    keys = (kept[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    keys = keys[keys < n]
    s = (qs @ np.asarray(k[keys], dtype=np.float64).T) * float(scale)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ np.asarray(v[keys], dtype=np.float64)) / p.sum(axis=1, keepdims=True)


def sparse_attention(q, k, v, mask_bits, scale, block=64, blocks=None):
    """Block-sparse attention.

    q, k, v   : [H, N, d] real arrays (exact input values).
    mask_bits : uint64 [H, nb, W] row masks (``crm`` layout).
    blocks    : optional list of (h, u) query blocks; when given, returns a list of
                float64 arrays (one per block, its real rows only); otherwise the
                full float64 output [H, N, d].
    """
    H, n, d = q.shape
    nb = -(-n // block)
    if blocks is None:
        keep = unpack_rows(mask_bits, nb)
        out = np.zeros((H, n, d), np.float64)
        for h in range(H):
            for u in range(nb):
                out[h, u * block: min(n, (u + 1) * block)] = block_output(
                    q[h], k[h], v[h], keep[h, u], u, scale, block)
        return out
    res = []
    for h, u in blocks:
        keep_row = unpack_rows(np.asarray(mask_bits[h, u])[None], nb)[0]
        res.append(block_output(q[h], k[h], v[h], keep_row, u, scale, block))
    return res


def kept_tiles(mask_bits, n_blocks) -> int:
    """Number of kept (query block, key block) pairs: the unit of work whose
    fraction of n_blocks^2 is the density (ScalingAttention, section 5.1)."""
    return int(unpack_rows(mask_bits, n_blocks).sum())
