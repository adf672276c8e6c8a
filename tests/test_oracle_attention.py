"""Pins for the float64 attention oracle: special cases that reduce to library
routines, closed forms, invariants and brute force on tiny inputs."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import workloads
from oracle import crm
from oracle.attention import sparse_attention, kept_tiles

B = 64


def _rand(H, n, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((H, n, d)) for _ in range(3)]


def _sdpa(q, k, v, scale):
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t, scale=scale).numpy()


@pytest.mark.parametrize("n", [64, 200, 257])
def test_all_ones_mask_is_dense_attention(n):
    H, d = 2, 16
    q, k, v = _rand(H, n, d, 1)
    nb = -(-n // B)
    bits = crm.pack_rows(np.ones((H, nb, nb), bool))
    out = sparse_attention(q, k, v, bits, 0.3)
    assert np.max(np.abs(out - _sdpa(q, k, v, 0.3))) <= 1e-12


@pytest.mark.parametrize("n", [128, 200])
def test_diagonal_mask_is_per_block_local_attention(n):
    H, d = 2, 8
    q, k, v = _rand(H, n, d, 2)
    nb = -(-n // B)
    keep = np.zeros((H, nb, nb), bool)
    keep[:, np.arange(nb), np.arange(nb)] = True
    out = sparse_attention(q, k, v, crm.pack_rows(keep), 0.5)
    for u in range(nb):
        sl = slice(u * B, min(n, (u + 1) * B))
        ref = _sdpa(q[:, sl], k[:, sl], v[:, sl], 0.5)
        assert np.max(np.abs(out[:, sl] - ref)) <= 1e-12


def _brute(q, k, v, words, scale, n, rows=None):
    """Per-query softmax over the explicitly listed kept keys, pure Python."""
    d = q.shape[-1]
    out = np.zeros((n, d))
    for i in (range(n) if rows is None else rows):
        blocks = list(crm.crm_active_blocks(words[i // B]))
        keys = [j for b in blocks for j in range(b * B, b * B + B) if j < n]
        if not keys:
            continue
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        for c in range(d):
            out[i, c] = math.fsum(w[t] * v[keys[t], c] for t in range(len(keys))) / z
    return out


def test_brute_force_tiny_random_masks():
    n, d = 4 * B - 17, 4
    q, k, v = _rand(1, n, d, 3)
    rng = np.random.default_rng(3)
    nb = -(-n // B)
    for trial in range(3):
        keep = rng.random((1, nb, nb)) < 0.5
        bits = crm.pack_rows(keep)
        out = sparse_attention(q, k, v, bits, 0.7)
        ref = _brute(q[0], k[0], v[0], bits[0], 0.7, n)
        assert np.max(np.abs(out[0] - ref)) <= 1e-12


def test_brute_force_tiny_workload_rows():
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.qkv(w)
    bits = workloads.pack_bits(workloads.masks(w))
    blocks = [(0, 0), (1, 3)]
    got = sparse_attention(q, k, v, bits, w.scale, blocks=blocks)
    for (h, u), g in zip(blocks, got):
        rows = range(u * B, (u + 1) * B, 7)
        ref = _brute(q[h].astype(np.float64), k[h].astype(np.float64),
                     v[h].astype(np.float64), bits[h], w.scale, w.seq_len, rows)
        g = g[::7]
        assert np.max(np.abs(g - ref[u * B:(u + 1) * B:7])) <= 1e-12


def test_empty_rows_are_zero():
    n, d = 3 * B, 8
    q, k, v = _rand(1, n, d, 4)
    keep = np.ones((1, 3, 3), bool)
    keep[0, 1] = False
    out = sparse_attention(q, k, v, crm.pack_rows(keep), 1.0)
    assert np.all(out[0, B:2 * B] == 0.0)
    assert np.all(np.abs(out[0, :B]) > 0)


def test_zero_queries_average_the_kept_values_closed_form():
    """With q = 0 every kept key has the same logit, so o_i is the plain mean of
    the kept v_j.  V encodes each key's block id in binary, so o_i[c] is the
    token-weighted mean of bit c of the kept block ids (the tail block has only
    its real tokens)."""
    n = 5 * B - 40
    nb = -(-n // B)
    d = 4
    q = np.zeros((1, n, d))
    k = np.random.default_rng(5).standard_normal((1, n, d))
    blk = np.arange(n) // B
    v = np.stack([(blk >> c) & 1 for c in range(d)], axis=1)[None].astype(np.float64)
    rng = np.random.default_rng(5)
    keep = rng.random((1, nb, nb)) < 0.5
    keep[0, 2] = False
    keep[0, 2, [0, 4]] = True
    out = sparse_attention(q, k, v, crm.pack_rows(keep), 1.0)
    tokens = np.array([min(n, (b + 1) * B) - b * B for b in range(nb)], np.float64)
    for u in range(nb):
        kept = np.flatnonzero(keep[0, u])
        if kept.size == 0:
            continue
        for c in range(d):
            want = sum(tokens[b] * ((b >> c) & 1) for b in kept) / tokens[kept].sum()
            assert np.all(np.abs(out[0, u * B:min(n, (u + 1) * B), c] - want) <= 1e-14)
    # row block 2 keeps blocks 0 (64 tokens, id 0) and 4 (24 tokens, id 4 -> bit 2)
    assert out[0, 2 * B, 2] == pytest.approx(24 / 88, abs=1e-15)


def test_constant_values_and_convex_hull():
    n, d = 3 * B + 5, 6
    q, k, v = _rand(1, n, d, 6)
    nb = -(-n // B)
    keep = np.random.default_rng(6).random((1, nb, nb)) < 0.6
    keep[0, :, 0] = True
    bits = crm.pack_rows(keep)
    const = np.full_like(v, 2.5)
    assert np.max(np.abs(sparse_attention(q, k, const, bits, 0.4) - 2.5)) <= 1e-14
    out = sparse_attention(q, k, v, bits, 0.4)
    for u in range(nb):
        keys = np.concatenate([np.arange(b * B, min(n, b * B + B)) for b in np.flatnonzero(keep[0, u])])
        lo, hi = v[0, keys].min(0), v[0, keys].max(0)
        blk = out[0, u * B:min(n, (u + 1) * B)]
        assert np.all(blk >= lo - 1e-12) and np.all(blk <= hi + 1e-12)


def test_merge_identity_over_disjoint_block_sets():
    """Splitting the kept set into A and B: o = (L_A o_A + L_B o_B) / (L_A + L_B)
    with L_X the row's exp-sum over X (log-sum-exp from scipy).  K is scaled so
    the row maximum rises block after block."""
    n, d = 4 * B, 8
    q, k, v = _rand(1, n, d, 7)
    k = k * (1.0 + np.arange(n) // B)[None, :, None]
    nb = 4
    keep = np.ones((1, nb, nb), bool)
    a = keep.copy(); a[..., 1::2] = False
    b = keep.copy(); b[..., 0::2] = False
    o = sparse_attention(q, k, v, crm.pack_rows(keep), 0.5)
    oa = sparse_attention(q, k, v, crm.pack_rows(a), 0.5)
    ob = sparse_attention(q, k, v, crm.pack_rows(b), 0.5)
    s = 0.5 * np.einsum("nd,md->nm", q[0], k[0])
    cols_a = np.concatenate([np.arange(x * B, x * B + B) for x in (0, 2)])
    cols_b = np.concatenate([np.arange(x * B, x * B + B) for x in (1, 3)])
    la = np.exp(logsumexp(s[:, cols_a], axis=1))[:, None]
    lb = np.exp(logsumexp(s[:, cols_b], axis=1))[:, None]
    merged = (la * oa[0] + lb * ob[0]) / (la + lb)
    assert np.max(np.abs(merged - o[0])) <= 1e-10


def test_scale_folds_into_queries():
    n, d = 2 * B + 3, 8
    q, k, v = _rand(2, n, d, 8)
    nb = -(-n // B)
    bits = crm.pack_rows(np.random.default_rng(8).random((2, nb, nb)) < 0.7)
    assert np.max(np.abs(sparse_attention(q, k, v, bits, 0.25) - sparse_attention(0.25 * q, k, v, bits, 1.0))) <= 1e-12


def test_padding_bits_are_ignored():
    n, d = 2 * B + 3, 4
    q, k, v = _rand(1, n, d, 9)
    nb = 3
    keep = np.ones((1, nb, nb), bool)
    bits = crm.pack_rows(keep)
    noisy = bits | np.uint64(0xFFFF_FFFF_FFFF_FFF8)
    assert np.array_equal(sparse_attention(q, k, v, bits, 1.0), sparse_attention(q, k, v, noisy, 1.0))


def test_block_subset_matches_full_output():
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.qkv(w)
    bits = workloads.pack_bits(workloads.masks(w))
    full = sparse_attention(q, k, v, bits, w.scale)
    sub = sparse_attention(q, k, v, bits, w.scale, blocks=[(1, 2)])
    assert np.array_equal(sub[0], full[1, 2 * B:3 * B])
    assert kept_tiles(bits, w.n_blocks) == int(workloads.masks(w).sum())


def test_planted_mistake_zero_padded_keys_is_caught():
    """A plausible oracle mistake -- treating the padding of the last block as
    zero keys -- changes every row that keeps the last block; the dense pin
    above (n not a multiple of 64) catches it."""
    n, d = 200, 16
    q, k, v = _rand(1, n, d, 10)
    npad = 256
    kp = np.concatenate([k, np.zeros((1, npad - n, d))], axis=1)
    vp = np.concatenate([v, np.zeros((1, npad - n, d))], axis=1)
    qp = np.concatenate([q, np.zeros((1, npad - n, d))], axis=1)
    wrong = sparse_attention(qp, kp, vp, crm.pack_rows(np.ones((1, 4, 4), bool)), 0.3)[:, :n]
    assert np.max(np.abs(wrong - _sdpa(q, k, v, 0.3))) > 1e-3
