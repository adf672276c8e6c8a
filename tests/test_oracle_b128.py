"""Pins for ScalingAttention's own mask granularity: 128-token blocks in 32-bit row-mask
words (ScalingAttention, section 4.3.2: one 32-bit load covers 32 KV blocks of
128 tokens; Appendix E, Algorithm 2 advances its base by the word width)."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import crm
from oracle.attention import sparse_attention

B = 128


def _rand(H, n, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((H, n, d)) for _ in range(3)]


def _sdpa(q, k, v, scale):
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t, scale=scale).numpy()


def test_32bit_decode_equals_algorithm_2_walk():
    rng = np.random.default_rng(11)
    for trial in range(300):
        wd = int(rng.integers(1, 5))
        kind = trial % 4
        if kind == 0:
            words = rng.integers(0, 2**32, size=wd, dtype=np.uint64).astype(np.uint32)
        elif kind == 1:
            words = np.zeros(wd, np.uint32)
            words[rng.integers(wd)] = np.uint32(1) << np.uint32(int(rng.integers(32)))
        elif kind == 2:
            words = np.full(wd, np.uint32(2**32 - 1))
        else:
            words = np.where(rng.random(wd) < 0.5, np.uint32(0), np.uint32(2**32 - 1))
        nb = int(rng.integers(max(1, 32 * (wd - 1) + 1), 32 * wd + 1))
        walked = [b for b in crm.crm_active_blocks(words, word_bits=32) if b < nb]
        dec = np.flatnonzero(crm.unpack_rows32(words[None], nb)[0]).tolist()
        assert walked == dec


def test_32bit_hand_examples_and_packer_roundtrip():
    w = np.array([[0b1011, 1 << 31]], np.uint32)
    assert np.flatnonzero(crm.unpack_rows32(w, 64)[0]).tolist() == [0, 1, 3, 63]
    rng = np.random.default_rng(12)
    for nk in (1, 31, 32, 33, 64, 591):
        keep = rng.random((2, 3, nk)) < 0.4
        words = workloads.pack_bits32(keep)
        assert words.dtype == np.uint32 and words.shape == (2, 3, -(-nk // 32))
        assert np.array_equal(crm.unpack_rows32(words, nk), keep)


def test_word_counts_coincide_across_formats():
    """ceil(ceil(N/128)/32) = ceil(N/4096) = ceil(ceil(N/64)/64): a 32-bit row of
    128-token blocks has as many words as a 64-bit row of 64-token blocks; the
    paper's 256k-token case needs 64."""
    assert crm.words_per_row(262144, 128, 32) == 64
    for n in (1, 64, 128, 4095, 4096, 4097, 32760, 75600, 126720, 262144):
        assert crm.words_per_row(n, 128, 32) == crm.words_per_row(n, 64, 64) == -(-n // 4096)


def test_refine_hand_example():
    keep = np.array([[True, False], [False, True]])
    # N = 200 tokens: two 128-blocks, four 64-blocks, the last 128-block short
    fine = crm.refine_blocks(keep, 2, 4)
    assert fine.astype(int).tolist() == [[1, 1, 0, 0], [1, 1, 0, 0], [0, 0, 1, 1], [0, 0, 1, 1]]
    # N = 150: the last 128-block holds 22 tokens, one 64-block
    assert crm.refine_blocks(keep, 2, 3).astype(int).tolist() == [[1, 1, 0], [1, 1, 0], [0, 0, 1]]


@pytest.mark.parametrize("n", [256, 300, 330, 4 * B + 1])
def test_all_ones_and_diagonal_at_128(n):
    H, d = 2, 8
    q, k, v = _rand(H, n, d, 21)
    nb = -(-n // B)
    ones = crm.pack_rows(np.ones((H, nb, nb), bool))
    assert np.max(np.abs(sparse_attention(q, k, v, ones, 0.4, block=B) - _sdpa(q, k, v, 0.4))) <= 1e-12
    diag = np.zeros((H, nb, nb), bool)
    diag[:, np.arange(nb), np.arange(nb)] = True
    out = sparse_attention(q, k, v, crm.pack_rows(diag), 0.4, block=B)
    for u in range(nb):
        sl = slice(u * B, min(n, (u + 1) * B))
        assert np.max(np.abs(out[:, sl] - _sdpa(q[:, sl], k[:, sl], v[:, sl], 0.4))) <= 1e-12


def test_brute_force_at_128_from_32bit_words():
    """Per-query softmax over the keys Algorithm 2 lists from the 32-bit words."""
    n, d, scale = 3 * B + 45, 4, 0.7
    rng = np.random.default_rng(22)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    nb = -(-n // B)
    keep = rng.random((nb, nb)) < 0.5
    keep[1] = False
    words = workloads.pack_bits32(keep)
    got = sparse_attention(q[None], k[None], v[None],
                           crm.pack_rows(crm.unpack_rows32(words, nb))[None], scale, block=B)[0]
    for i in range(0, n, 7):
        blocks = list(crm.crm_active_blocks(words[i // B], word_bits=32))
        keys = [j for b in blocks for j in range(b * B, b * B + B) if j < n]
        if not keys:
            assert np.all(got[i] == 0)
            continue
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        ref = [math.fsum(w[t] * v[keys[t], c] for t in range(len(keys))) / z for c in range(d)]
        assert np.max(np.abs(got[i] - ref)) <= 1e-12


@pytest.mark.parametrize("n", [5 * B, 5 * B - 40, 5 * B - 70])
def test_refined_mask_gives_the_same_attention(n):
    """The kept key set of every query is a union of whole 128-token blocks, so
    the same mask written over 64-token blocks must give the same output.  n is
    chosen so that the last 128-block is full, longer than 64, and shorter than
    64 (then it is a single 64-block)."""
    H, d = 2, 8
    q, k, v = _rand(H, n, d, 23)
    nb, nf = -(-n // B), -(-n // 64)
    rng = np.random.default_rng(24)
    keep = rng.random((H, nb, nb)) < 0.4
    keep[0, 2] = False
    coarse = sparse_attention(q, k, v, crm.pack_rows(keep), 0.5, block=B)
    fine = sparse_attention(q, k, v, crm.pack_rows(crm.refine_blocks(keep, 2, nf)), 0.5, block=64)
    assert np.max(np.abs(coarse - fine)) <= 1e-12


def test_planted_mistake_bits_read_as_64_token_blocks_is_caught():
    """Reading each bit of a 128-token row as a 64-token block (a plausible slip
    when both formats meet) keeps the wrong keys; the equality above fails."""
    n, H, d = 4 * B, 1, 8
    q, k, v = _rand(H, n, d, 25)
    keep = np.zeros((H, 4, 4), bool)
    keep[0, :, 0] = True
    keep[0, :, 3] = True
    coarse = sparse_attention(q, k, v, crm.pack_rows(keep), 0.5, block=B)
    nf = 2 * 4
    slip = np.zeros((H, nf, nf), bool)
    slip[..., :4] = np.repeat(keep, 2, axis=1)
    wrong = sparse_attention(q, k, v, crm.pack_rows(slip), 0.5, block=64)
    assert np.max(np.abs(coarse - wrong)) > 1e-3
