"""Compressed Row Mask (CRM): one bit per key block, packed into machine words.

ScalingAttention, section 4.3.2: each query-block row of the attention mask is a
bitmask held in aligned machine words, one bit per KV block, so one word load
covers as many blocks as the word has bits.  Appendix E, Algorithm 2 walks the
set bits of a row in ascending order: it skips all-zero words (advancing a base
index by the word width per word), reports base + count-trailing-zeros of the
current word, and clears the lowest set bit to advance.

The pages use 32-bit words with 128-token blocks; the library's main format is
64-bit words with 64-token blocks, and it also takes ScalingAttention's format.  Word
``w`` bit ``b`` (least significant bit = 0) is key block ``word_bits * w + b``;
bits at positions >= n_blocks are padding and carry no meaning.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def words_per_row(n_tokens: int, block: int, word_bits: int = 64) -> int:
    """Number of mask words per query-block row: ceil(ceil(N / block) / word_bits)."""
    n_blocks = -(-n_tokens // block)
    return -(-n_blocks // word_bits)


def crm_active_blocks(row_words, word_bits: int = 64):
    """Yield the active key-block indices of one mask row, ascending, by walking
    the words the way the CRM forward iterator does (Algorithm 2): the cursor
    starts one word before the row; zero words are skipped while the base
    advances by ``word_bits``; the current index is base + ctz(word); consuming a
    block clears the word's lowest set bit.  The walk ends when the row's words
    are exhausted."""
    words = [int(w) & ((1 << word_bits) - 1) for w in row_words]
    ptr, base, val = 0, -word_bits, 0

    def refill():
        nonlocal ptr, base, val
        while val == 0 and ptr != len(words):
            val = words[ptr]
            ptr += 1
            base += word_bits

    refill()
    while val != 0:
        lowest = val & -val
        yield base + lowest.bit_length() - 1
        val &= val - 1
        if val == 0:
            refill()


def unpack_rows(mask_bits: np.ndarray, n_blocks: int) -> np.ndarray:
    """Decode uint64 words [..., n_q, W] into a boolean mask [..., n_q, n_blocks];
    padding bits beyond ``n_blocks`` are dropped."""
    m = np.ascontiguousarray(mask_bits, dtype=np.uint64)
    shifts = np.arange(64, dtype=np.uint64)
    bits = (m[..., :, None] >> shifts) & np.uint64(1)           # [..., n_q, W, 64]
    bits = bits.reshape(m.shape[:-1] + (m.shape[-1] * 64,))
    return bits[..., :n_blocks].astype(bool)


def unpack_rows32(mask_words: np.ndarray, n_blocks: int) -> np.ndarray:
    """Decode ScalingAttention's 32-bit words [..., n_q, W] into a boolean mask
    [..., n_q, n_blocks] (bit b of word w is key block 32 w + b)."""
    m = np.ascontiguousarray(mask_words, dtype=np.uint32)
    shifts = np.arange(32, dtype=np.uint32)
    bits = (m[..., :, None] >> shifts) & np.uint32(1)           # [..., n_q, W, 32]
    bits = bits.reshape(m.shape[:-1] + (m.shape[-1] * 32,))
    return bits[..., :n_blocks].astype(bool)


def refine_blocks(keep: np.ndarray, factor: int, n_fine: int) -> np.ndarray:
    """The same block mask over blocks ``factor`` times smaller: fine block pair
    (u, v) is kept exactly when coarse pair (u // factor, v // factor) is.
    ``n_fine`` = ceil(N / fine block) may be less than factor * n_coarse when the
    last coarse block is short."""
    keep = np.asarray(keep, dtype=bool)
    u = np.arange(n_fine) // factor
    return keep[..., u[:, None], u[None, :]]


def pack_rows(keep: np.ndarray) -> np.ndarray:
    """Encode a boolean mask [..., n_q, n_k] as uint64 words [..., n_q, ceil(n_k/64)]
    (inverse of ``unpack_rows``; padding bits zero)."""
    keep = np.asarray(keep, dtype=bool)
    nk = keep.shape[-1]
    wd = -(-nk // 64)
    padded = np.zeros(keep.shape[:-1] + (wd * 64,), dtype=np.uint64)
    padded[..., :nk] = keep
    padded = padded.reshape(keep.shape[:-1] + (wd, 64))
    weights = np.uint64(1) << np.arange(64, dtype=np.uint64)
    # distinct powers of two: the sum is the bitwise OR
    return (padded * weights).sum(axis=-1, dtype=np.uint64)


def density(keep: np.ndarray) -> float:
    """Fraction of active blocks (ScalingAttention, Figure 1 caption: density is
    one minus sparsity, the active-block fraction)."""
    keep = np.asarray(keep, dtype=bool)
    return float(keep.sum()) / keep.size
