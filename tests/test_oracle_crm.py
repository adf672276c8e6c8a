"""Pins for the packed row-mask format (ScalingAttention, section 4.3.2 and
Appendix E, Algorithm 2)."""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import crm

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_word_counts_match_pages_and_shapes():
    g = json.load(open(os.path.join(GOLD, "crm_word_counts.json")))
    pc = g["paper_case"]
    assert crm.words_per_row(pc["n_tokens"], pc["block"], pc["word_bits"]) == pc["words"]
    for c in g["library_cases"]:
        assert crm.words_per_row(c["n_tokens"], c["block"], c["word_bits"]) == c["words"]
    for w in workloads.WORKLOADS.values():
        assert crm.words_per_row(w.seq_len, 64) == w.mask_words


def test_iterator_hand_examples():
    assert list(crm.crm_active_blocks([0b1011])) == [0, 1, 3]
    assert list(crm.crm_active_blocks([0, 1 << 63])) == [127]
    assert list(crm.crm_active_blocks([0, 0, 0])) == []
    assert list(crm.crm_active_blocks([(1 << 64) - 1])) == list(range(64))
    # ScalingAttention's 32-bit variant: base advances by 32 per word
    assert list(crm.crm_active_blocks([0, 0b10], word_bits=32)) == [33]


def test_iterator_equals_unpack_on_random_words():
    rng = np.random.default_rng(5)
    for trial in range(200):
        wd = int(rng.integers(1, 6))
        kind = trial % 4
        if kind == 0:
            words = rng.integers(0, 2**63, size=wd, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=wd).astype(np.uint64)
        elif kind == 1:
            words = np.zeros(wd, np.uint64)
            words[rng.integers(wd)] = np.uint64(1) << np.uint64(int(rng.integers(64)))
        elif kind == 2:
            words = np.full(wd, np.uint64(2**64 - 1))
        else:
            words = np.where(rng.random(wd) < 0.5, np.uint64(0), np.uint64(2**64 - 1))
        nb = int(rng.integers(max(1, 64 * (wd - 1) + 1), 64 * wd + 1))
        walked = [b for b in crm.crm_active_blocks(words) if b < nb]
        dec = np.flatnonzero(crm.unpack_rows(words[None], nb)[0]).tolist()
        assert walked == dec


def test_two_packers_agree_and_roundtrip():
    rng = np.random.default_rng(6)
    for nk in (1, 5, 63, 64, 65, 130, 1182):
        keep = rng.random((3, 4, nk)) < 0.3
        a = crm.pack_rows(keep)
        b = workloads.pack_bits(keep)
        assert a.dtype == np.uint64 and a.shape == (3, 4, -(-nk // 64))
        assert np.array_equal(a, b)
        assert np.array_equal(crm.unpack_rows(a, nk), keep)


def test_density_definition():
    keep = np.zeros((2, 4, 4), bool)
    keep[0, :, 0] = True
    assert crm.density(keep) == pytest.approx(4 / 32)
