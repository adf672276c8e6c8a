"""PSA stripe tuples expanded into a block mask.

PSA page (parameterized stripe attention), Figure 3 and Appendix Tables 7-9:
each head's pattern is either "full window" or a pair of stripe descriptions,
(width, offset, stride) along the temporal axis and (width, offset, stride)
along the spatial axis, covering both intra- and inter-frame stripes.  The page
names the parameters and prints the most frequent tuples but never writes the
predicate; the reading implemented here is:

* units: temporal distances in frames, spatial distances in spatial blocks of
  the flattened frame (token positions inside a frame, divided by the block);
* a stripe of width w is the band of w consecutive distances centred on the
  offset o: x = dist - o + floor(w/2) must satisfy 0 <= x < w;
* the stride is the gap between consecutive stripes, so the pattern repeats
  with period w + s: keep when (x mod (w + s)) < w, with a non-negative
  remainder; a stride of 0 stands for an infinite stride (a single band);
* distances are key minus query: dist_t = t(v) - t(u), dist_s = s(v) - s(u);
* a block pair is kept when the head is full window, or when both the temporal
  and the spatial predicate hold.

Block u's frame and spatial block: when the frame holds a whole number of
blocks (F mod B = 0), t(u) = u // (F/B) and s(u) = u mod (F/B); otherwise the
block is placed by its first token: t(u) = (uB) // F, s(u) = ((uB) mod F) // B.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .crm import pack_rows


def in_stripe(dist, width, offset, gap):
    """Stripe predicate on integer distances (numpy arrays)."""
    x = np.asarray(dist, dtype=np.int64) - int(offset) + int(width) // 2
    if gap == 0:
        return (x >= 0) & (x < width)
    return np.mod(x, int(width) + int(gap)) < width


def block_coords(n_blocks, frame_tokens, block=64):
    """(frame index, spatial block index) of every query/key block."""
    u = np.arange(n_blocks, dtype=np.int64)
    if frame_tokens % block == 0:
        per = frame_tokens // block
        return u // per, u % per
    first = u * block
    return first // frame_tokens, (first % frame_tokens) // block


def stripe_keep(params, n_frames, frame_tokens, seq_len, block=64):
    """Boolean block mask [H, nb, nb] from int tuples [H, 7] =
    {full, Tw, To, Ts, Sw, So, Ss}."""
    params = np.asarray(params, dtype=np.int64)
    nb = -(-seq_len // block)
    t, s = block_coords(nb, frame_tokens, block)
    dt = t[None, :] - t[:, None]
    ds = s[None, :] - s[:, None]
    out = np.zeros((params.shape[0], nb, nb), dtype=bool)
    for h, (full, tw, to, ts, sw, so, ss) in enumerate(params.tolist()):
        if full:
            out[h] = True
        else:
            out[h] = in_stripe(dt, tw, to, ts) & in_stripe(ds, sw, so, ss)
    return out


def stripe_mask_bits(params, n_frames, frame_tokens, seq_len, block=64):
    """Packed uint64 row masks [H, nb, ceil(nb/64)] of ``stripe_keep``."""
    return pack_rows(stripe_keep(params, n_frames, frame_tokens, seq_len, block))


def stripe_count_1d(n, width, offset, gap):
    """#{(a, b) in [0, n)^2 : in_stripe(b - a)} -- with whole frames the 2D keep
    count factorises into the temporal count times the spatial count."""
    a = np.arange(n)
    return int(in_stripe(a[None, :] - a[:, None], width, offset, gap).sum())
