"""Seeded synthetic inputs for block-sparse video-DiT attention.

This module is shared by the CPU oracle side (tests, the bench's CPU baseline)
and the GPU side (tests, bench, smoke).  It holds input construction only:
random tensors, bf16 rounding of those tensors, synthetic block masks and
stripe parameters drawn at random.  None of the method's arithmetic lives
here -- attention, mask decoding, stripe expansion, block scoring, top-p
selection and the Hilbert order are each implemented separately by the oracle
(``oracle/``) and by the HIP library.

Workloads (one attention layer each, batch folded into heads):

* ``tiny``         fp32, 2 heads, d=64, grid 4x8x8 = 256 tokens (4x4 blocks),
                   scale 1/8, Bernoulli(0.5) block bits with the diagonal on.
* ``wan13b_480p``  bf16, 12 heads, d=128, grid 21x30x52 = 32,760 tokens
                   (512 blocks of 64); band + temporal stripes + random fill,
                   per-head density ~ U[0.10, 0.50].
* ``wan14b_720p``  bf16, 40 heads, d=128, grid 21x45x80 = 75,600 tokens
                   (1182 blocks); 8 full heads, the rest band + random fill at
                   density ~ U[0.05, 0.40].
* ``hunyuan_768``  bf16, 24 heads, d=128, grid 33x48x80 = 126,720 tokens
                   (1980 blocks); per-head stripe tuples, 5 heads full window.
* ``topp_wan14b``  bf16, 40 heads, d=128, grid 21x45x80; Q and K carry a shared
                   per-frame rank-8 component (weight 0.5).

Draw order is fixed and documented per function so that any consumer can
regenerate the same bytes from the seed alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

BLOCK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    n_heads: int
    head_dim: int
    grid: tuple           # (frames, height, width) of latent tokens
    seed: int

    @property
    def seq_len(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def frame_tokens(self) -> int:
        return self.grid[1] * self.grid[2]

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // BLOCK)

    @property
    def mask_words(self) -> int:
        return -(-self.n_blocks // 64)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    "tiny": Workload("tiny", "f32", 2, 64, (4, 8, 8), 0),
    "wan13b_480p": Workload("wan13b_480p", "bf16", 12, 128, (21, 30, 52), 1),
    "wan14b_720p": Workload("wan14b_720p", "bf16", 40, 128, (21, 45, 80), 2),
    "hunyuan_768": Workload("hunyuan_768", "bf16", 24, 128, (33, 48, 80), 3),
    "topp_wan14b": Workload("topp_wan14b", "bf16", 40, 128, (21, 45, 80), 4),
}


# ---------------------------------------------------------------- bf16 plumbing
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw
    16-bit patterns as uint16.  Inputs are finite by construction."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 patterns (uint16) to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- mask plumbing
def pack_bits(keep: np.ndarray) -> np.ndarray:
    """Pack a boolean block mask [..., nq, nk] into uint64 words [..., nq, ceil(nk/64)],
    block b of a row at bit (b % 64) of word (b // 64); padding bits are zero."""
    keep = np.asarray(keep, dtype=bool)
    nk = keep.shape[-1]
    wd = -(-nk // 64)
    pad = wd * 64 - nk
    if pad:
        keep = np.concatenate([keep, np.zeros(keep.shape[:-1] + (pad,), bool)], axis=-1)
    by = np.packbits(keep, axis=-1, bitorder="little")          # [..., wd*8] bytes
    return np.ascontiguousarray(by).view("<u8").reshape(keep.shape[:-1] + (wd,))


def pack_bits32(keep: np.ndarray) -> np.ndarray:
    """Pack a boolean block mask [..., nq, nk] into uint32 words [..., nq, ceil(nk/32)]
    (the 32-bit row-mask format), block b at bit (b % 32) of word (b // 32)."""
    keep = np.asarray(keep, dtype=bool)
    nk = keep.shape[-1]
    wd = -(-nk // 32)
    pad = wd * 32 - nk
    if pad:
        keep = np.concatenate([keep, np.zeros(keep.shape[:-1] + (pad,), bool)], axis=-1)
    by = np.packbits(keep, axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view("<u4").reshape(keep.shape[:-1] + (wd,))


def _fill_random(rng, keep_row_major: np.ndarray, target: int) -> None:
    """Set uniformly random extra cells (without replacement) among the cells that
    are still off, until ``target`` cells are on (no-op when already there)."""
    flat = keep_row_major.reshape(-1)
    have = int(flat.sum())
    if target <= have:
        return
    key = rng.random(flat.size)
    key[flat] = 2.0                                  # never pick cells already on
    pick = np.argpartition(key, target - have - 1)[: target - have]
    flat[pick] = True


def _band(nb: int, half_width: int) -> np.ndarray:
    u = np.arange(nb)
    return np.abs(u[:, None] - u[None, :]) <= half_width


def mask_tiny(w: Workload) -> np.ndarray:
    """Each block bit Bernoulli(0.5), then the diagonal forced on (heads in order)."""
    rng = np.random.default_rng([w.seed, 1])
    nb = w.n_blocks
    keep = rng.random((w.n_heads, nb, nb)) < 0.5
    keep[:, np.arange(nb), np.arange(nb)] = True
    return keep


def mask_wan13b(w: Workload) -> np.ndarray:
    """Band |u-v|<=1, plus temporal stripes (the block holding token 64u + kF for
    every frame shift k != 0 in range), plus random fill to round(rho_h * nb^2),
    rho_h ~ U[0.10, 0.50].  Per head: draw rho_h, then the fill."""
    rng = np.random.default_rng([w.seed, 1])
    nb, n, f = w.n_blocks, w.seq_len, w.frame_tokens
    base = _band(nb, 1)
    for u in range(nb):
        first = BLOCK * u
        for kf in range(-(first // f), (n - 1 - first) // f + 1):
            if kf:
                base[u, (first + kf * f) // BLOCK] = True
    keep = np.empty((w.n_heads, nb, nb), bool)
    for h in range(w.n_heads):
        rho = rng.uniform(0.10, 0.50)
        keep[h] = base
        _fill_random(rng, keep[h], int(round(rho * nb * nb)))
    return keep


def mask_wan14b(w: Workload, block: int = BLOCK) -> np.ndarray:
    """round(0.2 H) heads full (first entries of a random permutation); every other
    head: band |u-v|<=1 plus random fill to round(rho_h nb^2), rho_h ~ U[0.05, 0.40],
    drawn in head order.  nb = ceil(N / block): 64-token blocks by default, 128 for
    ScalingAttention's own granularity (then the stream is seeded apart)."""
    rng = np.random.default_rng([w.seed, 1] if block == BLOCK else [w.seed, 1, block])
    nb = -(-w.seq_len // block)
    full = set(rng.permutation(w.n_heads)[: int(round(0.2 * w.n_heads))].tolist())
    base = _band(nb, 1)
    keep = np.empty((w.n_heads, nb, nb), bool)
    for h in range(w.n_heads):
        if h in full:
            keep[h] = True
            continue
        rho = rng.uniform(0.05, 0.40)
        keep[h] = base
        _fill_random(rng, keep[h], int(round(rho * nb * nb)))
    return keep


def uniform_mask(n_heads: int, nb: int, density: float, seed: int) -> np.ndarray:
    """Exactly round(density * nb^2) blocks on per head, uniformly at random."""
    rng = np.random.default_rng([seed, 7])
    keep = np.zeros((n_heads, nb, nb), bool)
    for h in range(n_heads):
        _fill_random(rng, keep[h], int(round(density * nb * nb)))
    return keep


def stripe_params(w: Workload) -> np.ndarray:
    """Per-head stripe tuples, int32 [H][7] = {full, Tw, To, Ts, Sw, So, Ss}
    (a stride of 0 stands for an infinite stride).  round(0.2 H) heads are full
    window (first entries of a random permutation); the others draw Tw from
    {1,5,7}, Sw from {1,3,5,10} and Ss from {1,3,6} in that order, head by head,
    with To = So = 0 and Ts infinite."""
    rng = np.random.default_rng([w.seed, 1])
    full = set(rng.permutation(w.n_heads)[: int(round(0.2 * w.n_heads))].tolist())
    out = np.zeros((w.n_heads, 7), np.int32)
    for h in range(w.n_heads):
        if h in full:
            out[h] = (1, 1, 0, 0, 1, 0, 0)
            continue
        tw = (1, 5, 7)[rng.integers(3)]
        sw = (1, 3, 5, 10)[rng.integers(4)]
        ss = (1, 3, 6)[rng.integers(3)]
        out[h] = (0, tw, 0, 0, sw, 0, ss)
    return out


def masks(w: Workload) -> np.ndarray:
    """Boolean block mask [H][nb][nb] for the workloads that carry a static mask."""
    if w.name == "tiny":
        return mask_tiny(w)
    if w.name == "wan13b_480p":
        return mask_wan13b(w)
    if w.name == "wan14b_720p":
        return mask_wan14b(w)
    raise ValueError(f"workload {w.name} builds its mask on the device")


# ---------------------------------------------------------------- tensors
def _normal_heads(rng, n_heads, n, d):
    for _ in range(n_heads):
        yield rng.standard_normal((n, d), dtype=np.float32)


def qkv(w: Workload, heads=None):
    """Q, K, V each [H][N][d], drawn N(0,1) as float32 in the order Q, K, V, head
    by head from one stream; bf16 workloads return raw bf16 patterns (uint16),
    the fp32 workload returns float32.  ``heads`` keeps only those heads (the
    stream is still consumed in full so the values do not depend on the
    selection).  The top-p workload adds its per-frame rank-8 component."""
    rng = np.random.default_rng([w.seed, 0])
    n, d, H = w.seq_len, w.head_dim, w.n_heads
    keep = list(range(H)) if heads is None else list(heads)
    lowrank = None
    if w.name == "topp_wan14b":
        lowrank = _frame_components(w)
    outs = []
    for ti in range(3):
        dt = np.float32 if w.dtype == "f32" else np.uint16
        arr = np.empty((len(keep), n, d), dt)
        for h, x in enumerate(_normal_heads(rng, H, n, d)):
            if h not in keep:
                continue
            if lowrank is not None and ti < 2:
                x = x + np.float32(0.5) * lowrank[h][np.arange(n) // w.frame_tokens]
            arr[keep.index(h)] = x if w.dtype == "f32" else bf16_bits(x)
        outs.append(arr)
    return tuple(outs)


def _frame_components(w: Workload) -> np.ndarray:
    """Per head C_h = A_h B_h, A_h [frames][8] ~ N(0,1), B_h [8][d] ~ N(0, 1/8):
    one unit-variance vector per frame, shared by Q and K."""
    rng = np.random.default_rng([w.seed, 2])
    t = w.grid[0]
    out = np.empty((w.n_heads, t, w.head_dim), np.float32)
    for h in range(w.n_heads):
        a = rng.standard_normal((t, 8))
        b = rng.standard_normal((8, w.head_dim)) / math.sqrt(8.0)
        out[h] = (a @ b).astype(np.float32)
    return out


def random_scores(n_heads: int, nq: int, nk: int, seed: int, spread: float = 3.0) -> np.ndarray:
    """Synthetic fp32 block-score matrices [H][nq][nk] for selection tests:
    N(0, spread^2) logits rounded to float32."""
    rng = np.random.default_rng([seed, 3])
    return (rng.standard_normal((n_heads, nq, nk)) * spread).astype(np.float32)


def threshold_map(n_heads: int, nb: int, seed: int):
    """Synthetic threshold maps and per-head levels for mask instantiation tests.

    Stand-in for the calibrated maps of ScalingAttention section 4.1.2 (none can
    be computed here: they need model weights and prompts).  T grows with the
    block distance |u - v| (local blocks become active at low levels, as in the
    pages' Figure 3) plus uniform noise, in [0, 1], float32; levels p*_h ~ U[0.1, 0.6].
    """
    rng = np.random.default_rng([seed, 5])
    u = np.arange(nb)
    dist = np.abs(u[:, None] - u[None, :]) / max(nb - 1, 1)
    T = np.empty((n_heads, nb, nb), dtype=np.float32)
    for h in range(n_heads):
        T[h] = np.clip(0.6 * dist ** rng.uniform(0.3, 1.0) + 0.4 * rng.random((nb, nb)), 0.0, 1.0)
    p = rng.uniform(0.1, 0.6, n_heads).astype(np.float32)
    return T, p


def stratified_rows(n_heads: int, n_tokens: int, n_rows: int, seed: int) -> np.ndarray:
    """Block-wise stratified row sample (ScalingAttention section 4.2.3): the
    token rows are cut into n_rows equal strata and one row is drawn uniformly
    from each, independently per head.  int32 [n_heads, n_rows]."""
    rng = np.random.default_rng([seed, 6])
    edges = (np.arange(n_rows + 1) * n_tokens) // n_rows
    out = np.empty((n_heads, n_rows), np.int32)
    for h in range(n_heads):
        for r in range(n_rows):
            lo, hi = edges[r], max(edges[r + 1], edges[r] + 1)
            out[h, r] = min(int(rng.integers(lo, hi)), n_tokens - 1)
    return out
