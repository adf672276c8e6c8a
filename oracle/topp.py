"""Hybrid top-p block selection with a fixed top-k minimum, as a fixed float32
procedure.

Pages: online top-p sparse attention keeps, per query block, the key blocks
whose softmax mass accumulates to a threshold p ("Competition Domains Matter"
abstract); a fixed top-k minimum guards rows whose proxy softmax is too
concentrated (SCOPE abstract); the cut-off itself is a sort followed by a
cumulative sum that stops where it reaches p (ScalingAttention, Appendix A,
Algorithm 1, local threshold discovery).

Because the kept set is an integer decision taken on floating-point sums, the
selection is defined by one float32 procedure that the GPU kernel also follows,
so both sides decide identically.  For one row of n scores s:

0. s = min(max(s, -FLT_MAX), FLT_MAX), with a NaN score taking -FLT_MAX (the
   pages only consider finite scores; this reading makes a row with NaN or
   infinite scores a row of finite ones, so the steps below stay defined)
1. m = max(s)
2. e_j = EXP(s_j - m)               (float32 subtraction, then EXP below)
3. order = indices by s descending, ties to the lower index
4. Z = e[order[0]] + e[order[1]] + ... in that sequence, float32
5. c = 0; for r = 0, 1, ...: c = c + e[order[r]] / Z (float32); the first r with
   c >= p gives k_p = r + 1 (k_p = n when c never reaches p)
6. k = max(k_p, min(min_blocks, n)); keep order[0 .. k)

EXP is this library's own float32 exponential: Cody-Waite range reduction with
a two-part ln 2 (W. J. Cody and W. Waite, Software Manual for the Elementary
Functions, 1980) and the degree-7 Taylor polynomial of e^r in Horner form;
2^n is assembled from exponent bits; arguments below -87 return 0.  Every step
is one IEEE float32 operation (+, -, *, /) rounded to nearest, never fused.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

from .crm import pack_rows

F = np.float32
LOG2E = F(1.4426950408889634)
LN2_HI = F(0.693359375)                # 355/512: n * LN2_HI is exact for |n| < 2^15
LN2_LO = F(0.6931471805599453 - 0.693359375)
TAYLOR = [F(1.0 / f) for f in (1.0, 1.0, 2.0, 6.0, 24.0, 120.0, 720.0, 5040.0)]
EXP_FLOOR = F(-87.0)


def exp32(x: np.ndarray) -> np.ndarray:
    """Element-wise float32 EXP (see module docstring); x <= 0 in use."""
    x = np.asarray(x, dtype=F)
    with np.errstate(invalid="ignore", over="ignore"):
        n = np.floor(x * LOG2E + F(0.5)).astype(F)
        r = (x - n * LN2_HI) - n * LN2_LO
        p = TAYLOR[7]
        for c in TAYLOR[6::-1]:
            p = p * r + c
        p = np.asarray(p, dtype=F)
        ni = np.nan_to_num(np.clip(n, -126, 127), nan=-126).astype(np.int32)
        two_n = ((ni + 127).astype(np.uint32) << np.uint32(23)).view(F)
        y = (p * two_n).astype(F)
    return np.where(x < EXP_FLOOR, F(0.0), y).astype(F)


FMAX = np.finfo(F).max


def clamp_scores(s: np.ndarray) -> np.ndarray:
    """Step 0: NaN -> -FLT_MAX, +-inf -> +-FLT_MAX (fmax / fmin drop a NaN operand)."""
    return np.fmin(np.fmax(np.asarray(s, dtype=F), -FMAX), FMAX).astype(F)


def select_row(s: np.ndarray, p: float, min_blocks: int) -> np.ndarray:
    """Kept key-block indices (in selection order) for one score row."""
    s = clamp_scores(s)
    n = s.size
    m = s.max()
    with np.errstate(over="ignore"):
        e = exp32((s - m).astype(F))          # -FLT_MAX - FLT_MAX overflows to -inf: EXP gives 0
    order = np.argsort(-s, kind="stable")
    e_sorted = e[order]
    z = np.cumsum(e_sorted, dtype=F)[-1]                  # sequential float32 sum
    c = np.cumsum((e_sorted / z).astype(F), dtype=F)      # sequential float32 scan
    hit = np.flatnonzero(c >= F(p))
    kp = int(hit[0]) + 1 if hit.size else n
    k = max(kp, min(int(min_blocks), n))
    return order[:k]


def topp_keep(scores: np.ndarray, p: float, min_blocks: int) -> np.ndarray:
    """Boolean mask [H, nq, nk] from float32 scores [H, nq, nk]."""
    scores = np.asarray(scores, dtype=F)
    out = np.zeros(scores.shape, dtype=bool)
    for h in range(scores.shape[0]):
        for u in range(scores.shape[1]):
            out[h, u, select_row(scores[h, u], p, min_blocks)] = True
    return out


def topp_mask_bits(scores, p, min_blocks):
    return pack_rows(topp_keep(scores, p, min_blocks))


def boundary_margin(scores_row: np.ndarray, p: float, min_blocks: int) -> float:
    """Distance, in float64 cumulative mass, between p and the partial sums on
    either side of the top-p cut-off of this row.  Kept sets computed in
    different precisions may only differ on rows where this is tiny."""
    s = np.asarray(scores_row, dtype=np.float64)
    order = np.argsort(-s, kind="stable")
    e = np.exp(s[order] - s.max())
    c = np.cumsum(e) / e.sum()
    return float(np.min(np.abs(c - p)))
