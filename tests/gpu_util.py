"""Helpers for the GPU parity tests: host<->device plumbing and the comparison
bars.  Device outputs are widened on the host (no device-side compute)."""
from __future__ import annotations

import numpy as np
import torch

import workloads

# bf16 parity bars (max / mean absolute error over all compared outputs), plus a
# per-row relative bar that a near-zero output would fail even where the
# absolute bars would let it pass.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_ROW_REL = 1e-2
F32_MAX_ABS = 1e-5


def dev():
    return torch.device("cuda", 0)


def to_dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(dev())
    return torch.from_numpy(a).to(dev())


def bf16_host(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> float64 host array (exact widening on the host)."""
    raw = t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return workloads.bf16_to_f32(raw).astype(np.float64)


def mask_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint64)


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """got/ref: [..., rows, d] float64.  Applies the three bars."""
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= BF16_MAX_ABS, f"{what}: max abs err {mx}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean abs err {mean}"
    rn = np.linalg.norm(ref, axis=-1)
    live = rn > 0
    if live.any():
        rel = np.linalg.norm(got - ref, axis=-1)[live] / rn[live]
        assert float(rel.max()) <= BF16_ROW_REL, f"{what}: row rel err {float(rel.max())}"
    dead = ~live
    if dead.any():
        assert np.all(got[dead] == 0.0), f"{what}: rows with no kept key must be 0"
    return mx, mean


def sample_blocks(keep: np.ndarray, n: int, seed: int):
    """(h, u) query blocks to compare at full size: the first and the last (ragged)
    block of the densest and of the sparsest head, plus n random blocks."""
    H, nb, _ = keep.shape
    per_head = keep.reshape(H, -1).sum(1)
    hd, hs = int(per_head.argmax()), int(per_head.argmin())
    rng = np.random.default_rng(seed)
    pick = {(hd, 0), (hd, nb - 1), (hs, 0), (hs, nb - 1)}
    while len(pick) < n + 4:
        pick.add((int(rng.integers(H)), int(rng.integers(nb))))
    return sorted(pick)
