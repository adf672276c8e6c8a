"""Python entry points with the C ABI's names.

Argument marshalling only: every function checks dtypes, shapes, devices and
contiguity, allocates outputs with torch (device memory is the only thing torch
provides here) and passes raw pointers plus torch's current HIP stream to the
library.  All computation happens in the library's kernels.

Masks travel as torch.int64 tensors holding the uint64 words bit for bit (and,
for the 32-bit format over 128-token blocks, torch.int32 tensors holding the
uint32 words).
"""
from __future__ import annotations

import ctypes
import functools
import math

import numpy as np
import torch

from ._lib import check, lib

BLOCK = 64


def mask_words(seq_len: int, block: int = BLOCK) -> int:
    return int(lib().bsa_mask_words(int(seq_len), int(block)))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    d = ts[0].device
    _need(d.type == "cuda", "tensors must live on a HIP device")
    for t in ts:
        _need(t.device == d, "all tensors must be on the same device")
        _need(t.is_contiguous(), "tensors must be contiguous")
    return d


def _on_device(fn):
    """Run fn with the device of its first device-tensor argument current: the
    library sizes launches and keeps its scratch memory per current device."""
    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        for a in (*args, *kwargs.values()):
            if isinstance(a, torch.Tensor) and a.device.type == "cuda":
                with torch.cuda.device(a.device):
                    return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return wrapped


def _check_mask(mask_bits, H, N):
    nb = -(-N // BLOCK)
    _need(mask_bits.dtype == torch.int64, "mask_bits must be int64 (uint64 words)")
    _need(tuple(mask_bits.shape) == (H, nb, mask_words(N)),
          f"mask_bits must be [{H}, {nb}, {mask_words(N)}], got {tuple(mask_bits.shape)}")


def workspace_bytes(n_heads: int, seq_len: int, head_dim: int) -> int:
    """Device workspace bytes sparse_attn_fwd_ws needs (0 for invalid sizes)."""
    return int(lib().sparse_attn_workspace_bytes(int(n_heads), int(seq_len), int(head_dim)))


@_on_device
def sparse_attn(q, k, v, mask_bits, scale=None, out=None, work_order=None, workspace=None):
    """Block-sparse attention (sparse_attn_fwd / sparse_attn_fwd_f32 /
    sparse_attn_fwd_planned / sparse_attn_fwd_ws).  q, k, v: [H, N, d] bf16 or fp32.
    ``workspace``: a caller-owned uint8 device tensor of at least
    workspace_bytes(H, N, d) bytes (bf16, no work order) used instead of the
    library's scratch buffer."""
    _dev(q, k, v, mask_bits)
    _need(q.dim() == 3 and q.shape == k.shape == v.shape, "q, k, v must share shape [H, N, d]")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    H, N, d = q.shape
    _check_mask(mask_bits, H, N)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _dev(q, out)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    s = _stream(q)
    _need(workspace is None or (q.dtype == torch.bfloat16 and work_order is None),
          "a workspace is taken by the bf16 entry point without a work order")
    if workspace is not None:
        _dev(q, workspace)
        _need(workspace.dtype == torch.uint8 and workspace.dim() == 1, "workspace must be a 1-D uint8 tensor")
        rc = lib().sparse_attn_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits), H, N, d, BLOCK, BLOCK,
                                      scale, _ptr(out), _ptr(workspace), workspace.numel(), s)
        check(rc, "sparse_attn_fwd_ws")
    elif q.dtype == torch.bfloat16:
        if work_order is None:
            rc = lib().sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits), H, N, d, BLOCK,
                                       BLOCK, scale, _ptr(out), s)
            check(rc, "sparse_attn_fwd")
        else:
            _dev(q, work_order)
            _need(work_order.dtype == torch.int32 and work_order.numel() == H * (-(-N // BLOCK)),
                  "work_order must be int32 [H * nb]")
            rc = lib().sparse_attn_fwd_planned(_ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits),
                                               _ptr(work_order), H, N, d, BLOCK, BLOCK, scale,
                                               _ptr(out), s)
            check(rc, "sparse_attn_fwd_planned")
    elif q.dtype == torch.float32:
        _need(work_order is None, "the fp32 path takes no work order")
        rc = lib().sparse_attn_fwd_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits), H, N, d, BLOCK,
                                       BLOCK, scale, _ptr(out), s)
        check(rc, "sparse_attn_fwd_f32")
    else:
        raise ValueError("q, k, v must be bfloat16 or float32")
    return out


@_on_device
def sparse_attn_noalloc(q, k, v, mask_bits, scale=None, out=None):
    """bf16 block-sparse attention through sparse_attn_fwd_noalloc: the library's
    scratch is its fixed device array, nothing is allocated inside the call (pass
    ``out`` to keep the binding from allocating the output)."""
    _dev(q, k, v, mask_bits)
    _need(q.dim() == 3 and q.shape == k.shape == v.shape, "q, k, v must share shape [H, N, d]")
    _need(q.dtype == k.dtype == v.dtype == torch.bfloat16, "q, k, v must be bfloat16")
    H, N, d = q.shape
    _check_mask(mask_bits, H, N)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _dev(q, out)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    rc = lib().sparse_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(mask_bits), H, N, d, BLOCK, BLOCK,
                                       scale, _ptr(out), _stream(q))
    check(rc, "sparse_attn_fwd_noalloc")
    return out


def _check_mask32(mask_words, H, N):
    nb = -(-N // 128)
    W = -(-nb // 32)
    _need(mask_words.dtype == torch.int32, "mask_words must be int32 (uint32 words)")
    _need(tuple(mask_words.shape) == (H, nb, W),
          f"mask_words must be [{H}, {nb}, {W}], got {tuple(mask_words.shape)}")


@_on_device
def sparse_attn_b128(q, k, v, mask_words, scale=None, out=None):
    """Block-sparse attention over 128 x 128-token blocks with 32-bit row-mask words
    (sparse_attn_fwd_b128).  q, k, v: bf16 [H, N, d]; mask_words int32
    [H, ceil(N/128), ceil(ceil(N/128)/32)]."""
    _dev(q, k, v, mask_words)
    _need(q.dim() == 3 and q.shape == k.shape == v.shape, "q, k, v must share shape [H, N, d]")
    _need(q.dtype == k.dtype == v.dtype == torch.bfloat16, "q, k, v must be bfloat16")
    H, N, d = q.shape
    _check_mask32(mask_words, H, N)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _dev(q, out)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    rc = lib().sparse_attn_fwd_b128(_ptr(q), _ptr(k), _ptr(v), _ptr(mask_words), H, N, d, scale,
                                    _ptr(out), _stream(q))
    check(rc, "sparse_attn_fwd_b128")
    return out


@_on_device
def mask_b128_to_b64(mask_words, seq_len: int, out=None):
    """32-bit rows over 128-token blocks -> the same mask as 64-bit rows over
    64-token blocks (int64 [H, ceil(N/64), ceil(ceil(N/64)/64)])."""
    _dev(mask_words)
    H = mask_words.shape[0]
    _check_mask32(mask_words, H, seq_len)
    nb = -(-seq_len // BLOCK)
    if out is None:
        out = torch.empty((H, nb, mask_words.shape[2]), dtype=torch.int64, device=mask_words.device)
    _dev(mask_words, out)
    _check_mask(out, H, seq_len)
    rc = lib().mask_b128_to_b64(_ptr(mask_words), H, int(seq_len), _ptr(out), _stream(mask_words))
    check(rc, "mask_b128_to_b64")
    return out


@_on_device
def plan(mask_bits, seq_len: int):
    """Tile scheduler (sparse_attn_plan): returns (row_counts int32 [H*nb],
    head_tiles int64 [H], work_order int32 [H*nb])."""
    _dev(mask_bits)
    H = mask_bits.shape[0]
    _check_mask(mask_bits, H, seq_len)
    nb = -(-seq_len // BLOCK)
    counts = torch.empty(H * nb, dtype=torch.int32, device=mask_bits.device)
    tiles = torch.empty(H, dtype=torch.int64, device=mask_bits.device)
    order = torch.empty(H * nb, dtype=torch.int32, device=mask_bits.device)
    rc = lib().sparse_attn_plan(_ptr(mask_bits), H, int(seq_len), BLOCK, _ptr(counts), _ptr(tiles),
                                _ptr(order), _stream(mask_bits))
    check(rc, "sparse_attn_plan")
    return counts, tiles, order


@_on_device
def mask_from_stripes(params, n_frames: int, frame_tokens: int, seq_len: int, out=None):
    """PSA stripe tuples int32 [H, 7] (device) -> int64 mask words [H, nb, W]."""
    _dev(params)
    _need(params.dtype == torch.int32 and params.dim() == 2 and params.shape[1] == 7,
          "params must be int32 [H, 7]")
    H = params.shape[0]
    nb = -(-seq_len // BLOCK)
    if out is None:
        out = torch.empty((H, nb, mask_words(seq_len)), dtype=torch.int64, device=params.device)
    _check_mask(out, H, seq_len)
    rc = lib().mask_from_stripes(_ptr(params), H, int(n_frames), int(frame_tokens), int(seq_len),
                                 BLOCK, _ptr(out), _stream(params))
    check(rc, "mask_from_stripes")
    return out


@_on_device
def block_scores_meanpool(q, k, scale=None, out=None):
    """Mean-pooled block scores fp32 [H, nb, nb] from bf16 q, k [H, N, d]."""
    _dev(q, k)
    _need(q.dtype == k.dtype == torch.bfloat16 and q.shape == k.shape and q.dim() == 3,
          "q, k must be bf16 [H, N, d]")
    H, N, d = q.shape
    nb = -(-N // BLOCK)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((H, nb, nb), dtype=torch.float32, device=q.device)
    _need(out.shape == (H, nb, nb) and out.dtype == torch.float32, "out must be fp32 [H, nb, nb]")
    rc = lib().block_scores_meanpool(_ptr(q), _ptr(k), H, N, d, BLOCK, scale, _ptr(out), _stream(q))
    check(rc, "block_scores_meanpool")
    return out


@_on_device
def mask_from_block_scores_topp(scores, p: float, min_blocks: int, out=None):
    """fp32 scores [H, nq, nk] -> int64 mask words [H, nq, ceil(nk/64)]."""
    _dev(scores)
    _need(scores.dtype == torch.float32 and scores.dim() == 3, "scores must be fp32 [H, nq, nk]")
    H, nq, nk = scores.shape
    if out is None:
        out = torch.empty((H, nq, -(-nk // 64)), dtype=torch.int64, device=scores.device)
    _need(out.shape == (H, nq, -(-nk // 64)) and out.dtype == torch.int64, "bad out")
    rc = lib().mask_from_block_scores_topp(_ptr(scores), H, nq, nk, float(p), int(min_blocks),
                                           _ptr(out), _stream(scores))
    check(rc, "mask_from_block_scores_topp")
    return out


@_on_device
def mask_from_threshold_map(thresholds, p_head, out=None):
    """fp32 threshold map [H, nq, nk] and fp32 levels [H] (device) -> int64 mask
    words [H, nq, ceil(nk/64)] with bit set where T <= p_head[h]."""
    _dev(thresholds, p_head)
    _need(thresholds.dtype == torch.float32 and thresholds.dim() == 3, "thresholds must be fp32 [H, nq, nk]")
    H, nq, nk = thresholds.shape
    _need(p_head.dtype == torch.float32 and p_head.shape == (H,), "p_head must be fp32 [H]")
    if out is None:
        out = torch.empty((H, nq, -(-nk // 64)), dtype=torch.int64, device=thresholds.device)
    _need(out.shape == (H, nq, -(-nk // 64)) and out.dtype == torch.int64, "bad out")
    rc = lib().mask_from_threshold_map(_ptr(thresholds), _ptr(p_head), H, nq, nk, _ptr(out),
                                       _stream(thresholds))
    check(rc, "mask_from_threshold_map")
    return out


@_on_device
def mask_resize(mask_bits, nb_base: int, nb_target: int, out=None):
    """Region maps int64 [H, nb_base, ceil(nb_base/64)] -> [H, nb_target, ceil(nb_target/64)]
    (Eq. 7: bilinear interpolation with a ceiling)."""
    _dev(mask_bits)
    H = mask_bits.shape[0]
    _need(mask_bits.dtype == torch.int64 and mask_bits.shape == (H, nb_base, -(-nb_base // 64)),
          "mask_bits must be int64 [H, nb_base, ceil(nb_base/64)]")
    if out is None:
        out = torch.empty((H, nb_target, -(-nb_target // 64)), dtype=torch.int64, device=mask_bits.device)
    _need(out.shape == (H, nb_target, -(-nb_target // 64)) and out.dtype == torch.int64, "bad out")
    rc = lib().mask_resize(_ptr(mask_bits), H, int(nb_base), int(nb_target), _ptr(out), _stream(mask_bits))
    check(rc, "mask_resize")
    return out


@_on_device
def threshold_map_resize(thresholds, nb_target: int, out=None):
    """Threshold maps fp32 [H, nb, nb] -> [H, nb_target, nb_target] (min over the
    positive-weight bilinear samples)."""
    _dev(thresholds)
    _need(thresholds.dtype == torch.float32 and thresholds.dim() == 3 and
          thresholds.shape[1] == thresholds.shape[2], "thresholds must be fp32 [H, nb, nb]")
    H, nb, _ = thresholds.shape
    if out is None:
        out = torch.empty((H, nb_target, nb_target), dtype=torch.float32, device=thresholds.device)
    _need(out.shape == (H, nb_target, nb_target) and out.dtype == torch.float32, "bad out")
    rc = lib().threshold_map_resize(_ptr(thresholds), H, nb, int(nb_target), _ptr(out), _stream(thresholds))
    check(rc, "threshold_map_resize")
    return out


@_on_device
def attn_fidelity(q, k, mask_bits, rows, scale=None):
    """Hellinger distance per sampled row fp32 [H, R] and Fidelity Score per head fp32
    [H] between dense and sparse attention; rows int32 [H, R] token indices (device)."""
    _dev(q, k, mask_bits, rows)
    _need(q.dtype == k.dtype == torch.bfloat16 and q.shape == k.shape and q.dim() == 3,
          "q, k must be bf16 [H, N, d]")
    H, N, d = q.shape
    _check_mask(mask_bits, H, N)
    _need(rows.dtype == torch.int32 and rows.dim() == 2 and rows.shape[0] == H, "rows must be int32 [H, R]")
    R = rows.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    row_h = torch.empty((H, R), dtype=torch.float32, device=q.device)
    head_f = torch.empty((H,), dtype=torch.float32, device=q.device)
    rc = lib().attn_fidelity(_ptr(q), _ptr(k), _ptr(mask_bits), _ptr(rows), H, N, d, BLOCK, R, scale,
                             _ptr(row_h), _ptr(head_f), _stream(q))
    check(rc, "attn_fidelity")
    return row_h, head_f


@_on_device
def permute_tokens(x, perm, inverse: bool = False, out=None):
    """Gather (inverse=False) or scatter (inverse=True) token rows of x [H, N, d]."""
    _dev(x, perm)
    _need(x.dim() == 3 and perm.dtype == torch.int32 and perm.numel() == x.shape[1],
          "x must be [H, N, d] and perm int32 [N]")
    if out is None:
        out = torch.empty_like(x)
    _dev(x, out)
    H, N, d = x.shape
    rc = lib().permute_tokens(_ptr(x), _ptr(perm), H, N, d, x.element_size(), int(bool(inverse)),
                              _ptr(out), _stream(x))
    check(rc, "permute_tokens")
    return out


def hilbert3d_order(T: int, H: int, W: int) -> np.ndarray:
    """Host-only: int32 [T*H*W] token ids in 3D Hilbert order."""
    perm = np.empty(T * H * W, dtype=np.int32)
    rc = lib().hilbert3d_order(int(T), int(H), int(W), perm.ctypes.data_as(ctypes.c_void_p))
    check(rc, "hilbert3d_order")
    return perm


@_on_device
def mfma_probe(sink: torch.Tensor, iterations: int) -> float:
    """Measurement aid beside the path: enqueue the register-only bf16 MFMA loop of
    bsa_mfma_probe on the current stream of ``sink``'s device (fp32, at least
    512 x compute units elements) and return the flops it performs; time the call
    with events on that stream for the rate."""
    _dev(sink)
    _need(sink.dtype == torch.float32, "sink must be float32")
    flops = ctypes.c_double(0.0)
    rc = lib().bsa_mfma_probe(int(iterations), _ptr(sink), ctypes.c_longlong(sink.numel()),
                              ctypes.byref(flops), _stream(sink))
    check(rc, "bsa_mfma_probe")
    return flops.value
