"""GPU parity of attn_fidelity (Hellinger distance / Fidelity Score between dense and
sparse attention rows, ScalingAttention Eqs. 3-4) against the float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_07_amd as bsa
import workloads
from oracle import crm
from oracle.fidelity import head_fidelity, row_hellinger
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bars(got, ref):
    # fp32 logits from bf16 inputs: relative error of the dropped mass ~1e-6, so
    # |dH| <= 1e-4 * H + 1e-6 is a wide margin; empty rows are exactly 1.
    assert np.all(np.abs(got - ref) <= 1e-4 * ref + 1e-6), np.max(np.abs(got - ref))


def _case(H, N, d, n_rows, density, seed, empty_block=None):
    rng = np.random.default_rng(seed)
    q = workloads.bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    k = workloads.bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    nb = -(-N // 64)
    keep = rng.random((H, nb, nb)) < density
    if empty_block is not None:
        keep[:, empty_block, :] = False
    bits = crm.pack_rows(keep)
    rows = workloads.stratified_rows(H, N, n_rows, seed)
    scale = 1.0 / np.sqrt(d)
    row_h, head_f = bsa.attn_fidelity(gu.to_dev(q, bf16=True), gu.to_dev(k, bf16=True), gu.to_dev(bits),
                                      gu.to_dev(rows), scale)
    torch.cuda.synchronize()
    qf, kf = workloads.bf16_to_f32(q), workloads.bf16_to_f32(k)
    ref = row_hellinger(qf, kf, bits, rows, scale)
    return row_h.cpu().numpy(), head_f.cpu().numpy(), ref, rows, keep


@pytest.mark.parametrize("H,N,d,n_rows,density", [
    (2, 200, 64, 5, 0.4), (3, 1000, 128, 16, 0.3), (2, 3000, 128, 20, 0.15), (1, 4133, 64, 33, 0.6),
])
def test_fidelity_matches_oracle(H, N, d, n_rows, density):
    got, gf, ref, _, _ = _case(H, N, d, n_rows, density, seed=N + n_rows)
    _bars(got, ref)
    assert np.all(np.abs(gf - head_fidelity(ref)) <= 1e-4)


def test_empty_and_full_rows():
    got, _, ref, rows, keep = _case(2, 700, 128, 11, 0.5, seed=3, empty_block=2)
    empty = (rows // 64) == 2
    assert empty.any() and np.all(got[empty] == 1.0) and np.all(ref[empty] == 1.0)
    _bars(got, ref)
    # all-ones mask: nothing is dropped, so H is exactly 0
    rng = np.random.default_rng(4)
    H, N, d = 2, 700, 64
    q = workloads.bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    nb = -(-N // 64)
    full = crm.pack_rows(np.ones((H, nb, nb), bool))
    rows_d = gu.to_dev(workloads.stratified_rows(H, N, 16, 5))
    row_h, head_f = bsa.attn_fidelity(gu.to_dev(q, bf16=True), gu.to_dev(q, bf16=True), gu.to_dev(full), rows_d)
    assert torch.all(row_h == 0).item() and torch.all(head_f == 1).item()


def test_out_of_range_row_gives_nan():
    rng = np.random.default_rng(6)
    H, N, d = 1, 300, 64
    q = gu.to_dev(workloads.bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32)), bf16=True)
    nb = -(-N // 64)
    bits = gu.to_dev(crm.pack_rows(np.ones((H, nb, nb), bool)))
    rows = gu.to_dev(np.array([[0, 299, 300, -1]], np.int32))
    row_h, _ = bsa.attn_fidelity(q, q, bits, rows)
    r = row_h.cpu().numpy()[0]
    assert r[0] == 0 and r[1] == 0 and np.isnan(r[2]) and np.isnan(r[3])


def test_fidelity_on_layer_shape_sampled_heads():
    """Wan2.1-14B 720p layer mask, 16 stratified rows per head (the pages' sample
    size), checked on 6 heads (2 full, 4 sparse)."""
    w = workloads.WORKLOADS["wan14b_720p"]
    keep = workloads.masks(w)
    heads = [int(h) for h in np.nonzero(keep.reshape(w.n_heads, -1).all(1))[0][:2]]
    heads += [h for h in range(w.n_heads) if h not in heads][:4]
    q, k, _ = workloads.qkv(w, heads=heads)
    bits = workloads.pack_bits(keep[heads])
    rows = workloads.stratified_rows(len(heads), w.seq_len, 16, seed=11)
    row_h, head_f = bsa.attn_fidelity(gu.to_dev(q, bf16=True), gu.to_dev(k, bf16=True), gu.to_dev(bits),
                                      gu.to_dev(rows), w.scale)
    torch.cuda.synchronize()
    ref = row_hellinger(workloads.bf16_to_f32(q), workloads.bf16_to_f32(k), bits, rows, w.scale)
    got = row_h.cpu().numpy()
    _bars(got, ref)
    assert np.all(got[:2] == 0)          # full heads drop nothing
