"""GPU parity of ScalingAttention's own mask format -- 128 x 128-token blocks in 32-bit
row words -- through the C ABI: the word-for-word expansion is bit-exact, and
attention over it matches the float64 oracle evaluated at 128-token blocks."""
import numpy as np
import pytest
import torch

import block_sparse_attention_07_amd as bsa
import workloads
from oracle import crm
from oracle.attention import sparse_attention
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
B = 128


def _f(x):
    return workloads.bf16_to_f32(x).astype(np.float64)


def _words_dev(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(gu.dev())


def _random_words(H, n, density, seed, junk_padding=True):
    nb = -(-n // B)
    rng = np.random.default_rng(seed)
    keep = rng.random((H, nb, nb)) < density
    words = workloads.pack_bits32(keep)
    if junk_padding and nb % 32:
        # set every padding bit of the last word: the library must ignore them
        words[..., -1] |= np.uint32(~((1 << (nb % 32)) - 1) & 0xFFFFFFFF)
    return keep, words


@pytest.mark.parametrize("n", [1, 100, 128, 129, 64 * 37 + 13, 128 * 20 - 70, 4096, 4097, 64 * 130 + 7])
def test_expansion_is_bit_exact(n):
    H = 3
    keep, words = _random_words(H, n, 0.4, seed=n)
    got = gu.mask_host(bsa.mask_b128_to_b64(_words_dev(words), n))
    nf = -(-n // 64)
    ref = crm.pack_rows(crm.refine_blocks(keep, 2, nf))
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [128, 300, 128 * 9 - 70, 128 * 9 + 40, 1000, 128 * 33])
def test_attention_all_rows(d, n):
    H = 3
    nb = -(-n // B)
    rng = np.random.default_rng(n + d)
    q, k, v = (workloads.bf16_bits(rng.standard_normal((H, n, d)).astype(np.float32)) for _ in range(3))
    keep, words = _random_words(H, n, 0.45, seed=n * d)
    keep[0, 0] = False                      # an empty row (both 64-halves)
    keep[1, -1] = True                      # a full row ending in the ragged block
    keep[2, :, -1] = True                   # every row keeps the ragged block
    words = workloads.pack_bits32(keep)
    scale = 1.0 / np.sqrt(d)
    out = bsa.sparse_attn_b128(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True),
                               _words_dev(words), scale)
    torch.cuda.synchronize()
    got = gu.bf16_host(out)
    ref = sparse_attention(_f(q), _f(k), _f(v), crm.pack_rows(keep), scale, block=B)
    for h in range(H):
        gu.assert_bf16_close(got[h], ref[h], f"d={d} n={n} head {h}")
    assert np.all(got[0, :min(n, B)] == 0.0)


def test_every_row_pair_is_planned_as_a_pair():
    """Both 64-token halves of a 128-row are identical after expansion, so the
    planner pairs every non-empty 128-row except a last one that has a single
    64-token half."""
    n, H = 128 * 12 - 30, 2
    keep, words = _random_words(H, n, 0.3, seed=5, junk_padding=False)
    keep[1, 4] = False
    words = workloads.pack_bits32(keep)
    m64 = bsa.mask_b128_to_b64(_words_dev(words), n)
    _, _, order = bsa.plan(m64, n)
    o = order.cpu().numpy()
    nf = -(-n // 64)
    pairs = sorted((int(e) - H * nf) for e in o if e >= H * nf)
    singles = sorted(int(e) for e in o if 0 <= e < H * nf)
    assert len(pairs) == H * (nf // 2)
    assert all(p % 2 == 0 for p in pairs)
    assert singles == ([h * nf + nf - 1 for h in range(H)] if nf % 2 else [])


def test_wan14b_shape_sampled_rows():
    """The Wan2.1-14B 720p layer (40 heads, 75,600 tokens, d = 128) under the same
    mask recipe drawn over 128-token blocks; sampled 128-query blocks, including the
    ragged last one, against the oracle."""
    w = workloads.WORKLOADS["wan14b_720p"]
    keep = workloads.mask_wan14b(w, block=B)
    words = workloads.pack_bits32(keep)
    q, k, v = workloads.qkv(w)
    got = bsa.sparse_attn_b128(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True),
                               _words_dev(words), w.scale)
    torch.cuda.synchronize()
    blocks = gu.sample_blocks(keep, 16, seed=w.seed)
    hs = sorted({h for h, _ in blocks})
    hmap = {h: i for i, h in enumerate(hs)}
    qf, kf, vf = (np.stack([_f(x[h]) for h in hs]) for x in (q, k, v))
    ref = sparse_attention(qf, kf, vf, crm.pack_rows(keep[hs]), w.scale, block=B,
                           blocks=[(hmap[h], u) for h, u in blocks])
    out = got.cpu()
    for (h, u), r in zip(blocks, ref):
        gu.assert_bf16_close(gu.bf16_host(out[h, u * B:u * B + r.shape[0]]), r, f"b128 ({h},{u})")
