"""GPU parity of the block-sparse attention kernels against the float64 oracle,
through the C ABI (python binding -> libbsattn.so)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_07_amd as bsa
import workloads
from oracle import crm, stripes
from oracle.attention import sparse_attention
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
B = 64


def _rand_bf16(H, n, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [workloads.bf16_bits((rng.standard_normal((H, n, d)) * scale).astype(np.float32)) for _ in range(3)]


def _run_bf16(q, k, v, bits, scale, **kw):
    out = bsa.sparse_attn(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True),
                          gu.to_dev(bits), scale, **kw)
    torch.cuda.synchronize()
    return gu.bf16_host(out)


def _f(x):
    return workloads.bf16_to_f32(x).astype(np.float64)


def test_tiny_fp32_workload_matches_oracle():
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.qkv(w)
    bits = workloads.pack_bits(workloads.masks(w))
    out = bsa.sparse_attn(gu.to_dev(q), gu.to_dev(k), gu.to_dev(v), gu.to_dev(bits), w.scale)
    ref = sparse_attention(q, k, v, bits, w.scale)
    got = out.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ref)) <= gu.F32_MAX_ABS


@pytest.mark.parametrize("d,n", [(64, 200), (128, 64 * 7 + 5), (128, 1000)])
def test_fp32_ragged_random_masks(d, n):
    rng = np.random.default_rng(n)
    q, k, v = [rng.standard_normal((2, n, d)).astype(np.float32) for _ in range(3)]
    nb = -(-n // B)
    keep = rng.random((2, nb, nb)) < 0.5
    keep[0, 1] = False
    bits = crm.pack_rows(keep)
    out = bsa.sparse_attn(gu.to_dev(q), gu.to_dev(k), gu.to_dev(v), gu.to_dev(bits), 0.125)
    ref = sparse_attention(q, k, v, bits, 0.125)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= gu.F32_MAX_ABS


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [64, 200, 64 * 7 + 5, 1000, 64 * 33])
def test_bf16_random_masks_all_rows(d, n):
    q, k, v = _rand_bf16(3, n, d, seed=n + d)
    nb = -(-n // B)
    rng = np.random.default_rng(n * d)
    keep = rng.random((3, nb, nb)) < 0.5
    keep[0, 0] = False                 # an empty row
    keep[1, -1] = True                 # a full row ending in the ragged block
    keep[2, :, -1] = True              # every row keeps the ragged block
    bits = crm.pack_rows(keep)
    scale = 1.0 / np.sqrt(d)
    got = _run_bf16(q, k, v, bits, scale)
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, scale)
    gu.assert_bf16_close(got, ref, f"d={d} n={n}")
    assert np.all(got[0, :B] == 0.0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 17, 63, 65, 127])
def test_short_sequences(d, n):
    """Shorter than one or two blocks: the only or the last block is ragged.  Head 0
    keeps every block (with two blocks its rows are identical and run as a pair),
    head 1 keeps nothing, head 2 keeps only the ragged last block in every row."""
    H = 3
    nb = -(-n // B)
    q, k, v = _rand_bf16(H, n, d, seed=7 * n + d)
    keep = np.ones((H, nb, nb), bool)
    keep[1] = False
    keep[2, :, :nb - 1] = False
    bits = crm.pack_rows(keep)
    scale = 1.0 / np.sqrt(d)
    got = _run_bf16(q, k, v, bits, scale)
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, scale)
    gu.assert_bf16_close(got, ref, f"d={d} n={n}")
    assert np.all(got[1] == 0.0)


@pytest.mark.parametrize("n", [1, 33])
def test_fp32_short_sequences(n):
    rng = np.random.default_rng(n)
    q, k, v = [rng.standard_normal((2, n, 64)).astype(np.float32) for _ in range(3)]
    keep = np.ones((2, 1, 1), bool)
    keep[1] = False
    bits = crm.pack_rows(keep)
    out = bsa.sparse_attn(gu.to_dev(q), gu.to_dev(k), gu.to_dev(v), gu.to_dev(bits), 0.125)
    ref = sparse_attention(q, k, v, bits, 0.125)
    got = out.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= gu.F32_MAX_ABS
    assert np.all(got[1] == 0.0)


def test_bf16_sharpened_logits():
    """Peaked softmax (scale x 4, and Q/K with a shared component) exposes a
    wrong running max or a missed rescale that flat logits would hide."""
    n, d = 64 * 9 + 17, 128
    rng = np.random.default_rng(11)
    base = rng.standard_normal((1, n, d)).astype(np.float32)
    q = workloads.bf16_bits(base + rng.standard_normal((1, n, d)).astype(np.float32))
    k = workloads.bf16_bits(base + rng.standard_normal((1, n, d)).astype(np.float32))
    v = workloads.bf16_bits(rng.standard_normal((1, n, d)).astype(np.float32))
    nb = -(-n // B)
    keep = rng.random((1, nb, nb)) < 0.6
    keep[0, np.arange(nb), np.arange(nb)] = True
    bits = crm.pack_rows(keep)
    scale = 4.0 / np.sqrt(d)
    gu.assert_bf16_close(_run_bf16(q, k, v, bits, scale), sparse_attention(_f(q), _f(k), _f(v), bits, scale), "sharp")


def test_bf16_rescale_stress_growing_keys():
    """Keys grow block after block so the running max rises on every kept tile."""
    n, d = 64 * 12, 128
    rng = np.random.default_rng(12)
    growth = (1.0 + 0.6 * (np.arange(n) // B))[None, :, None]
    q = workloads.bf16_bits(rng.standard_normal((2, n, d)).astype(np.float32))
    k = workloads.bf16_bits((rng.standard_normal((2, n, d)) * growth).astype(np.float32))
    v = workloads.bf16_bits(rng.standard_normal((2, n, d)).astype(np.float32))
    keep = np.ones((2, 12, 12), bool)
    keep[1, :, ::3] = False
    bits = crm.pack_rows(keep)
    scale = 1.0 / np.sqrt(d)
    gu.assert_bf16_close(_run_bf16(q, k, v, bits, scale), sparse_attention(_f(q), _f(k), _f(v), bits, scale), "rescale")


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_rescale_stress_single_rows(d):
    """Growing keys on distinct random rows, all run as single rows (an identity
    work order pairs nothing): logits in later tiles exceed the first tile's max by
    far more than the fast tile walk accepts, so those rows go through the
    max-tracking walk; flat rows beside them stay on the fast one."""
    n = 64 * 12 + 5
    nb = -(-n // B)
    rng = np.random.default_rng(21)
    growth = (1.0 + 0.6 * (np.arange(n) // B))[None, :, None]
    q = workloads.bf16_bits(rng.standard_normal((2, n, d)).astype(np.float32))
    kf = rng.standard_normal((2, n, d))
    kf[0] *= growth[0]                       # head 0 grows, head 1 stays flat
    k = workloads.bf16_bits(kf.astype(np.float32))
    v = workloads.bf16_bits(rng.standard_normal((2, n, d)).astype(np.float32))
    keep = rng.random((2, nb, nb)) < 0.5
    keep[:, np.arange(nb), np.arange(nb)] = True
    keep[:, :, 0] = True                     # every row starts at the smallest keys
    bits = crm.pack_rows(keep)
    scale = 1.0 / np.sqrt(d)
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, scale)
    order = torch.arange(2 * nb, dtype=torch.int32, device="cuda")
    got = _run_bf16(q, k, v, bits, scale, work_order=order)
    gu.assert_bf16_close(got, ref, "rescale single rows")
    gu.assert_bf16_close(_run_bf16(q, k, v, bits, scale), ref, "rescale planned")


def test_bf16_zero_query_probe_pins_the_kept_set():
    """q = 0: each output is the token-weighted mean of the kept blocks' values;
    V carries each key's block id in binary, so a dropped or extra block shows up
    as a wrong average of block-id bits."""
    n, d = 64 * 20 - 13, 64
    nb = -(-n // B)
    blk = np.arange(n) // B
    v = np.zeros((1, n, d), np.float32)
    for c in range(5):
        v[0, :, c] = (blk >> c) & 1
    q = np.zeros((1, n, d), np.float32)
    k = np.random.default_rng(13).standard_normal((1, n, d)).astype(np.float32)
    keep = np.random.default_rng(13).random((1, nb, nb)) < 0.3
    keep[0, np.arange(nb), np.arange(nb)] = True
    bits = crm.pack_rows(keep)
    got = _run_bf16(workloads.bf16_bits(q), workloads.bf16_bits(k), workloads.bf16_bits(v), bits, 0.1)
    tokens = np.array([min(n, (b + 1) * B) - b * B for b in range(nb)], np.float64)
    for u in range(nb):
        kept = np.flatnonzero(keep[0, u])
        for c in range(5):
            want = sum(tokens[b] * ((b >> c) & 1) for b in kept) / tokens[kept].sum()
            blk_out = got[0, u * B:min(n, (u + 1) * B), c]
            assert np.all(np.abs(blk_out - want) <= 4e-3 * max(want, 1e-3) + 1e-6), (u, c)


def test_empty_rows_padding_bits_plan_and_determinism():
    n, d = 64 * 10 + 3, 128
    q, k, v = _rand_bf16(3, n, d, seed=14)
    nb = -(-n // B)
    keep = np.random.default_rng(14).random((3, nb, nb)) < 0.4
    keep[1, 4] = False
    keep[2] = False
    bits = crm.pack_rows(keep)
    scale = 1.0 / np.sqrt(d)
    a = _run_bf16(q, k, v, bits, scale)
    noisy = bits | np.uint64(~((1 << nb) - 1) & (2**64 - 1))
    b = _run_bf16(q, k, v, noisy, scale)
    assert np.array_equal(a, b)
    assert np.all(a[1, 4 * B:5 * B] == 0.0) and np.all(a[2] == 0.0)
    c = _run_bf16(q, k, v, bits, scale)
    assert np.array_equal(a, c)
    mdev = gu.to_dev(bits)
    counts, tiles, order = bsa.plan(mdev, n)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), keep.reshape(-1, nb).sum(1))
    assert np.array_equal(tiles.cpu().numpy(), keep.reshape(3, -1).sum(1))
    out = bsa.sparse_attn(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True), mdev, scale,
                          work_order=order)
    torch.cuda.synchronize()
    assert np.array_equal(gu.bf16_host(out), a)
    # any permutation of the rows gives the same bits (single entries only)
    rev = torch.arange(3 * nb - 1, -1, -1, dtype=torch.int32, device=order.device)
    out2 = bsa.sparse_attn(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True), mdev, scale,
                           work_order=rev)
    torch.cuda.synchronize()
    assert np.array_equal(gu.bf16_host(out2), a)


def test_plan_order_is_heads_by_decreasing_work():
    rng = np.random.default_rng(15)
    H, n = 7, 64 * 50
    nb = 50
    keep = np.zeros((H, nb, nb), bool)
    for h, dens in enumerate([0.1, 0.5, 0.5, 1.0, 0.0, 0.3, 0.05]):
        keep[h] = rng.random((nb, nb)) < dens
    keep[2] = keep[1]           # a tie: lower head index first
    counts, tiles, order = bsa.plan(gu.to_dev(crm.pack_rows(keep)), n)
    torch.cuda.synchronize()
    t = keep.reshape(H, -1).sum(1)
    rc = keep.sum(2)
    heads = sorted(range(H), key=lambda h: (-t[h], h))
    # each head's segment: pairs of identical adjacent rows (u even) first, then the
    # other rows, each by decreasing count (ties by u), then -1 for the slots pairs free
    want = []
    for h in heads:
        paired = [u for u in range(0, nb - 1, 2) if np.array_equal(keep[h, u], keep[h, u + 1])]
        covered = set(paired) | {u + 1 for u in paired}
        singles = [u for u in range(nb) if u not in covered]
        want += [H * nb + h * nb + u for u in sorted(paired, key=lambda u: (-rc[h, u], u))]
        want += [h * nb + u for u in sorted(singles, key=lambda u: (-rc[h, u], u))]
        want += [-1] * len(paired)
    assert sum(np.array_equal(keep[3, u], keep[3, u + 1]) for u in range(0, nb - 1, 2)) == nb // 2
    assert np.array_equal(order.cpu().numpy(), np.array(want))
    assert np.array_equal(tiles.cpu().numpy(), t)
    assert np.array_equal(counts.cpu().numpy(), rc.reshape(-1))


def test_rows_beyond_one_decode_chunk():
    """More than 2048 key blocks: the row list is decoded in several passes."""
    n, d = 64 * 2100 + 10, 64
    nb = -(-n // B)
    q, k, v = _rand_bf16(1, n, d, seed=16)
    rng = np.random.default_rng(16)
    keep = rng.random((1, nb, nb)) < 0.02
    keep[0, :, 2047:2050] = True
    keep[0, :, nb - 1] = True
    bits = crm.pack_rows(keep)
    got = _run_bf16(q, k, v, bits, 0.125)
    blocks = [(0, 0), (0, 1), (0, 2048), (0, nb - 1)] + [(0, int(x)) for x in rng.integers(0, nb, 6)]
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, 0.125, blocks=blocks)
    for (h, u), r in zip(blocks, ref):
        gu.assert_bf16_close(got[h, u * B:u * B + r.shape[0]], r, f"block {u}")


def test_decode_chunks_first_empty_and_growing_keys():
    """Rows spanning two 2048-block decode chunks, all run as single rows.  Some
    rows keep nothing in the first chunk, so the running max comes from the
    second chunk's first tile.  Others keep nothing in the second chunk.  In
    head 1, the keys of the second chunk are scaled up so that its logits pass
    the first chunk's max by far more than the fast walk accepts, and those rows
    are walked again, across both chunks, with the max tracked tile by tile."""
    n, d = 64 * 2100 + 10, 64
    nb = -(-n // B)
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((2, n, d)).astype(np.float32) for _ in range(3))
    k[1, 2048 * B:] *= 6.0
    q, k, v = (workloads.bf16_bits(x) for x in (q, k, v))
    keep = rng.random((2, nb, nb)) < 0.02
    keep[:, :, 10] = True
    keep[:, :, 2060] = True
    keep[:, 3, :2048] = False                        # first chunk empty
    keep[:, 4, 2048:] = False                        # second chunk empty
    keep[:, 5] = False                               # empty row
    keep[:, 5, nb - 1] = True                        # ... but for the ragged last block
    bits = crm.pack_rows(keep)
    order = torch.arange(2 * nb, dtype=torch.int32, device="cuda")
    got = _run_bf16(q, k, v, bits, 0.125, work_order=order)
    blocks = [(h, u) for h in (0, 1) for u in (0, 3, 4, 5, 2047, nb - 1)]
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, 0.125, blocks=blocks)
    for (h, u), r in zip(blocks, ref):
        gu.assert_bf16_close(got[h, u * B:u * B + r.shape[0]], r, f"head {h} block {u}")


@pytest.mark.parametrize("H,n,d", [(8, 64 * 70 + 17, 128), (12, 64 * 45, 64), (6, 64 * 90 + 3, 128),
                                   (5, 64 * 110, 64)])
def test_every_row_once_across_xcd_groups(H, n, d):
    """Single rows go out in slices whose XCD groups walk different heads (4
    groups when H % 4 == 0, else 2 or 1); with more rows than one slice takes,
    holes from paired rows and an empty row, every row is written once and
    matches the oracle (the output starts as NaN)."""
    nb = -(-n // B)
    q, k, v = _rand_bf16(H, n, d, seed=H * n)
    rng = np.random.default_rng(H + n)
    keep = rng.random((H, nb, nb)) < 0.3
    for h in range(H):
        for u in range(0, nb - 1, 2):
            if rng.random() < 0.2:
                keep[h, u + 1] = keep[h, u]
    keep[H - 1, 3] = False
    bits = crm.pack_rows(keep)
    out = torch.full((H, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = _run_bf16(q, k, v, bits, 1.0 / np.sqrt(d), out=out)
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, 1.0 / np.sqrt(d))
    gu.assert_bf16_close(got, ref, f"H={H} n={n} d={d}")
    assert np.all(got[H - 1, 3 * B:4 * B] == 0.0)
    # a caller's plain permutation of the rows, read through the same XCD groups:
    # every row written once and matching the oracle (rows the planner paired now
    # run as single rows, whose sums are ordered differently, so not bit for bit)
    perm = gu.to_dev(np.random.default_rng(H).permutation(H * nb).astype(np.int32))
    out2 = torch.full((H, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    got2 = _run_bf16(q, k, v, bits, 1.0 / np.sqrt(d), out=out2, work_order=perm)
    gu.assert_bf16_close(got2, ref, f"H={H} n={n} d={d} permuted")


@pytest.mark.parametrize("H,n", [(6, 64 * 800 + 9), (8, 64 * 600 + 33), (6, 64 * 1400 + 9),
                                 (8, 64 * 1100 + 33)])
def test_slices_beyond_the_pair_launch(H, n):
    """Single-row slices with two XCD groups (H = 6) and four (H = 8).  At the
    smaller lengths (10 slices) every slice rides in the pair launch.  At the
    larger ones (more than 16 slices) the last eight do, and the others go out
    one launch each.  Pairs, the pair launch's slices and the later slice
    launches together write every row once (the output starts as NaN), and
    sampled blocks, the ragged last one included, match the oracle."""
    d = 64
    nb = -(-n // B)
    q, k, v = _rand_bf16(H, n, d, seed=H * 1000 + n % 1000)
    rng = np.random.default_rng(H + n)
    u = np.arange(nb)
    keep = np.abs(u[:, None] - u[None, :]) <= 1
    keep = np.broadcast_to(keep, (H, nb, nb)) | (rng.random((H, nb, nb)) < rng.uniform(0.02, 0.08, (H, 1, 1)))
    for h in range(H):
        for uu in range(0, nb - 1, 2):
            if rng.random() < 0.1:
                keep[h, uu + 1] = keep[h, uu]
    keep[H - 1, 7] = False
    bits = crm.pack_rows(keep)
    out = torch.full((H, n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    got = _run_bf16(q, k, v, bits, 0.125, out=out)
    assert not np.isnan(got).any()
    assert np.all(got[H - 1, 7 * B:8 * B] == 0.0)
    blocks = [(0, 0), (H - 1, nb - 1), (H // 2, nb // 2)] + [(int(a), int(b)) for a, b in
                                                            zip(rng.integers(0, H, 9), rng.integers(0, nb, 9))]
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, 0.125, blocks=blocks)
    for (h, uu), r in zip(blocks, ref):
        gu.assert_bf16_close(got[h, uu * B:uu * B + r.shape[0]], r, f"H={H} block ({h}, {uu})")


def test_long_rows_past_the_planner_sort_limit():
    """More than 8192 query blocks per head: the planner keeps the rows in block
    order without pairs (its LDS sort covers 8192 rows), and the attention still
    matches the oracle; identical adjacent rows are included."""
    n, d = 64 * 8200 + 5, 64
    nb = -(-n // B)
    q, k, v = _rand_bf16(1, n, d, seed=17)
    rng = np.random.default_rng(17)
    u = np.arange(nb)
    keep = (np.abs(u[:, None] - u[None, :]) <= 1)[None].copy()
    extra = rng.integers(0, nb, size=(nb, 3))
    keep[0, u[:, None], extra] = True
    keep[0, 11] = keep[0, 10]                        # identical adjacent rows (no pair here)
    keep[0, 4000] = False                            # an empty row
    bits = crm.pack_rows(keep)
    mdev = gu.to_dev(bits)
    counts, tiles, order = bsa.plan(mdev, n)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), np.arange(nb))
    assert np.array_equal(counts.cpu().numpy(), keep[0].sum(1))
    assert int(tiles.cpu().numpy()[0]) == int(keep.sum())
    got = _run_bf16(q, k, v, bits, 0.125)
    blocks = [(0, 0), (0, 10), (0, 11), (0, 4000), (0, nb - 1)] + [(0, int(x)) for x in rng.integers(0, nb, 5)]
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, 0.125, blocks=blocks)
    for (h, uu), r in zip(blocks, ref):
        gu.assert_bf16_close(got[h, uu * B:uu * B + r.shape[0]], r, f"block {uu}")
    assert np.all(got[0, 4000 * B:4001 * B] == 0.0)


@pytest.mark.parametrize("name", ["wan13b_480p", "wan14b_720p"])
def test_workload_sampled_rows(name):
    w = workloads.WORKLOADS[name]
    keep = workloads.masks(w)
    bits = workloads.pack_bits(keep)
    q, k, v = workloads.qkv(w)
    print(f"[{name}] density {keep.mean():.3f}", flush=True)
    got = bsa.sparse_attn(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True), gu.to_dev(bits), w.scale)
    torch.cuda.synchronize()
    blocks = gu.sample_blocks(keep, 24, seed=w.seed)
    hs = sorted({h for h, _ in blocks})
    qf, kf, vf = (np.stack([_f(x[h]) for h in hs]) for x in (q, k, v))
    hmap = {h: i for i, h in enumerate(hs)}
    ref = sparse_attention(qf, kf, vf, bits[hs], w.scale, blocks=[(hmap[h], u) for h, u in blocks])
    out = got.cpu()
    for (h, u), r in zip(blocks, ref):
        g = gu.bf16_host(out[h, u * B:u * B + r.shape[0]])
        gu.assert_bf16_close(g, r, f"{name} block ({h},{u})")


def test_hunyuan_stripe_pipeline():
    w = workloads.WORKLOADS["hunyuan_768"]
    params = workloads.stripe_params(w)
    T, F = w.grid[0], w.frame_tokens
    mdev = bsa.mask_from_stripes(gu.to_dev(params), T, F, w.seq_len)
    torch.cuda.synchronize()
    bits_ref = stripes.stripe_mask_bits(params, T, F, w.seq_len)
    assert np.array_equal(gu.mask_host(mdev), bits_ref)
    q, k, v = workloads.qkv(w)
    got = bsa.sparse_attn(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True), mdev, w.scale)
    torch.cuda.synchronize()
    keep = crm.unpack_rows(bits_ref, w.n_blocks)
    blocks = gu.sample_blocks(keep, 16, seed=w.seed)
    hs = sorted({h for h, _ in blocks})
    hmap = {h: i for i, h in enumerate(hs)}
    qf, kf, vf = (np.stack([_f(x[h]) for h in hs]) for x in (q, k, v))
    ref = sparse_attention(qf, kf, vf, bits_ref[hs], w.scale, blocks=[(hmap[h], u) for h, u in blocks])
    out = got.cpu()
    for (h, u), r in zip(blocks, ref):
        gu.assert_bf16_close(gu.bf16_host(out[h, u * B:u * B + r.shape[0]]), r, f"hunyuan ({h},{u})")


@pytest.mark.parametrize("n,d", [(64 * 37 + 13, 128), (64 * 40, 64), (64 * 9 + 1, 128)])
def test_pairs_of_identical_rows(n, d):
    """Adjacent query blocks with identical mask rows run as one 128-query workgroup
    (planner pair entries); some pairs, some singles, empty pairs, a ragged last
    block inside a pair, all rows compared with the oracle."""
    nb = -(-n // B)
    H = 3
    q, k, v = _rand_bf16(H, n, d, seed=n + d)
    rng = np.random.default_rng(n)
    keep = rng.random((H, nb, nb)) < 0.3
    for h in range(H):
        for u in range(0, nb - 1, 2):
            if rng.random() < 0.6:
                keep[h, u + 1] = keep[h, u]
    keep[1, :] = True                      # a full head: every row paired
    keep[2, 0:2] = False                   # an empty pair
    if nb % 2 == 0:
        keep[0, nb - 1] = keep[0, nb - 2]  # the ragged last block inside a pair
    bits = crm.pack_rows(keep)
    _, _, order = bsa.plan(gu.to_dev(bits), n)
    o = order.cpu().numpy()
    assert (o >= H * nb).sum() > 0 and (o == -1).sum() == (o >= H * nb).sum()
    got = _run_bf16(q, k, v, bits, 1 / np.sqrt(d))
    ref = sparse_attention(_f(q), _f(k), _f(v), bits, 1 / np.sqrt(d))
    for h in range(H):
        gu.assert_bf16_close(got[h], ref[h], f"head {h}")
    assert np.all(got[2, :128] == 0)
    # the same result through a plain permutation (no pair entries)
    perm = gu.to_dev(np.random.default_rng(1).permutation(H * nb).astype(np.int32))
    got2 = _run_bf16(q, k, v, bits, 1 / np.sqrt(d), work_order=perm)
    for h in range(H):
        gu.assert_bf16_close(got2[h], ref[h], f"head {h} permuted")


def test_caller_workspace_matches_library_scratch():
    """sparse_attn_fwd_ws with a caller workspace gives the same bits as
    sparse_attn_fwd (same plan, same kernels), on two shapes in a row with one
    workspace sized for the larger, and matches the oracle."""
    cases = [(3, 64 * 21 + 9, 128), (2, 64 * 6 + 1, 64)]
    need = max(bsa.workspace_bytes(H, n, d) for H, n, d in cases)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for H, n, d in cases:
        q, k, v = _rand_bf16(H, n, d, seed=31 + n)
        nb = -(-n // B)
        keep = np.random.default_rng(n).random((H, nb, nb)) < 0.35
        keep[0, 1] = False
        bits = crm.pack_rows(keep)
        scale = 1.0 / np.sqrt(d)
        a = _run_bf16(q, k, v, bits, scale)
        b = _run_bf16(q, k, v, bits, scale, workspace=ws)
        assert np.array_equal(a, b)
        gu.assert_bf16_close(b, sparse_attention(_f(q), _f(k), _f(v), bits, scale), f"ws H={H} n={n} d={d}")
    with pytest.raises(bsa.BsaError):
        bsa.sparse_attn(gu.to_dev(q, True), gu.to_dev(k, True), gu.to_dev(v, True), gu.to_dev(bits), scale,
                        workspace=ws[:16])


def test_host_threads_growing_the_scratch_buffer():
    """Several host threads call the attention on the default stream at sizes larger
    than any earlier test's, so the library's scratch buffer is replaced (device
    synchronised, old buffer freed) while other threads are enqueueing work on it;
    every result equals the one computed through a caller workspace, which leaves
    the scratch buffer alone."""
    import threading
    H, d = 64, 128
    sizes = [50000, 54000, 58000, 62000]            # transposed V 0.82 .. 1.02 GB, above every other test
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    cases, want = [], []
    ws = torch.empty(bsa.workspace_bytes(H, max(sizes), d), dtype=torch.uint8, device="cuda")
    for n in sizes:
        q, k, v = (torch.randn((H, n, d), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
        nb = -(-n // B)
        keep = torch.rand((H, nb, nb), generator=g, device="cuda") < 0.02
        W = -(-nb // 64)
        pad = torch.zeros((H, nb, W * 64), dtype=torch.int64, device="cuda")
        pad[..., :nb] = keep.to(torch.int64)
        words = (pad.view(H, nb, W, 64) << torch.arange(64, device="cuda", dtype=torch.int64)).sum(-1)
        cases.append((q, k, v, words))
        want.append(bsa.sparse_attn(q, k, v, words, 1 / np.sqrt(d), workspace=ws))
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            torch.cuda.set_device(0)
            for j in range(len(cases)):
                out = bsa.sparse_attn(*cases[j], 1 / np.sqrt(d))
                torch.cuda.synchronize()
                if not torch.equal(out, want[j]):
                    errors.append((t, j))
        except Exception as e:          # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
