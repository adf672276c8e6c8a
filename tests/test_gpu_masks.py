"""GPU parity of the mask producers and the token permutation: bit-exact where
the result is an integer (stripes, top-p, permutation), within a derived
tolerance for the float block scores; plus the full dynamic top-p pipeline."""
import json
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_07_amd as bsa
import workloads
from oracle import block_scores, crm, hilbert, resize, stripes, threshold, topp
from oracle.attention import sparse_attention
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
B = 64
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _stripe_case(params, T, F):
    params = np.asarray(params, np.int32)
    m = bsa.mask_from_stripes(gu.to_dev(params), T, F, T * F)
    torch.cuda.synchronize()
    assert np.array_equal(gu.mask_host(m), stripes.stripe_mask_bits(params, T, F, T * F))


def test_stripes_printed_tuples_bit_exact():
    g = json.load(open(os.path.join(GOLD, "psa_stripe_tuples.json")))
    rows = [[1, 1, 0, 0, 1, 0, 0]] + [[0] + t for tab in g["tables"].values() for t in tab]
    _stripe_case(rows, 33, 60 * 64)          # HunyuanVideo 768x1280 latent grid
    _stripe_case(rows, 21, 3600)             # Wan 720p: 3600-token frames (not whole blocks)


def test_stripes_random_tuples_and_odd_frames():
    rng = np.random.default_rng(21)
    params = np.zeros((20, 7), np.int32)
    for i in range(20):
        params[i] = (int(rng.random() < 0.1), rng.integers(1, 12), rng.integers(-3, 4), rng.integers(0, 5),
                     rng.integers(1, 11), rng.integers(-2, 3), rng.integers(0, 7))
    for T, F in [(5, 64 * 7), (7, 100), (3, 1560), (1, 130)]:
        _stripe_case(params, T, F)


def test_stripes_whole_block_frames_and_degenerate_tuples():
    """Frames of 1, 2, 63, 64 whole blocks (one wave per row, words assembled from
    the frames they overlap) and 65 blocks (one thread per word); tuples with a
    zero or negative width keep nothing unless the head is full."""
    rng = np.random.default_rng(23)
    params = np.zeros((11, 7), np.int32)
    for i in range(9):
        params[i] = (int(i == 0), rng.integers(1, 9), rng.integers(-3, 4), rng.integers(0, 4),
                     rng.integers(1, 70), rng.integers(-5, 6), rng.integers(0, 9))
    params[9] = (0, 0, 0, 0, 3, 0, 0)
    params[10] = (0, 3, 0, 0, -1, 0, 0)
    for T, F in [(70, 64), (33, 128), (3, 64 * 63), (2, 64 * 64), (2, 64 * 65)]:
        _stripe_case(params, T, F)


@pytest.mark.parametrize("nk", [1, 5, 64, 65, 200, 300, 777, 1025, 1182, 1280, 1281, 1536, 1537, 2048, 4096])
def test_topp_bit_exact_random_scores(nk):
    """Row lengths cover every per-lane width of the one-wave-per-row kernel
    (1 .. 32 blocks per lane), both widths of the two-part kernel (1025 .. 1280
    and 1281 .. 1536 blocks, with their edges) and the workgroup kernel for
    longer rows; 51 rows leave a partial last workgroup."""
    s = workloads.random_scores(3, 17, nk, seed=nk)
    s[0, 0] = 0.0                                   # all ties
    s[0, 1] = np.round(s[0, 1])                     # many ties
    s[2, 3] = np.where(np.arange(nk) % 2 == 0, np.float32(-0.0), np.float32(0.0))   # -0 and +0 are equal
    s[1, 2, nk // 2] = 40.0                         # one dominant block
    sd = gu.to_dev(s)
    for p, mb in [(0.9, 8), (0.5, 0), (0.99, 3), (1.0, 8), (1e-6, 8)]:
        m = bsa.mask_from_block_scores_topp(sd, p, mb)
        torch.cuda.synchronize()
        assert np.array_equal(gu.mask_host(m), topp.topp_mask_bits(s, p, mb)), (p, mb)


@pytest.mark.parametrize("nk", [300, 1182, 1400, 2048, 3000])
def test_topp_non_finite_scores_bit_exact(nk):
    """NaN and +-inf scores take the clamp rule (NaN -> -FLT_MAX, +-inf -> +-FLT_MAX)
    in every kernel width: the one-wave rows (300, 2048 blocks), the two-part rows
    (1182, 1400) and the workgroup rows (3000), bit for bit with the oracle."""
    s = workloads.random_scores(2, 9, nk, seed=nk + 1)
    rng = np.random.default_rng(nk)
    for r in range(9):
        idx = rng.choice(nk, size=12, replace=False)
        s[0, r, idx[:4]] = np.nan
        s[0, r, idx[4:8]] = -np.inf
        s[0, r, idx[8:10]] = np.float32(-np.nan)     # negative-signed NaN
        if r % 3 == 0:
            s[0, r, idx[10]] = np.inf
        if r % 3 == 1:
            s[0, r, idx[10:12]] = np.inf               # two tied infinities
    s[1, 0] = np.nan                                    # a whole row of NaN
    s[1, 1] = -np.inf
    s[1, 2, :] = np.inf
    sd = gu.to_dev(s)
    for p, mb in [(0.9, 8), (1e-6, 8), (1.0, 0), (0.5, nk - 3)]:
        m = bsa.mask_from_block_scores_topp(sd, p, mb)
        torch.cuda.synchronize()
        assert np.array_equal(gu.mask_host(m), topp.topp_mask_bits(s, p, mb)), (p, mb)


def test_block_scores_within_fp32_bound():
    n, d = 64 * 37 + 9, 128
    rng = np.random.default_rng(22)
    q = workloads.bf16_bits(rng.standard_normal((3, n, d)).astype(np.float32))
    k = workloads.bf16_bits(rng.standard_normal((3, n, d)).astype(np.float32))
    scale = 1.0 / np.sqrt(d)
    got = bsa.block_scores_meanpool(gu.to_dev(q, True), gu.to_dev(k, True), scale)
    torch.cuda.synchronize()
    qf, kf = workloads.bf16_to_f32(q).astype(np.float64), workloads.bf16_to_f32(k).astype(np.float64)
    ref = block_scores.block_scores(qf, kf, scale)
    # error budget, relative to sum_c |qbar_c kbar_c|: the fp32 means (<= 64 eps
    # each), the three partial products dropped from the exact three-part bf16
    # split (<= 3 * 2^-24), fp32 accumulation over 48 MFMA steps of 16 products
    # (<= 64 eps) -- below 1.2e-5 in all, inside the 4e-5 bar
    qb, kb = block_scores.block_means(qf), block_scores.block_means(kf)
    bound = 4e-5 * scale * np.einsum("hud,hvd->huv", np.abs(qb), np.abs(kb)) + 1e-12
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())


def test_permute_gather_scatter_exact():
    rng = np.random.default_rng(23)
    n, d = 1000, 128
    x = workloads.bf16_bits(rng.standard_normal((2, n, d)).astype(np.float32))
    perm = rng.permutation(n).astype(np.int32)
    xd, pd = gu.to_dev(x, True), gu.to_dev(perm)
    y = bsa.permute_tokens(xd, pd)
    z = bsa.permute_tokens(y, pd, inverse=True)
    torch.cuda.synchronize()
    yh = y.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yh, hilbert.permute_rows(x, perm))
    assert np.array_equal(z.cpu().view(torch.int16).numpy().view(np.uint16), x)
    xf = rng.standard_normal((1, n, 64)).astype(np.float32)
    yf = bsa.permute_tokens(gu.to_dev(xf), pd, inverse=True)
    torch.cuda.synchronize()
    assert np.array_equal(yf.cpu().numpy(), hilbert.permute_rows(xf, perm, inverse=True))


@pytest.mark.parametrize("nb,d", [(1300, 128), (1300, 64), (2600, 64)])
def test_block_scores_strip_and_tile_forms(nb, d):
    """Row counts whose 32-row strips do not fit in LDS (16-row strips) and whose
    16-row strips do not either (128 x 128 tiles), against the same bound."""
    n = 64 * nb - 23
    rng = np.random.default_rng(nb + d)
    q = workloads.bf16_bits(rng.standard_normal((1, n, d)).astype(np.float32))
    k = workloads.bf16_bits(rng.standard_normal((1, n, d)).astype(np.float32))
    scale = 1.0 / np.sqrt(d)
    got = bsa.block_scores_meanpool(gu.to_dev(q, True), gu.to_dev(k, True), scale)
    torch.cuda.synchronize()
    qf, kf = workloads.bf16_to_f32(q).astype(np.float64), workloads.bf16_to_f32(k).astype(np.float64)
    ref = block_scores.block_scores(qf, kf, scale)
    qb, kb = block_scores.block_means(qf), block_scores.block_means(kf)
    bound = 4e-5 * scale * np.einsum("hud,hvd->huv", np.abs(qb), np.abs(kb)) + 1e-12
    err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), float((err / bound).max())


def test_topp_pipeline_end_to_end():
    """Hilbert permute -> block scores -> top-p mask -> attention -> unpermute, at
    the Wan2.1-14B 720p shape, against the oracle pipeline."""
    w = workloads.WORKLOADS["topp_wan14b"]
    T, Hh, Ww = w.grid
    p, mb = 0.9, 8
    perm = bsa.hilbert3d_order(T, Hh, Ww)
    assert np.array_equal(perm, hilbert.hilbert_order(T, Hh, Ww))
    q, k, v = workloads.qkv(w)
    pd = gu.to_dev(perm)
    qd, kd, vd = (bsa.permute_tokens(gu.to_dev(x, True), pd) for x in (q, k, v))
    sc = bsa.block_scores_meanpool(qd, kd, w.scale)
    mask = bsa.mask_from_block_scores_topp(sc, p, mb)
    yd = bsa.sparse_attn(qd, kd, vd, mask, w.scale)
    out = bsa.permute_tokens(yd, pd, inverse=True)
    torch.cuda.synchronize()
    bits_gpu = gu.mask_host(mask)
    # the selection itself is bit-exact: the oracle's float32 procedure on the GPU's
    # own scores gives the GPU's mask on every one of the 47,280 rows
    assert np.array_equal(bits_gpu, topp.topp_mask_bits(sc.cpu().numpy(), p, mb))
    # oracle pipeline: float64 scores, rounded once to float32, then the float32 selection
    qp = hilbert.permute_rows(q, perm)
    kp = hilbert.permute_rows(k, perm)
    vp = hilbert.permute_rows(v, perm)
    f = lambda x: workloads.bf16_to_f32(x).astype(np.float64)
    s_ref = np.stack([block_scores.block_scores(f(qp[h:h + 1]), f(kp[h:h + 1]), w.scale)[0]
                      for h in range(w.n_heads)])
    bits_ref = topp.topp_mask_bits(s_ref.astype(np.float32), p, mb)
    same = np.all(bits_gpu == bits_ref, axis=-1)
    print(f"[topp] density {crm.unpack_rows(bits_gpu, w.n_blocks).mean():.4f}, "
          f"rows differing {int((~same).sum())} of {same.size}", flush=True)
    assert (~same).sum() <= max(5, same.size // 1000)
    # A row may differ where the float32 cumulative mass passes p within reach of
    # rounding, or where blocks whose scores are equal within the block-score
    # tolerance straddle the cut-off (their order is not fixed by fp32-accurate
    # scores): then both sides keep the same number of blocks.
    keep = crm.unpack_rows(bits_ref, w.n_blocks)
    keep_gpu = crm.unpack_rows(bits_gpu, w.n_blocks)
    for h, u in zip(*np.nonzero(~same)):
        if topp.boundary_margin(s_ref[h, u], p, mb) < 1e-4:
            continue
        kr, kg = keep[h, u], keep_gpu[h, u]
        assert kr.sum() == kg.sum(), (h, u)
        d = np.nonzero(kr != kg)[0]
        cut = np.sort(s_ref[h, u])[::-1][int(kr.sum()) - 1]
        qb = block_scores.block_means(f(qp[h:h + 1]))[0, u]
        kb = block_scores.block_means(f(kp[h:h + 1]))[0, d]
        tol = 4e-5 * w.scale * (np.abs(kb) @ np.abs(qb))
        assert np.all(np.abs(s_ref[h, u, d] - cut) <= tol), (h, u, d)
    blocks = [b for b in gu.sample_blocks(keep, 16, seed=w.seed) if same[b]]
    hs = sorted({h for h, _ in blocks})
    hmap = {h: i for i, h in enumerate(hs)}
    qf, kf, vf = (np.stack([f(x[h]) for h in hs]) for x in (qp, kp, vp))
    ref = sparse_attention(qf, kf, vf, bits_ref[hs], w.scale, blocks=[(hmap[h], u) for h, u in blocks])
    outh = out.cpu()
    for (h, u), r in zip(blocks, ref):
        rows = perm[u * B:u * B + r.shape[0]]
        g = gu.bf16_host(outh[h][torch.from_numpy(rows.astype(np.int64))])
        gu.assert_bf16_close(g, r, f"topp ({h},{u})")


def _threshold_case(T, p):
    T = np.ascontiguousarray(T, np.float32)
    p = np.ascontiguousarray(p, np.float32)
    m = bsa.mask_from_threshold_map(gu.to_dev(T), gu.to_dev(p))
    torch.cuda.synchronize()
    assert np.array_equal(gu.mask_host(m), threshold.threshold_mask_bits(T, p))


def test_threshold_hand_example_bit_exact():
    g = json.load(open(os.path.join(GOLD, "threshold_hand_example.json")))
    T = np.array([[[float(x) for x in row] for row in head] for head in g["T"]], dtype=np.float32)
    _threshold_case(T, g["p"])


@pytest.mark.parametrize("nk", [1, 63, 64, 65, 1182])
def test_threshold_random_maps_with_ties_bit_exact(nk):
    rng = np.random.default_rng(100 + nk)
    H, nq = 3, 37
    # levels on a coarse grid so exact ties with p* are frequent; a few NaN / inf entries
    T = (rng.integers(0, 21, size=(H, nq, nk)) / 20.0).astype(np.float32)
    flat = T.reshape(-1)
    idx = rng.choice(flat.size, size=min(flat.size, 9), replace=False)
    flat[idx[:3]] = np.nan
    flat[idx[3:6]] = np.inf
    flat[idx[6:]] = -np.inf
    _threshold_case(T, [0.35, 0.5, 1.0])


def test_threshold_workload_map_at_layer_shape():
    w = workloads.WORKLOADS["wan14b_720p"]
    T, p = workloads.threshold_map(w.n_heads, w.n_blocks, seed=7)
    _threshold_case(T, p)


@pytest.mark.parametrize("nb,nt", [(6, 12), (9, 9), (20, 13), (70, 131), (100, 64), (33, 200), (512, 1182), (1500, 700)])
def test_resize_maps_match_oracle(nb, nt):
    rng = np.random.default_rng(nb * 1000 + nt)
    H = 2
    keep = rng.random((H, nb, nb)) < 0.15
    got = bsa.mask_resize(gu.to_dev(crm.pack_rows(keep)), nb, nt)
    torch.cuda.synchronize()
    assert np.array_equal(gu.mask_host(got), crm.pack_rows(resize.resize_region(keep, nt)))
    T = rng.random((H, nb, nb), dtype=np.float32)
    T[0, 0, nb - 1] = np.nan
    Tt = bsa.threshold_map_resize(gu.to_dev(T), nt).cpu().numpy()
    ref = resize.resize_threshold(T, nt)
    assert np.array_equal(np.isnan(Tt), np.isnan(ref))
    assert np.array_equal(Tt[~np.isnan(Tt)], ref[~np.isnan(ref)])


def test_resize_commutes_with_threshold_masks_on_device():
    """Resizing the threshold map then instantiating equals instantiating then resizing
    the region map (the conservative reading of Eq. 7), at the 480p -> 720p block counts."""
    T, p = workloads.threshold_map(4, 512, seed=8)
    Td, pd = gu.to_dev(T), gu.to_dev(p)
    a = bsa.mask_from_threshold_map(bsa.threshold_map_resize(Td, 1182), pd)
    b = bsa.mask_resize(bsa.mask_from_threshold_map(Td, pd), 512, 1182)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
