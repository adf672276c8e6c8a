"""Benchmark: block-sparse attention at the Wan2.1-14B 720p layer shape on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--profile]
                    [--sweep] [--aux] [--topp] [--b128] [--cold] [--ceiling]

Workload (synthetic, seeded): 40 heads, head_dim 128, bf16, latent grid
21x45x80 = 75,600 tokens (1182 blocks of 64); 8 heads keep every block, the
other 32 keep a band |u-v| <= 1 plus uniformly random blocks up to a per-head
density drawn from U[0.05, 0.40].

One step = one pass of the hot path on that layer: the tile scheduler (row
popcounts, head order) and the block-sparse attention kernel, via
sparse_attn_fwd.  Inputs are resident in HBM before timing starts.

Reported on one JSON line:
  value      effective TFLOP/s on kept blocks = kept tiles * 4*64*64*128 / step time
  speedup_vs_full_mask   step time with an all-ones mask / step time with the workload mask
  roofline   one planned call of the attention path (V transpose, pair launch,
             single-row slices; events on its stream): algorithmic flops per call /
             average call time vs the bf16 MFMA peak
  cpu_baseline  the float64 CPU oracle on a bounded sample of query blocks

--sweep  (extra, to stderr) uniform random masks at 5 .. 100 % density on the same
         shape: speedup against 1/density (the analogue of ScalingAttention Fig. 5).
--aux    (extra, to stderr) the HBM-bound kernels of the path (mask producers,
         block scores, top-p, permutation, resize, fidelity) in GB/s vs 8 TB/s.
--topp   (extra, to stderr) the dynamic top-p layer end to end on its workload:
         Hilbert gather of Q, K, V, block scores, top-p mask, attention, scatter.
--b128   (extra, to stderr) the same layer under the same mask recipe drawn over
         128x128-token blocks and passed as 32-bit row words (ScalingAttention's CRM format).
--cold   (extra, to stderr) steps timed one by one after a 512 MiB device write that
         evicts the 256 MB last-level cache (MALL), median against back-to-back steps.
--ceiling (extra, to stderr) a reference point for the roofline, not part of the path:
         a dense bf16 GEMM from the vendor library (torch.matmul) at 8192^3 and 16384^3,
         and the effective rate of one planned call as a fraction of it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_wan14b_720p_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_07_amd", "csrc", "attn_bf16.hip")


def tile_flops(d: int) -> float:
    return 4.0 * 64 * 64 * d


def read_traffic():
    """HBM bytes per attention launch from the committed counter summary, or None
    when the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    src_hash = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, q, k, v, bits, keep, budget_s=12.0):
    """Time the float64 oracle on a seeded sample of query blocks until about
    budget_s seconds of CPU work; report kept-tile flops per second."""
    from oracle.attention import sparse_attention
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(1234)
    nb = w.n_blocks
    order = rng.permutation(w.n_heads * nb)
    cache = {}
    tiles = 0
    blocks = 0
    t0 = time.perf_counter()
    spent = 0.0
    for rid in order:
        h, u = divmod(int(rid), nb)
        if h not in cache:
            cache[h] = tuple(workloads.bf16_to_f32(x[h]).astype(np.float64)[None] for x in (q, k, v))
        qh, kh, vh = cache[h]
        ts = time.perf_counter()
        sparse_attention(qh, kh, vh, bits[h:h + 1], w.scale, blocks=[(0, u)])
        spent += time.perf_counter() - ts
        tiles += int(keep[h, u].sum())
        blocks += 1
        if spent >= budget_s and blocks >= 8:
            break
    value = tiles * tile_flops(w.head_dim) / spent / 1e12
    return {
        "value": round(value, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{blocks} random (head, query block) rows of the same layer, {tiles} kept tiles, "
                  f"{spent:.1f} s of float64 numpy/BLAS",
    }


def device_uniform_mask(torch, H, nb, density, seed, dev):
    """Bernoulli(density) blocks drawn on the device (seeded), packed to int64 words."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    keep = torch.rand((H, nb, nb), generator=g, device=dev) < density
    W = -(-nb // 64)
    pad = torch.zeros((H, nb, W * 64), dtype=torch.int64, device=dev)
    pad[..., :nb] = keep.to(torch.int64)
    shifts = torch.arange(64, device=dev, dtype=torch.int64)
    words = (pad.view(H, nb, W, 64) << shifts).sum(-1)      # distinct bits: the sum is the OR
    return words, int(keep.sum().item())


def density_sweep(bsa, torch, w, qd, kd, vd, out, timed, ms_full):
    dev = qd.device
    for dens in (0.05, 0.10, 0.20, 0.40, 0.60, 0.80, 1.00):
        md, kept = device_uniform_mask(torch, w.n_heads, w.n_blocks, dens, 100 + int(dens * 100), dev)
        f = lambda: bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out)
        f()
        ms = timed(f, 5)
        rec = {"sweep_density": dens, "kept_tiles": kept, "ms": round(ms, 3),
               "tflops": round(kept * tile_flops(w.head_dim) / (ms * 1e-3) / 1e12, 1),
               "speedup_vs_full": round(ms_full / ms, 3), "ideal_speedup": round(1 / dens, 3)}
        print(json.dumps(rec), file=sys.stderr, flush=True)
        del md


def b128_layer(bsa, torch, w, qd, kd, vd, out, timed, ms_full):
    """The same layer with the mask recipe drawn over ScalingAttention's 128-token blocks,
    passed as 32-bit row words.  Flops count the kept 64-token tiles of the same
    mask (the expanded form), as the headline metric does."""
    import workloads
    keep = workloads.mask_wan14b(w, block=128)
    words = workloads.pack_bits32(keep)
    wd = torch.from_numpy(words.view(np.int32)).to(qd.device)
    m64 = bsa.mask_b128_to_b64(wd, w.seq_len)
    kept = int(sum(int(x).bit_count() for x in m64.cpu().numpy().view(np.uint64).ravel()))
    f = lambda: bsa.sparse_attn_b128(qd, kd, vd, wd, w.scale, out=out)
    f()
    ms = timed(f, 10)
    print(json.dumps({"b128_layer": "Wan2.1-14B 720p, 128x128 blocks, 32-bit words",
                      "density": round(float(keep.mean()), 4), "kept_64_tiles": kept, "ms": round(ms, 3),
                      "tflops": round(kept * tile_flops(w.head_dim) / (ms * 1e-3) / 1e12, 1),
                      "speedup_vs_full": round(ms_full / ms, 3)}), file=sys.stderr, flush=True)


def topp_layer(bsa, torch, timed):
    """The dynamic top-p layer end to end on its own workload (Q and K carry the
    per-frame rank-8 component): Hilbert gather of Q, K, V, mean-pooled block
    scores, top-p 0.9 with at least 8 blocks, planner + block-sparse attention,
    scatter of O back to token order.  Per-stage and whole-chain times (stderr)."""
    import workloads
    dev = torch.device("cuda", 0)
    w = workloads.WORKLOADS["topp_wan14b"]
    q, k, v = workloads.qkv(w)
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = tb(q), tb(k), tb(v)
    del q, k, v
    perm = torch.from_numpy(bsa.hilbert3d_order(*w.grid)).to(dev)
    qp, kp, vp, o, y = (torch.empty_like(qd) for _ in range(5))
    H, N, nb = w.n_heads, w.seq_len, w.n_blocks
    scores = torch.empty((H, nb, nb), dtype=torch.float32, device=dev)
    mask = torch.empty((H, nb, bsa.mask_words(N)), dtype=torch.int64, device=dev)
    stages = {
        "hilbert_gather_qkv": lambda: [bsa.permute_tokens(a, perm, out=b) for a, b in ((qd, qp), (kd, kp), (vd, vp))],
        "block_scores": lambda: bsa.block_scores_meanpool(qp, kp, w.scale, out=scores),
        "topp_mask": lambda: bsa.mask_from_block_scores_topp(scores, 0.9, 8, out=mask),
        "plan_and_attention": lambda: bsa.sparse_attn(qp, kp, vp, mask, w.scale, out=o),
        "scatter_o": lambda: bsa.permute_tokens(o, perm, inverse=True, out=y),
    }
    for fn in stages.values():
        fn()
    torch.cuda.synchronize()
    kept = int(np.unpackbits(mask.cpu().numpy().view(np.uint8)).sum())
    rec = {"topp_layer": "Wan2.1-14B 720p, Hilbert order, top-p 0.9, min 8 blocks",
           "density": round(kept / (H * nb * nb), 4), "kept_tiles": kept}
    for name, fn in stages.items():
        rec[name + "_ms"] = round(timed(fn, 5), 3)
    total = timed(lambda: [fn() for fn in stages.values()], 5)
    rec["total_ms"] = round(total, 3)
    rec["attention_share"] = round(rec["plan_and_attention_ms"] / total, 3)
    rec["layer_tflops_on_kept_tiles"] = round(kept * tile_flops(w.head_dim) / (total * 1e-3) / 1e12, 1)
    print(json.dumps(rec), file=sys.stderr, flush=True)


def aux_kernels(bsa, torch, timed):
    """Effective bandwidth of the HBM-bound kernels on the configs' shapes."""
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    H, N, d = 40, 75600, 128
    nb = -(-N // 64)
    W = -(-nb // 64)
    x = torch.randn((H, N, d), generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)

    def report(name, fn, nbytes, n=5):
        fn()
        ms = timed(fn, n)
        print(json.dumps({"aux": name, "ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "frac_of_8TBps": round(nbytes / (ms * 1e-3) / 8e12, 3)}), file=sys.stderr, flush=True)

    perm = torch.randperm(N, generator=g, device=dev).to(torch.int32)
    report("permute_tokens gather [40,75600,128] bf16", lambda: bsa.permute_tokens(x, perm, out=y), 2 * x.numel() * 2)
    scores = torch.empty((H, nb, nb), dtype=torch.float32, device=dev)
    report("block_scores_meanpool q,k [40,75600,128]", lambda: bsa.block_scores_meanpool(x, x, out=scores),
           2 * x.numel() * 2 + scores.numel() * 4)
    scores.normal_(generator=g)
    mw = torch.empty((H, nb, W), dtype=torch.int64, device=dev)
    report("mask_from_block_scores_topp p=0.9 min 8", lambda: bsa.mask_from_block_scores_topp(scores, 0.9, 8, out=mw),
           scores.numel() * 4 + mw.numel() * 8)
    pth = torch.rand((H,), generator=g, device=dev)
    report("mask_from_threshold_map [40,1182,1182]", lambda: bsa.mask_from_threshold_map(scores, pth, out=mw),
           scores.numel() * 4 + mw.numel() * 8)
    tb = torch.rand((H, 512, 512), generator=g, device=dev)
    tt = torch.empty((H, nb, nb), dtype=torch.float32, device=dev)
    report("threshold_map_resize 512 -> 1182", lambda: bsa.threshold_map_resize(tb, nb, out=tt),
           tb.numel() * 4 + tt.numel() * 4)
    mb = torch.zeros((H, 512, 8), dtype=torch.int64, device=dev)
    report("mask_resize 512 -> 1182", lambda: bsa.mask_resize(mb, 512, nb, out=mw), mb.numel() * 8 + mw.numel() * 8)
    rows = torch.randint(0, N, (H, 16), generator=g, device=dev, dtype=torch.int32)
    report("attn_fidelity 16 rows per head", lambda: bsa.attn_fidelity(x, x, mw, rows), x.numel() * 2)
    Hh, T, F = 24, 33, 3840
    nbh = T * F // 64
    params = torch.tensor([[0, 5, 0, 0, 3, 0, 3]] * Hh, dtype=torch.int32, device=dev)
    ms_out = torch.empty((Hh, nbh, -(-nbh // 64)), dtype=torch.int64, device=dev)
    report("mask_from_stripes HunyuanVideo 24 heads", lambda: bsa.mask_from_stripes(params, T, F, T * F, out=ms_out),
           ms_out.numel() * 8)


def gemm_ceiling(torch, timed, achieved):
    """A dense bf16 GEMM from the vendor library (context for the roofline only)."""
    dev = torch.device("cuda", 0)
    best = 0.0
    for n in (8192, 16384):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        fn = lambda: torch.matmul(a, b, out=c)
        fn()
        ms = timed(fn, 10 if n == 8192 else 4)
        tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
        best = max(best, tf)
        print(json.dumps({"ceiling": f"vendor bf16 GEMM {n}^3 (torch.matmul)", "ms": round(ms, 3),
                          "tflops": round(tf, 1)}), file=sys.stderr, flush=True)
        del a, b, c
    print(json.dumps({"ceiling_best_tflops": round(best, 1), "planned_call_tflops": round(achieved, 1),
                      "frac_of_ceiling": round(achieved / best, 3)}), file=sys.stderr, flush=True)


def cold_steps(torch, fn, stream, n, ms_warm):
    """Median single-step time after a 512 MiB write that evicts the 256 MB MALL."""
    junk = torch.empty(1 << 28, dtype=torch.int16, device=stream.device)
    times = []
    for _ in range(n):
        junk.fill_(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    print(json.dumps({"cold_step_ms": round(times[len(times) // 2], 3), "steps": n,
                      "warm_step_ms": round(ms_warm, 3)}), file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="short run for counter collection: a few planned launches plus a 1 GiB copy")
    ap.add_argument("--sweep", action="store_true", help="also run the density sweep (stderr)")
    ap.add_argument("--aux", action="store_true", help="also time the HBM-bound kernels (stderr)")
    ap.add_argument("--topp", action="store_true", help="also time the dynamic top-p layer end to end (stderr)")
    ap.add_argument("--b128", action="store_true",
                    help="also time the layer under a 128x128-block mask in 32-bit words (stderr)")
    ap.add_argument("--cold", action="store_true",
                    help="also time single steps after evicting the last-level cache (stderr)")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time a vendor-library bf16 GEMM as a practical MFMA ceiling (stderr)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads would shard across GPUs with no exchange step; not built here)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_07_amd as bsa
    import workloads

    dev = torch.device("cuda", 0)
    w = workloads.WORKLOADS["wan14b_720p"]
    keep = workloads.masks(w)
    bits = workloads.pack_bits(keep)
    q, k, v = workloads.qkv(w)
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = tb(q), tb(k), tb(v)
    md = torch.from_numpy(bits.view(np.int64)).to(dev)
    full_bits = workloads.pack_bits(np.ones((1, w.n_blocks, w.n_blocks), bool))
    fd = torch.from_numpy(np.repeat(full_bits, w.n_heads, axis=0).view(np.int64)).to(dev)
    out = torch.empty_like(qd)
    kept = int(keep.sum())
    flops = kept * tile_flops(w.head_dim)
    full_flops = w.n_heads * w.n_blocks ** 2 * tile_flops(w.head_dim)
    stream = torch.cuda.current_stream(dev)

    def step(mask):
        bsa.sparse_attn(qd, kd, vd, mask, w.scale, out=out)

    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    if args.profile:
        _, _, order = bsa.plan(md, w.seq_len)
        for _ in range(3):
            bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out, work_order=order)
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)    # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "done", "attn_launches": 3, "copy_bytes": 1 << 30}), flush=True)
        return

    for _ in range(args.warmup):
        step(md)
    ms = timed(lambda: step(md), args.steps)
    print(f"[bench] sparse step {ms:.3f} ms", file=sys.stderr, flush=True)

    for _ in range(max(1, args.warmup // 2)):
        step(fd)
    ms_full = timed(lambda: step(fd), max(3, args.steps // 3))
    print(f"[bench] full-mask step {ms_full:.3f} ms", file=sys.stderr, flush=True)

    _, _, order = bsa.plan(md, w.seq_len)
    planned = lambda: bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out, work_order=order)
    planned()
    ms_k = timed(planned, args.steps)
    achieved = flops / (ms_k * 1e-3) / 1e12

    rec = {
        "metric": "effective bf16 TFLOP/s on kept blocks + speedup vs full mask, Wan-14B 720p shape",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "Wan2.1-14B 720p attention layer: 40 heads, head_dim 128, 21x45x80=75600 "
                        "tokens, 64x64 blocks, 8 full heads + banded-random heads (density U[0.05,0.40])",
            "n_heads": w.n_heads, "seq_len": w.seq_len, "head_dim": w.head_dim, "block": 64,
            "kept_tiles": kept, "density": round(kept / (w.n_heads * w.n_blocks ** 2), 4),
            "parallelism": "single GPU",
        },
        "speedup_vs_full_mask": round(ms_full / ms, 3),
        "full_mask_ms": round(ms_full, 4),
        "full_mask_tflops": round(full_flops / (ms_full * 1e-3) / 1e12, 3),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic(),
            "kernel": "attn_pair_kernel<128> (pair rows) + attn_fwd_bf16_kernel<128> (single rows), one planned call",
            "kernel_ms": round(ms_k, 4),
        },
    }
    if args.sweep:
        density_sweep(bsa, torch, w, qd, kd, vd, out, timed, ms_full)
    if args.aux:
        aux_kernels(bsa, torch, timed)
    if args.topp:
        topp_layer(bsa, torch, timed)
    if args.b128:
        b128_layer(bsa, torch, w, qd, kd, vd, out, timed, ms_full)
    if args.cold:
        cold_steps(torch, lambda: step(md), stream, max(5, args.steps), ms)
    if args.ceiling:
        gemm_ceiling(torch, timed, achieved)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, bits, keep)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
