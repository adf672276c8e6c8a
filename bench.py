"""Benchmark: block-sparse attention on one GPU at the shapes of the video-DiT layers.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
                    [--profile] [--aux] [--b128] [--cold] [--ceiling]

Headline workload (synthetic, seeded): the Wan2.1-14B 720p layer, 40 heads,
head_dim 128, bf16, latent grid 21x45x80 = 75,600 tokens (1182 blocks of 64);
8 heads keep every block, the other 32 keep a band |u-v| <= 1 plus uniformly
random blocks up to a per-head density drawn from U[0.05, 0.40].

One step = one pass of the hot path on that layer: the tile scheduler (row
popcounts, head order) and the block-sparse attention kernel, via
sparse_attn_fwd.  Inputs are resident in HBM before timing starts.

Reported on one JSON line:
  value      effective TFLOP/s on kept blocks = kept tiles * 4*64*64*128 / step time
             (mean over the K timed steps); median_ms_per_step from per-step events
  speedup_vs_full_mask   step time with an all-ones mask / step time with the workload mask
  roofline   one planned call of the attention path (V transpose, pairs plus the last
             single-row slices, the other slices; events on its stream): algorithmic flops per call /
             average call time vs the bf16 MFMA peak
  cpu_baseline  the float64 CPU oracle on a bounded sample of query blocks
  wan13b_480p, hunyuan_768   the other layer shapes, each with its step time,
             effective TFLOP/s, speedup over the all-ones mask and roofline fraction
             (HunyuanVideo: stripe masks expanded on the device by mask_from_stripes;
             the expansion is timed on its own and is not inside the attention step)
  topp_wan14b   the dynamic top-p layer end to end (Hilbert gather of Q, K, V, block
             scores, top-p mask, planner + attention, scatter of O) with per-stage times
  density_sweep  uniform random masks at 5 .. 100 % density on the headline shape:
             speedup against 1/density (the analogue of ScalingAttention Fig. 5)
  gpu_clock  SCLK / MCLK read by amd-smi while the headline step runs
  --quick skips the extra layers, the top-p layer and the sweep.

--aux    (extra, to stderr) the HBM-bound kernels of the path (mask producers,
         block scores, top-p, permutation, resize, fidelity) in GB/s vs 8 TB/s.
--b128   (extra, to stderr) the same layer under the same mask recipe drawn over
         128x128-token blocks and passed as 32-bit row words (ScalingAttention's CRM format).
cold     (default run; with --quick only under --cold) steps timed one by one after a
         512 MiB device write that evicts the 256 MB last-level cache (MALL), median
         against the median of the back-to-back steps.
dense_sdpa  (default run) dense attention at the headline shape from PyTorch's fused
         kernels (flash / memory-efficient backend, never the math backend), and how much
         faster the all-ones and workload masks run here: context, not part of the path.
mfma_ceiling  (default run; with --quick only under --ceiling) reference points for the
         roofline, not part of the path, measured on the same GPU: the library's
         register-only MFMA probe (bsa_mfma_probe) and a dense bf16 GEMM from the vendor
         library (torch.matmul) at 8192^3 and 16384^3, with the headline and all-ones
         rates as fractions of each.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
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


def host_cpu():
    """Threads this process may run on, and the CPU model (lscpu)."""
    cores = len(os.sched_getaffinity(0))
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return cores, model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return None


def cpu_baseline(w, q, k, v, bits, keep, budget_s=12.0):
    """Time the float64 oracle on a seeded sample of query blocks until about
    budget_s seconds of CPU work; report kept-tile flops per second."""
    from oracle.attention import sparse_attention
    import workloads
    cores, model = host_cpu()
    rng = np.random.default_rng(1234)
    nb = w.n_blocks
    order = rng.permutation(w.n_heads * nb)
    cache = {}
    tiles = 0
    blocks = 0
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
    threads = blas_threads()
    return {
        "value": round(value, 6), "unit": "TFLOP/s", "cores": min(cores, threads) if threads else cores,
        "kind": "oracle",
        "sample": f"{blocks} random (head, query block) rows of the same layer, {tiles} kept tiles, "
                  f"{spent:.1f} s of float64 numpy/BLAS",
        "affinity_cores": cores, "blas_threads": threads, "cpu_model": model,
    }


class Timer:
    """HIP events on one stream: mean over a run of back-to-back steps, and the
    median of the per-step intervals between consecutive events."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, fn, n):
        torch = self.torch
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(self.stream)
        for i in range(n):
            fn()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
        return ev[0].elapsed_time(ev[n]) / n, per[n // 2]

    def __call__(self, fn, n):
        return self.run(fn, n)[0]


def gpu_clock_while(fn, seconds=2.0):
    """SCLK and MCLK as amd-smi reports them while fn runs back to back (None when
    the tool is missing or its output is not understood)."""
    import torch
    try:
        proc = subprocess.Popen(["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except Exception:
        return None
    t0 = time.perf_counter()
    while proc.poll() is None and time.perf_counter() - t0 < seconds + 20:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    try:
        out, _ = proc.communicate(timeout=5)
        return parse_amdsmi_clock(json.loads(out))
    except Exception:
        proc.kill()
        proc.wait()
        return None


def parse_amdsmi_clock(js):
    """Current GFX clock of each XCD (SCLK) and the memory clock (MCLK), in MHz, from
    amd-smi's metric JSON (gpu_data[0].clock.gfx_N.clk and mem_0.clk)."""
    clocks = js["gpu_data"][0]["clock"] if isinstance(js, dict) else js[0]["clock"]
    cur = lambda dom: clocks[dom]["clk"]["value"] if isinstance(clocks[dom].get("clk"), dict) else None
    gfx = [cur(k) for k in sorted(clocks) if k.startswith("gfx_") and cur(k) is not None]
    mem = cur("mem_0") if "mem_0" in clocks else None
    if not gfx:
        return None
    return {"sclk_mhz_per_xcd": gfx, "sclk_mhz_mean": round(sum(gfx) / len(gfx), 1), "mclk_mhz": mem,
            "source": "amd-smi metric --clock, sampled once while the headline step runs back to back"}


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


def full_mask(torch, H, nb, dev):
    W = -(-nb // 64)
    words = np.zeros((nb, W), np.uint64)
    words[:, :] = np.uint64(2 ** 64 - 1)
    if nb % 64:
        words[:, -1] = np.uint64((1 << (nb % 64)) - 1)
    return torch.from_numpy(np.ascontiguousarray(np.broadcast_to(words, (H, nb, W))).view(np.int64)).to(dev)


def density_sweep(bsa, torch, w, qd, kd, vd, out, timer, ms_full):
    res = []
    for dens in (0.05, 0.10, 0.20, 0.40, 0.60, 0.80, 1.00):
        md, kept = device_uniform_mask(torch, w.n_heads, w.n_blocks, dens, 100 + int(dens * 100), qd.device)
        f = lambda: bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out)
        f()
        ms = timer(f, 5)
        rec = {"density": dens, "kept_tiles": kept, "ms": round(ms, 3),
               "tflops": round(kept * tile_flops(w.head_dim) / (ms * 1e-3) / 1e12, 1),
               "speedup_vs_full": round(ms_full / ms, 3), "ideal_speedup": round(1 / dens, 3)}
        print("[bench] sweep " + json.dumps(rec), file=sys.stderr, flush=True)
        res.append(rec)
        del md
    return res


def layer_record(w, kept, ms, ms_med, ms_full):
    full = w.n_heads * w.n_blocks ** 2
    tf = kept * tile_flops(w.head_dim) / (ms * 1e-3) / 1e12
    return {
        "n_heads": w.n_heads, "seq_len": w.seq_len, "head_dim": w.head_dim, "kept_tiles": kept,
        "density": round(kept / full, 4), "ms": round(ms, 4), "median_ms": round(ms_med, 4),
        "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "full_mask_ms": round(ms_full, 4),
        "full_mask_tflops": round(full * tile_flops(w.head_dim) / (ms_full * 1e-3) / 1e12, 1),
        "speedup_vs_full_mask": round(ms_full / ms, 3), "ideal_speedup": round(full / kept, 3),
    }


def static_layer(bsa, torch, name, timer, steps):
    """A layer with a host-built static mask (Wan2.1-1.3B 480p recipe)."""
    import workloads
    dev = torch.device("cuda", 0)
    w = workloads.WORKLOADS[name]
    keep = workloads.masks(w)
    bits = workloads.pack_bits(keep)
    q, k, v = workloads.qkv(w)
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = tb(q), tb(k), tb(v)
    del q, k, v
    md = torch.from_numpy(bits.view(np.int64)).to(dev)
    fd = full_mask(torch, w.n_heads, w.n_blocks, dev)
    out = torch.empty_like(qd)
    f = lambda: bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out)
    ff = lambda: bsa.sparse_attn(qd, kd, vd, fd, w.scale, out=out)
    for _ in range(3):
        f()
    ms, med = timer.run(f, steps)
    ff()
    ms_full = timer(ff, max(3, steps // 3))
    rec = layer_record(w, int(keep.sum()), ms, med, ms_full)
    rec["workload"] = ("Wan2.1-1.3B 480p attention layer: 12 heads, head_dim 128, 21x30x52=32760 tokens, "
                       "band + temporal stripes + random fill, density U[0.10,0.50] per head")
    print(f"[bench] {name} " + json.dumps(rec), file=sys.stderr, flush=True)
    return rec


def hunyuan_layer(bsa, torch, timer, steps):
    """HunyuanVideo 768x1280 layer under PSA stripe masks expanded on the device."""
    import workloads
    dev = torch.device("cuda", 0)
    w = workloads.WORKLOADS["hunyuan_768"]
    params = torch.from_numpy(workloads.stripe_params(w)).to(dev)
    T, F = w.grid[0], w.frame_tokens
    md = bsa.mask_from_stripes(params, T, F, w.seq_len)
    build = lambda: bsa.mask_from_stripes(params, T, F, w.seq_len, out=md)
    build()
    ms_build = timer(build, 10)
    kept = int(np.unpackbits(md.cpu().numpy().view(np.uint8)).sum())
    q, k, v = workloads.qkv(w)
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    qd, kd, vd = tb(q), tb(k), tb(v)
    del q, k, v
    fd = full_mask(torch, w.n_heads, w.n_blocks, dev)
    out = torch.empty_like(qd)
    f = lambda: bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out)
    ff = lambda: bsa.sparse_attn(qd, kd, vd, fd, w.scale, out=out)
    for _ in range(3):
        f()
    ms, med = timer.run(f, steps)
    ff()
    ms_full = timer(ff, 3)
    rec = layer_record(w, kept, ms, med, ms_full)
    rec["workload"] = ("HunyuanVideo 768x1280 attention layer: 24 heads, head_dim 128, 33x48x80=126720 tokens, "
                       "PSA stripe tuples (5 heads full window)")
    rec["mask_from_stripes_ms"] = round(ms_build, 4)
    rec["mask_build_in_step"] = False
    print("[bench] hunyuan_768 " + json.dumps(rec), file=sys.stderr, flush=True)
    return rec


def topp_layer(bsa, torch, timer):
    """The dynamic top-p layer end to end on its own workload (Q and K carry the
    per-frame rank-8 component): Hilbert gather of Q, K, V, mean-pooled block
    scores, top-p 0.9 with at least 8 blocks, planner + block-sparse attention,
    scatter of O back to token order.  Per-stage and whole-chain times."""
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
    rec = {"workload": "Wan2.1-14B 720p, Q/K with a per-frame rank-8 component, Hilbert order, top-p 0.9, min 8 blocks",
           "density": round(kept / (H * nb * nb), 4), "kept_tiles": kept}
    for name, fn in stages.items():
        rec[name + "_ms"] = round(timer(fn, 5), 3)
    total = timer(lambda: [fn() for fn in stages.values()], 5)
    rec["total_ms"] = round(total, 3)
    rec["attention_share"] = round(rec["plan_and_attention_ms"] / total, 3)
    rec["layer_tflops_on_kept_tiles"] = round(kept * tile_flops(w.head_dim) / (total * 1e-3) / 1e12, 1)
    rec["frac_of_peak"] = round(rec["layer_tflops_on_kept_tiles"] / PEAK_BF16_TFLOPS, 4)
    rec["block_scores_GBps"] = round((2 * H * N * w.head_dim * 2 + H * nb * nb * 4) / (rec["block_scores_ms"] * 1e-3) / 1e9, 1)
    print("[bench] topp_wan14b " + json.dumps(rec), file=sys.stderr, flush=True)
    return rec


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


def gemm_ceiling(bsa, torch, timed):
    """Two practical MFMA ceilings on the same GPU in the same run (context for the
    roofline fraction, not part of the path): the library's register-only MFMA
    probe (the issue rate at the clock the chip holds under MFMA load) and a dense
    bf16 GEMM from the vendor library."""
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(512 * cus, dtype=torch.float32, device=dev)
    bsa.mfma_probe(sink, 2000)
    iters = 100000
    probe_flops = bsa.mfma_probe(sink, iters)
    ms = timed(lambda: bsa.mfma_probe(sink, iters), 2)
    probe = round(probe_flops / (ms * 1e-3) / 1e12, 1)
    del sink
    sizes = {}
    for n in (8192, 16384):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        fn = lambda: torch.matmul(a, b, out=c)
        fn()
        ms = timed(fn, 10 if n == 8192 else 4)
        sizes[str(n)] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    torch.cuda.empty_cache()
    return {"mfma_probe_tflops": probe,
            "mfma_probe": "bsa_mfma_probe: 16 bf16 32x32x16 MFMAs per wave and iteration on "
                          "register operands, 2 x 4-wave workgroups per CU, no memory traffic",
            "gemm_kind": "vendor bf16 GEMM n^3 (torch.matmul, vendor BLAS)",
            "gemm_tflops_by_n": sizes, "gemm_best_tflops": max(sizes.values())}


def dense_sdpa(torch, timed, qd, kd, vd, ms_sparse, ms_full):
    """Dense attention at the same shape from PyTorch's fused kernels (flash or
    memory-efficient backend; the math backend, which would materialise every
    score, is never allowed): context for the all-ones mask, not part of the path."""
    from torch.nn.attention import sdpa_kernel, SDPBackend
    H, N, d = qd.shape
    q, k, v = (x.view(1, H, N, d) for x in (qd, kd, vd))
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            fn = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v)
            fn()
            ms = timed(fn, 3)
    except (RuntimeError, NotImplementedError) as ex:
        return {"available": False, "reason": str(ex)[:160]}
    torch.cuda.empty_cache()
    return {"kind": "torch scaled_dot_product_attention, fused backend, every key kept, same shape",
            "ms": round(ms, 3), "tflops": round(4 * H * N * N * d / (ms * 1e-3) / 1e12, 1),
            "all_ones_mask_speedup": round(ms / ms_full, 3), "workload_speedup": round(ms / ms_sparse, 3)}


def cold_steps(torch, fn, stream, n, ms_warm):
    """Median single-step time after a 512 MiB write that evicts the 256 MB MALL,
    next to the median of the back-to-back (warm) steps."""
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
    del junk
    times.sort()
    return {"cold_median_ms": round(times[len(times) // 2], 3), "steps": n,
            "warm_median_ms": round(ms_warm, 3),
            "evict": "512 MiB device write before each step (the MALL holds 256 MB)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=25)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="headline layer only (no other layers, top-p layer or density sweep)")
    ap.add_argument("--profile", action="store_true",
                    help="short run for counter collection: a few planned launches plus a 1 GiB copy")
    ap.add_argument("--aux", action="store_true", help="also time the HBM-bound kernels (stderr)")
    ap.add_argument("--b128", action="store_true",
                    help="also time the layer under a 128x128-block mask in 32-bit words (stderr)")
    ap.add_argument("--cold", action="store_true",
                    help="also time single steps after evicting the last-level cache (stderr)")
    ap.add_argument("--ceiling", action="store_true",
                    help="time the vendor-library bf16 GEMM ceiling also with --quick")
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
    fd = full_mask(torch, w.n_heads, w.n_blocks, dev)
    out = torch.empty_like(qd)
    kept = int(keep.sum())
    flops = kept * tile_flops(w.head_dim)
    full_flops = w.n_heads * w.n_blocks ** 2 * tile_flops(w.head_dim)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(torch, stream)
    print("[bench] inputs ready", file=sys.stderr, flush=True)

    def step(mask):
        bsa.sparse_attn(qd, kd, vd, mask, w.scale, out=out)

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
    ms, ms_med = timer.run(lambda: step(md), args.steps)
    print(f"[bench] sparse step {ms:.3f} ms (median {ms_med:.3f})", file=sys.stderr, flush=True)

    for _ in range(max(1, args.warmup // 2)):
        step(fd)
    ms_full = timer(lambda: step(fd), max(3, args.steps // 3))
    print(f"[bench] full-mask step {ms_full:.3f} ms", file=sys.stderr, flush=True)

    _, _, order = bsa.plan(md, w.seq_len)
    planned = lambda: bsa.sparse_attn(qd, kd, vd, md, w.scale, out=out, work_order=order)
    planned()
    ms_k = timer(planned, args.steps)
    achieved = flops / (ms_k * 1e-3) / 1e12
    clock = gpu_clock_while(lambda: step(md))
    print(f"[bench] clock {clock}", file=sys.stderr, flush=True)

    rec = {
        "metric": "effective bf16 TFLOP/s on kept blocks + speedup vs full mask, Wan-14B 720p shape",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "median_ms_per_step": round(ms_med, 4),
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
        "ideal_speedup": round(w.n_heads * w.n_blocks ** 2 / kept, 3),
        "full_mask_ms": round(ms_full, 4),
        "full_mask_tflops": round(full_flops / (ms_full * 1e-3) / 1e12, 3),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic(),
            "kernel": "attn_mixed_kernel<128> (pair rows + last single-row slices) + attn_fwd_bf16_kernel<128> (other single-row slices), one planned call",
            "kernel_ms": round(ms_k, 4),
        },
        "gpu_clock": clock,
    }
    if args.aux:
        aux_kernels(bsa, torch, timer)
    if args.b128:
        b128_layer(bsa, torch, w, qd, kd, vd, out, timer, ms_full)
    if args.cold or not args.quick:
        rec["cold"] = cold_steps(torch, lambda: step(md), stream, 7, ms_med)
    if not args.quick:
        rec["dense_sdpa"] = dense_sdpa(torch, timer, qd, kd, vd, ms, ms_full)
    if args.ceiling or not args.quick:
        ceil = gemm_ceiling(bsa, torch, timer)
        for key, ref in (("probe", ceil["mfma_probe_tflops"]), ("gemm", ceil["gemm_best_tflops"])):
            ceil[f"headline_frac_of_{key}"] = round(rec["value"] / ref, 3)
            ceil[f"full_mask_frac_of_{key}"] = round(rec["full_mask_tflops"] / ref, 3)
        rec["mfma_ceiling"] = ceil
    if not args.quick:
        rec["density_sweep"] = density_sweep(bsa, torch, w, qd, kd, vd, out, timer, ms_full)
    del qd, kd, vd, out, md, fd
    torch.cuda.empty_cache()
    if not args.quick:
        rec["wan13b_480p"] = static_layer(bsa, torch, "wan13b_480p", timer, args.steps)
        torch.cuda.empty_cache()
        rec["hunyuan_768"] = hunyuan_layer(bsa, torch, timer, args.steps)
        torch.cuda.empty_cache()
        rec["topp_wan14b"] = topp_layer(bsa, torch, timer)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, bits, keep)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
