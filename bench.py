"""Benchmark of the GDLA forward on one MI355X: one step = one gdla_prefill_prepared call over the
8192-token single-layer workload (batch 1, d_model 4096, 64 signal + 16 noise heads, 16 KV heads,
latents 1024 / 512, head dim 128, rotary dim 64, full causal; the layer's weights transposed once
beforehand by gdla_prepare_weights), inputs seeded and resident in HBM.

Prints one JSON line: whole-step throughput (algorithmic FLOP of the layer / step time), the
roofline of the dominant kernel (signal-head attention, timed with HIP events recorded by the
library around it in the timed steps, which record no other events; `stages_ms` comes from further
untimed steps that record every stage), and the fp64 CPU oracle timed on a bounded sample of the
same workload.
The line also carries the other half of the metric, `decode`: one decode step of 64 sequences at
65536 positions (latent-cache GB/s, the roofline of the split-L attention kernel against HBM and
its own CPU-oracle baseline), and `ceilings`: the bf16 matrix-core rate with random operands (on
the prefill attention's MFMA instruction) and the HBM read rate measured on this GPU, against which
both fractions are also given.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-ceilings]
                    [--no-cpu-baseline] [--transpose-per-call]
                    [--workload prefill_8k|swa_prefill_2x32k|chunked_prefill_4k_256k|decode_64x64k]
                    [--tokens T] [--page-rows R] [--window W] [--docs MEAN] [--backward]
                    [--decode-only] [--copy-probe]

--workload picks another workload for the timed line (2 x 32K prefill with a 4096 window; a
4096-token chunk against a 256K cache; one decode step of 64 sequences at 64K context, reported
in GB/s of latent cache).  With the decode workload (or --decode-only, which prints only the
decode object): --tokens T > 1 times the multi-token decode (T draft tokens per sequence, ending
at position 65535), --page-rows R a paged cache of shuffled R-row pages, --window W a layer with
a W-position sliding window.  --docs MEAN packs the prefill tokens into seeded documents of that
mean length; --backward times gdla_backward on the workload's shape; --transpose-per-call times
gdla_prefill (weights transposed inside every call); --copy-probe only copies 1 GiB three times
(the known-size reference of the traffic counters).  bench.py measures one GPU: --gpus N > 1 exits
with a message.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "GDLA prefill TFLOP/s (% bf16 MFMA peak); decode latent-KV GB/s (% HBM peak)"


def visible_pairs(p0, t, window, docs=None):
    """Number of (query, key) pairs with key <= query position and, for window W, within W (and,
    with packed documents, inside the query's document: docs[i] = first position of its document)."""
    total = 0
    for i in range(t):
        p = p0 + i
        lo = max(0, p - window + 1) if window > 0 else 0
        if docs is not None:
            lo = max(lo, docs[i])
        total += p + 1 - lo
    return total


def packed_documents(t, mean, seed=0):
    """Document starts of t packed tokens, document lengths drawn from a seeded exponential
    distribution of the given mean (at least one token each)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    starts, pos = [], 0
    while pos < t:
        n = max(1, int(round(rng.exponential(mean))))
        starts += [pos] * min(n, t - pos)
        pos += n
    return starts


def layer_flops(cfg, t, p0, window, docs=None):
    """Algorithmic FLOP of one GDLA layer call on one sequence (attention counts visible pairs)."""
    d, dcq, dc, nh, ns = cfg["d_model"], cfg["d_q_latent"], cfg["d_kv_latent"], cfg["n_heads"], cfg["n_signal"]
    nkv, dh, dr = cfg["n_kv"], cfg["d_head"], cfg["d_rope"]
    pairs = visible_pairs(p0, t, window, docs)
    attn_signal = 2.0 * ns * pairs * (2 * dh + dr)
    attn_noise = 2.0 * (nh - ns) * pairs * (2 * dh + dr)
    keys = p0 + t - (max(0, p0 - window + 1) if window > 0 else 0)
    proj = 2.0 * t * (d * (dcq + dc + dr + ns) + dcq * (nh * dh + nh * dr + ns * dh) + ns * dh * d)
    expand = 2.0 * keys * dc * (2 * nkv * dh)
    return {"attn_signal": attn_signal, "attn_noise": attn_noise, "proj": proj, "expand": expand,
            "total": attn_signal + attn_noise + proj + expand, "pairs": pairs}


def backward_flops(cfg, t, window, docs=None):
    """Algorithmic FLOP of one backward call on one sequence at positions 0..t-1: the forward it
    recomputes plus the gradients (per visible pair and head: the score, dP = dH V^T, dq, dK and
    dV products; every projection and the expansion twice, for the data and the weight gradient)."""
    f = layer_flops(cfg, t, 0, window, docs)
    dqk, dh = cfg["d_head"] + cfg["d_rope"], cfg["d_head"]
    attn = 2.0 * cfg["n_heads"] * f["pairs"] * (3 * dqk + 2 * dh)
    return {"forward": f["total"], "attention": attn, "proj": 2.0 * (f["proj"] + f["expand"]),
            "total": f["total"] + attn + 2.0 * (f["proj"] + f["expand"])}


def bench_backward(args):
    """Times gdla_backward on the workload's shape (training sequences from position 0)."""
    import torch
    import synth
    import attention_gdla_prefill_decode_amd as gd
    cfg = synth.WORKLOADS[args.workload]
    bsz, t, win = cfg["batch"], cfg["seq"], cfg["window"]
    inp = synth.make_inputs(cfg, "cuda", p0=0)
    dims = gd.make_dims(cfg)
    w = gd.make_weights(inp["weights"])
    tensors = dict(inp["weights"], gamma_q=None, gamma_kv=None)
    gen = torch.Generator(device="cuda").manual_seed(5)
    dout = torch.randn(inp["x"].shape, generator=gen, device="cuda").to(inp["x"].dtype)
    docs = None
    doc_t = None
    if args.docs > 0:
        docs = packed_documents(t, args.docs)
        doc_t = torch.tensor([docs] * bsz, dtype=torch.int32, device="cuda")
    ws = torch.empty(gd.gdla_workspace_bytes(dims, gd.GDLA_OP_BACKWARD, bsz, t, None, t), dtype=torch.uint8,
                     device="cuda")
    for _ in range(args.warmup):
        g = gd.gdla_backward(dims, w, tensors, inp["x"], dout, doc_start=doc_t, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g = gd.gdla_backward(dims, w, tensors, inp["x"], dout, doc_start=doc_t, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    fl = {k: v * bsz for k, v in backward_flops(cfg, t, win, docs).items()}
    return {"workload": args.workload + "_backward", "batch": bsz, "seq_len": t, "window": win,
            "ms_per_call": round(ms, 3), "TFLOPs": round(fl["total"] / (ms * 1e-3) / 1e12, 2),
            "flop_per_call": fl, "grads_finite": bool(all(torch.isfinite(v).all().item() for v in g.values()))}


def source_sha(rel):
    h = hashlib.sha256()
    with open(os.path.join(ROOT, rel), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name):
    """HBM bytes per launch of a dominant kernel from its committed counter summary
    (profiles/<name>), if the counters were taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != source_sha(t["kernel_source"]):
        return None
    return t.get("bytes_per_launch")


def traffic_source(name):
    """Where `traffic` comes from: the committed counter summary, taken on this kernel source."""
    return (f"profiles/{name}: rocprofv3 FETCH_SIZE / WRITE_SIZE of the kernel, scaled by a 1 GiB "
            f"copy's counts, taken on the committed kernel source (its SHA-256 matches the current "
            f"file); not measured in this run")


def ceilings(reps=3):
    """Measured ceilings of this GPU (libgdla_ceiling.so): v_mfma_f32_16x16x32_bf16 (the prefill
    attention's instruction) back to back on pseudo-random operands (8 chains per wave, 8 waves
    per workgroup); a streaming read of 4 GiB
    through LDS rings of direct global-to-LDS loads, one workgroup per CU.
    Returns the best of `reps` runs of each, timed with HIP events on the current stream."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "attention_gdla_prefill_decode_amd", "libgdla_ceiling.so")
    L = ctypes.CDLL(path)
    L.ceiling_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = 1024, 4000
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    flop = float(blocks) * 8 * iters * 8 * 16384

    def timed(fn):
        best = None
        for _ in range(reps + 1):  # the first run warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if fn() != 0:
                raise RuntimeError("ceiling probe launch failed")
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    ms_mfma = timed(lambda: L.ceiling_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, stream))
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    rblocks = 256  # one workgroup per CU
    ms_read = timed(lambda: L.ceiling_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                           rblocks, stream))
    del buf
    return {"mfma_bf16_random_TFLOPs": round(flop / ms_mfma / 1e9, 1),
            "hbm_read_GBps": round(nbytes / ms_read / 1e6, 1),
            "how": "libgdla_ceiling.so: ceiling_mfma (1024 x 512 threads, 8 x 4000 v_mfma_f32_16x16x32_bf16 "
                   "per wave on random bf16 operands) and ceiling_read (4 GiB: 256 workgroups, one per CU, each "
                   "streaming 16 MiB through a 4-slot LDS ring of 32 KiB with direct global-to-LDS 16-byte "
                   "loads, three slots in flight); best of 3 after a warm-up"}


def cpu_baseline_decode(nseq=8):
    """The fp64 oracle (absorbed form, as it stands) on nseq sequences drawn with the recipe of the
    64 x 64K decode workload: each a 65535-row N(0, 1) latent prefix and one new token at position
    65535.  Returns latent-cache GB/s of the oracle (the bytes of the GPU metric: each cached row of
    576 bf16 values read once per sequence)."""
    import numpy as np
    import synth
    import oracle.gdla_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    cfg = synth.WORKLOADS["decode_64x64k"]
    inp = synth.make_inputs(cfg, "cpu", batch=nseq)
    w = {k: v.double().numpy() for k, v in inp["weights"].items()}
    dims = ref.Dims(cfg["n_heads"], cfg["n_signal"], cfg["n_noise"], cfg["n_kv"], cfg["d_head"],
                    cfg["d_rope"], 0)
    p0 = cfg["p0"]
    dt = 0.0
    for b in range(nseq):
        prefix = inp["cache"][b, :p0].double().numpy()
        x = inp["x"][b, :1].double().numpy()
        t0 = time.perf_counter()
        ref.gdla_decode(x, w, dims, [prefix], [p0])
        dt += time.perf_counter() - t0
        del prefix
    row = cfg["d_kv_latent"] + cfg["d_rope"]
    nbytes = nseq * (p0 + 1) * row * 2
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"fp64 NumPy oracle, absorbed form, {nseq} sequences of the 64 x 64K decode step "
                      f"(same recipe, seed of the workload, drawn as a batch of {nseq}): 65535-row "
                      f"prefix + 1 new token each, {nbytes / 1e9:.3f} GB of latent cache"}


def cpu_baseline(rows=2048):
    """The fp64 oracle on the last `rows` query rows of the 8K workload with their full causal
    context, drawn with the same recipe on the CPU; returns its throughput in TFLOP/s."""
    import numpy as np
    import synth
    import oracle.gdla_ref as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    cfg = synth.WORKLOADS["prefill_8k"]
    t = cfg["seq"]
    inp = synth.make_inputs(cfg, "cpu")
    w = {k: v.double().numpy() for k, v in inp["weights"].items()}
    x = inp["x"][0].double().numpy()
    dims = ref.Dims(cfg["n_heads"], cfg["n_signal"], cfg["n_noise"], cfg["n_kv"], cfg["d_head"],
                    cfg["d_rope"], 0)
    sel = np.arange(t - rows, t)
    t0 = time.perf_counter()
    ref.gdla_forward(x, w, dims, None, 0, rows=sel)
    dt = time.perf_counter() - t0
    d, dcq, dc, nh, ns = cfg["d_model"], cfg["d_q_latent"], cfg["d_kv_latent"], cfg["n_heads"], cfg["n_signal"]
    dh, dr, nkv = cfg["d_head"], cfg["d_rope"], cfg["n_kv"]
    pairs = sum(p + 1 for p in range(t - rows, t))
    flops = (2.0 * nh * pairs * (2 * dh + dr)                       # attention of the rows
             + 2.0 * rows * (d * (dcq + ns) + dcq * (nh * dh + nh * dr + ns * dh) + ns * dh * d)
             + 2.0 * t * d * (dc + dr)                              # latents of every key
             + 2.0 * t * dc * (2 * nkv * dh))                       # K/V expansion of every key
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"fp64 NumPy oracle, last {rows} of 8192 query rows of the same layer with "
                      f"their full causal context (latents and K/V of all 8192 keys), "
                      f"{flops / 1e12:.3f} TFLOP of algorithmic work"}


def paged_copy(cache, page_rows, seed=0):
    """The cache [B, L, row] in a pool of B L / page_rows pages in shuffled order (the block table
    of a serving system after many allocations)."""
    import torch
    import attention_gdla_prefill_decode_amd as gd
    B, L, row = cache.shape
    blocks = L // page_rows
    gen = torch.Generator().manual_seed(seed)
    table = torch.randperm(B * blocks, generator=gen).to(torch.int32).reshape(B, blocks).to(cache.device)
    pages = torch.empty((B * blocks, page_rows, row), dtype=cache.dtype, device=cache.device)
    pages[table.reshape(-1).long()] = cache.reshape(B * blocks, page_rows, row)
    return gd.PagedCache(pages, table.contiguous())


def stage_breakdown(run, args, kwargs, steps):
    """Per-stage milliseconds (mean of `steps` calls, every stage's events recorded), from steps
    outside the timed region."""
    import attention_gdla_prefill_decode_amd as gd
    timers = [gd.StageTimer() for _ in range(steps)]
    for i in range(steps):
        run(*args, **kwargs, timer=timers[i])
    tot = {k: 0.0 for k in gd.STAGES}
    for tm in timers:
        for k, v in tm.elapsed().items():
            tot[k] += v
    return {k: round(v / steps, 4) for k, v in tot.items()}


# What a decode step runs in each stage slot of the library (the prefill names of gdla.STAGES);
# a decode step expands no K/V.
DECODE_STAGE_NAMES = {"proj_in": "proj_in", "norm_append": "norm_append", "expand_kv": None,
                      "proj_q": "proj_q_and_absorb", "attn_noise": "latent_attention",
                      "attn_signal": "merge_unabsorb_combine", "proj_out": "proj_out"}


def bench_decode(steps, warmup, tokens=1, page_rows=0, window=0):
    """64 sequences with a 65536-position context.  tokens = 1: one decode step (gdla_decode, the
    new token at position 65535); tokens = T > 1: T draft tokens per sequence at positions
    65536 - T .. 65535 in one gdla_decode_tokens call.  page_rows > 0: the same over a paged
    cache (gdla_decode_paged, shuffled pages of page_rows rows).  window > 0: sliding-window
    attention over the last `window` positions (the same cache, a layer with that window)."""
    import torch
    import synth
    import attention_gdla_prefill_decode_amd as gd
    cfg = synth.WORKLOADS["decode_64x64k"]
    if window > 0:
        cfg = dict(cfg, window=window)
    inp = synth.make_inputs(cfg, "cuda", seq=tokens, p0=cfg["max_len"] - tokens)
    w = gd.make_weights(inp["weights"])
    dims = gd.make_dims(cfg)
    pos = inp["p0"]
    cache = inp["cache"]
    if page_rows > 0:
        x = inp["x"]
        cache = paged_copy(inp["cache"], page_rows)
        del inp["cache"]
        run = gd.gdla_decode_paged
    elif tokens == 1:
        x = inp["x"][:, 0].contiguous()
        run = gd.gdla_decode
    else:
        x = inp["x"]
        run = gd.gdla_decode_tokens
    ws = torch.empty(gd.gdla_workspace_bytes(dims, gd.GDLA_OP_DECODE, len(pos), tokens, pos, cfg["max_len"]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    for _ in range(warmup):
        run(dims, w, x, pos, cache, out=out, ws=ws)
    torch.cuda.synchronize()
    # the timed steps record events around the split-L kernel only
    timers = [gd.StageTimer(("attn_noise",)) for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(dims, w, x, pos, cache, out=out, ws=ws, timer=timers[i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kern_ms = sum(tm.elapsed()["attn_noise"] for tm in timers) / steps
    stages = stage_breakdown(run, (dims, w, x, pos, cache), dict(out=out, ws=ws), steps)
    # Algorithmic bytes of the latent-attention kernel: every cache row visible to the last token
    # once per sequence, the absorbed query of every head and token (bf16) and the attended
    # latent o of every head and token (fp32).
    last = [p + tokens - 1 for p in pos]
    keys = sum(min(p + 1, cfg["window"]) if cfg["window"] > 0 else p + 1 for p in last)
    row = cfg["d_kv_latent"] + cfg["d_rope"]
    nbytes = keys * row * 2 + len(pos) * tokens * cfg["n_heads"] * (row * 2 + cfg["d_kv_latent"] * 4)
    gbs = nbytes / kern_ms / 1e6
    # Algorithmic FLOP: per head, token and visible key a 576-long score dot product and a
    # 512-long weighted sum.  Above the ridge (312.5 FLOP/B) the kernel is MFMA-bound: from two
    # tokens per sequence on, since every token multiplies the work on each cache row.
    vis = sum(min(p + i + 1, cfg["window"]) if cfg["window"] > 0 else p + i + 1
              for p in pos for i in range(tokens))
    flop = 2.0 * cfg["n_heads"] * vis * (row + cfg["d_kv_latent"])
    if flop / nbytes > PEAK_MFMA_TFLOPS * 1e3 / PEAK_HBM_GBS:
        tfs = flop / kern_ms / 1e9
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfs / PEAK_MFMA_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    name = "decode_64x64k" if tokens == 1 else f"decode_tokens_64x64k_t{tokens}"
    if page_rows > 0:
        name += f"_paged{page_rows}"
    if window > 0:
        name += f"_window{window}"
    return {"workload": name, "batch": len(pos), "tokens": tokens, "context": int(last[0]) + 1,
            "ms_per_step": round(ms, 4),
            "latent_GBps_whole_step": round(nbytes / ms / 1e6, 1),
            "tokens_per_s": round(len(pos) * tokens / ms * 1e3, 1),
            "roofline": dict({"kernel": "latent_decode_kernel<shared>"}, **roof,
                             traffic=(traffic_from_profile("latent_decode_64x64k_traffic.json")
                                      if tokens == 1 and page_rows == 0 and window == 0 else None),
                             traffic_source=traffic_source("latent_decode_64x64k_traffic.json"),
                             bytes_per_launch=nbytes, flop_per_launch=flop,
                             avg_launch_ms=round(kern_ms, 4)),
            # the library's stage slots under what a decode step runs in each
            "stages_ms": {DECODE_STAGE_NAMES[k]: round(v, 4) for k, v in stages.items()
                          if DECODE_STAGE_NAMES.get(k)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true",
                    help="leave the 64 x 64K decode step out of the prefill line")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured MFMA / HBM ceilings")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the 64 x 64K decode workload (prints its JSON object)")
    ap.add_argument("--workload", default="prefill_8k",
                    choices=["prefill_8k", "swa_prefill_2x32k", "chunked_prefill_4k_256k", "decode_64x64k"],
                    help="workload of the timed line (default: the 8K prefill)")
    ap.add_argument("--tokens", type=int, default=1,
                    help="with --workload decode_64x64k or --decode-only: draft tokens per sequence "
                         "(T > 1 times gdla_decode_tokens, the multi-token verification step)")
    ap.add_argument("--page-rows", type=int, default=0,
                    help="with the decode workload: run over a paged cache of this page size "
                         "(gdla_decode_paged)")
    ap.add_argument("--window", type=int, default=0,
                    help="with the decode workload: a layer with this sliding window (decode over "
                         "the last W positions of the 64K cache)")
    ap.add_argument("--docs", type=float, default=0,
                    help="prefill workloads: pack the tokens into documents of this mean length "
                         "(seeded exponential lengths; gdla_prefill_packed)")
    ap.add_argument("--backward", action="store_true",
                    help="time gdla_backward (training sequences from position 0) on the workload's "
                         "shape instead of the forward; prints its JSON object")
    ap.add_argument("--transpose-per-call", action="store_true",
                    help="time gdla_prefill (weights transposed inside every call) instead of "
                         "gdla_prefill_prepared (transposed once beforehand)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 1 GiB device to device three times (a known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import attention_gdla_prefill_decode_amd as gd

    if args.copy_probe:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_launch": n, "launches": 3}), flush=True)
        return

    if args.backward:
        print(json.dumps(bench_backward(args)), flush=True)
        return

    if args.decode_only:
        print(json.dumps(bench_decode(args.steps, args.warmup, args.tokens, args.page_rows, args.window)), flush=True)
        return

    if args.workload == "decode_64x64k":
        d = bench_decode(args.steps, args.warmup, args.tokens, args.page_rows, args.window)
        result = {
            "metric": METRIC, "value": round(d["latent_GBps_whole_step"], 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": d["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16 (fp32 accumulate)", "data": "synthetic",
            "config": {"workload": d["workload"], "batch": 64, "tokens_per_sequence": args.tokens,
                       "context": 65536, "window": args.window, "parallelism": "none (1 GPU)"},
            "roofline": d["roofline"], "stages_ms": d["stages_ms"], "tokens_per_s": d["tokens_per_s"],
        }
        print(json.dumps(result), flush=True)
        return

    cfg = synth.WORKLOADS[args.workload]
    bsz, t, p0, win = cfg["batch"], cfg["seq"], cfg["p0"], cfg["window"]
    inp = synth.make_inputs(cfg, "cuda")
    w = gd.make_weights(inp["weights"])
    dims = gd.make_dims(cfg)
    x, cache = inp["x"], inp["cache"]
    pos = inp["p0"]
    ws = torch.empty(gd.gdla_workspace_bytes(dims, gd.GDLA_OP_PREFILL, bsz, t, pos, cfg["max_len"]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    docs = None
    if args.transpose_per_call:
        run = gd.gdla_prefill
    else:  # the layer's weights transposed once, as a deployment keeps them resident
        prepared = gd.gdla_prepare_weights(dims, w)

        def run(*a, **k):
            return gd.gdla_prefill_prepared(a[0], a[1], prepared, *a[2:], **k)
    if args.docs > 0:  # documents packed from the chunk's first token
        docs = [p0 + v for v in packed_documents(t, args.docs)]
        doc_t = torch.tensor([docs] * bsz, dtype=torch.int32, device="cuda")

        def run(*a, **k):
            return gd.gdla_prefill_packed(a[0], a[1], a[2], a[3], doc_t, a[4], **k)
    for _ in range(args.warmup):
        run(dims, w, x, pos, cache, out=out, ws=ws)
    torch.cuda.synchronize()
    # The timed steps record events around the two attention kernels only (each record is a packet
    # on the stream); they are read after the timed region (no host sync inside).
    timers = [gd.StageTimer(("attn_noise", "attn_signal")) for _ in range(args.steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        run(dims, w, x, pos, cache, out=out, ws=ws, timer=timers[i])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    timed = {k: sum(tm.elapsed()[k] for tm in timers) / args.steps for k in ("attn_noise", "attn_signal")}
    # every stage's time, from further untimed steps with all stage events
    stages = stage_breakdown(run, (dims, w, x, pos, cache), dict(out=out, ws=ws), args.steps)
    fl = {k: v * bsz for k, v in layer_flops(cfg, t, p0, win, docs).items()}
    value = fl["total"] / (ms * 1e-3) / 1e12
    attn_ms = round(timed["attn_signal"], 4)
    achieved = fl["attn_signal"] / (attn_ms * 1e-3) / 1e12
    noise_ms = round(timed["attn_noise"], 4)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16+fp16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": args.workload, "batch": bsz, "seq_len": t, "cached_before": p0,
                   "d_model": cfg["d_model"], "heads": "64 signal + 16 noise, 16 KV",
                   "latents": "1024 / 512", "head_dim": cfg["d_head"], "rope_dim": cfg["d_rope"],
                   "window": win, "parallelism": "none (1 GPU)",
                   "weights": ("transposed inside every call" if args.transpose_per_call or docs
                               else "transposed once beforehand (gdla_prepare_weights)"),
                   **({"documents": len(set(docs)), "mean_document": args.docs} if docs else {})},
        "frac_of_mfma_peak_whole_step": round(value / PEAK_MFMA_TFLOPS, 4),
        "roofline": {"kernel": "attn_prefill_kernel<signal>", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": (traffic_from_profile("attn_signal_prefill_8k_traffic.json")
                                 if args.workload == "prefill_8k" and not docs else None),
                     "traffic_source": traffic_source("attn_signal_prefill_8k_traffic.json"),
                     "flop_per_launch": fl["attn_signal"], "avg_launch_ms": attn_ms},
        "attention_core": {"kernels": "noise + signal attention", "ms": round(attn_ms + noise_ms, 4),
                           "TFLOPs": round((fl["attn_signal"] + fl["attn_noise"])
                                           / ((attn_ms + noise_ms) * 1e-3) / 1e12, 2)},
        "stages_ms": stages,
        "out_finite": bool(torch.isfinite(out).all().item()),
    }
    del inp, x, cache, ws, out
    if not args.transpose_per_call:
        del prepared
    torch.cuda.empty_cache()
    if not args.no_decode and args.workload == "prefill_8k" and not docs:
        result["decode"] = bench_decode(max(5, args.steps), 3)
    if not args.no_ceilings:
        c = ceilings()
        result["ceilings"] = c
        roof = result["roofline"]
        roof["measured_ceiling"] = c["mfma_bf16_random_TFLOPs"]
        roof["frac_of_measured_ceiling"] = round(roof["achieved"] / c["mfma_bf16_random_TFLOPs"], 4)
        if "decode" in result:
            droof = result["decode"]["roofline"]
            if droof["bound"] == "hbm":
                droof["measured_ceiling"] = c["hbm_read_GBps"]
                droof["frac_of_measured_ceiling"] = round(droof["achieved"] / c["hbm_read_GBps"], 4)
    if not args.no_cpu_baseline and args.workload == "prefill_8k" and not docs:
        result["cpu_baseline"] = cpu_baseline()
        if "decode" in result:
            result["decode"]["cpu_baseline"] = cpu_baseline_decode()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
