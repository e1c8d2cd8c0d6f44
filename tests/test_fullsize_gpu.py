"""GPU parity at the full workload sizes (8K prefill, 2 x 32K windowed prefill, 64 x 64K decode,
4K chunk against a 256K cache), in the launch configuration the benchmark times.  The library
computes every row; the fp64 oracle evaluates a row sample one by one (absorbed form, which the
CPU pins equate with the expanded form).  The sample always holds the first and last rows, rows
on both sides of the 64- and 256-row query tiles, the window edge rows W-2 .. W+1 and seeded
random rows."""

import numpy as np
import pytest
import torch

import synth
import oracle.gdla_ref as ref
import attention_gdla_prefill_decode_amd as gd
from tests import harness as H

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _rows(t, extra, seed, n_random=4):
    rng = np.random.default_rng(seed)
    base = {0, 1, 63, 64, 255, 256, t - 2, t - 1} | set(extra)
    base |= set(int(v) for v in rng.integers(0, t, n_random))
    return sorted(r for r in base if 0 <= r < t)


def _prefill_rows(name, window_rows=()):
    cfg = synth.WORKLOADS[name]
    inp = synth.make_inputs(cfg, "cuda")
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    cache0 = inp["cache"].clone()  # the prefix as the oracle must see it (before the append)
    _say(f"{name}: GPU prefill B={cfg['batch']} T={cfg['seq']} P0={cfg['p0']} W={cfg['window']}")
    out = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    w = H.oracle_weights(inp)
    od = H.oracle_dims(cfg, cfg["window"])
    got, exp = [], []
    for b in range(cfg["batch"]):
        rows = _rows(cfg["seq"], window_rows, seed=100 + b)
        p0 = inp["p0"][b]
        prefix = H.to_np(cache0[b, :p0]) if p0 > 0 else None
        _say(f"  oracle sequence {b}: rows {rows}")
        r = ref.gdla_forward(H.to_np(inp["x"][b]), w, od, prefix, p0, form="absorbed", rows=rows)
        got.append(H.to_np(out[b, rows]))
        exp.append(r["out"])
        H.check_rows(H.to_np(dev["cache"][b, p0:p0 + cfg["seq"]])[rows], r["cache_rows"][rows],
                     "bf16", f"{name} cache rows")
    _say(H.check(np.concatenate(got), np.concatenate(exp), "bf16", f"{name} sampled rows"))


@pytest.mark.timeout(600)
def test_prefill_8k_sampled_rows():
    _prefill_rows("prefill_8k", window_rows=(4095, 4096, 8127, 8128))


@pytest.mark.timeout(600)
def test_swa_prefill_2x32k_sampled_rows():
    w = synth.WORKLOADS["swa_prefill_2x32k"]["window"]
    _prefill_rows("swa_prefill_2x32k", window_rows=(w - 2, w - 1, w, w + 1, 2 * w, 16383, 16384))


@pytest.mark.timeout(600)
def test_chunked_prefill_4k_256k_sampled_rows():
    _prefill_rows("chunked_prefill_4k_256k", window_rows=(2047, 2048, 4031, 4032))


@pytest.mark.timeout(600)
def test_decode_64x64k_sampled_sequences():
    cfg = synth.WORKLOADS["decode_64x64k"]
    inp = synth.make_inputs(cfg, "cuda")
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    _say(f"decode_64x64k: GPU decode B={cfg['batch']} at position {cfg['p0']}")
    seqs = [0, 1, 31, 62, 63]
    prefixes = [H.to_np(inp["cache"][b, :inp["p0"][b]]) for b in seqs]
    out = gd.gdla_decode(dims, dev["wstruct"], dev["x"][:, 0].contiguous(), inp["p0"], dev["cache"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    w = H.oracle_weights(inp)
    od = H.oracle_dims(cfg, 0)
    _say(f"  oracle sequences {seqs}")
    r = ref.gdla_decode(H.to_np(inp["x"][seqs, 0]), w, od, prefixes, [inp["p0"][b] for b in seqs])
    _say(H.check(H.to_np(out[seqs]), r["out"], "bf16", "decode_64x64k sampled sequences"))
    H.check_rows(np.stack([H.to_np(dev["cache"][b, inp["p0"][b]]) for b in seqs]), r["cache_rows"],
                 "bf16", "decode_64x64k appended rows")


@pytest.mark.timeout(900)
def test_backward_8k_full():
    """The benchmark's backward configuration (one 8192-token training sequence of the 8K prefill
    layer, full causal, the fused fp16 path) against the oracle's backward over every gradient.
    The oracle forms one head's 8192 x 8192 probability matrix at a time; its 80 heads run on
    spawned worker processes (which never touch the GPU), two BLAS threads each."""
    import multiprocessing as mp
    import os
    cfg = synth.WORKLOADS["prefill_8k"]
    workers = max(1, min(8, (os.cpu_count() or 2) // 2))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        for k in saved:
            os.environ[k] = "2"
        with mp.get_context("spawn").Pool(workers) as pool:
            _say(f"8K backward: GPU call, then the oracle's 80 heads on {workers} workers")
            got, exp = H.backward_case(cfg, cfg["seq"], 1, map_fn=pool.imap)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    for line in H.check_grads(got, exp, 1e-2, "8K fused backward"):
        _say(line)

