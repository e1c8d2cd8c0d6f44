"""Host-side checks of bench.py's command line (no GPU): the single-GPU contract and the
algorithmic FLOP and byte counts the roofline figures divide by."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_attention_flop_of_the_8k_prefill():
    # causal pairs of 8192 tokens, 64 signal heads, 2 (2 d_h + d_r) per pair and head
    cfg = synth.WORKLOADS["prefill_8k"]
    f = bench.layer_flops(cfg, 8192, 0, 0)
    pairs = 8192 * 8193 // 2
    assert f["pairs"] == pairs
    assert f["attn_signal"] == 2.0 * 64 * pairs * (2 * 128 + 64)


def test_backward_flop_counts_five_products_per_pair():
    cfg = synth.WORKLOADS["prefill_8k"]
    f = bench.layer_flops(cfg, 8192, 0, 0)
    bw = bench.backward_flops(cfg, 8192, 0)
    assert bw["attention"] == 2.0 * 80 * f["pairs"] * (3 * 192 + 2 * 128)
    assert bw["total"] == f["total"] + bw["attention"] + bw["proj"]


def test_ceiling_library_exports_its_probes():
    # the measured-ceiling probes live in a library of their own next to libgdla.so (no launch here)
    import ctypes
    path = os.path.join(ROOT, "attention_gdla_prefill_decode_amd", "libgdla_ceiling.so")
    assert os.path.exists(path), "build the libraries first (__graft_entry__.build())"
    lib = ctypes.CDLL(path)
    for name in ("ceiling_mfma", "ceiling_read"):
        assert hasattr(lib, name), name


def test_decode_cpu_baseline_counts_the_latent_cache_bytes():
    # the decode baseline's bytes: every cached row (576 bf16 values) of each sampled sequence once
    cfg = synth.WORKLOADS["decode_64x64k"]
    row = cfg["d_kv_latent"] + cfg["d_rope"]
    assert row * 2 == 1152
    assert (cfg["p0"] + 1) * row * 2 == 65536 * 1152
