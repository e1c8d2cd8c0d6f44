"""Seeded synthetic inputs for the GDLA layer: the only module both the oracle side and the GPU
side read.  It draws random numbers and fixes shapes; it contains none of the method's arithmetic.

Recipe (one torch.Generator per workload, seeded with the workload's seed):
  draw order x, then the weights in the order of WEIGHT_NAMES, then the cache prefix;
  each draw is fp32 standard normal, multiplied by its scale, then cast once to the workload dtype
  (bf16 casts round to nearest even);
  x ~ N(0, 1); each weight ~ N(0, 1/fan_in) with fan_in its input dimension; the cache prefix
  (rows 0 .. p0-1, both the latent and the rotary part) ~ N(0, 1); RMSNorm gains are 1 unless a
  test asks for random gains (1 + 0.1 N(0, 1)).
"""

import math

import torch

WEIGHT_NAMES = ("w_qa", "w_qc", "w_qr", "w_dkv", "w_kr", "w_uk", "w_uv", "w_lambda", "w_gate", "w_o")

# Layer shapes: d_model 4096, 80 query heads, 16 KV heads, latents 1024 / 512 come from the pages
# (hotpaper.ai summary, "technical approach" list); head dim 128, rotary dim 64, the 64 + 16
# signal/noise split and the window of 4096 are choices of this library's workloads.
_BIG = dict(d_model=4096, n_heads=80, n_signal=64, n_noise=16, n_kv=16, d_q_latent=1024,
            d_kv_latent=512, d_head=128, d_rope=64)

WORKLOADS = {
    "tiny_fp32": dict(d_model=256, n_heads=8, n_signal=6, n_noise=2, n_kv=2, d_q_latent=64,
                      d_kv_latent=32, d_head=32, d_rope=16, batch=1, seq=128, p0=0,
                      max_len=128, window=0, dtype="f32", seed=1),
    "prefill_8k": dict(_BIG, batch=1, seq=8192, p0=0, max_len=8192, window=0, dtype="bf16",
                       seed=2),
    "swa_prefill_2x32k": dict(_BIG, batch=2, seq=32768, p0=0, max_len=32768, window=4096,
                              dtype="bf16", seed=3),
    "decode_64x64k": dict(_BIG, batch=64, seq=1, p0=65535, max_len=65536, window=0,
                          dtype="bf16", seed=4),
    "chunked_prefill_4k_256k": dict(_BIG, batch=1, seq=4096, p0=258048, max_len=262144,
                                    window=0, dtype="bf16", seed=5),
}

DIM_KEYS = ("d_model", "n_heads", "n_signal", "n_noise", "n_kv", "d_q_latent", "d_kv_latent",
            "d_head", "d_rope")


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def weight_shapes(cfg):
    d, dcq, dc = cfg["d_model"], cfg["d_q_latent"], cfg["d_kv_latent"]
    nh, ns, nkv, dh, dr = cfg["n_heads"], cfg["n_signal"], cfg["n_kv"], cfg["d_head"], cfg["d_rope"]
    return {
        "w_qa": (d, dcq), "w_qc": (dcq, nh * dh), "w_qr": (dcq, nh * dr), "w_dkv": (d, dc),
        "w_kr": (d, dr), "w_uk": (dc, nkv * dh), "w_uv": (dc, nkv * dh), "w_lambda": (d, ns),
        "w_gate": (dcq, ns * dh), "w_o": (ns * dh, d),
    }


def _normal(shape, gen, device, scale, dtype):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype)


def make_inputs(cfg, device="cpu", seed=None, batch=None, seq=None, p0=None, max_len=None,
                random_gamma=False, x_scale=1.0):
    """Draw one workload's inputs on `device`.

    Returns a dict: x [B, T, d_model]; weights {name: [in, out]}; gamma_q, gamma_kv (or None);
    cache [B, max_len, d_c + d_R] with rows [0, p0[b]) drawn and the rest zero; p0 (list of B).
    batch / seq / p0 / max_len override the workload's values (p0 may be an int or a list).
    """
    seed = cfg["seed"] if seed is None else seed
    bsz = cfg["batch"] if batch is None else batch
    t = cfg["seq"] if seq is None else seq
    p0 = cfg["p0"] if p0 is None else p0
    p0s = [int(p0)] * bsz if isinstance(p0, int) else [int(v) for v in p0]
    if len(p0s) != bsz:
        raise ValueError("p0 list must have one entry per sequence")
    max_len = max(max(p0s) + t, cfg["max_len"] if max_len is None else max_len)
    dt = torch_dtype(cfg["dtype"])
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = _normal((bsz, t, cfg["d_model"]), gen, device, x_scale, dt)
    weights = {}
    for name, shape in weight_shapes(cfg).items():
        weights[name] = _normal(shape, gen, device, 1.0 / math.sqrt(shape[0]), dt)
    row = cfg["d_kv_latent"] + cfg["d_rope"]
    cache = torch.zeros((bsz, max_len, row), device=device, dtype=dt)
    for b, p in enumerate(p0s):
        if p > 0:
            cache[b, :p] = _normal((p, row), gen, device, 1.0, dt)
    gamma_q = gamma_kv = None
    if random_gamma:
        gamma_q = (1.0 + 0.1 * torch.randn((cfg["d_q_latent"],), generator=gen, device=device)).to(dt)
        gamma_kv = (1.0 + 0.1 * torch.randn((cfg["d_kv_latent"],), generator=gen, device=device)).to(dt)
    return {"x": x, "weights": weights, "gamma_q": gamma_q, "gamma_kv": gamma_kv,
            "cache": cache, "p0": p0s, "max_len": max_len}


def small_cfg(dtype="f32", n_heads=8, n_signal=6, n_noise=2, n_kv=2, d_model=64, d_q_latent=32,
              d_kv_latent=16, d_head=8, d_rope=4, seed=11):
    """A workload dict with arbitrary small dims (tests only)."""
    return dict(d_model=d_model, n_heads=n_heads, n_signal=n_signal, n_noise=n_noise, n_kv=n_kv,
                d_q_latent=d_q_latent, d_kv_latent=d_kv_latent, d_head=d_head, d_rope=d_rope,
                batch=1, seq=16, p0=0, max_len=16, window=0, dtype=dtype, seed=seed)
