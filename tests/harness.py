"""Shared helpers of the GPU tests, the smoke check and the benchmark: run the GDLA library and the
fp64 oracle on the same seeded inputs and measure the difference."""

import numpy as np
import torch

import oracle.gdla_grad as grad_ref
import oracle.gdla_ref as ref
import synth
import attention_gdla_prefill_decode_amd as gd

# Tolerances on `out` (max-abs and relative L2 over the whole output).
TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 5e-3)}

# A small layer with the big head sizes (d_head 128, d_rope 64, d_kv_latent 512): 8 signal heads,
# 2 noise heads, 2 KV heads, so g = 4 as in the 80-head layer.
SMALL_BF16 = dict(d_model=256, n_heads=10, n_signal=8, n_noise=2, n_kv=2, d_q_latent=128,
                  d_kv_latent=512, d_head=128, d_rope=64, batch=1, seq=64, p0=0, max_len=64,
                  window=0, dtype="bf16", seed=7)


# The widest fast-path head layouts: five blocks of 16 heads (the fifth shared by all waves) and
# a partly filled fifth block.
BF80 = dict(SMALL_BF16, n_heads=80, n_signal=64, n_noise=16, n_kv=16)
BF72 = dict(SMALL_BF16, n_heads=72, n_signal=64, n_noise=8, n_kv=4)


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_weights(inp):
    w = {k: to_np(v) for k, v in inp["weights"].items()}
    w["gamma_q"] = None if inp["gamma_q"] is None else to_np(inp["gamma_q"])
    w["gamma_kv"] = None if inp["gamma_kv"] is None else to_np(inp["gamma_kv"])
    return w


def oracle_dims(cfg, window):
    return ref.Dims(cfg["n_heads"], cfg["n_signal"], cfg["n_noise"], cfg["n_kv"], cfg["d_head"],
                    cfg["d_rope"], window)


def errors(got, exp):
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    diff = got - exp
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(exp))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(exp * exp))) if exp.size else 0.0
    return max_abs, rel, rms


def check(got, exp, dtype, what):
    max_abs, rel, rms = errors(got, exp)
    tol_abs, tol_rel = TOL[dtype]
    msg = f"{what}: max-abs {max_abs:.3e} (tol {tol_abs:g}), rel-L2 {rel:.3e} (tol {tol_rel:g}), ref RMS {rms:.3e}"
    assert max_abs <= tol_abs and rel <= tol_rel, msg
    return msg


def device_inputs(inp, device="cuda"):
    d = {"x": inp["x"].to(device), "cache": inp["cache"].to(device),
         "weights": {k: v.to(device).contiguous() for k, v in inp["weights"].items()},
         "gamma_q": None if inp["gamma_q"] is None else inp["gamma_q"].to(device),
         "gamma_kv": None if inp["gamma_kv"] is None else inp["gamma_kv"].to(device)}
    d["wstruct"] = gd.make_weights(d["weights"], d["gamma_q"], d["gamma_kv"])
    return d


def doc_starts(p0, lens, first=None):
    """Per-token document starts of one sequence whose new tokens (from position p0) hold documents
    of the given lengths; the first document began at `first` (default p0)."""
    out, start = [], p0
    for n in lens:
        out += [start] * n
        start += n
    if first is not None:
        out[:lens[0]] = [first] * lens[0]
    return out


def prefill_case(cfg, seq, p0, window=0, seed=None, random_gamma=True, lam_zero=False,
                 want_heads=False, entry="prefill", docs=None, prep=None, rows=None):
    """Runs gdla_prefill (or, with entry="decode_tokens", the multi-token absorbed decode) on GPU
    and the oracle's one-call forward on CPU for every sequence; returns both outputs.  docs: per
    sequence, the document start of every new token (gdla_prefill_packed).  `prep(inp)` may rewrite
    the CPU inputs before both sides see them; `rows` limits the oracle to those query rows (the
    returned "out" then holds the GPU's rows of the same indices)."""
    batch = len(p0)
    inp = synth.make_inputs(cfg, "cpu", seed=seed, batch=batch, seq=seq, p0=p0,
                            random_gamma=random_gamma)
    if prep is not None:
        prep(inp)
    dev = device_inputs(inp)
    dims = gd.make_dims(cfg, window=window)
    lam = None
    if lam_zero:
        lam = torch.zeros((batch, seq, cfg["n_signal"]), dtype=torch.float32, device="cuda")
    heads = None
    if want_heads:
        heads = torch.empty((batch, seq, cfg["n_heads"], cfg["d_head"]), dtype=torch.float32,
                            device="cuda")
    if docs is not None:
        ds = torch.tensor(docs, dtype=torch.int32, device="cuda")
        out = gd.gdla_prefill_packed(dims, dev["wstruct"], dev["x"], inp["p0"], ds, dev["cache"],
                                     lambda_override=lam, out_heads=heads)
    else:
        run = gd.gdla_prefill if entry == "prefill" else gd.gdla_decode_tokens
        out = run(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"], lambda_override=lam,
                  out_heads=heads)
    torch.cuda.synchronize()
    w = oracle_weights(inp)
    od = oracle_dims(cfg, window)
    exp_out, exp_rows, exp_heads = [], [], []
    for b in range(batch):
        pre = to_np(inp["cache"][b, :inp["p0"][b]]) if inp["p0"][b] > 0 else None
        r = ref.gdla_forward(to_np(inp["x"][b]), w, od, pre, inp["p0"][b],
                             None if lam is None else np.zeros((seq, cfg["n_signal"])),
                             rows=rows, doc_start=None if docs is None else np.array(docs[b]))
        exp_out.append(r["out"])
        exp_rows.append(r["cache_rows"])
        exp_heads.append(r["heads"])
    got_rows = [to_np(dev["cache"][b, inp["p0"][b]:inp["p0"][b] + seq]) for b in range(batch)]
    got = to_np(out)
    got_heads = None if heads is None else to_np(heads)
    if rows is not None:
        got = got[:, rows]
        got_heads = None if got_heads is None else got_heads[:, rows]
    return {"out": got, "exp_out": np.stack(exp_out), "rows": got_rows, "out_all": to_np(out),
            "exp_rows": exp_rows, "heads": got_heads,
            "exp_heads": np.stack(exp_heads), "inp": inp, "dev": dev, "dims": dims}


def decode_case(cfg, p0, seed=None, random_gamma=True, want_heads=False, prep=None):
    """One decode step per sequence (token b at position p0[b]) on GPU and in the oracle.
    `prep(inp)` may rewrite the CPU inputs (e.g. the cache prefix) before both sides see them."""
    batch = len(p0)
    inp = synth.make_inputs(cfg, "cpu", seed=seed, batch=batch, seq=1, p0=p0,
                            random_gamma=random_gamma)
    if prep is not None:
        prep(inp)
    dev = device_inputs(inp)
    dims = gd.make_dims(cfg, window=cfg.get("window", 0))
    heads = None
    if want_heads:
        heads = torch.empty((batch, cfg["n_heads"], cfg["d_head"]), dtype=torch.float32,
                            device="cuda")
    out = gd.gdla_decode(dims, dev["wstruct"], dev["x"][:, 0].contiguous(), inp["p0"],
                         dev["cache"], out_heads=heads)
    torch.cuda.synchronize()
    w = oracle_weights(inp)
    od = oracle_dims(cfg, cfg.get("window", 0))
    prefixes = [to_np(inp["cache"][b, :inp["p0"][b]]) if inp["p0"][b] > 0 else None
                for b in range(batch)]
    r = ref.gdla_decode(to_np(inp["x"][:, 0]), w, od, prefixes, inp["p0"])
    return {"out": to_np(out), "exp_out": r["out"], "heads": None if heads is None else to_np(heads),
            "exp_heads": r["heads"],
            "rows": np.stack([to_np(dev["cache"][b, inp["p0"][b]]) for b in range(batch)]),
            "exp_rows": r["cache_rows"]}


def check_rows(got, exp, dtype, what):
    """Cache rows: fp32 to 1e-5; bf16 rows are rounded once (a near-tie may round the other way
    after fp32 arithmetic), so within one bf16 ulp, 2^-7 relative, plus 1e-5."""
    got = np.asarray(got, dtype=np.float64)
    exp = np.asarray(exp, dtype=np.float64)
    if dtype == "f32":
        err = float(np.max(np.abs(got - exp)))
        assert err <= 1e-5, f"{what}: cache rows max-abs {err:.3e}"
    else:
        bound = np.abs(exp) * 2.0 ** -7 + 1e-5
        bad = np.abs(got - exp) > bound
        assert not bad.any(), f"{what}: {int(bad.sum())} cache entries beyond one bf16 rounding"


def to_pages(cache, page_rows, seed=0, spare=3):
    """Copies a contiguous cache [B, L, row] into a shuffled pool of pages: returns a
    gd.PagedCache whose block table maps every block of every sequence to a distinct page (plus
    `spare` unused pages, so page indices are not dense)."""
    B, L, row = cache.shape
    blocks = (L + page_rows - 1) // page_rows
    n_pages = B * blocks + spare
    gen = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=gen)[:B * blocks].to(torch.int32)
    table = perm.reshape(B, blocks).contiguous()
    pages = torch.zeros((n_pages, page_rows, row), dtype=cache.dtype, device=cache.device)
    padded = torch.zeros((B, blocks * page_rows, row), dtype=cache.dtype, device=cache.device)
    padded[:, :L] = cache
    pages[table.reshape(-1).long().to(cache.device)] = padded.reshape(B * blocks, page_rows, row)
    return gd.PagedCache(pages, table.to(cache.device))


def from_pages(pc, B, L):
    """The contiguous [B, L, row] view of a paged cache (a copy)."""
    rows = pc.pages[pc.block_table.long()]  # [B, blocks, page_rows, row]
    return rows.reshape(B, -1, pc.pages.shape[-1])[:, :L]


def backward_case(cfg, seq, batch, window=0, docs=None, seed=None, random_gamma=True, lam_zero=False,
                  prep=None, dout_scale=1.0, map_fn=map):
    """gdla_backward on GPU and the oracle's backward on CPU (sequences at positions 0..T-1) for
    a seeded upstream gradient dout (N(0, 1) times dout_scale); weight gradients are summed over
    the batch.  `prep(inp)` may rewrite the CPU inputs before both sides see them; `map_fn` maps
    the oracle's per-head work (e.g. over worker processes)."""
    inp = synth.make_inputs(cfg, "cpu", seed=seed, batch=batch, seq=seq, p0=0, random_gamma=random_gamma)
    if prep is not None:
        prep(inp)
    gen = torch.Generator().manual_seed(1000 + (cfg["seed"] if seed is None else seed))
    dout = (torch.randn((batch, seq, cfg["d_model"]), generator=gen) * dout_scale).to(inp["x"].dtype)
    dev = device_inputs(inp)
    dims = gd.make_dims(cfg, window=window)
    tensors = dict(dev["weights"], gamma_q=dev["gamma_q"], gamma_kv=dev["gamma_kv"])
    ds = None if docs is None else torch.tensor(docs, dtype=torch.int32, device="cuda")
    lam = torch.zeros((batch, seq, cfg["n_signal"]), dtype=torch.float32, device="cuda") if lam_zero else None
    got = gd.gdla_backward(dims, dev["wstruct"], tensors, dev["x"], dout.to("cuda"), doc_start=ds,
                           lambda_override=lam)
    torch.cuda.synchronize()
    w = oracle_weights(inp)
    od = oracle_dims(cfg, window)
    exp = {}
    for b in range(batch):
        r = grad_ref.gdla_backward(to_np(inp["x"][b]), w, od, to_np(dout[b]),
                                   doc_start=None if docs is None else np.array(docs[b]),
                                   lam_override=np.zeros((seq, cfg["n_signal"])) if lam_zero else None,
                                   map_fn=map_fn)
        for k, v in r.items():
            if v is None or not (k == "dx" or k.startswith("dw_") or k.startswith("dgamma")):
                continue
            if k == "dx":
                exp.setdefault(k, []).append(v)
            else:
                exp[k] = exp.get(k, 0) + v
    exp["dx"] = np.stack(exp["dx"])
    return {k: to_np(v) for k, v in got.items()}, exp


def check_grads(got, exp, rel_l2, what):
    """Every gradient within rel_l2 of the oracle's (relative L2 over the tensor), and its max-abs
    error within 2 rel_l2 of the tensor's largest entry; returns one line per gradient."""
    lines = []
    for k in sorted(exp):
        g, e = np.asarray(got[k], dtype=np.float64), np.asarray(exp[k], dtype=np.float64)
        assert g.shape == e.shape, f"{what} {k}: shape {g.shape} vs {e.shape}"
        assert np.all(np.isfinite(g)), f"{what} {k}: non-finite gradient entries"
        den = float(np.linalg.norm(e))
        rel = float(np.linalg.norm(g - e)) / (den if den > 0 else 1.0)
        mx = float(np.max(np.abs(g - e)))
        big = float(np.max(np.abs(e))) if e.size else 0.0
        lines.append(f"{k}: rel-L2 {rel:.2e}, max-abs {mx:.2e} (max |ref| {big:.2e}, "
                     f"ratio {mx / max(big, 1e-300):.2e})")
        assert rel <= rel_l2 and mx <= 2 * rel_l2 * max(big, 1e-30), f"{what} {k}: " + lines[-1]
    return lines
