"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin takes the oracle module (`ref`, normally oracle.gdla_ref) and raises AssertionError when
the oracle disagrees with: the pages' worked example, a library routine (torch's fp64 RMSNorm and
scaled-dot-product attention), a 50-digit brute force, an independently written gated-MLA program,
or a closed form / invariant of the mathematics.  Readings that a pin needs (which head is signal,
which KV head a query head reads, the RoPE convention) are restated here, not imported, so a
mistake planted in the oracle's own helpers is still caught (tests/test_oracle_mutations.py).
"""

import json
import math
import os

import numpy as np
import torch

from oracle.mla_ref import mla_forward
import synth
from tests.brute_gdla import brute_gdla

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_problem(n_heads=6, n_signal=4, n_noise=2, n_kv=2, d_model=16, d_q_latent=8,
                  d_kv_latent=8, d_head=4, d_rope=4, seq=7, p0=0, seed=5, random_gamma=True):
    cfg = synth.small_cfg("f32", n_heads, n_signal, n_noise, n_kv, d_model, d_q_latent,
                          d_kv_latent, d_head, d_rope, seed)
    inp = synth.make_inputs(cfg, "cpu", seq=seq, p0=p0, batch=1, random_gamma=random_gamma)
    w = {k: v.double().numpy() for k, v in inp["weights"].items()}
    w["gamma_q"] = None if inp["gamma_q"] is None else inp["gamma_q"].double().numpy()
    w["gamma_kv"] = None if inp["gamma_kv"] is None else inp["gamma_kv"].double().numpy()
    x = inp["x"][0].double().numpy()
    prefix = inp["cache"][0, :p0].double().numpy() if p0 > 0 else None
    return cfg, w, x, prefix


def make_dims(ref, cfg, window=0):
    return ref.Dims(cfg["n_heads"], cfg["n_signal"], cfg["n_noise"], cfg["n_kv"], cfg["d_head"],
                    cfg["d_rope"], window)


def _kv_reading(h, n_signal, n_kv):
    return h % n_kv if h < n_signal else (h - n_signal) % n_kv


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {a.shape} vs {b.shape}")
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    if not err <= tol * scale:
        raise AssertionError(f"{what}: max abs err {err:.3e} > {tol:.1e} (scale {scale:.3g})")


# --------------------------------------------------------------------------------------------
def pin_worked_example(ref):
    """The pages' worked example of Eq.(8) and the gate (fixture with citation)."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    pr, dv = ex["printed"], ex["derived"]
    h_n = np.array(dv["noise_outputs"]).reshape(1, 2, 1)
    _close(ref.repeat_noise(h_n, 2).reshape(-1), pr["repeat_2_of_noise"], 1e-15, "Repeat_2")
    dims = ref.Dims(6, 4, 2, 2, 1, 2)
    heads = np.array(dv["signal_outputs"] + dv["noise_outputs"]).reshape(1, 6, 1)
    lam = np.array(dv["lambda"]).reshape(1, 4)
    d = ref.differential_combine(heads, lam, dims)
    _close(d.reshape(-1), pr["D"], 1e-12, "worked example D")
    gp = np.array(pr["gate_G"])
    y = ref.gate_output(d, np.log(gp / (1.0 - gp)).reshape(1, 4, 1)).reshape(-1)
    if np.max(np.abs(y - np.array(pr["gated"]))) > ex["tolerance_printed_2dp"] + 1e-12:
        raise AssertionError(f"worked example gated output {y} vs printed {pr['gated']}")


def pin_rmsnorm_library(ref):
    """RMSNorm equals torch.nn.functional.rms_norm in fp64."""
    g = torch.Generator().manual_seed(3)
    v = torch.randn(5, 33, generator=g, dtype=torch.float64) * 3.0
    gamma = 1.0 + 0.2 * torch.randn(33, generator=g, dtype=torch.float64)
    for eps in (1e-6, 0.5):
        exp = torch.nn.functional.rms_norm(v, (33,), gamma, eps).numpy()
        _close(ref.rms_norm(v.numpy(), gamma.numpy(), eps), exp, 1e-13, "rms_norm vs torch")


def pin_attention_sdpa(ref):
    """Per-head attention equals torch SDPA (fp64 CPU, boolean mask, scale 1/sqrt(d_h + d_R))."""
    g = torch.Generator().manual_seed(7)
    for n_heads, n_signal, n_noise, n_kv, window, p0, t in (
            (8, 6, 2, 2, 0, 0, 9), (8, 6, 2, 2, 0, 6, 5), (8, 6, 2, 2, 3, 4, 7),
            (8, 6, 2, 2, 1, 0, 4), (8, 6, 2, 2, 20, 2, 6), (12, 8, 4, 2, 0, 3, 6)):
        dh, dr = 5, 4
        dims = ref.Dims(n_heads, n_signal, n_noise, n_kv, dh, dr, window)
        big_l = p0 + t
        q_c = torch.randn(t, n_heads, dh, generator=g, dtype=torch.float64)
        q_r = torch.randn(t, n_heads, dr, generator=g, dtype=torch.float64)
        k_c = torch.randn(big_l, n_kv, dh, generator=g, dtype=torch.float64)
        k_r = torch.randn(big_l, dr, generator=g, dtype=torch.float64)
        v = torch.randn(big_l, n_kv, dh, generator=g, dtype=torch.float64)
        qpos = np.arange(p0, p0 + t)
        got = ref.attention_expanded(q_c.numpy(), q_r.numpy(), k_c.numpy(), k_r.numpy(),
                                     v.numpy(), qpos, dims)
        p = torch.arange(p0, p0 + t)[:, None]
        s = torch.arange(big_l)[None, :]
        mask = s <= p
        if window > 0:
            mask = mask & (p - s < window)
        for h in range(n_heads):
            j = _kv_reading(h, n_signal, n_kv)
            q = torch.cat([q_c[:, h], q_r[:, h]], dim=1)[None]
            k = torch.cat([k_c[:, j], k_r], dim=1)[None]
            exp = torch.nn.functional.scaled_dot_product_attention(
                q, k, v[:, j][None], attn_mask=mask[None], scale=1.0 / math.sqrt(dh + dr))[0]
            _close(got[:, h], exp.numpy(), 1e-12, f"attention vs SDPA (W={window}, h={h})")


def pin_brute_force(ref):
    """The whole layer equals the 50-digit scalar-loop brute force on tiny shapes."""
    cases = [  # (n_heads, n_signal, n_noise, n_kv, seq, p0, window)
        (3, 2, 1, 1, 1, 0, 0), (3, 2, 1, 1, 5, 0, 0), (4, 3, 1, 1, 2, 3, 0),
        (6, 4, 2, 2, 5, 3, 2), (6, 4, 2, 1, 4, 0, 1), (4, 3, 1, 1, 5, 3, 2),
        (12, 8, 4, 2, 3, 1, 0),
    ]
    for i, (nh, ns, nn, nkv, t, p0, win) in enumerate(cases):
        cfg, w, x, prefix = small_problem(nh, ns, nn, nkv, d_model=6, d_q_latent=5,
                                          d_kv_latent=4, d_head=4, d_rope=2, seq=t, p0=p0,
                                          seed=100 + i)
        dims = make_dims(ref, cfg, win)
        got = ref.gdla_forward(x, w, dims, prefix, p0)
        out, heads = brute_gdla(x, w, ns, nn, nkv, 4, 2, win, prefix=prefix, p0=p0)
        exp_out = np.array([[float(v) for v in r] for r in out])
        exp_h = np.array([[[float(v) for v in hh] for hh in r] for r in heads])
        _close(got["heads"], exp_h, 1e-12, f"brute force heads case {i}")
        _close(got["out"], exp_out, 1e-12, f"brute force out case {i}")


def pin_lambda_zero_is_mla(ref):
    """lambda = 0 gives the independently written gated MLA over the signal heads."""
    for window, p0 in ((0, 0), (3, 4), (0, 5)):
        cfg, w, x, prefix = small_problem(8, 6, 2, 2, seq=6, p0=p0, seed=21 + p0)
        dims = make_dims(ref, cfg, window)
        got = ref.gdla_forward(x, w, dims, prefix, p0, lam_override=np.zeros((6, 6)))
        exp = mla_forward(x, w, 6, 2, 2, cfg["d_head"], cfg["d_rope"], window,
                          prefix=prefix, p0=p0)
        _close(got["out"], exp, 1e-12, f"lambda=0 vs MLA (W={window}, p0={p0})")


def pin_absorbed_equals_expanded(ref):
    """Attention on the latent (absorbed) equals attention on expanded K/V (associativity)."""
    for window, p0 in ((0, 0), (2, 3)):
        cfg, w, x, prefix = small_problem(6, 4, 2, 2, seq=5, p0=p0, seed=31)
        dims = make_dims(ref, cfg, window)
        a = ref.gdla_forward(x, w, dims, prefix, p0, form="expanded")
        b = ref.gdla_forward(x, w, dims, prefix, p0, form="absorbed")
        _close(a["heads"], b["heads"], 1e-12, "absorbed vs expanded heads")
        _close(a["out"], b["out"], 1e-12, "absorbed vs expanded out")


def pin_window_special_cases(ref):
    """W >= L equals full causal; W = 1 makes every head output its own token's value."""
    cfg, w, x, prefix = small_problem(6, 4, 2, 2, seq=6, p0=2, seed=41)
    full = ref.gdla_forward(x, w, make_dims(ref, cfg, 0), prefix, 2)
    wide = ref.gdla_forward(x, w, make_dims(ref, cfg, 8), prefix, 2)
    _close(wide["out"], full["out"], 0.0, "W >= L vs full")
    one = ref.gdla_forward(x, w, make_dims(ref, cfg, 1), prefix, 2)
    dh = cfg["d_head"]
    c_bar = one["cache_rows"][:, :cfg["d_kv_latent"]]
    v_own = c_bar @ w["w_uv"]
    for h in range(cfg["n_heads"]):
        j = _kv_reading(h, cfg["n_signal"], cfg["n_kv"])
        _close(one["heads"][:, h], v_own[:, j * dh:(j + 1) * dh], 1e-13, f"W=1 head {h}")


def pin_closed_forms(ref):
    """T = 1 at position 0 sees only itself; with zero query weights every score is equal and the
    head output is the plain mean of the visible values."""
    cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=1, p0=0, seed=51)
    r = ref.gdla_forward(x, w, make_dims(ref, cfg), None, 0)
    dh = cfg["d_head"]
    v0 = r["cache_rows"][:, :cfg["d_kv_latent"]] @ w["w_uv"]
    for h in range(cfg["n_heads"]):
        j = _kv_reading(h, cfg["n_signal"], cfg["n_kv"])
        _close(r["heads"][0, h], v0[0, j * dh:(j + 1) * dh], 1e-13, "T=1 closed form")
    for window in (0, 3):
        cfg, w, x, prefix = small_problem(6, 4, 2, 2, seq=7, p0=2, seed=52)
        w0 = dict(w)
        w0["w_qc"] = np.zeros_like(w["w_qc"])
        w0["w_qr"] = np.zeros_like(w["w_qr"])
        r = ref.gdla_forward(x, w0, make_dims(ref, cfg, window), prefix, 2)
        rows = np.concatenate([prefix, r["cache_rows"]])
        vals = rows[:, :cfg["d_kv_latent"]] @ w["w_uv"]
        for t in range(7):
            p = 2 + t
            lo = 0 if window == 0 else max(0, p - window + 1)
            mean = vals[lo:p + 1].mean(axis=0)
            for h in range(cfg["n_heads"]):
                j = _kv_reading(h, cfg["n_signal"], cfg["n_kv"])
                _close(r["heads"][t, h], mean[j * dh:(j + 1) * dh], 1e-13, "equal-score mean")


def pin_chunk_consistency(ref):
    """One call over T tokens = the same tokens in two chunks = T-1 tokens then a decode step."""
    cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=9, p0=0, seed=61)
    for window in (0, 3):
        dims = make_dims(ref, cfg, window)
        mono = ref.gdla_forward(x, w, dims, None, 0)
        a = ref.gdla_forward(x[:4], w, dims, None, 0)
        b = ref.gdla_forward(x[4:], w, dims, a["cache_rows"], 4)
        _close(np.concatenate([a["out"], b["out"]]), mono["out"], 1e-12, "chunked vs one call")
        _close(np.concatenate([a["cache_rows"], b["cache_rows"]]), mono["cache_rows"], 1e-13,
               "chunked cache rows")
        c = ref.gdla_forward(x[:8], w, dims, None, 0)
        dec = ref.gdla_decode(x[8:9], w, dims, [c["cache_rows"]], [8])
        _close(dec["out"][0], mono["out"][8], 1e-12, "prefill + decode vs one call")


def pin_pairing(ref):
    """With noise head j's query weights copied from signal head j, H_N,j = H_S,j (both read KV
    head j mod n_KV) and D_j = (1 - lambda_j) H_S,j."""
    cfg, w, x, _ = small_problem(8, 6, 2, 2, seq=5, p0=0, seed=71)
    dh, dr, ns = cfg["d_head"], cfg["d_rope"], cfg["n_signal"]
    w2 = dict(w)
    w2["w_qc"] = w["w_qc"].copy()
    w2["w_qr"] = w["w_qr"].copy()
    for j in range(cfg["n_noise"]):
        n = ns + j
        w2["w_qc"][:, n * dh:(n + 1) * dh] = w["w_qc"][:, j * dh:(j + 1) * dh]
        w2["w_qr"][:, n * dr:(n + 1) * dr] = w["w_qr"][:, j * dr:(j + 1) * dr]
    r = ref.gdla_forward(x, w2, make_dims(ref, cfg), None, 0)
    for j in range(cfg["n_noise"]):
        _close(r["heads"][:, ns + j], r["heads"][:, j], 1e-13, "noise copy = signal")
        _close(r["D"][:, j], (1.0 - r["lam"][:, j:j + 1]) * r["heads"][:, j], 1e-13,
               "D = (1 - lambda) H_S")


def pin_rope_mechanics(ref):
    """RoPE is a rotation (norm kept, identity at 0) that pairs dim j with j + d/2, and q.k after
    RoPE depends on positions only through their difference."""
    g = np.random.default_rng(5)
    d = 8
    u = g.standard_normal((6, d))
    pos = np.array([0, 1, 5, 17, 123, 4095])
    r = ref.rope(u, pos)
    _close(np.linalg.norm(r, axis=1), np.linalg.norm(u, axis=1), 1e-12, "rope keeps norms")
    _close(r[0], u[0], 0.0, "rope at position 0")
    e0 = np.zeros((1, d))
    e0[0, 0] = 1.0
    re0 = ref.rope(e0, np.array([7]))[0]
    if np.any(np.abs(np.delete(re0, [0, d // 2])) > 0) or abs(re0[0] - math.cos(7.0)) > 1e-13:
        raise AssertionError("rope must rotate (j, j + d/2) by p * theta^(-2j/d)")
    q = g.standard_normal((1, d))
    k = g.standard_normal((1, d))
    for p, s, delta in ((9, 4, 100), (3, 3, 50), (1000, 10, 7)):
        a = ref.rope(q, np.array([p])) @ ref.rope(k, np.array([s])).T
        b = ref.rope(q, np.array([p + delta])) @ ref.rope(k, np.array([s + delta])).T
        _close(a, b, 1e-11, "rope relative-position invariance")


def pin_row_sums(ref):
    """Every softmax row sums to one: with all values 1 every head outputs exactly 1."""
    g = np.random.default_rng(9)
    dims = ref.Dims(6, 4, 2, 2, 4, 2, 3)
    t, big_l = 5, 9
    h = ref.attention_expanded(g.standard_normal((t, 6, 4)), g.standard_normal((t, 6, 2)),
                               g.standard_normal((big_l, 2, 4)), g.standard_normal((big_l, 2)),
                               np.ones((big_l, 2, 4)), np.arange(4, 9), dims)
    _close(h, np.ones_like(h), 1e-14, "row sums")


def _doc_starts(lengths, first=0):
    """Per-token document start for documents of the given lengths packed from position `first`."""
    out, start = [], first
    for n in lengths:
        out += [start] * n
        start += n
    return np.array(out)


def pin_documents_brute_force(ref):
    """Packed documents: the layer equals the 50-digit brute force whose visible set also starts
    at the token's document (tiny shapes; with a window; a document that began in the prefix)."""
    cases = [  # (seq, p0, window, document lengths of the new tokens, first document start)
        (6, 0, 0, (2, 3, 1), 0), (5, 3, 2, (2, 3), 1), (4, 2, 0, (3, 1), 0),
    ]
    for i, (t, p0, win, lens, first) in enumerate(cases):
        cfg, w, x, prefix = small_problem(4, 3, 1, 1, d_model=6, d_q_latent=5, d_kv_latent=4,
                                          d_head=4, d_rope=2, seq=t, p0=p0, seed=140 + i)
        ds = _doc_starts(lens, p0)
        ds[:lens[0]] = first  # the first document may have started before the new tokens
        got = ref.gdla_forward(x, w, make_dims(ref, cfg, win), prefix, p0, doc_start=ds)
        out, heads = brute_gdla(x, w, 3, 1, 1, 4, 2, win, prefix=prefix, p0=p0, doc_start=list(ds))
        exp_out = np.array([[float(v) for v in r] for r in out])
        _close(got["out"], exp_out, 1e-12, f"documents brute force case {i}")


def pin_documents_are_separate_sequences(ref):
    """A packed sequence of documents gives, on each document's rows, the forward of that document
    alone from position 0: attention stays inside the document and RoPE scores depend only on
    relative positions (the pages' packed training sequence, paperglide Figure 4 (a))."""
    lens = (5, 1, 7, 3)
    cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=sum(lens), seed=77)
    for win in (0, 3):
        dims = make_dims(ref, cfg, win)
        packed = ref.gdla_forward(x, w, dims, doc_start=_doc_starts(lens))
        absorbed = ref.gdla_forward(x, w, dims, doc_start=_doc_starts(lens), form="absorbed")
        _close(absorbed["out"], packed["out"], 1e-12, "documents absorbed vs expanded")
        start = 0
        for n in lens:
            alone = ref.gdla_forward(x[start:start + n], w, dims)
            _close(packed["out"][start:start + n], alone["out"], 1e-11,
                   f"document at {start} (W={win}) vs the document alone")
            start += n
    # no document boundary inside the new tokens: the same as no documents
    plain = ref.gdla_forward(x, w, make_dims(ref, cfg, 0))
    one = ref.gdla_forward(x, w, make_dims(ref, cfg, 0), doc_start=np.zeros(sum(lens), dtype=int))
    _close(one["out"], plain["out"], 0.0, "one document vs no documents")


ALL_PINS = [pin_worked_example, pin_rmsnorm_library, pin_attention_sdpa, pin_brute_force,
            pin_lambda_zero_is_mla, pin_absorbed_equals_expanded, pin_window_special_cases,
            pin_closed_forms, pin_chunk_consistency, pin_pairing, pin_rope_mechanics,
            pin_row_sums, pin_documents_brute_force, pin_documents_are_separate_sequences]


# -------------------------------------------------------------------------------- backward
# Pins of the backward oracle (oracle/gdla_grad.py).  Each takes the backward module `gg`; the
# forward they differentiate is oracle.gdla_ref, pinned above.
def _loss_fd(ref_fwd, x, w, dims, dout, docs, name, direction, eps=1e-6):
    """Central difference of L = sum(out (.) dout) along `direction` of input `name`."""
    def f(xx, ww):
        return float(np.sum(ref_fwd.gdla_forward(xx, ww, dims, doc_start=docs)["out"] * dout))
    if name == "x":
        return (f(x + eps * direction, w) - f(x - eps * direction, w)) / (2 * eps)
    wp, wm = dict(w), dict(w)
    wp[name] = w[name] + eps * direction
    wm[name] = w[name] - eps * direction
    return (f(x, wp) - f(x, wm)) / (2 * eps)


def pin_backward_finite_differences(gg):
    """Every gradient matches the central finite difference of the pinned forward along a random
    direction (full causal; with a window and packed documents)."""
    import oracle.gdla_ref as ref_fwd
    for i, (win, docs) in enumerate(((0, None), (3, [0, 0, 0, 3, 3, 3, 3, 7]))):
        cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=8, seed=61 + i)
        dims = make_dims(ref_fwd, cfg, win)
        rng = np.random.default_rng(70 + i)
        dout = rng.standard_normal((8, cfg["d_model"]))
        g = gg.gdla_backward(x, w, dims, dout, doc_start=None if docs is None else np.array(docs))
        names = ["x"] + sorted(k for k in w if w[k] is not None)
        for name in names:
            base = x if name == "x" else w[name]
            direction = rng.standard_normal(base.shape)
            fd = _loss_fd(ref_fwd, x, w, dims, dout, docs, name, direction)
            an = float(np.sum(g["d" + name] * direction))
            if not abs(fd - an) <= 1e-7 * max(1.0, abs(fd)):
                raise AssertionError(f"backward vs finite difference, {name} (case {i}): {an} vs {fd}")


def pin_backward_entries(gg):
    """Single entries of dx and of several weight gradients against one-coordinate differences."""
    import oracle.gdla_ref as ref_fwd
    cfg, w, x, _ = small_problem(4, 3, 1, 1, seq=5, seed=83)
    dims = make_dims(ref_fwd, cfg, 0)
    dout = np.random.default_rng(84).standard_normal((5, cfg["d_model"]))
    g = gg.gdla_backward(x, w, dims, dout)
    for name, idx in (("x", (4, 3)), ("x", (0, 0)), ("w_qc", (2, 5)), ("w_uk", (1, 2)),
                      ("w_kr", (3, 1)), ("w_lambda", (0, 2)), ("gamma_kv", (5,))):
        base = x if name == "x" else w[name]
        e = np.zeros(base.shape)
        e[idx] = 1.0
        fd = _loss_fd(ref_fwd, x, w, dims, dout, None, name, e)
        an = float(g["d" + name][idx])
        if not abs(fd - an) <= 1e-7 * max(1.0, abs(fd)):
            raise AssertionError(f"d{name}{idx}: {an} vs finite difference {fd}")


def pin_backward_lambda_zero(gg):
    """With lambda fixed at 0 the noise heads do not reach the output: the columns of W_qc and W_qr
    that feed the noise heads get exactly zero gradient, and so does every noise head's dH."""
    import oracle.gdla_ref as ref_fwd
    cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=6, seed=91)
    dims = make_dims(ref_fwd, cfg, 0)
    dout = np.random.default_rng(92).standard_normal((6, cfg["d_model"]))
    g = gg.gdla_backward(x, w, dims, dout, lam_override=np.zeros((6, 4)))
    dh, dr = cfg["d_head"], cfg["d_rope"]
    _close(g["dH"][:, 4:], np.zeros_like(g["dH"][:, 4:]), 0.0, "noise dH with lambda = 0")
    _close(g["dw_qc"][:, 4 * dh:], np.zeros((cfg["d_q_latent"], 2 * dh)), 0.0, "noise W_qc grad")
    _close(g["dw_qr"][:, 4 * dr:], np.zeros((cfg["d_q_latent"], 2 * dr)), 0.0, "noise W_qr grad")
    if not np.all(np.abs(g["dw_qc"][:, :4 * dh]) > 0):
        raise AssertionError("signal W_qc grad vanished")


def pin_backward_matches_stored(gg):
    """The oracle, which forms one head's probability matrix at a time, reproduces the gradients the
    earlier version (every head's probabilities kept for the whole call) wrote to
    tests/golden/backward_small.npz (tests/golden/make_backward_golden.py), on a full-causal problem
    and on a windowed one with packed documents."""
    import oracle.gdla_ref as ref_fwd
    stored = np.load(os.path.join(GOLDEN, "backward_small.npz"))
    cases = ((0, None, 101), (3, [0, 0, 0, 3, 3, 3, 3, 7, 7], 102))
    for i, (win, docs, seed) in enumerate(cases):
        cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=9, seed=seed)
        dims = make_dims(ref_fwd, cfg, win)
        dout = np.random.default_rng(seed + 1000).standard_normal((9, cfg["d_model"]))
        g = gg.gdla_backward(x, w, dims, dout, doc_start=None if docs is None else np.array(docs))
        names = sorted(k[len(f"case{i}_"):] for k in stored.files if k.startswith(f"case{i}_"))
        if len(names) < 15:
            raise AssertionError(f"stored case {i} holds only {names}")
        for name in names:
            _close(g[name], stored[f"case{i}_{name}"], 1e-12, f"case {i} {name} vs stored")


def pin_backward_process_map(gg):
    """The heads' maps evaluated by two worker processes give exactly the sequential result."""
    import multiprocessing as mp
    import oracle.gdla_ref as ref_fwd
    cfg, w, x, _ = small_problem(6, 4, 2, 2, seq=9, seed=111)
    dims = make_dims(ref_fwd, cfg, 4)
    dout = np.random.default_rng(112).standard_normal((9, cfg["d_model"]))
    seq = gg.gdla_backward(x, w, dims, dout)
    with mp.get_context("spawn").Pool(2) as pool:
        par = gg.gdla_backward(x, w, dims, dout, map_fn=pool.imap)
    for name, val in seq.items():
        if val is not None:
            _close(par[name], val, 0.0, f"{name}: process map vs sequential")


# pins of the gradient values (the planted-mistake tests run these), and all backward pins
GRAD_VALUE_PINS = [pin_backward_finite_differences, pin_backward_entries, pin_backward_lambda_zero,
                   pin_backward_matches_stored]
GRAD_PINS = GRAD_VALUE_PINS + [pin_backward_process_map]
