"""Plain fp64 CPU oracle of the Grouped Differential Latent Attention (GDLA) forward pass.

TEST INFRASTRUCTURE ONLY.  This module is the correctness oracle of the GDLA library: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import it.  The GPU product
path never imports, calls or links anything here, and nothing here imports the product package.

What it computes follows the Motif 3 Technical Report pages:

* picx.dev summary, section 2.2 "Grouped Differential Latent Attention", display equations
  numbered in order of appearance:
    Eq.(1)  c^Q_t = RMSNorm(x_t W^Q_a)
    Eq.(2)  [q^C_t ; q^R_t] = c^Q_t W^Q_b
    Eq.(3)  [c^KV_t ; k^R_t] = x_t W^KV_a              (k^R is the decoupled rotary key)
    Eq.(4)  cbar^KV_t = RMSNorm(c^KV_t)
    Eq.(5)  [K^C_t ; V_t] = Reshape_heads(cbar^KV_t W^KV_b)
    Eq.(6)  n_N = n_H / (g + 1),  n_S = g n_N
    Eq.(7)  lambda_t = sigmoid(x_t W^lambda) in (0,1)^{n_S}
    Eq.(8)  D_t = H_{S,t} - lambda_t (.) Repeat_g(H_{N,t})
    Eq.(9)  G_t = Reshape_heads(c^Q_t W^G)
    Eq.(10) GDLA(x_t) = vec(sigmoid(G_t) (.) D_t) W^O
* paperglide reader, section "Model Architecture": the worked numeric example of the combine
  (Repeat tiles the noise outputs) and the Figure 1 caption (one RMS-normalised KV latent expanded
  into the KV heads shared by the signal and noise query paths; one rotary key shared by all heads;
  an element-wise gate from the normalised query latent; one lambda per signal head and token).
* the same section's MLA answer: the cache holds the latent only and the full K/V are rebuilt
  inside attention, which is the "absorbed" form evaluated by `attention_absorbed`.

Where the pages are silent the oracle takes these readings (the GPU library takes the same ones):

* Heads 0..n_S-1 of W_qc / W_qr are the signal heads, n_S..n_H-1 the noise heads.
* Repeat_g tiles: signal head i pairs with noise head (i mod n_N).
* Query head -> KV head: signal i -> i mod n_KV, noise j -> j mod n_KV (requires n_KV | n_N, so a
  signal head and its noise partner read the same KV head).
* RMSNorm(v) = v / sqrt(mean(v^2) + eps) * gamma, applied to c^Q and c^KV only.
* RoPE: rotate-half pairs (j, j + d_R/2) with angle p * theta^(-2j/d_R), absolute 0-based
  positions p = P0 + t.
* Softmax scale 1/sqrt(d_head + d_rope); key s is visible from query p iff s <= p and, when a
  window W > 0 is set, p - s < W.
* Packed documents (paperglide reader, Figure 4 (a): a training sequence holding 473 documents,
  drawn on the QK^T score matrix): when a token's document start d(p) is given, key s is visible
  from query p only if also s >= d(p), i.e. attention stays inside the document.
* A cache row is [cbar^KV (after norm and gamma) ; k^R (after RoPE)].

The softmax is evaluated exactly per row in two passes (max, then exp / sum); a matmul is used as
a library step; the only blocking is over query rows, to bound memory.
"""

import math

import numpy as np

__all__ = [
    "Dims", "rms_norm", "sigmoid", "rope", "kv_head_of", "noise_partner", "repeat_noise",
    "query_path", "latent_path", "lambda_path", "expand_kv", "visible_mask",
    "attention_expanded", "attention_absorbed", "differential_combine", "gate_output",
    "output_projection", "gdla_forward", "gdla_forward_batch", "gdla_decode",
]


class Dims:
    """Head and latent sizes of one GDLA layer (picx.dev summary section 2.2, Eq.(6))."""

    def __init__(self, n_heads, n_signal, n_noise, n_kv, d_head, d_rope, window=0,
                 eps=1e-6, theta=10000.0, scale=None):
        if n_signal + n_noise != n_heads:
            raise ValueError("n_signal + n_noise must equal n_heads")
        if n_noise <= 0 or n_signal % n_noise != 0:
            raise ValueError("n_signal must be a multiple g of n_noise (Eq.(6))")
        if n_kv <= 0 or n_noise % n_kv != 0:
            raise ValueError("n_kv must divide n_noise (KV-head reading)")
        if d_rope % 2 != 0:
            raise ValueError("d_rope must be even (rotate-half RoPE)")
        self.n_heads, self.n_signal, self.n_noise, self.n_kv = n_heads, n_signal, n_noise, n_kv
        self.d_head, self.d_rope = d_head, d_rope
        self.window = int(window)
        self.eps = float(eps)
        self.theta = float(theta)
        self.g = n_signal // n_noise
        self.scale = (1.0 / math.sqrt(d_head + d_rope)) if not scale else float(scale)

    def with_window(self, window):
        return Dims(self.n_heads, self.n_signal, self.n_noise, self.n_kv, self.d_head,
                    self.d_rope, window, self.eps, self.theta, self.scale)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def rms_norm(v, gamma=None, eps=1e-6):
    """RMSNorm over the last axis (Eq.(1) and Eq.(4)): v / sqrt(mean(v^2) + eps) * gamma."""
    v = _f64(v)
    r = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return r if gamma is None else r * _f64(gamma)


def sigmoid(z):
    """Logistic function, evaluated without overflow for either sign of z."""
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def rope(u, pos, theta=10000.0):
    """Rotary encoding of the decoupled rotary dims (Eq.(2)-(3); convention is a reading).

    u has shape [T, ..., d] and pos has shape [T].  Pair (j, j + d/2) is rotated by the angle
    pos * theta^(-2j/d): (a, b) -> (a cos - b sin, a sin + b cos).
    """
    u = _f64(u)
    d = u.shape[-1]
    half = d // 2
    freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = _f64(pos).reshape((-1,) + (1,) * (u.ndim - 1)) * freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def kv_head_of(h, dims):
    """KV head read by query head h: signal i -> i mod n_KV, noise j -> j mod n_KV."""
    if h < dims.n_signal:
        return h % dims.n_kv
    return (h - dims.n_signal) % dims.n_kv


def noise_partner(i, dims):
    """Index (among all heads) of the noise head whose output is subtracted from signal head i."""
    return dims.n_signal + (i % dims.n_noise)


def repeat_noise(h_noise, g):
    """Repeat_g of Eq.(8): tile the n_N noise outputs g times along the head axis (axis -2)."""
    h_noise = _f64(h_noise)
    reps = [1] * h_noise.ndim
    reps[-2] = g
    return np.tile(h_noise, reps)


def query_path(x, w, dims, pos):
    """Eq.(1), (2), (9): latent query c^Q, per-head q^C, rotated q^R and gate logits G."""
    x = _f64(x)
    t = x.shape[0]
    c_q = rms_norm(x @ _f64(w["w_qa"]), w.get("gamma_q"), dims.eps)
    q_c = (c_q @ _f64(w["w_qc"])).reshape(t, dims.n_heads, dims.d_head)
    q_r = rope((c_q @ _f64(w["w_qr"])).reshape(t, dims.n_heads, dims.d_rope), pos, dims.theta)
    gate = (c_q @ _f64(w["w_gate"])).reshape(t, dims.n_signal, dims.d_head)
    return c_q, q_c, q_r, gate


def latent_path(x, w, dims, pos):
    """Eq.(3), (4): normalised KV latent cbar and the rotated shared key k^R, one per token."""
    x = _f64(x)
    c_bar = rms_norm(x @ _f64(w["w_dkv"]), w.get("gamma_kv"), dims.eps)
    k_r = rope(x @ _f64(w["w_kr"]), pos, dims.theta)
    return c_bar, k_r


def lambda_path(x, w):
    """Eq.(7): one coefficient per signal head and token, sigmoid(x W^lambda)."""
    return sigmoid(_f64(x) @ _f64(w["w_lambda"]))


def expand_kv(c_bar, w, dims):
    """Eq.(5): K^C and V of every KV head from the latent; head j is column block j."""
    c_bar = _f64(c_bar)
    n = c_bar.shape[0]
    k_c = (c_bar @ _f64(w["w_uk"])).reshape(n, dims.n_kv, dims.d_head)
    v = (c_bar @ _f64(w["w_uv"])).reshape(n, dims.n_kv, dims.d_head)
    return k_c, v


def visible_mask(qpos, kpos, window, qdoc=None):
    """Key s is visible from query p iff s <= p and (window == 0 or p - s < window) and, with
    document starts qdoc, s >= qdoc[p's row]."""
    p = np.asarray(qpos)[:, None]
    s = np.asarray(kpos)[None, :]
    m = s <= p
    if window > 0:
        m &= (p - s) < window
    if qdoc is not None:
        m &= s >= np.asarray(qdoc)[:, None]
    return m


def _key_range(qpos, window, qdoc=None):
    lo = 0 if window <= 0 else max(0, int(np.min(qpos)) - window + 1)
    if qdoc is not None:
        lo = max(lo, int(np.min(qdoc)))
    return lo, int(np.max(qpos)) + 1


def _softmax_rows(scores, mask):
    """Exact two-pass softmax of each row over its visible entries."""
    scores = np.where(mask, scores, -np.inf)
    m = np.max(scores, axis=1, keepdims=True)
    e = np.where(mask, np.exp(scores - m), 0.0)
    p = e / np.sum(e, axis=1, keepdims=True)
    if np.any(np.abs(np.sum(p, axis=1) - 1.0) > 1e-12):
        raise AssertionError("softmax row does not sum to 1")
    return p


def attention_expanded(q_c, q_r, k_c, k_r, v, qpos, dims, block=256, qdoc=None):
    """Per-head softmax attention over expanded keys [K^C ; k^R] and values V.

    q_c [T, n_H, d_h], q_r [T, n_H, d_R]; k_c, v [L, n_KV, d_h]; k_r [L, d_R] (shared by all
    heads); qpos [T] absolute positions; qdoc [T] optional document starts; keys are positions
    0..L-1.  Returns H [T, n_H, d_h].
    """
    q_c, q_r, k_c, k_r, v = map(_f64, (q_c, q_r, k_c, k_r, v))
    qpos = np.asarray(qpos)
    t = q_c.shape[0]
    out = np.zeros((t, dims.n_heads, dims.d_head))
    for t0 in range(0, t, block):
        t1 = min(t, t0 + block)
        p = qpos[t0:t1]
        qd = None if qdoc is None else np.asarray(qdoc)[t0:t1]
        lo, hi = _key_range(p, dims.window, qd)
        mask = visible_mask(p, np.arange(lo, hi), dims.window, qd)
        for h in range(dims.n_heads):
            j = kv_head_of(h, dims)
            s = dims.scale * (q_c[t0:t1, h] @ k_c[lo:hi, j].T + q_r[t0:t1, h] @ k_r[lo:hi].T)
            out[t0:t1, h] = _softmax_rows(s, mask) @ v[lo:hi, j]
    return out


def attention_absorbed(q_c, q_r, c_bar, k_r, w, dims, qpos, block=256, qdoc=None):
    """The same attention evaluated on the latent cache (the MLA 'reconstruct inside attention').

    q~ = q^C_h W_uk[:, j]^T scores against cbar directly, o = sum_s P_s cbar_s, H = o W_uv[:, j].
    """
    q_c, q_r, c_bar, k_r = map(_f64, (q_c, q_r, c_bar, k_r))
    w_uk, w_uv = _f64(w["w_uk"]), _f64(w["w_uv"])
    qpos = np.asarray(qpos)
    t = q_c.shape[0]
    dh = dims.d_head
    out = np.zeros((t, dims.n_heads, dh))
    for t0 in range(0, t, block):
        t1 = min(t, t0 + block)
        p = qpos[t0:t1]
        qd = None if qdoc is None else np.asarray(qdoc)[t0:t1]
        lo, hi = _key_range(p, dims.window, qd)
        mask = visible_mask(p, np.arange(lo, hi), dims.window, qd)
        for h in range(dims.n_heads):
            j = kv_head_of(h, dims)
            q_abs = q_c[t0:t1, h] @ w_uk[:, j * dh:(j + 1) * dh].T
            s = dims.scale * (q_abs @ c_bar[lo:hi].T + q_r[t0:t1, h] @ k_r[lo:hi].T)
            o = _softmax_rows(s, mask) @ c_bar[lo:hi]
            out[t0:t1, h] = o @ w_uv[:, j * dh:(j + 1) * dh]
    return out


def differential_combine(h, lam, dims):
    """Eq.(8): D = H_S - lambda (.) Repeat_g(H_N); h [T, n_H, d_h], lam [T, n_S] -> [T, n_S, d_h]."""
    h = _f64(h)
    h_s = h[:, :dims.n_signal]
    h_n = h[:, dims.n_signal:]
    return h_s - _f64(lam)[:, :, None] * repeat_noise(h_n, dims.g)


def gate_output(d, gate_logits):
    """Eq.(10), before W^O: the element-wise sigmoid gate."""
    return sigmoid(gate_logits) * _f64(d)


def output_projection(y, w_o):
    """Eq.(10): vec over heads, then W^O."""
    y = _f64(y)
    return y.reshape(y.shape[0], -1) @ _f64(w_o)


def gdla_forward(x, w, dims, prefix=None, p0=0, lam_override=None, form="expanded", rows=None,
                 doc_start=None):
    """GDLA layer forward for one sequence: T new tokens at positions p0 .. p0+T-1.

    prefix: [p0, d_c + d_R] cache rows already present (None when p0 == 0).
    rows:   optional indices of the query rows to evaluate (all rows by default); the cache rows of
            all T tokens are always produced, since later rows attend to them.
    doc_start: optional [T] position of the first token of each new token's document (packed
            documents); attention then stays inside the document.
    Returns a dict with out [R, d_model], cache_rows [T, d_c + d_R], heads H [R, n_H, d_h],
    lam [R, n_S], and the intermediates of the R evaluated rows.
    """
    x = _f64(x)
    t = x.shape[0]
    pos = p0 + np.arange(t)
    sel = np.arange(t) if rows is None else np.asarray(rows)
    # queries, gates and lambdas only for the evaluated rows; latents for every new token
    c_q, q_c, q_r, gate = query_path(x[sel], w, dims, pos[sel])
    c_bar_new, k_r_new = latent_path(x, w, dims, pos)
    lam = lambda_path(x[sel], w) if lam_override is None else _f64(lam_override)[sel]
    cache_rows = np.concatenate([c_bar_new, k_r_new], axis=1)
    d_c = c_bar_new.shape[1]
    if p0 > 0:
        prefix = _f64(prefix)
        if prefix.shape[0] != p0 or prefix.shape[1] != cache_rows.shape[1]:
            raise ValueError("prefix must be [p0, d_c + d_R]")
        keys = np.concatenate([prefix, cache_rows], axis=0)
    else:
        keys = cache_rows
    c_bar_all, k_r_all = keys[:, :d_c], keys[:, d_c:]
    qpos = pos[sel]
    qdoc = None if doc_start is None else np.asarray(doc_start)[sel]
    if qdoc is not None and np.any((qdoc < 0) | (qdoc > qpos)):
        raise ValueError("a document must start at or before its token")
    hi = int(np.max(qpos)) + 1
    if form == "expanded":
        k_c, v = expand_kv(c_bar_all[:hi], w, dims)
        heads = attention_expanded(q_c, q_r, k_c, k_r_all[:hi], v, qpos, dims, qdoc=qdoc)
    elif form == "absorbed":
        heads = attention_absorbed(q_c, q_r, c_bar_all[:hi], k_r_all[:hi], w, dims, qpos, qdoc=qdoc)
    else:
        raise ValueError("form must be 'expanded' or 'absorbed'")
    d = differential_combine(heads, lam, dims)
    y = gate_output(d, gate)
    out = output_projection(y, w["w_o"])
    return {"out": out, "cache_rows": cache_rows, "heads": heads, "lam": lam, "gate": gate,
            "D": d, "Y": y, "c_q": c_q, "q_c": q_c, "q_r": q_r}


def gdla_forward_batch(x, w, dims, prefixes=None, p0s=None, lam_override=None, form="expanded"):
    """gdla_forward over a batch [B, T, d]; prefixes[b] is [p0s[b], d_c + d_R] or None."""
    x = _f64(x)
    bsz = x.shape[0]
    p0s = [0] * bsz if p0s is None else list(p0s)
    outs, rows, heads = [], [], []
    for b in range(bsz):
        pre = None if prefixes is None else prefixes[b]
        lo = None if lam_override is None else lam_override[b]
        r = gdla_forward(x[b], w, dims, pre, p0s[b], lo, form)
        outs.append(r["out"])
        rows.append(r["cache_rows"])
        heads.append(r["heads"])
    return {"out": np.stack(outs), "cache_rows": rows, "heads": np.stack(heads)}


def gdla_decode(x, w, dims, prefixes, positions, lam_override=None, form="absorbed"):
    """One new token per sequence: x [B, d]; token b sits at positions[b] and sees prefixes[b]."""
    x = _f64(x)
    outs, rows, heads = [], [], []
    for b in range(x.shape[0]):
        lo = None if lam_override is None else _f64(lam_override)[b:b + 1]
        r = gdla_forward(x[b:b + 1], w, dims, prefixes[b], int(positions[b]), lo, form)
        outs.append(r["out"][0])
        rows.append(r["cache_rows"][0])
        heads.append(r["heads"][0])
    return {"out": np.stack(outs), "cache_rows": np.stack(rows), "heads": np.stack(heads)}
