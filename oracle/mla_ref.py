"""Gated multi-head latent attention (MLA) over the signal heads only: an independent reference.

TEST INFRASTRUCTURE ONLY (see the package header).  Written separately from gdla_ref.py and
sharing none of its helpers, so that "lambda = 0 reduces GDLA to gated MLA" is a check between two
independently written programs.

Motif 3 Technical Report pages: MLA keeps one latent per token and rebuilds K/V inside attention
(paperglide reader, section "Model Architecture", the MLA answer); GDLA adds noise heads and the
lambda term on top of it (picx.dev summary section 2.2, Eq.(8)).  With lambda = 0, Eq.(8) leaves
D = H_S, so Eq.(10) becomes vec(sigmoid(G) (.) H_S) W^O: plain MLA over the signal heads with the
same query-dependent gate.  Noise heads never influence the result.

Style on purpose differs from gdla_ref: the whole [T, L] score matrix of a head is built at once
with an explicit additive mask, RoPE is applied by complex multiplication, and the softmax uses the
log-sum-exp form.
"""

import numpy as np


def _norm(v, gamma, eps):
    ms = np.einsum("...i,...i->...", v, v) / v.shape[-1]
    out = v * (1.0 / np.sqrt(ms + eps))[..., None]
    return out if gamma is None else out * np.asarray(gamma, dtype=np.float64)


def _rotate(u, pos, theta):
    # pair (j, j + d/2) as the complex number a + i b, multiplied by exp(i * pos * theta^(-2j/d))
    d = u.shape[-1]
    half = d // 2
    z = u[..., :half] + 1j * u[..., half:]
    freq = np.power(theta, -np.arange(0, d, 2, dtype=np.float64) / d)
    ph = np.exp(1j * np.multiply.outer(pos.astype(np.float64), freq))
    ph = ph.reshape(ph.shape[:1] + (1,) * (u.ndim - 2) + ph.shape[1:])
    r = z * ph
    return np.concatenate([r.real, r.imag], axis=-1)


def mla_forward(x, w, n_signal, n_kv, n_noise, d_head, d_rope, window=0, eps=1e-6,
                theta=10000.0, scale=None, prefix=None, p0=0):
    """Gated MLA over the signal heads for one sequence x [T, d_model]; returns out [T, d_model].

    Uses the same weights as the GDLA layer; signal head i reads KV head i mod n_kv.  Keys are the
    prefix rows (latent after norm, rotary key after RoPE) followed by this call's own rows.
    """
    x = np.asarray(x, dtype=np.float64)
    f = lambda k: np.asarray(w[k], dtype=np.float64)
    t = x.shape[0]
    pos = p0 + np.arange(t)
    tau = scale if scale else 1.0 / np.sqrt(d_head + d_rope)
    cq = _norm(x @ f("w_qa"), w.get("gamma_q"), eps)
    n_heads = n_signal + n_noise
    qc = (cq @ f("w_qc")).reshape(t, n_heads, d_head)[:, :n_signal]
    qr = _rotate((cq @ f("w_qr")).reshape(t, n_heads, d_rope), pos, theta)[:, :n_signal]
    gates = 1.0 / (1.0 + np.exp(-(cq @ f("w_gate")).reshape(t, n_signal, d_head)))
    cb = _norm(x @ f("w_dkv"), w.get("gamma_kv"), eps)
    kr = _rotate(x @ f("w_kr"), pos, theta)
    if p0 > 0:
        pre = np.asarray(prefix, dtype=np.float64)
        d_c = cb.shape[1]
        cb = np.vstack([pre[:, :d_c], cb])
        kr = np.vstack([pre[:, d_c:], kr])
    big_l = cb.shape[0]
    kc_all = (cb @ f("w_uk")).reshape(big_l, n_kv, d_head)
    v_all = (cb @ f("w_uv")).reshape(big_l, n_kv, d_head)
    keys = np.arange(big_l)
    rel = pos[:, None] - keys[None, :]
    allowed = rel >= 0
    if window > 0:
        allowed = allowed & (rel < window)
    bias = np.where(allowed, 0.0, -np.inf)
    ys = np.empty((t, n_signal, d_head))
    for i in range(n_signal):
        j = i % n_kv
        logits = tau * (np.einsum("td,sd->ts", qc[:, i], kc_all[:, j])
                        + np.einsum("td,sd->ts", qr[:, i], kr)) + bias
        mx = logits.max(axis=1, keepdims=True)
        lse = mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True))
        probs = np.exp(logits - lse)
        ys[:, i] = gates[:, i] * (probs @ v_all[:, j])
    return ys.reshape(t, n_signal * d_head) @ f("w_o")
