"""Plain fp64 CPU oracle of the GDLA layer's backward pass (gradients of a training step).

TEST INFRASTRUCTURE ONLY, like gdla_ref.py: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the GPU product path never does.

The pages train Motif 3 with GDLA layers and recompute each block's forward pass during the
backward pass (paperglide reader, section "Distributed Training System": activation recomputation);
they give no gradient formulas.  This module differentiates the forward of gdla_ref.py
(picx.dev summary section 2.2, Eq.(1)-(10), with the same readings) by the chain rule, one
equation at a time, in the reverse order of the forward:

    out = vec(Y) W_O                       Eq.(10)   -> dW_O, dY
    Y = sigmoid(G) (.) D                   Eq.(10)   -> dD, dG
    D_i = H_i - lambda_i H_(n_S + i mod n_N)   Eq.(8) -> dH (signal and noise), dlambda
    H_h = softmax(tau S_h) V                (two softmax maps, both kinds of head)
                                                     -> dq^C, dq^R, dK^C, dk^R, dV
    lambda = sigmoid(x W_lambda)           Eq.(7)
    [K^C ; V] = cbar [W_uk | W_uv]         Eq.(5)    -> dcbar, dW_uk, dW_uv
    cbar = RMSNorm(c^KV) gamma_KV          Eq.(4)
    k^R = RoPE(x W_kr)                     Eq.(3)
    q^C, q^R = c^Q W_qc, RoPE(c^Q W_qr)    Eq.(2);  G = c^Q W_gate  Eq.(9)
    c^Q = RMSNorm(x W_qa) gamma_Q          Eq.(1)

Softmax backward: with P = softmax(s) and dH = P V's upstream gradient, dP = dH V^T and
ds = P (.) (dP - rowsum(dP (.) P)); masked keys have P = 0 and so receive no gradient.  RoPE is a
rotation, so its backward rotates by the negative angle.  RMSNorm backward of y = v / r (.) gamma,
r = sqrt(mean(v^2) + eps): with u = dy (.) gamma, dv = u / r - v (sum_j u_j v_j) / (n r^3) and
dgamma = sum over rows of dy (.) v / r.

The reference is the loss L = sum(out (.) dout) for a given upstream gradient dout; every returned
gradient is dL/d(that input).  Only new-token sequences starting at position 0 are covered (a
training sequence), with the optional window and packed documents of the forward.

dH of every head is known before any head's map is evaluated (dY = dout W_O^T does not depend on
the maps; Eq.(8) routes it with lambda and sigmoid(G)), so each head's probability matrix is formed
once, used for its output and its gradients, and dropped: one T x T matrix at a time.  The heads are
independent, and gdla_backward can map them over worker processes (`map_fn`).
"""

import numpy as np

from oracle import gdla_ref as ref

__all__ = ["rms_norm_backward", "rope_backward", "head_attention_backward", "gdla_backward"]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def rms_norm_backward(v, gamma, dy, eps):
    """Gradient of y = v / sqrt(mean(v^2) + eps) (.) gamma over the last axis: returns (dv, dgamma);
    dgamma is None when gamma is None (a fixed gain of 1)."""
    v, dy = _f64(v), _f64(dy)
    n = v.shape[-1]
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    u = dy if gamma is None else dy * _f64(gamma)
    dv = u / r - v * np.sum(u * v, axis=-1, keepdims=True) / (n * r ** 3)
    dgamma = None if gamma is None else np.sum(dy * v / r, axis=tuple(range(v.ndim - 1)))
    return dv, dgamma


def rope_backward(du, pos, theta):
    """Gradient through RoPE: the transpose of a rotation is the rotation by the negative angle."""
    return ref.rope(du, -_f64(pos), theta)


def head_attention_backward(q_c, q_r, k_c, k_r, v, d_h, tau, pos, window, doc_start):
    """One head's softmax map, forward and backward, for queries and keys at positions `pos`:
    s = tau (q_c k_c^T + q_r k_r^T) on the visible (query, key) pairs, P = softmax(s) per row,
    H = P v; dP = d_h v^T, ds = P (.) (dP - rowsum(dP (.) P)).
    Returns (H, dq_c, dq_r, dk_c, dk_r, dv); the last three are this head's contributions to its KV
    head's K^C and V and to the shared rotary key."""
    hidden = ~ref.visible_mask(pos, pos, window, doc_start)
    s = q_c @ k_c.T
    s += q_r @ k_r.T
    s *= tau
    np.copyto(s, -np.inf, where=hidden)
    s -= np.max(s, axis=1, keepdims=True)
    p = np.exp(s, out=s)  # masked keys: exp(-inf) = 0
    p /= np.sum(p, axis=1, keepdims=True)
    h = p @ v
    ds = d_h @ v.T  # dP
    ds -= np.einsum("ij,ij->i", ds, p)[:, None]  # rowsum(dP (.) P)
    ds *= p
    return h, tau * ds @ k_c, tau * ds @ k_r, tau * ds.T @ q_c, tau * ds.T @ q_r, p.T @ d_h


def _head_task(args):
    return head_attention_backward(*args)


def gdla_backward(x, w, dims, dout, doc_start=None, lam_override=None, map_fn=map):
    """Gradients of L = sum(out (.) dout) for one sequence x [T, d_model] at positions 0..T-1.

    Returns a dict: dx [T, d_model]; dw_qa, dw_qc, dw_qr, dw_dkv, dw_kr, dw_uk, dw_uv, dw_lambda,
    dw_gate, dw_o (shaped like the weights); dgamma_q, dgamma_kv (None for fixed gains of 1); and
    the intermediate gradients dY, dH (per head), dlam, dq_c, dq_r, dk_c, dk_r, dv.
    map_fn(f, tasks) evaluates the heads' maps (in head order), e.g. a process pool's map.
    """
    x, dout = _f64(x), _f64(dout)
    t = x.shape[0]
    pos = np.arange(t)
    nh, ns, nn, nkv = dims.n_heads, dims.n_signal, dims.n_noise, dims.n_kv
    dh, dr, tau = dims.d_head, dims.d_rope, dims.scale
    W = {k: _f64(v) for k, v in w.items() if k.startswith("w_")}
    gq = None if w.get("gamma_q") is None else _f64(w["gamma_q"])
    gkv = None if w.get("gamma_kv") is None else _f64(w["gamma_kv"])

    # ---- forward, keeping what the backward needs (the recomputation)
    a_q = x @ W["w_qa"]
    c_q = ref.rms_norm(a_q, gq, dims.eps)                                        # Eq.(1)
    q_c = (c_q @ W["w_qc"]).reshape(t, nh, dh)                                   # Eq.(2)
    q_r = ref.rope((c_q @ W["w_qr"]).reshape(t, nh, dr), pos, dims.theta)
    g_logit = (c_q @ W["w_gate"]).reshape(t, ns, dh)                             # Eq.(9)
    c_kv = x @ W["w_dkv"]
    c_bar = ref.rms_norm(c_kv, gkv, dims.eps)                                    # Eq.(3), (4)
    k_r = ref.rope(x @ W["w_kr"], pos, dims.theta)
    k_c = (c_bar @ W["w_uk"]).reshape(t, nkv, dh)                                # Eq.(5)
    v = (c_bar @ W["w_uv"]).reshape(t, nkv, dh)
    lam = ref.sigmoid(x @ W["w_lambda"]) if lam_override is None else _f64(lam_override)  # Eq.(7)
    partner = np.arange(ns) % nn                                                 # Repeat_g tiles
    sg = ref.sigmoid(g_logit)

    # ---- Eq.(10): out = vec(Y) W_O and the gate; dY needs no head output
    d_y = (dout @ W["w_o"].T).reshape(t, ns, dh)
    d_d = d_y * sg

    # ---- Eq.(8): signal heads take dD, the noise head of pair i takes -lambda_i dD_i
    d_heads = np.zeros((t, nh, dh))
    d_heads[:, :ns] = d_d
    for i in range(ns):
        d_heads[:, ns + partner[i]] -= lam[:, i:i + 1] * d_d[:, i]

    # ---- the softmax maps of every head: outputs and gradients, one head at a time
    docs = None if doc_start is None else doc_start
    tasks = ((q_c[:, h], q_r[:, h], k_c[:, ref.kv_head_of(h, dims)], k_r, v[:, ref.kv_head_of(h, dims)],
              d_heads[:, h], tau, pos, dims.window, docs) for h in range(nh))
    heads = np.zeros((t, nh, dh))
    d_qc = np.zeros_like(q_c)
    d_qr = np.zeros_like(q_r)
    d_kc = np.zeros_like(k_c)
    d_kr = np.zeros_like(k_r)
    d_v = np.zeros_like(v)
    for h, (hh, dqc, dqr, dkc, dkr, dvv) in enumerate(map_fn(_head_task, tasks)):
        j = ref.kv_head_of(h, dims)
        heads[:, h] = hh
        d_qc[:, h] = dqc
        d_qr[:, h] = dqr
        d_kc[:, j] += dkc
        d_kr += dkr
        d_v[:, j] += dvv

    # ---- the terms that need the head outputs: Eq.(8) and (10) forward, dG, dlambda, dW_O
    h_s, h_n = heads[:, :ns], heads[:, ns:]
    d = h_s - lam[:, :, None] * h_n[:, partner]                                  # Eq.(8)
    y = sg * d                                                                   # Eq.(10)
    dw_o = y.reshape(t, ns * dh).T @ dout
    d_g = d_y * d * sg * (1.0 - sg)
    d_lam = -np.sum(d_d * h_n[:, partner], axis=2)

    # ---- Eq.(5), (4), (3): back into the latent and the rotary key
    dw_uk = c_bar.T @ d_kc.reshape(t, nkv * dh)
    dw_uv = c_bar.T @ d_v.reshape(t, nkv * dh)
    d_cbar = d_kc.reshape(t, nkv * dh) @ W["w_uk"].T + d_v.reshape(t, nkv * dh) @ W["w_uv"].T
    d_ckv, dgamma_kv = rms_norm_backward(c_kv, gkv, d_cbar, dims.eps)
    d_kr_pre = rope_backward(d_kr, pos, dims.theta)

    # ---- Eq.(2), (9), (1): back into the query latent
    d_qr_pre = rope_backward(d_qr, pos, dims.theta).reshape(t, nh * dr)
    d_qc_flat = d_qc.reshape(t, nh * dh)
    d_g_flat = d_g.reshape(t, ns * dh)
    dw_qc = c_q.T @ d_qc_flat
    dw_qr = c_q.T @ d_qr_pre
    dw_gate = c_q.T @ d_g_flat
    d_cq = d_qc_flat @ W["w_qc"].T + d_qr_pre @ W["w_qr"].T + d_g_flat @ W["w_gate"].T
    d_aq, dgamma_q = rms_norm_backward(a_q, gq, d_cq, dims.eps)

    # ---- Eq.(7): lambda (a fixed override receives no gradient path into x)
    d_lam_logit = d_lam * lam * (1.0 - lam) if lam_override is None else np.zeros_like(d_lam)

    # ---- x and the x-side weights
    dw_qa = x.T @ d_aq
    dw_dkv = x.T @ d_ckv
    dw_kr = x.T @ d_kr_pre
    dw_lambda = x.T @ d_lam_logit
    dx = (d_aq @ W["w_qa"].T + d_ckv @ W["w_dkv"].T + d_kr_pre @ W["w_kr"].T
          + d_lam_logit @ W["w_lambda"].T)
    return {"dx": dx, "dw_qa": dw_qa, "dw_qc": dw_qc, "dw_qr": dw_qr, "dw_dkv": dw_dkv,
            "dw_kr": dw_kr, "dw_uk": dw_uk, "dw_uv": dw_uv, "dw_lambda": dw_lambda,
            "dw_gate": dw_gate, "dw_o": dw_o, "dgamma_q": dgamma_q, "dgamma_kv": dgamma_kv,
            "dY": d_y, "dH": d_heads, "dlam": d_lam, "dq_c": d_qc, "dq_r": d_qr, "dk_c": d_kc,
            "dk_r": d_kr, "dv": d_v}
