"""Brute-force GDLA layer in 50-digit arithmetic with explicit scalar loops (tiny shapes only).

Independent of the oracle: no NumPy, no shared helpers.  It evaluates the equations of the
picx.dev summary of the Motif 3 Technical Report, section 2.2, Eq.(1)-(10), element by element,
with the same readings the oracle documents (signal heads first, tiled Repeat_g, KV head
i mod n_KV, rotate-half RoPE, scale 1/sqrt(d_head + d_rope), visibility s <= p and p - s < W).
"""

import mpmath

mpmath.mp.dps = 50
mpf = mpmath.mpf


def _mat(a):
    """Nested lists of mpf from anything indexable (array, tensor or list)."""
    return [[mpf(float(v)) for v in row] for row in a]


def _vec(a):
    return [mpf(float(v)) for v in a]


def _matvec(v, w):  # row vector times matrix w[in][out]
    n_out = len(w[0])
    return [mpmath.fsum(v[i] * w[i][o] for i in range(len(v))) for o in range(n_out)]


def _rms(v, gamma, eps):
    r = mpmath.sqrt(mpmath.fsum(e * e for e in v) / len(v) + eps)
    return [v[i] / r * (gamma[i] if gamma is not None else 1) for i in range(len(v))]


def _rope(u, p, theta):
    d = len(u)
    half = d // 2
    out = [mpf(0)] * d
    for j in range(half):
        ang = p * mpmath.power(theta, mpf(-2 * j) / d)
        c, s = mpmath.cos(ang), mpmath.sin(ang)
        out[j] = u[j] * c - u[j + half] * s
        out[j + half] = u[j] * s + u[j + half] * c
    return out


def _sig(z):
    return 1 / (1 + mpmath.exp(-z))


def brute_gdla(x, w, n_signal, n_noise, n_kv, d_head, d_rope, window=0, eps=1e-6,
               theta=10000.0, prefix=None, p0=0, lam_override=None, doc_start=None):
    """Returns (out [T][d_model], heads [T][n_H][d_head]) as nested lists of mpf.  doc_start[t]
    (optional) is the first position of token t's document: keys before it are not visible."""
    n_heads = n_signal + n_noise
    g = n_signal // n_noise
    eps, theta = mpf(eps), mpf(theta)
    tau = 1 / mpmath.sqrt(d_head + d_rope)
    W = {k: _mat(v) for k, v in w.items() if k.startswith("w_")}
    gq = _vec(w["gamma_q"]) if w.get("gamma_q") is not None else None
    gkv = _vec(w["gamma_kv"]) if w.get("gamma_kv") is not None else None
    xs = _mat(x)
    T = len(xs)
    rows_c, rows_r = [], []
    if p0 > 0:
        pre = _mat(prefix)
        d_c = len(W["w_dkv"][0])
        for r in pre:
            rows_c.append(r[:d_c])
            rows_r.append(r[d_c:])
    qc, qr, gate, lam = [], [], [], []
    for t in range(T):
        p = p0 + t
        cq = _rms(_matvec(xs[t], W["w_qa"]), gq, eps)
        qcf = _matvec(cq, W["w_qc"])
        qrf = _matvec(cq, W["w_qr"])
        qc.append([qcf[h * d_head:(h + 1) * d_head] for h in range(n_heads)])
        qr.append([_rope(qrf[h * d_rope:(h + 1) * d_rope], p, theta) for h in range(n_heads)])
        gf = _matvec(cq, W["w_gate"])
        gate.append([gf[i * d_head:(i + 1) * d_head] for i in range(n_signal)])
        rows_c.append(_rms(_matvec(xs[t], W["w_dkv"]), gkv, eps))
        rows_r.append(_rope(_matvec(xs[t], W["w_kr"]), p, theta))
        if lam_override is None:
            lam.append([_sig(z) for z in _matvec(xs[t], W["w_lambda"])])
        else:
            lam.append([mpf(float(v)) for v in lam_override[t]])
    L = len(rows_c)
    kc = [_matvec(rows_c[s], W["w_uk"]) for s in range(L)]
    vv = [_matvec(rows_c[s], W["w_uv"]) for s in range(L)]
    heads = []
    for t in range(T):
        p = p0 + t
        first = 0 if doc_start is None else doc_start[t]
        vis = [s for s in range(L) if first <= s <= p and (window == 0 or p - s < window)]
        ht = []
        for h in range(n_heads):
            j = (h % n_kv) if h < n_signal else ((h - n_signal) % n_kv)
            sc = []
            for s in vis:
                dot = mpmath.fsum(qc[t][h][e] * kc[s][j * d_head + e] for e in range(d_head))
                dot += mpmath.fsum(qr[t][h][e] * rows_r[s][e] for e in range(d_rope))
                sc.append(tau * dot)
            m = max(sc)
            ex = [mpmath.exp(v - m) for v in sc]
            z = mpmath.fsum(ex)
            ht.append([mpmath.fsum(ex[k] / z * vv[s][j * d_head + e] for k, s in enumerate(vis))
                       for e in range(d_head)])
        heads.append(ht)
    out = []
    for t in range(T):
        y = []
        for i in range(n_signal):
            nz = heads[t][n_signal + (i % n_noise)]
            for e in range(d_head):
                dval = heads[t][i][e] - lam[t][i] * nz[e]
                y.append(_sig(gate[t][i][e]) * dval)
        out.append(_matvec(y, W["w_o"]))
    return out, heads
