"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that the pins catch
every one of them: a dropped term, a wrong sign, a wrong index or pairing, a transposed or swapped
operand, an off-by-one mask, a missing scale or normalisation."""

import os
import types

import pytest

from tests.oracle_pins import ALL_PINS, GRAD_VALUE_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "gdla_ref.py")

MUTATIONS = {
    "drop_rotary_score_term": ("s = dims.scale * (q_c[t0:t1, h] @ k_c[lo:hi, j].T + q_r[t0:t1, h] @ k_r[lo:hi].T)",
                               "s = dims.scale * (q_c[t0:t1, h] @ k_c[lo:hi, j].T)"),
    "combine_sign": ("return h_s - _f64(lam)", "return h_s + _f64(lam)"),
    "repeat_interleaved": ("return np.tile(h_noise, reps)", "return np.repeat(h_noise, g, axis=-2)"),
    "missing_scale": ("s = dims.scale * (q_c[t0:t1, h]", "s = (q_c[t0:t1, h]"),
    "window_off_by_one": ("m &= (p - s) < window", "m &= (p - s) <= window"),
    "signal_kv_contiguous": ("return h % dims.n_kv", "return (h // dims.g) % dims.n_kv"),
    "noise_kv_contiguous": ("return (h - dims.n_signal) % dims.n_kv",
                            "return ((h - dims.n_signal) * dims.n_kv) // dims.n_noise"),
    "rmsnorm_sum": ("np.mean(v * v, axis=-1, keepdims=True)", "np.sum(v * v, axis=-1, keepdims=True)"),
    "gate_without_sigmoid": ("return sigmoid(gate_logits) * _f64(d)", "return _f64(gate_logits) * _f64(d)"),
    "value_from_key_weights": ('v = (c_bar @ _f64(w["w_uv"]))', 'v = (c_bar @ _f64(w["w_uk"]))'),
    "rope_sign": ("a * s + b * c], axis=-1)", "b * c - a * s], axis=-1)"),
    "key_not_rotated": ('k_r = rope(x @ _f64(w["w_kr"]), pos, dims.theta)', 'k_r = x @ _f64(w["w_kr"])'),
    "causal_excludes_self": ("m = s <= p", "m = s < p"),
    "lambda_not_sigmoid": ('return sigmoid(_f64(x) @ _f64(w["w_lambda"]))', 'return _f64(x) @ _f64(w["w_lambda"])'),
    "gamma_ignored": ("return r if gamma is None else r * _f64(gamma)", "return r"),
    "absorbed_wrong_value_proj": ("out[t0:t1, h] = o @ w_uv[:, j * dh:(j + 1) * dh]",
                                  "out[t0:t1, h] = o @ w_uk[:, j * dh:(j + 1) * dh]"),
    "document_mask_ignored": ("m &= s >= np.asarray(qdoc)[:, None]", "pass"),
    "document_off_by_one": ("m &= s >= np.asarray(qdoc)[:, None]", "m &= s > np.asarray(qdoc)[:, None]"),
    "document_key_range_from_last_row": ("lo = max(lo, int(np.min(qdoc)))", "lo = max(lo, int(np.max(qdoc)))"),
}


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("gdla_ref_mutant")
    exec(compile(src.replace(old, new), "gdla_ref_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # any failure of a pin counts as catching the mistake
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"planted mistake {name} escaped every pin"


GRAD_SRC = os.path.join(os.path.dirname(SRC), "gdla_grad.py")

GRAD_MUTATIONS = {
    "softmax_backward_no_rowsum": ("    ds -= np.einsum(\"ij,ij->i\", ds, p)[:, None]  # rowsum(dP (.) P)\n", ""),
    "rope_backward_same_angle": ("return ref.rope(du, -_f64(pos), theta)", "return ref.rope(du, _f64(pos), theta)"),
    "rms_backward_first_term_only": ("dv = u / r - v * np.sum(u * v, axis=-1, keepdims=True) / (n * r ** 3)", "dv = u / r"),
    "lambda_grad_sign": ("d_lam = -np.sum(d_d * h_n[:, partner], axis=2)", "d_lam = np.sum(d_d * h_n[:, partner], axis=2)"),
    "noise_grad_missing": ("d_heads[:, ns + partner[i]] -= lam[:, i:i + 1] * d_d[:, i]", "pass"),
    "gate_grad_without_sigmoid_slope": ("d_g = d_y * d * sg * (1.0 - sg)", "d_g = d_y * d"),
    "shared_rotary_key_grad_last_head_only": ("d_kr += dkr", "d_kr = dkr"),
    "value_grad_transposed": ("tau * ds.T @ q_r, p.T @ d_h", "tau * ds.T @ q_r, p @ d_h"),
}


def _grad_mutant(old, new):
    with open(GRAD_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("gdla_grad_mutant")
    exec(compile(src.replace(old, new), "gdla_grad_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(GRAD_MUTATIONS))
def test_planted_backward_mistake_is_caught(name):
    mod = _grad_mutant(*GRAD_MUTATIONS[name])
    caught = []
    for pin in GRAD_VALUE_PINS:
        try:
            pin(mod)
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"planted mistake {name} escaped every backward pin"
