"""GPU numerics beyond random N(0, 1) data: the online-softmax branches that random scores never
reach (a running maximum that jumps mid-sequence, a head whose every score underflows), NaN
propagation, operands near the edges of fp16's range, and training-scale upstream gradients.
Each case is compared with the fp64 oracle on the same inputs."""

import numpy as np
import pytest
import torch

import synth
import oracle
import attention_gdla_prefill_decode_amd as gd
from tests import harness as H

pytestmark = pytest.mark.gpu

BF = H.SMALL_BF16
LOG2E = 1.0 / np.log(2.0)


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- a jump of the running maximum
# A key whose rotary part k^R is multiplied by f moves every later query's score against it by up
# to f times its rotary part, so after two or more key tiles have been accumulated the running
# maximum jumps.  In the prefill the planted keys are cached prefix rows (exact bf16 inputs on both
# sides, so the large scores carry no rounding of their own); the backward takes no prefix, so
# there the keys are new tokens scaled by f (their latent and query pass an RMSNorm and do not
# change, their k^R is multiplied by f and rounded once into the bf16 cache, which is why the
# factors are smaller there: each score's rounding error grows with its size).
def _jump_fraction(inp, cfg, b, key, before, p0):
    """Fraction of (query, head) pairs, over the queries that see `key`, whose score against it
    exceeds their maximum over keys 0 .. before - 1 by more than 8 log2 units (the prefill kernel's
    rescale threshold), and the fraction where it does so by less than 24 (the earlier keys still
    weigh in)."""
    w = H.oracle_weights(inp)
    od = H.oracle_dims(cfg, 0)
    x = H.to_np(inp["x"][b])
    T = x.shape[0]
    pos = p0 + np.arange(T)
    _, q_c, q_r, _ = oracle.gdla_ref.query_path(x, w, od, pos)
    c_new, k_new = oracle.gdla_ref.latent_path(x, w, od, pos)
    rows = np.concatenate([c_new, k_new], axis=1)
    if p0 > 0:
        rows = np.concatenate([H.to_np(inp["cache"][b, :p0]), rows], axis=0)
    d_c = cfg["d_kv_latent"]
    k_c, _ = oracle.gdla_ref.expand_kv(rows[:, :d_c], w, od)
    tq = np.arange(max(0, key - p0), T)
    big, mid = [], []
    for h in range(cfg["n_heads"]):
        kv = oracle.gdla_ref.kv_head_of(h, od)
        s = (q_c[tq, h] @ k_c[:, kv].T + q_r[tq, h] @ rows[:, d_c:].T) * od.scale * LOG2E
        jump = s[:, key] - s[:, :before].max(axis=1)
        big.append(jump > 8.0)
        mid.append((jump > 8.0) & (jump < 24.0))
    return float(np.mean(big)), float(np.mean(mid))


def _check_heads(got, exp, what):
    """Per-head H (values of the size of V, unlike out): rel-L2 within 5e-3 and max-abs within
    2e-2 of the largest |H|."""
    max_abs, rel, rms = H.errors(got, exp)
    big = float(np.max(np.abs(exp)))
    msg = f"{what}: max-abs {max_abs:.3e} (max |ref| {big:.3e}), rel-L2 {rel:.3e}, ref RMS {rms:.3e}"
    assert rel <= 5e-3 and max_abs <= 2e-2 * big, msg
    return msg


def test_bf16_prefill_score_jump():
    """The lazy rescale of the prefill kernel (running maximum up by more than 2^8, accumulators
    already holding two or more key tiles) against the oracle: 200 new tokens after a 320-row
    prefix whose rows 150 (key tile 2) and 290 (key tile 4) have k^R multiplied by 16 and 32."""
    cfg, p0 = H.BF80, 320
    planted = ((150, 128, 16.0), (290, 256, 32.0))

    def prep(inp):
        for key, _, f in planted:
            inp["cache"][:, key, cfg["d_kv_latent"]:] *= f

    r = H.prefill_case(cfg, 200, [p0], seed=101, prep=prep, want_heads=True)
    for key, before, _ in planted:
        big, mid = _jump_fraction(r["inp"], cfg, 0, key, before, p0)
        _say(f"key {key}: {big:.2f} of (query, head) pairs jump by > 8 log2 units, {mid:.2f} by 8..24")
        assert big > 0.15 and mid > 0.1
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 prefill after score jumps"))
    _say(_check_heads(r["heads"], r["exp_heads"], "per-head H after score jumps"))


def test_fused_backward_score_jump():
    """Planted jumps through the fused backward (its forward recompute, the per-row log-sum-exp it
    returns and the probabilities the backward kernels rebuild from it): tokens 150 and 260 of 300
    scaled by 8 and 16."""
    cfg = H.BF80
    planted = ((150, 128, 8.0), (260, 256, 16.0))

    def prep(inp):
        for t, _, f in planted:
            inp["x"][:, t] *= f

    inp = synth.make_inputs(cfg, "cpu", seed=101, batch=1, seq=300, p0=0, random_gamma=True)
    prep(inp)
    for key, before, _ in planted:
        big, _ = _jump_fraction(inp, cfg, 0, key, before, 0)
        _say(f"key {key}: {big:.2f} of (query, head) pairs jump by > 8 log2 units")
        assert big > 0.05
    got, exp = H.backward_case(cfg, 300, 1, seed=101, prep=prep)
    for line in H.check_grads(got, exp, 1e-2, "fused backward after score jumps"):
        _say(line)


# ---------------------------------------------------------------- every score of a head underflows
def test_bf16_decode_underflow_redo():
    """All scores of one head about 2^-200 below the decode kernel's fixed reference: without the
    second pass against the exact maximum every probability of that head would be 0 and its
    output 0/0.  Ten heads (one head block) and 4001 keys over three key splits.  The rotary keys
    of the cached rows are set to k with q^R_h . k = -A for the chosen head h* and 0 for the other
    nine heads (ten equations in 64 unknowns), and W^KR is changed so that the new token's own
    rotary key does the same; the latent parts stay random, so the head still attends
    non-uniformly."""
    cfg = BF
    p0 = 4000
    hstar = 3
    A = 200.0  # log2 units

    def prep(inp):
        w = H.oracle_weights(inp)
        od = H.oracle_dims(cfg, 0)
        d_c = cfg["d_kv_latent"]
        x = H.to_np(inp["x"][0, 0])
        # rotated queries at the token's position, and unrotated ones (RoPE at the same position
        # cancels between the token's query and its own key)
        _, _, q_rot, _ = oracle.gdla_ref.query_path(x[None], w, od, np.array([p0]))
        _, _, q_un, _ = oracle.gdla_ref.query_path(x[None], w, od, np.array([0]))
        tgt = np.zeros(cfg["n_heads"])
        tgt[hstar] = -A / (od.scale * LOG2E)
        k_cache = np.linalg.lstsq(q_rot[0], tgt, rcond=None)[0]
        inp["cache"][0, :p0, d_c:] = torch.from_numpy(k_cache).to(inp["cache"].dtype)
        k_self = np.linalg.lstsq(q_un[0], tgt, rcond=None)[0]
        wkr = w["w_kr"]
        wkr = wkr + np.outer(x, k_self - x @ wkr) / float(x @ x)
        inp["weights"]["w_kr"] = torch.from_numpy(wkr).to(inp["weights"]["w_kr"].dtype)

    r = H.decode_case(cfg, [p0], seed=103, prep=prep, want_heads=True)
    # the planted scores, from the oracle's own paths on the rewritten inputs
    inp = synth.make_inputs(cfg, "cpu", seed=103, batch=1, seq=1, p0=[p0], random_gamma=True)
    prep(inp)
    w = H.oracle_weights(inp)
    od = H.oracle_dims(cfg, 0)
    x = H.to_np(inp["x"][0])
    _, q_c, q_r, _ = oracle.gdla_ref.query_path(x, w, od, np.array([p0]))
    c_bar, k_r = oracle.gdla_ref.latent_path(x, w, od, np.array([p0]))
    rows = np.concatenate([H.to_np(inp["cache"][0, :p0]), np.concatenate([c_bar, k_r], 1)], 0)
    k_c, _ = oracle.gdla_ref.expand_kv(rows[:, :cfg["d_kv_latent"]], w, od)
    top = []
    for h in range(cfg["n_heads"]):
        kv = oracle.gdla_ref.kv_head_of(h, od)
        s = (k_c[:, kv] @ q_c[0, h] + rows[:, cfg["d_kv_latent"]:] @ q_r[0, h]) * od.scale * LOG2E
        top.append(float(s.max()))
    _say("per-head maximum score (log2 units): " + ", ".join(f"{v:.1f}" for v in top))
    assert top[hstar] < -150.0 and max(top[:hstar] + top[hstar + 1:]) < 50.0
    assert np.all(np.isfinite(r["out"])) and np.all(np.isfinite(r["heads"]))
    _say(H.check(r["heads"][:, hstar], r["exp_heads"][:, hstar], "bf16", "the underflowing head's H"))
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 decode with an underflowing head"))


# ---------------------------------------------------------------- NaN propagation
def test_nan_input_propagates_prefill():
    """A NaN in one token's input reaches every output row that sees that token (its cache row
    becomes NaN) instead of being turned into finite values.  Rows whose key tiles end before the
    token's tile are unaffected and still match the oracle."""
    cfg, T, tn = H.BF80, 200, 130

    def prep(inp):
        inp["x"][0, tn, 7] = float("nan")

    r = H.prefill_case(cfg, T, [0], seed=107, prep=prep, rows=np.arange(128))
    out = r["out_all"][0]
    assert not np.isfinite(out[tn:]).any(), "rows that see the NaN token must not be finite"
    assert np.isnan(H.to_np(r["dev"]["cache"][0, tn])).any(), "the NaN token's cache row"
    _say(H.check(r["out"], r["exp_out"], "bf16", "rows before the NaN token's key tile"))


def test_nan_input_propagates_decode():
    """A NaN in one sequence's new token makes that sequence's output non-finite; the other
    sequences of the batch are untouched and match the oracle."""
    cfg = H.BF80
    p0 = [300, 1200, 64]

    def prep(inp):
        inp["x"][1, 0, 5] = float("nan")

    inp = synth.make_inputs(cfg, "cpu", seed=109, batch=3, seq=1, p0=p0, random_gamma=True)
    prep(inp)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    out = H.to_np(gd.gdla_decode(dims, dev["wstruct"], dev["x"][:, 0].contiguous(), p0, dev["cache"]))
    torch.cuda.synchronize()
    assert not np.isfinite(out[1]).any()
    w = H.oracle_weights(inp)
    od = H.oracle_dims(cfg, 0)
    keep = [0, 2]
    exp = oracle.gdla_ref.gdla_decode(H.to_np(inp["x"][keep, 0]), w, od,
                                      [H.to_np(inp["cache"][b, :p0[b]]) for b in keep], [p0[b] for b in keep])
    _say(H.check(out[keep], exp["out"], "bf16", "decode rows of the other sequences"))


# ---------------------------------------------------------------- operands far from unit scale
# Powers of two that cancel in exact arithmetic: x * 2^5 with W^KR, W^lambda / 2^5 (the RMSNorms
# absorb the rest of x's scale); gamma_Q * 2^6 with W^QC, W^QR, W^G / 2^6; W^UV * 2^6 with
# W^O / 2^6.  Inside the fp16 path c^Q and V then reach a few hundred while the query-side and
# output weights sit low in fp16's normal range (their typical size about 2^-11, the smallest normal
# 2^-14).  fp16 rounding is relative, so the result must match the oracle on the same scaled
# inputs as closely as at unit scale.  (Shrinking weights much further would leave them among
# fp16's subnormals, whose absolute spacing of 2^-24 no longer keeps 11 significant bits.)
def _scale_layer(inp):
    inp["x"].mul_(2.0 ** 5)
    for k in ("w_kr", "w_lambda"):
        inp["weights"][k].mul_(2.0 ** -5)
    inp["gamma_q"].mul_(2.0 ** 6)
    for k in ("w_qc", "w_qr", "w_gate"):
        inp["weights"][k].mul_(2.0 ** -6)
    inp["weights"]["w_uv"].mul_(2.0 ** 6)
    inp["weights"]["w_o"].mul_(2.0 ** -6)


@pytest.mark.parametrize("cfg,T,p0,window", [(H.BF80, 300, [0], 0), (BF, 260, [40, 0], 64)],
                         ids=["80h", "10h-window"])
def test_large_operands_prefill(cfg, T, p0, window):
    r = H.prefill_case(cfg, T, p0, window=window, seed=113, prep=_scale_layer)
    _say(H.check(r["out"], r["exp_out"], "bf16", f"prefill with operands scaled by powers of two, {cfg['n_heads']} heads"))


def test_large_operands_decode():
    r = H.decode_case(H.BF80, [0, 700, 2047], seed=113, prep=_scale_layer)
    _say(H.check(r["out"], r["exp_out"], "bf16", "decode with operands scaled by powers of two"))


def test_fp16_overflow_is_not_silent():
    """Values beyond fp16's range in the prefill's fp16 operands (V from W^UV * 2^17, about 10^5)
    become infinities, so the output is not finite, rather than saturating to finite wrong values."""
    def prep(inp):
        inp["weights"]["w_uv"].mul_(2.0 ** 17)

    r = H.prefill_case(H.BF80, 300, [0], seed=127, prep=prep)
    assert np.all(np.isfinite(r["exp_out"]))
    assert not np.all(np.isfinite(r["out"])), "an fp16 overflow must surface as a non-finite output"


# ---------------------------------------------------------------- training-scale gradients
@pytest.mark.parametrize("dout_scale", [1e-4, 1e-6, 1e3])
def test_fused_backward_gradient_scale(dout_scale):
    """Upstream gradients far from unit scale (1e-4 and 1e-6 sit in or below fp16's subnormal
    range once multiplied through the layer) through the fused backward, whose fp16 operands are
    scaled by a power of two computed from the largest |dout| on the device."""
    got, exp = H.backward_case(BF, 300, 1, seed=117, dout_scale=dout_scale)
    for line in H.check_grads(got, exp, 1e-2, f"fused backward, dout x {dout_scale:g}"):
        _say(line)
