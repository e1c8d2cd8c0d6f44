"""GPU parity of the GDLA library against the fp64 oracle, element by element, at sizes the
oracle finishes in seconds (several tiles and a ragged tail), plus GPU-side invariants."""

import numpy as np
import pytest
import torch

import synth
import oracle
import attention_gdla_prefill_decode_amd as gd
from tests import harness as H

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny_fp32"]
BF = H.SMALL_BF16


def setup_module(module):
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- fp32 (tolerance 1e-5)
def test_tiny_fp32_prefill_full():
    r = H.prefill_case(TINY, 128, [0], random_gamma=False)
    _say(H.check(r["out"], r["exp_out"], "f32", "tiny fp32 T=128"))
    H.check_rows(r["rows"][0], r["exp_rows"][0], "f32", "tiny fp32 cache rows")


@pytest.mark.parametrize("seq,p0,window", [
    (37, [0, 11], 0), (50, [20], 16), (7, [0], 1), (64, [3, 0, 60], 5), (1, [0], 0), (1, [90], 0),
    (100, [0], 200),
])
def test_fp32_prefill_variants(seq, p0, window):
    r = H.prefill_case(TINY, seq, p0, window=window, seed=13)
    _say(H.check(r["out"], r["exp_out"], "f32", f"fp32 T={seq} p0={p0} W={window}"))
    for b in range(len(p0)):
        H.check_rows(r["rows"][b], r["exp_rows"][b], "f32", "fp32 cache rows")


def test_fp32_heads_debug_output():
    r = H.prefill_case(TINY, 40, [9], window=12, want_heads=True)
    err = np.max(np.abs(r["heads"] - r["exp_heads"]))
    assert err <= 1e-5, err


def test_fp32_decode():
    r = H.decode_case(TINY, [0, 5, 127, 64], want_heads=True)
    _say(H.check(r["out"], r["exp_out"], "f32", "fp32 decode"))
    assert np.max(np.abs(r["heads"] - r["exp_heads"])) <= 1e-5
    H.check_rows(r["rows"], r["exp_rows"], "f32", "fp32 decode cache rows")


# ---------------------------------------------------------------- bf16 (2e-2 / 5e-3)
@pytest.mark.parametrize("seq,p0,window", [
    (300, [0], 0), (200, [0, 77], 0), (257, [5], 64), (129, [0], 1), (64, [40], 100000),
])
def test_bf16_prefill(seq, p0, window):
    r = H.prefill_case(BF, seq, p0, window=window, seed=17)
    _say(H.check(r["out"], r["exp_out"], "bf16", f"bf16 T={seq} p0={p0} W={window}"))
    for b in range(len(p0)):
        H.check_rows(r["rows"][b], r["exp_rows"][b], "bf16", "bf16 cache rows")


# A layer with the full query latent (d_cq 1024): A2 runs on the row-wise kernel (one wave per token
# row) rather than the general one; its cache rows and outputs against the oracle, in prefill (T =
# 300, so the query-side latent leaves in fp16 for the transposed-weight GEMM, and T = 40 on the
# general GEMMs) and in decode (latent with its bf16 remainder for the skinny projections).
BF_CQ1024 = dict(BF, d_q_latent=1024)


@pytest.mark.parametrize("seq,p0", [(300, [0]), (40, [3, 0])])
def test_bf16_prefill_full_query_latent(seq, p0):
    r = H.prefill_case(BF_CQ1024, seq, p0, seed=41)
    _say(H.check(r["out"], r["exp_out"], "bf16", f"bf16 d_cq 1024 T={seq} p0={p0}"))
    for b in range(len(p0)):
        H.check_rows(r["rows"][b], r["exp_rows"][b], "bf16", "bf16 d_cq 1024 cache rows")


def test_bf16_decode_full_query_latent():
    r = H.decode_case(BF_CQ1024, [50, 0, 17], seed=43)
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 d_cq 1024 decode"))
    H.check_rows(r["rows"], r["exp_rows"], "bf16", "bf16 d_cq 1024 decode cache rows")


def test_bf16_prefill_odd_signal_heads():
    # 12 signal heads: the lambda projection's 12 columns cannot leave the transposed-weight GEMM
    # as 16-byte segments and go to the general GEMM (>= 256 rows take the transposed path)
    cfg = dict(BF, n_heads=16, n_signal=12, n_noise=4, n_kv=4)
    r = H.prefill_case(cfg, 288, [0], seed=23)
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 12+4 heads T=288"))


def test_bf16_prefill_many_short_sequences():
    # 12 sequences of 24 tokens: >= 256 rows but sequences shorter than 32 (no RoPE epilogue)
    r = H.prefill_case(BF, 24, [0, 3, 10, 0, 1, 7, 30, 2, 0, 5, 9, 4], seed=31)
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 12 x 24 tokens"))
    for b in range(12):
        H.check_rows(r["rows"][b], r["exp_rows"][b], "bf16", "bf16 cache rows")


def test_bf16_heads_debug_output():
    r = H.prefill_case(BF, 160, [0], want_heads=True)
    _say(H.check(r["heads"], r["exp_heads"], "bf16", "bf16 per-head H"))


@pytest.mark.parametrize("cfg,p0", [
    (H.BF80, [0, 700, 2047]), (H.BF72, [3000, 5]), (dict(H.BF80, window=1000), [2500, 40, 999]),
    (dict(H.BF72, window=64), [63, 64, 1300]),
], ids=["80h", "72h", "80h-window", "72h-window64"])
def test_bf16_decode_wide(cfg, p0):
    r = H.decode_case(cfg, p0, seed=23, want_heads=True)
    _say(H.check(r["out"], r["exp_out"], "bf16", f"bf16 decode {cfg['n_heads']} heads p0={p0}"))
    _say(H.check(r["heads"], r["exp_heads"], "bf16", "per-head H"))


def _max_logit_log2(inp, cfg, b, keys):
    """Largest scaled score (log2 units) of any head of sequence b over the given cache rows."""
    w = H.oracle_weights(inp)
    od = H.oracle_dims(cfg, cfg.get("window", 0))
    p = inp["p0"][b]
    _, q_c, q_r, _ = oracle.gdla_ref.query_path(H.to_np(inp["x"][b:b + 1, 0]), w, od, np.array([p]))
    rows = H.to_np(inp["cache"][b, keys])
    d_c = cfg["d_kv_latent"]
    best = -np.inf
    for h in range(cfg["n_heads"]):
        kv = oracle.gdla_ref.kv_head_of(h, od)
        w_uk = w["w_uk"][:, kv * cfg["d_head"]:(kv + 1) * cfg["d_head"]]
        s = rows[:, :d_c] @ (w_uk @ q_c[0, h]) + rows[:, d_c:] @ q_r[0, h]
        best = max(best, float(np.max(s)) * od.scale / np.log(2.0))
    return best


def test_bf16_decode_score_jump_recomputes_split():
    """Keys far above the first tile's maximum (more than 2^64 in probability) force the
    second pass against the exact maximum; the result must still match the oracle.  The later
    keys all repeat one row, so their scores tie and bf16 rounding cannot tip the balance, and
    only its k^R part is scaled up, which raises the scores but leaves the values (cbar) alone."""
    p0 = 900  # one key split
    d_c = H.BF80["d_kv_latent"]

    def prep(inp):
        cache = inp["cache"]
        cache[0, :64] = 0  # first tile: every score exactly 0
        row = cache[0, 64].clone().double()
        for _ in range(4):  # scale k^R until some head scores about 80 (log2 units)
            cache[0, 64] = row.to(cache.dtype)
            top = _max_logit_log2(inp, H.BF80, 0, slice(64, 65))
            if top > 75.0:
                break
            row[d_c:] *= max(2.0, 80.0 / max(top, 0.5))
        cache[0, 64:p0] = row.to(cache.dtype)
        assert _max_logit_log2(inp, H.BF80, 0, slice(64, 65)) > 70.0

    r = H.decode_case(H.BF80, [p0], seed=29, prep=prep)
    assert np.all(np.isfinite(r["out"]))
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 decode after a score jump"))


@pytest.mark.parametrize("p0", [[0, 1, 300, 1000], [4095]])
def test_bf16_decode(p0):
    r = H.decode_case(BF, p0, want_heads=True)
    _say(H.check(r["out"], r["exp_out"], "bf16", f"bf16 decode p0={p0}"))
    _say(H.check(r["heads"], r["exp_heads"], "bf16", "bf16 decode per-head H"))
    H.check_rows(r["rows"], r["exp_rows"], "bf16", "bf16 decode cache rows")


def test_bf16_decode_batch_over_64():
    # 72 sequences: the skinny projection kernel's second row block holds 8 rows
    r = H.decode_case(BF, [(37 * b) % 500 for b in range(72)], seed=41)
    _say(H.check(r["out"], r["exp_out"], "bf16", "bf16 decode B=72"))
    H.check_rows(r["rows"], r["exp_rows"], "bf16", "bf16 decode cache rows")


# ---------------------------------------------------------------- multi-token decode
# T draft tokens per sequence on the absorbed path (token i at position p0 + i sees the cache and
# tokens 0..i), against the oracle's one-call forward over the same T tokens.
@pytest.mark.parametrize("T,p0,window", [(3, [0, 5, 120], 0), (2, [64], 0), (16, [40], 0), (4, [90, 7], 9)])
def test_fp32_decode_tokens(T, p0, window):
    r = H.prefill_case(TINY, T, p0, window=window, seed=29, want_heads=True, entry="decode_tokens")
    _say(H.check(r["out"], r["exp_out"], "f32", f"fp32 decode_tokens T={T} p0={p0} W={window}"))
    err = float(np.max(np.abs(r["heads"] - r["exp_heads"])))
    assert err <= 1e-5, f"per-head H max-abs {err:.3e}"
    for b in range(len(p0)):
        H.check_rows(r["rows"][b], r["exp_rows"][b], "f32", "fp32 cache rows")


@pytest.mark.parametrize("cfg,T,p0", [
    (BF, 2, [0, 33, 1000]),            # ten heads (one head block), first token at position 0
    (BF, 4, [4095, 31, 64]),           # tokens across a tile boundary
    (H.BF80, 4, [0, 700, 2047]),       # five head blocks, the fifth shared
    (H.BF72, 3, [3000, 5]),            # partly filled fifth block
    (dict(H.BF80, window=1000), 4, [2500, 40, 998]),  # window edge inside the draft
    (BF, 16, [100, 4, 300, 50]),       # 64 query rows (one row block of the skinny projection)
    (BF, 5, [10] * 13),                # 65 query rows (a second row block of one row)
    (BF, 16, [3 * b for b in range(17)]),  # 272 query rows (general projection GEMM)
])
def test_bf16_decode_tokens(cfg, T, p0):
    r = H.prefill_case(cfg, T, p0, window=cfg.get("window", 0), seed=31, want_heads=True,
                       entry="decode_tokens")
    _say(H.check(r["out"], r["exp_out"], "bf16", f"bf16 decode_tokens n_H={cfg['n_heads']} T={T}"))
    H.check(r["heads"], r["exp_heads"], "bf16", "per-head H")
    for b in range(len(p0)):
        H.check_rows(r["rows"][b], r["exp_rows"][b], "bf16", "bf16 cache rows")


def test_decode_tokens_matches_decode_and_prefill():
    """T = 1 is gdla_decode bit for bit; T = 4 agrees with gdla_prefill of the same tokens."""
    cfg = H.BF80
    inp = synth.make_inputs(cfg, "cpu", batch=3, seq=4, p0=[500, 9, 1999], random_gamma=True)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    c1, c2 = dev["cache"].clone(), dev["cache"].clone()
    one = gd.gdla_decode(dims, dev["wstruct"], dev["x"][:, 0].contiguous(), inp["p0"], c1)
    tok = gd.gdla_decode_tokens(dims, dev["wstruct"], dev["x"][:, :1].contiguous(), inp["p0"], c2)
    torch.cuda.synchronize()
    assert torch.equal(one, tok[:, 0]) and torch.equal(c1, c2)
    c3, c4 = dev["cache"].clone(), dev["cache"].clone()
    pre = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], c3)
    dec = gd.gdla_decode_tokens(dims, dev["wstruct"], dev["x"], inp["p0"], c4)
    torch.cuda.synchronize()
    _say(H.check(H.to_np(dec), H.to_np(pre), "bf16", "decode_tokens vs prefill"))
    for bi, p in enumerate(inp["p0"]):  # the same rows, up to the projection GEMMs' rounding
        H.check_rows(H.to_np(c4[bi, p:p + 4]), H.to_np(c3[bi, p:p + 4]), "bf16", "appended rows")


# ---------------------------------------------------------------- packed documents
@pytest.mark.parametrize("cfg,T,p0,window,lens,first", [
    (BF, 300, [0], 0, (37, 113, 150), None),          # document edges inside query blocks and tiles
    (BF, 200, [0, 77], 40, (1, 64, 135), None),       # a one-token document; window inside documents
    (BF, 160, [300], 0, (100, 60), 120),              # the first document began in the cached prefix
    (H.BF80, 130, [0], 0, (65, 65), None),
    (TINY, 70, [0, 9], 12, (20, 3, 47), None),        # fp32 generic path
])
def test_packed_prefill(cfg, T, p0, window, lens, first):
    docs = [H.doc_starts(p, lens, first) for p in p0]
    r = H.prefill_case(cfg, T, p0, window=window, seed=47, want_heads=True, docs=docs)
    dt = cfg["dtype"]
    _say(H.check(r["out"], r["exp_out"], dt, f"packed prefill {dt} lens={lens} W={window}"))
    if dt == "f32":
        err = float(np.max(np.abs(r["heads"] - r["exp_heads"])))
        assert err <= 1e-5, f"per-head H max-abs {err:.3e}"
    else:
        H.check(r["heads"], r["exp_heads"], dt, "per-head H")


def test_packed_prefill_single_document_is_prefill():
    """One document from position 0 masks nothing: bit for bit the plain prefill."""
    inp = synth.make_inputs(BF, "cpu", batch=2, seq=150, p0=[0, 40], random_gamma=True, seed=53)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(BF, window=70)
    c2 = dev["cache"].clone()
    ref_out = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"])
    zero = torch.zeros((2, 150), dtype=torch.int32, device="cuda")
    out = gd.gdla_prefill_packed(dims, dev["wstruct"], dev["x"], inp["p0"], zero, c2)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)


# ---------------------------------------------------------------- backward
# The general backward path recomputes the forward and runs every step in fp32 from the stored
# (fp32 or bf16) values, which the oracle reads exactly: fp32 rounding alone, 1e-5 relative.
@pytest.mark.parametrize("cfg,T,batch,window,lens", [
    (TINY, 40, 2, 0, None),
    (TINY, 33, 1, 7, (10, 1, 22)),
    (BF, 64, 1, 0, None),
    (BF, 70, 2, 20, (30, 40)),
])
def test_backward_matches_oracle(cfg, T, batch, window, lens):
    docs = None if lens is None else [H.doc_starts(0, lens) for _ in range(batch)]
    got, exp = H.backward_case(cfg, T, batch, window=window, docs=docs, seed=67)
    for line in H.check_grads(got, exp, 1e-5, f"backward {cfg['dtype']} T={T} W={window}"):
        _say(line)


# With at least 256 rows the backward runs fused: fp16 MFMA operands (gradients, activations and
# weights each rounded once to fp16, 2^-11 relative), fp32 accumulation, on top of the forward's
# own roundings (bf16 cache rows, 2^-9).  The deepest gradients pass about eight such roundings:
# about 2.3e-3 in quadrature, so 1e-2 leaves a factor of four.
# The short cases put one token, or a ragged 13, in each sequence's last 32-query block, with
# the transposed copies of q and dH padded per sequence.
@pytest.mark.parametrize("cfg,T,batch,window,lens", [
    (BF, 300, 1, 0, None),
    (BF, 160, 2, 20, (37, 90, 33)),
    (H.BF80, 256, 1, 0, None),
    (H.BF72, 270, 1, 64, (200, 70)),
    (BF, 33, 8, 0, None),
    (BF, 45, 6, 12, (20, 25)),
])
def test_backward_fused_matches_oracle(cfg, T, batch, window, lens):
    docs = None if lens is None else [H.doc_starts(0, lens) for _ in range(batch)]
    got, exp = H.backward_case(cfg, T, batch, window=window, docs=docs, seed=73)
    for line in H.check_grads(got, exp, 1e-2, f"fused backward n_H={cfg['n_heads']} T={T} W={window}"):
        _say(line)


# Enough tokens that the weight-gradient products are split along the token axis (8192 rows: up
# to 8 slices of 1024; 4096 rows: up to 4), summed in order, on the fused path; with a window, and
# with packed documents (a one-token document among them).
@pytest.mark.parametrize("batch,window,lens", [(4, 300, None), (2, 0, (700, 1, 900, 447))])
def test_backward_fused_split_k(batch, window, lens):
    docs = None if lens is None else [H.doc_starts(0, lens) for _ in range(batch)]
    got, exp = H.backward_case(BF, 2048, batch, window=window, docs=docs, seed=79)
    for line in H.check_grads(got, exp, 1e-2, f"fused backward, {batch} x 2048 tokens (split-K products)"):
        _say(line)


# Every gradient has one writer and the K slices are summed in order: repeated calls (fused path
# with split products, and the general path) give identical bits.
@pytest.mark.parametrize("cfg,T,batch", [(BF, 2048, 2), (BF, 64, 1)])
def test_backward_is_deterministic(cfg, T, batch):
    inp = synth.make_inputs(cfg, "cpu", seed=83, batch=batch, seq=T, p0=0, random_gamma=True)
    gen = torch.Generator().manual_seed(84)
    dout = torch.randn((batch, T, cfg["d_model"]), generator=gen).to(inp["x"].dtype).to("cuda")
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    tensors = dict(dev["weights"], gamma_q=dev["gamma_q"], gamma_kv=dev["gamma_kv"])
    first = gd.gdla_backward(dims, dev["wstruct"], tensors, dev["x"], dout)
    first = {k: v.clone() for k, v in first.items()}
    second = gd.gdla_backward(dims, dev["wstruct"], tensors, dev["x"], dout)
    torch.cuda.synchronize()
    for k in first:
        assert torch.equal(first[k], second[k]), f"backward {k} differs between two calls"


def test_backward_lambda_zero():
    got, exp = H.backward_case(BF, 48, 1, seed=71, lam_zero=True)
    H.check_grads(got, exp, 1e-5, "backward, lambda = 0")
    assert float(np.max(np.abs(got["dw_lambda"]))) == 0.0


# ---------------------------------------------------------------- paged latent cache
# The same calls over a shuffled pool of pages: the kernels read and write exactly the rows of the
# contiguous layout, so the outputs must equal the contiguous path's bit for bit (windowed decode
# excepted: its paged tiles are aligned to the pages, so the sums run in another order), and the
# rows written through the block table must land in the right pages.
@pytest.mark.parametrize("cfg,T,p0,page_rows", [
    (H.BF80, 1, [0, 700, 2047], 64),
    (H.BF80, 4, [31, 1000, 2], 32),
    (dict(H.BF80, window=1000), 3, [2500, 40, 998], 96),
    (TINY, 2, [0, 50, 127], 32),
])
def test_paged_decode_matches_contiguous(cfg, T, p0, page_rows):
    dt = cfg["dtype"]
    inp = synth.make_inputs(cfg, "cpu", batch=len(p0), seq=T, p0=p0, random_gamma=True, seed=37)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg, window=cfg.get("window", 0))
    B, L = dev["cache"].shape[0], dev["cache"].shape[1]
    pc = H.to_pages(dev["cache"], page_rows, seed=5)
    ref = gd.gdla_decode_tokens(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"])
    out = gd.gdla_decode_paged(dims, dev["wstruct"], dev["x"], inp["p0"], pc)
    torch.cuda.synchronize()
    if cfg.get("window", 0) == 0:
        assert torch.equal(out, ref), "paged and contiguous decode must agree bit for bit"
    else:  # paged tiles start on page boundaries, contiguous ones at the window start
        H.check(H.to_np(out), H.to_np(ref), dt, "paged vs contiguous decode")
    assert torch.equal(H.from_pages(pc, B, L), dev["cache"]), "appended rows must land in their pages"
    # and against the oracle's one-call forward
    r = H.prefill_case(cfg, T, p0, window=cfg.get("window", 0), seed=37, entry="decode_tokens")
    _say(H.check(H.to_np(out), r["exp_out"], dt, f"paged decode {dt} T={T} page_rows={page_rows}"))


@pytest.mark.parametrize("cfg,T,p0,window,page_rows", [
    (BF, 100, [0, 150], 0, 32),
    (BF, 64, [300, 7], 40, 64),
    (TINY, 37, [0, 11], 0, 32),
])
def test_paged_prefill_matches_contiguous(cfg, T, p0, window, page_rows):
    inp = synth.make_inputs(cfg, "cpu", batch=len(p0), seq=T, p0=p0, random_gamma=True, seed=41)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg, window=window)
    B, L = dev["cache"].shape[0], dev["cache"].shape[1]
    pc = H.to_pages(dev["cache"], page_rows, seed=9)
    ref = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"])
    out = gd.gdla_prefill_paged(dims, dev["wstruct"], dev["x"], inp["p0"], pc)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "paged and contiguous prefill must agree bit for bit"
    assert torch.equal(H.from_pages(pc, B, L), dev["cache"])
    r = H.prefill_case(cfg, T, p0, window=window, seed=41)
    _say(H.check(H.to_np(out), r["exp_out"], cfg["dtype"], f"paged prefill T={T} W={window}"))


@pytest.mark.parametrize("entry", ["decode", "prefill"])
def test_paged_window_never_reads_recycled_pages(entry):
    """Sliding-window layer over a ring of pages: the blocks wholly before every new token's window
    are remapped to a page of NaNs (as a serving system would recycle them).  Neither path may read
    them: the outputs stay finite and equal the contiguous cache's."""
    cfg, W, page = dict(H.BF80, window=96), 96, 32
    T = 3 if entry == "decode" else 40
    p0 = [500, 1000, 130]
    inp = synth.make_inputs(cfg, "cpu", batch=3, seq=T, p0=p0, random_gamma=True, seed=59)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg, window=W)
    pc = H.to_pages(dev["cache"], page, seed=13)
    poison = pc.pages.shape[0] - 1  # a spare page: no block maps to it yet
    pc.pages[poison] = float("nan")
    for b, p in enumerate(p0):
        first_visible = max(0, p - W + 1)  # the first new token's window start (later ones start later)
        pc.block_table[b, :first_visible // page] = poison
    if entry == "decode":
        ref = gd.gdla_decode_tokens(dims, dev["wstruct"], dev["x"], p0, dev["cache"])
        out = gd.gdla_decode_paged(dims, dev["wstruct"], dev["x"], p0, pc)
    else:
        ref = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], p0, dev["cache"])
        out = gd.gdla_prefill_paged(dims, dev["wstruct"], dev["x"], p0, pc)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "a recycled (NaN) page was read"
    _say(H.check(H.to_np(out), H.to_np(ref), "bf16", f"ring of pages, {entry}"))


def test_paged_append():
    cfg = BF
    inp = synth.make_inputs(cfg, "cpu", batch=3, seq=45, p0=[0, 20, 99], seed=43)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    B, L = dev["cache"].shape[0], dev["cache"].shape[1]
    pc = H.to_pages(dev["cache"], 32, seed=11)
    gd.gdla_latent_append(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"])
    gd.gdla_latent_append_paged(dims, dev["wstruct"], dev["x"], inp["p0"], pc)
    torch.cuda.synchronize()
    assert torch.equal(H.from_pages(pc, B, L), dev["cache"])


def test_bf16_lambda_zero_is_gated_mla():
    r = H.prefill_case(BF, 96, [0, 20], window=32, lam_zero=True)
    inp = r["inp"]
    w = H.oracle_weights(inp)
    for b, p in enumerate(inp["p0"]):
        pre = H.to_np(inp["cache"][b, :p]) if p > 0 else None
        exp = oracle.mla_forward(H.to_np(inp["x"][b]), w, BF["n_signal"], BF["n_kv"], BF["n_noise"],
                                 BF["d_head"], BF["d_rope"], 32, prefix=pre, p0=p)
        _say(H.check(r["out"][b], exp, "bf16", f"lambda=0 vs gated MLA, seq {b}"))


def test_latent_append():
    for cfg, dt in ((TINY, "f32"), (BF, "bf16")):
        inp = synth.make_inputs(cfg, "cpu", batch=2, seq=33, p0=[0, 50], random_gamma=True)
        dev = H.device_inputs(inp)
        dims = gd.make_dims(cfg)
        gd.gdla_latent_append(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"])
        torch.cuda.synchronize()
        w = H.oracle_weights(inp)
        od = H.oracle_dims(cfg, 0)
        for b, p in enumerate(inp["p0"]):
            c_bar, k_r = oracle.latent_path(H.to_np(inp["x"][b]), w, od, p + np.arange(33))
            exp = np.concatenate([c_bar, k_r], axis=1)
            H.check_rows(H.to_np(dev["cache"][b, p:p + 33]), exp, dt, f"append {dt} seq {b}")
            # rows outside [p, p + 33) are untouched
            assert torch.equal(dev["cache"][b, :p].cpu(), inp["cache"][b, :p])
            assert torch.equal(dev["cache"][b, p + 33:].cpu(), inp["cache"][b, p + 33:])


# ---------------------------------------------------------------- GPU-side invariants
def test_chunked_and_decode_match_one_call():
    cfg = BF
    inp = synth.make_inputs(cfg, "cpu", batch=1, seq=130, p0=0, random_gamma=True)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg, window=48)
    base = dev["cache"].clone()
    mono = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], [0], base)
    c2 = dev["cache"].clone()
    a = gd.gdla_prefill(dims, dev["wstruct"], dev["x"][:, :70].contiguous(), [0], c2)
    b = gd.gdla_prefill(dims, dev["wstruct"], dev["x"][:, 70:129].contiguous(), [70], c2)
    dec = gd.gdla_decode(dims, dev["wstruct"], dev["x"][:, 129].contiguous(), [129], c2)
    torch.cuda.synchronize()
    got = torch.cat([a, b, dec[:, None]], dim=1)
    _say(H.check(H.to_np(got), H.to_np(mono), "bf16", "chunks + decode vs one call"))
    assert torch.equal(base[:, :130], c2[:, :130]), "cache rows must not depend on chunking"


def test_window_at_least_length_equals_full():
    inp = synth.make_inputs(BF, "cpu", batch=1, seq=150, p0=0)
    dev = H.device_inputs(inp)
    outs = []
    for window in (0, 150, 1 << 20):
        cache = dev["cache"].clone()
        outs.append(gd.gdla_prefill(gd.make_dims(BF, window=window), dev["wstruct"], dev["x"], [0],
                                    cache))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_repeat_runs_are_bitwise_identical():
    for cfg, seq in ((TINY, 70), (BF, 140)):
        inp = synth.make_inputs(cfg, "cpu", batch=2, seq=seq, p0=[0, 9])
        dev = H.device_inputs(inp)
        dims = gd.make_dims(cfg, window=0)
        o1 = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"].clone())
        o2 = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], dev["cache"].clone())
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


def test_workspace_reuse_and_explicit_stream():
    inp = synth.make_inputs(BF, "cpu", batch=1, seq=64, p0=0)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(BF)
    need = gd.gdla_workspace_bytes(dims, gd.GDLA_OP_PREFILL, 1, 64, [0], 64)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # garbage-filled workspace
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1 = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], [0], dev["cache"].clone(), ws=ws, stream=s)
    s.synchronize()
    o2 = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], [0], dev["cache"].clone())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_explicit_stream_without_workspace():
    """stream= with neither ws= nor out=, called outside any stream context: the binding allocates
    the workspace and the output on that stream, so memory freed when the call returns is not handed
    to work queued meanwhile on the current stream while the call's kernels still run on the other."""
    inp = synth.make_inputs(BF, "cpu", batch=1, seq=300, p0=0, seed=61)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(BF)
    ref = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], [0], dev["cache"].clone())
    need = gd.gdla_workspace_bytes(dims, gd.GDLA_OP_PREFILL, 1, 300, [0], dev["cache"].shape[1])
    cache = dev["cache"].clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(20_000_000)  # keep the side stream busy so its kernels run late
    out = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], [0], cache, stream=s)
    # blocks of exactly the workspace's size, filled on the current stream right away
    junk = [torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda") for _ in range(4)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out, ref)


@pytest.mark.parametrize("cfg,T,p0,window", [(H.BF80, 300, [0], 0), (BF, 260, [40, 0], 64), (BF, 64, [5], 0)],
                         ids=["80h", "10h-window", "short"])
def test_prefill_prepared_weights_match_prefill(cfg, T, p0, window):
    """gdla_prefill_prepared (weights transposed once by gdla_prepare_weights) gives gdla_prefill's
    output and cache rows bit for bit; below 256 rows the prepared copies are not read at all."""
    inp = synth.make_inputs(cfg, "cpu", batch=len(p0), seq=T, p0=p0, random_gamma=True, seed=131)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg, window=window)
    prepared = gd.gdla_prepare_weights(dims, dev["wstruct"])
    c1, c2 = dev["cache"].clone(), dev["cache"].clone()
    ref = gd.gdla_prefill(dims, dev["wstruct"], dev["x"], inp["p0"], c1)
    out = gd.gdla_prefill_prepared(dims, dev["wstruct"], prepared, dev["x"], inp["p0"], c2)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(c1, c2)
    r = H.prefill_case(cfg, T, p0, window=window, seed=131)
    _say(H.check(H.to_np(out), r["exp_out"], "bf16", f"prepared-weight prefill T={T}"))
