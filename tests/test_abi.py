"""CPU tests of the C-ABI boundary: the library loads, exports every function include/gdla.h
declares, and every argument error is reported before any GPU work (these calls never reach a
launch, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

import attention_gdla_prefill_decode_amd as gd
from attention_gdla_prefill_decode_amd import gdla as gb
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdla.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdla_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = gd.lib()
    names = declared_functions()
    assert set(names) == set(gd.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def test_status_strings():
    lib = gd.lib()
    for code, name in enumerate(["GDLA_OK", "GDLA_ERR_INVALID_ARG", "GDLA_ERR_UNSUPPORTED",
                                 "GDLA_ERR_WORKSPACE", "GDLA_ERR_OUT_OF_RANGE", "GDLA_ERR_HIP"]):
        assert lib.gdla_status_string(code).decode() == name
    assert lib.gdla_status_string(99).decode() == "unknown gdla_status"


def big_dims(**kw):
    cfg = dict(synth.WORKLOADS["prefill_8k"])
    cfg.update(kw)
    return gd.make_dims(cfg)


def test_workspace_bytes():
    d = big_dims()
    pre = gd.gdla_workspace_bytes(d, gd.GDLA_OP_PREFILL, 1, 8192, [0], 8192)
    assert pre > 0 and pre % 256 == 0
    # the expanded K/V of 8192 keys x 16 heads x 128 x 2 (K, V) in bf16 alone is 64 MiB
    assert pre >= 8192 * 16 * 128 * 2 * 2
    assert gd.gdla_workspace_bytes(d, gd.GDLA_OP_PREFILL, 1, 8192, None, 8192) == pre
    dec = gd.gdla_workspace_bytes(d, gd.GDLA_OP_DECODE, 64, 1, [65535] * 64, 65536)
    assert dec > 0
    app = gd.gdla_workspace_bytes(d, gd.GDLA_OP_APPEND, 2, 10, [0, 5], 64)
    assert 0 < app < pre
    # windowed prefill needs keys from p0 - W + 1 only
    dw = big_dims(window=4096)
    assert gd.gdla_workspace_bytes(dw, gd.GDLA_OP_PREFILL, 1, 4096, [100000], 262144) < \
        gd.gdla_workspace_bytes(d, gd.GDLA_OP_PREFILL, 1, 4096, [100000], 262144)
    # invalid requests report 0
    assert gd.gdla_workspace_bytes(d, gd.GDLA_OP_PREFILL, 1, 10, [8190], 8192) == 0
    # several tokens per sequence on the decode path: workspace grows with B T
    dec4 = gd.gdla_workspace_bytes(d, gd.GDLA_OP_DECODE, 64, 4, [65532] * 64, 65536)
    assert dec4 > dec
    assert gd.gdla_workspace_bytes(d, gd.GDLA_OP_DECODE, 4, gd.MAX_DECODE_TOKENS, None, 64) > 0
    assert gd.gdla_workspace_bytes(d, gd.GDLA_OP_DECODE, 4, gd.MAX_DECODE_TOKENS + 1, None, 64) == 0
    assert gd.gdla_workspace_bytes(d, gd.GDLA_OP_DECODE, 1, 4, [61], 64) == 0
    assert gd.gdla_workspace_bytes(d, 7, 1, 1, None, 64) == 0
    assert gd.gdla_workspace_bytes(big_dims(n_noise=15), gd.GDLA_OP_PREFILL, 1, 1, None, 8) == 0


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def call_prefill(dims, weights=None, x=FAKE, B=1, T=4, pos=(0,), cache=FAKE, max_len=64, out=FAKE,
                 ws=FAKE, ws_bytes=1 << 40):
    lib = gd.lib()
    w = weights if weights is not None else gb.GdlaWeights(*([FAKE] * 12))
    pa = (ctypes.c_int32 * len(pos))(*pos) if pos is not None else None
    st = lib.gdla_prefill(ctypes.byref(dims), ctypes.byref(w), x, B, T, pa, cache, max_len, out,
                          ws, ws_bytes, None, None)
    return st, lib.gdla_last_error().decode()


@pytest.mark.parametrize("case,expect", [
    ("bad_split", gb.GDLA_ERR_INVALID_ARG),
    ("noise_not_divisor", gb.GDLA_ERR_INVALID_ARG),
    ("kv_not_divisor", gb.GDLA_ERR_INVALID_ARG),
    ("odd_rope", gb.GDLA_ERR_INVALID_ARG),
    ("negative_window", gb.GDLA_ERR_INVALID_ARG),
    ("bad_dtype", gb.GDLA_ERR_INVALID_ARG),
    ("huge_head", gb.GDLA_ERR_UNSUPPORTED),
    ("null_x", gb.GDLA_ERR_INVALID_ARG),
    ("null_out", gb.GDLA_ERR_INVALID_ARG),
    ("null_weight", gb.GDLA_ERR_INVALID_ARG),
    ("null_pos", gb.GDLA_ERR_INVALID_ARG),
    ("misaligned_x", gb.GDLA_ERR_INVALID_ARG),
    ("pos_past_end", gb.GDLA_ERR_OUT_OF_RANGE),
    ("negative_pos", gb.GDLA_ERR_OUT_OF_RANGE),
    ("small_workspace", gb.GDLA_ERR_WORKSPACE),
    ("misaligned_workspace", gb.GDLA_ERR_INVALID_ARG),
])
def test_prefill_argument_errors(case, expect):
    kw = {}
    dims = big_dims()
    if case == "bad_split":
        dims = big_dims(n_signal=60)
    elif case == "noise_not_divisor":
        dims = big_dims(n_signal=62, n_noise=18)
    elif case == "kv_not_divisor":
        dims = big_dims(n_kv=5)
    elif case == "odd_rope":
        dims = big_dims(d_rope=63)
    elif case == "negative_window":
        dims = big_dims(window=-1)
    elif case == "bad_dtype":
        dims.dtype = 9
    elif case == "huge_head":
        dims = big_dims(d_head=512)
    elif case == "null_x":
        kw["x"] = None
    elif case == "null_out":
        kw["out"] = None
    elif case == "null_weight":
        w = gb.GdlaWeights(*([FAKE] * 12))
        w.w_uv = None
        kw["weights"] = w
    elif case == "null_pos":
        kw["pos"] = None
    elif case == "misaligned_x":
        kw["x"] = FAKE + 2
    elif case == "pos_past_end":
        kw["pos"] = (61,)
    elif case == "negative_pos":
        kw["pos"] = (-1,)
    elif case == "small_workspace":
        kw["ws_bytes"] = 1024
    elif case == "misaligned_workspace":
        kw["ws"] = FAKE + 16
    st, msg = call_prefill(dims, **kw)
    assert st == expect, (st, msg)
    assert msg, "a failure must leave a description in gdla_last_error()"


def test_empty_inputs_are_noops():
    # B = 0 or T = 0: nothing to do, nothing launched, GDLA_OK, no pointers needed
    st, _ = call_prefill(big_dims(), x=None, B=0, pos=None, cache=None, out=None, ws=None)
    assert st == gb.GDLA_OK
    st, _ = call_prefill(big_dims(), x=None, T=0, cache=None, out=None, ws=None)
    assert st == gb.GDLA_OK


def test_decode_and_append_argument_errors():
    lib = gd.lib()
    d = big_dims()
    w = gb.GdlaWeights(*([FAKE] * 12))
    pos = (ctypes.c_int32 * 2)(5, 64)
    st = lib.gdla_decode(ctypes.byref(d), ctypes.byref(w), FAKE, 2, pos, FAKE, 64, FAKE, FAKE,
                         1 << 40, None, None)
    assert st == gb.GDLA_ERR_OUT_OF_RANGE
    pos = (ctypes.c_int32 * 2)(5, 6)
    st = lib.gdla_decode(ctypes.byref(d), ctypes.byref(w), FAKE, 2, pos, FAKE, 64, FAKE, FAKE, 16,
                         None, None)
    assert st == gb.GDLA_ERR_WORKSPACE
    w.w_kr = None
    st = lib.gdla_latent_append(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 3, pos, FAKE, 64, FAKE,
                                1 << 40, None)
    assert st == gb.GDLA_ERR_INVALID_ARG
    w.w_kr = FAKE
    w.w_qa = None  # the query weights are not needed to append latents
    st = lib.gdla_latent_append(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 3, pos, FAKE, 64, FAKE,
                                16, None)
    assert st == gb.GDLA_ERR_WORKSPACE


def test_decode_noalloc_refuses_calls_beyond_its_scratch():
    # 256 sequences of the 80-head layer need about 185 MiB of workspace, above the 96 MiB static
    # scratch: refused with GDLA_ERR_WORKSPACE before any GPU call (so this runs without a GPU)
    lib = gd.lib()
    d = big_dims()
    w = gb.GdlaWeights(*([FAKE] * 12))
    B = 256
    pos = (ctypes.c_int32 * B)(*([100] * B))
    need = lib.gdla_workspace_bytes(ctypes.byref(d), gb.GDLA_OP_DECODE, B, 1, pos, 4096)
    assert need > gd.NOALLOC_SCRATCH_BYTES
    st = lib.gdla_decode_noalloc(ctypes.byref(d), ctypes.byref(w), FAKE, B, pos, FAKE, 4096, FAKE, None, None)
    assert st == gb.GDLA_ERR_WORKSPACE
    assert b"static scratch" in lib.gdla_last_error()
    # and 64 sequences at the 64K context fit
    B = 64
    pos = (ctypes.c_int32 * B)(*([65535] * B))
    assert lib.gdla_workspace_bytes(ctypes.byref(d), gb.GDLA_OP_DECODE, B, 1, pos, 65536) <= gd.NOALLOC_SCRATCH_BYTES


def test_decode_tokens_argument_errors():
    lib = gd.lib()
    d = big_dims()
    w = gb.GdlaWeights(*([FAKE] * 12))
    pos = (ctypes.c_int32 * 2)(5, 60)

    def call(T, pos=pos, ws_bytes=1 << 40):
        return lib.gdla_decode_tokens(ctypes.byref(d), ctypes.byref(w), FAKE, 2, T, pos, FAKE, 64,
                                      FAKE, FAKE, ws_bytes, None, None)

    assert call(gd.MAX_DECODE_TOKENS + 1) == gb.GDLA_ERR_INVALID_ARG
    assert lib.gdla_last_error().decode()
    assert call(-1) == gb.GDLA_ERR_INVALID_ARG
    assert call(5) == gb.GDLA_ERR_OUT_OF_RANGE  # 60 + 5 > 64
    assert call(4, ws_bytes=16) == gb.GDLA_ERR_WORKSPACE
    # T = 0: nothing to do
    assert lib.gdla_decode_tokens(ctypes.byref(d), ctypes.byref(w), None, 2, 0, pos, None, 64, None,
                                  None, 0, None, None) == gb.GDLA_OK


def test_paged_argument_errors():
    lib = gd.lib()
    d = big_dims()
    w = gb.GdlaWeights(*([FAKE] * 12))
    pos = (ctypes.c_int32 * 2)(5, 60)

    def paged(page_rows=64, n_pages=8, max_blocks=2, pages=FAKE, table=FAKE):
        return gb.GdlaPagedCache(pages, table, n_pages, page_rows, max_blocks)

    def dec(pc, T=1, ws_bytes=1 << 40):
        return lib.gdla_decode_paged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, T, pos,
                                     None if pc is None else ctypes.byref(pc), FAKE, FAKE, ws_bytes,
                                     None, None)

    assert dec(None) == gb.GDLA_ERR_INVALID_ARG
    assert dec(paged(page_rows=48)) == gb.GDLA_ERR_INVALID_ARG      # not a multiple of 32
    assert dec(paged(n_pages=0)) == gb.GDLA_ERR_INVALID_ARG
    assert dec(paged(table=None)) == gb.GDLA_ERR_INVALID_ARG
    assert dec(paged(table=FAKE + 2)) == gb.GDLA_ERR_INVALID_ARG    # misaligned block table
    assert dec(paged(max_blocks=1), T=5) == gb.GDLA_ERR_OUT_OF_RANGE  # 60 + 5 > 1 * 64
    assert dec(paged(), T=gd.MAX_DECODE_TOKENS + 1) == gb.GDLA_ERR_INVALID_ARG
    assert dec(paged(), T=2, ws_bytes=16) == gb.GDLA_ERR_WORKSPACE
    assert lib.gdla_last_error().decode()
    pc = paged()
    st = lib.gdla_prefill_paged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 8, pos, ctypes.byref(pc), FAKE,
                                FAKE, 16, None, None)
    assert st == gb.GDLA_ERR_WORKSPACE
    st = lib.gdla_latent_append_paged(ctypes.byref(d), ctypes.byref(w), FAKE, 2, 70, pos, ctypes.byref(pc),
                                      FAKE, 1 << 40, None)
    assert st == gb.GDLA_ERR_OUT_OF_RANGE  # 60 + 70 > 2 * 64
    # a paged prefill stages the visible rows: more workspace than the contiguous prefill
    pre = gd.gdla_workspace_bytes(d, gd.GDLA_OP_PREFILL, 2, 8, [5, 60], 128)
    prp = gd.gdla_workspace_bytes(d, gd.GDLA_OP_PREFILL_PAGED, 2, 8, [5, 60], 128)
    assert prp >= pre + 2 * 68 * 576 * 2


def test_packed_prefill_argument_errors():
    lib = gd.lib()
    d = big_dims()
    w = gb.GdlaWeights(*([FAKE] * 12))
    pos = (ctypes.c_int32 * 1)(0)

    def call(doc, ws_bytes=1 << 40, T=4):
        return lib.gdla_prefill_packed(ctypes.byref(d), ctypes.byref(w), FAKE, 1, T, pos, doc, FAKE, 64,
                                       FAKE, FAKE, ws_bytes, None, None)

    assert call(None) == gb.GDLA_ERR_INVALID_ARG
    assert lib.gdla_last_error().decode()
    assert call(FAKE + 2) == gb.GDLA_ERR_INVALID_ARG
    assert call(FAKE, ws_bytes=16) == gb.GDLA_ERR_WORKSPACE
    assert call(FAKE, T=65) == gb.GDLA_ERR_OUT_OF_RANGE


def test_backward_argument_errors():
    lib = gd.lib()
    d = big_dims()
    w = gb.GdlaWeights(*([FAKE] * 12))
    full = gb.GdlaGrads(*([FAKE] * 13))

    def call(grads=full, x=FAKE, dout=FAKE, doc=None, ws_bytes=1 << 40, T=16):
        return lib.gdla_backward(ctypes.byref(d), ctypes.byref(w), x, 1, T, doc, dout, ctypes.byref(grads), FAKE,
                                 ws_bytes, None, None)

    assert call(x=None) == gb.GDLA_ERR_INVALID_ARG
    assert call(dout=None) == gb.GDLA_ERR_INVALID_ARG
    no_dx = gb.GdlaGrads(*([None] + [FAKE] * 12))
    assert call(grads=no_dx) == gb.GDLA_ERR_INVALID_ARG
    no_dgamma = gb.GdlaGrads(*([FAKE] * 11 + [None, FAKE]))  # gamma_q is set, dgamma_q missing
    assert call(grads=no_dgamma) == gb.GDLA_ERR_INVALID_ARG
    assert call(doc=FAKE + 2) == gb.GDLA_ERR_INVALID_ARG
    assert call(x=FAKE + 2) == gb.GDLA_ERR_INVALID_ARG
    assert call(ws_bytes=16) == gb.GDLA_ERR_WORKSPACE
    assert lib.gdla_last_error().decode()
    assert call(T=0, x=None, dout=None) == gb.GDLA_OK
    assert gd.gdla_workspace_bytes(d, gd.GDLA_OP_BACKWARD, 1, 16, None, 16) > 0


def test_prepared_weights_sizes_and_errors():
    lib = gd.lib()
    d = big_dims()
    need = gd.gdla_prepared_weights_bytes(d)
    # ten transposed weights of the 80-head layer, 2 bytes per value
    vals = (4096 * (1024 + 512 + 64 + 64) + 1024 * (80 * 128 + 80 * 64 + 64 * 128) + 512 * 2 * 16 * 128
            + 64 * 128 * 4096)
    assert need >= 2 * vals and need < 2 * vals + 10 * 256
    assert gd.gdla_prepared_weights_bytes(big_dims(dtype="f32")) == 0
    w = gb.GdlaWeights(*([FAKE] * 12))
    st = lib.gdla_prepare_weights(ctypes.byref(big_dims(dtype="f32")), ctypes.byref(w), FAKE, 1 << 40, None)
    assert st == gb.GDLA_ERR_UNSUPPORTED
    st = lib.gdla_prepare_weights(ctypes.byref(d), ctypes.byref(w), None, 1 << 40, None)
    assert st == gb.GDLA_ERR_INVALID_ARG
    st = lib.gdla_prepare_weights(ctypes.byref(d), ctypes.byref(w), FAKE, need - 1, None)
    assert st == gb.GDLA_ERR_WORKSPACE
    w.w_o = None
    st = lib.gdla_prepare_weights(ctypes.byref(d), ctypes.byref(w), FAKE, need, None)
    assert st == gb.GDLA_ERR_INVALID_ARG
    w.w_o = FAKE
    pos = (ctypes.c_int32 * 1)(0)
    st = lib.gdla_prefill_prepared(ctypes.byref(d), ctypes.byref(w), None, need, FAKE, 1, 8, pos, FAKE, 8, FAKE,
                                   FAKE, 1 << 40, None, None)
    assert st == gb.GDLA_ERR_INVALID_ARG
    st = lib.gdla_prefill_prepared(ctypes.byref(d), ctypes.byref(w), FAKE, 16, FAKE, 1, 8, pos, FAKE, 8, FAKE,
                                   FAKE, 1 << 40, None, None)
    assert st == gb.GDLA_ERR_WORKSPACE
