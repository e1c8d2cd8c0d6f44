"""Thin ctypes binding of libgdla.so (include/gdla.h).

Argument marshalling only: torch tensors supply device memory and the current stream; every step
of the GDLA forward runs in the library's HIP kernels.  There is no fallback: if libgdla.so is
missing, or a call fails, an exception is raised.
"""

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdla.so")

GDLA_OK, GDLA_ERR_INVALID_ARG, GDLA_ERR_UNSUPPORTED, GDLA_ERR_WORKSPACE, GDLA_ERR_OUT_OF_RANGE, \
    GDLA_ERR_HIP = range(6)
GDLA_F32, GDLA_BF16 = 0, 1
GDLA_OP_PREFILL, GDLA_OP_DECODE, GDLA_OP_APPEND, GDLA_OP_PREFILL_PAGED, GDLA_OP_BACKWARD = 0, 1, 2, 3, 4

GRAD_FIELDS = ("dx", "dw_qa", "dw_qc", "dw_qr", "dw_dkv", "dw_kr", "dw_uk", "dw_uv", "dw_lambda",
               "dw_gate", "dw_o", "dgamma_q", "dgamma_kv")

WEIGHT_FIELDS = ("w_qa", "gamma_q", "w_qc", "w_qr", "w_dkv", "w_kr", "gamma_kv", "w_uk", "w_uv",
                 "w_lambda", "w_gate", "w_o")

EXPORTED = ("gdla_workspace_bytes", "gdla_latent_append", "gdla_prefill", "gdla_decode",
            "gdla_decode_tokens", "gdla_prefill_packed", "gdla_latent_append_paged",
            "gdla_prefill_paged", "gdla_decode_paged", "gdla_backward", "gdla_decode_noalloc",
            "gdla_prepared_weights_bytes", "gdla_prepare_weights", "gdla_prefill_prepared",
            "gdla_status_string", "gdla_last_error")

MAX_DECODE_TOKENS = 16  # GDLA_MAX_DECODE_TOKENS
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024  # GDLA_NOALLOC_SCRATCH_BYTES


class GdlaDims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_signal", ctypes.c_int32), ("n_noise", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("d_q_latent", ctypes.c_int32),
                ("d_kv_latent", ctypes.c_int32), ("d_head", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class GdlaWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class GdlaPagedCache(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("n_pages", ctypes.c_int32), ("page_rows", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32)]


class GdlaGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class GdlaDebug(ctypes.Structure):
    _fields_ = [("lambda_override", ctypes.c_void_p), ("out_heads", ctypes.c_void_p),
                ("stage_events", ctypes.c_void_p)]


STAGES = ("proj_in", "norm_append", "expand_kv", "proj_q", "attn_noise", "attn_signal", "proj_out")


class StageTimer:
    """2 x len(STAGES) HIP events for gdla_debug.stage_events; elapsed() gives per-stage ms.
    stages: the stage names to time (default: all); the others' entries stay NULL, so the call
    records no event for them."""

    def __init__(self, stages=None):
        self.stages = tuple(STAGES if stages is None else stages)
        if any(n not in STAGES for n in self.stages):
            raise ValueError(f"unknown stage in {self.stages}")
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = (ctypes.c_void_p * (2 * len(STAGES)))()
        for k, name in enumerate(STAGES):
            if name not in self.stages:
                continue
            for i in (2 * k, 2 * k + 1):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                self.events[i] = ev
        self.ptr = ctypes.cast(self.events, ctypes.c_void_p).value

    def elapsed(self):
        """Per-stage milliseconds of the last call that recorded these events."""
        out = {}
        for k, name in enumerate(STAGES):
            if name not in self.stages:
                continue
            self.hip.hipEventSynchronize(self.events[2 * k + 1])
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * k],
                                            self.events[2 * k + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = ms.value
        return out

    def __del__(self):
        try:
            for i in range(2 * len(STAGES)):
                if self.events[i]:
                    self.hip.hipEventDestroy(self.events[i])
        except Exception:
            pass


class GdlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_lib = None


def lib():
    """The loaded libgdla.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first with "
                               "`python -m attention_gdla_prefill_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.gdla_workspace_bytes.restype = ctypes.c_size_t
        L.gdla_workspace_bytes.argtypes = [P(GdlaDims), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32]
        L.gdla_latent_append.restype = ctypes.c_int
        L.gdla_latent_append.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
        L.gdla_prefill.restype = ctypes.c_int
        L.gdla_prefill.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_size_t, P(GdlaDebug), ctypes.c_void_p]
        L.gdla_decode.restype = ctypes.c_int
        L.gdla_decode.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  P(GdlaDebug), ctypes.c_void_p]
        L.gdla_prepared_weights_bytes.restype = ctypes.c_size_t
        L.gdla_prepared_weights_bytes.argtypes = [P(GdlaDims)]
        L.gdla_prepare_weights.restype = ctypes.c_int
        L.gdla_prepare_weights.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]
        L.gdla_prefill_prepared.restype = ctypes.c_int
        L.gdla_prefill_prepared.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_size_t, P(GdlaDebug), ctypes.c_void_p]
        L.gdla_decode_noalloc.restype = ctypes.c_int
        L.gdla_decode_noalloc.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p, P(GdlaDebug), ctypes.c_void_p]
        L.gdla_decode_tokens.restype = ctypes.c_int
        L.gdla_decode_tokens.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, P(GdlaDebug), ctypes.c_void_p]
        L.gdla_prefill_packed.restype = ctypes.c_int
        L.gdla_prefill_packed.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_size_t, P(GdlaDebug),
                                          ctypes.c_void_p]
        L.gdla_latent_append_paged.restype = ctypes.c_int
        L.gdla_latent_append_paged.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                               P(GdlaPagedCache), ctypes.c_void_p, ctypes.c_size_t,
                                               ctypes.c_void_p]
        for name in ("gdla_prefill_paged", "gdla_decode_paged"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                          ctypes.c_int32, ctypes.c_void_p, P(GdlaPagedCache), ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_size_t, P(GdlaDebug), ctypes.c_void_p]
        L.gdla_backward.restype = ctypes.c_int
        L.gdla_backward.argtypes = [P(GdlaDims), P(GdlaWeights), ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, P(GdlaGrads),
                                    ctypes.c_void_p, ctypes.c_size_t, P(GdlaDebug), ctypes.c_void_p]
        L.gdla_status_string.restype = ctypes.c_char_p
        L.gdla_status_string.argtypes = [ctypes.c_int]
        L.gdla_last_error.restype = ctypes.c_char_p
        L.gdla_last_error.argtypes = []
        _lib = L
    return _lib


def make_dims(cfg, window=None, dtype=None, eps=1e-6, theta=10000.0, scale=0.0):
    """gdla_dims from a workload dict (keys d_model, n_heads, ..., dtype 'f32' / 'bf16')."""
    dt = cfg["dtype"] if dtype is None else dtype
    return GdlaDims(cfg["d_model"], cfg["n_heads"], cfg["n_signal"], cfg["n_noise"], cfg["n_kv"],
                    cfg["d_q_latent"], cfg["d_kv_latent"], cfg["d_head"], cfg["d_rope"],
                    cfg.get("window", 0) if window is None else window, eps, theta, scale,
                    GDLA_F32 if dt == "f32" else GDLA_BF16)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_weights(weights, gamma_q=None, gamma_kv=None):
    """gdla_weights from a dict of device tensors ([in, out] row-major, contiguous).  The returned
    struct keeps references to the tensors, so their memory lives as long as the struct does."""
    vals = dict(weights)
    vals["gamma_q"], vals["gamma_kv"] = gamma_q, gamma_kv
    for k, v in vals.items():
        if v is not None and not v.is_contiguous():
            raise ValueError(f"weight {k} must be contiguous")
    w = GdlaWeights(*[None if vals.get(n) is None else vals[n].data_ptr() for n in WEIGHT_FIELDS])
    w._tensors = {n: vals.get(n) for n in WEIGHT_FIELDS}
    return w


def _pos_array(pos):
    arr = (ctypes.c_int32 * len(pos))(*[int(p) for p in pos])
    return arr


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context for the memory a call allocates (workspace, outputs): with an explicit stream they
    are allocated on that stream, so the caching allocator hands their blocks to no other work
    before the call's kernels on that stream have finished with them."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check(status):
    if status != GDLA_OK:
        L = lib()
        raise GdlaError(status, "%s: %s" % (L.gdla_status_string(status).decode(),
                                            L.gdla_last_error().decode()))


def gdla_workspace_bytes(dims, op, B, T, pos, max_len):
    pa = None if pos is None else _pos_array(pos)
    return int(lib().gdla_workspace_bytes(ctypes.byref(dims), op, B, T, pa, max_len))


def _workspace(dims, op, B, T, pos, max_len, ws, device):
    need = gdla_workspace_bytes(dims, op, B, T, pos, max_len)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


def _debug(lambda_override, out_heads, timer=None):
    if lambda_override is None and out_heads is None and timer is None:
        return None
    return GdlaDebug(None if lambda_override is None else lambda_override.data_ptr(),
                     None if out_heads is None else out_heads.data_ptr(),
                     None if timer is None else timer.ptr)


def gdla_latent_append(dims, weights, x, pos, cache, ws=None, stream=None):
    """Writes cache rows [pos[b], pos[b] + T) from x [B, T, d_model]."""
    B, T = x.shape[0], x.shape[1]
    max_len = cache.shape[1]
    with _on(stream):
        ws, nbytes = _workspace(dims, GDLA_OP_APPEND, B, T, pos, max_len, ws, x.device)
    _check(lib().gdla_latent_append(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                    _pos_array(pos), _ptr(cache), max_len, _ptr(ws), nbytes,
                                    _stream(stream)))


def gdla_prefill(dims, weights, x, pos, cache, out=None, ws=None, lambda_override=None,
                 out_heads=None, stream=None, timer=None):
    """x [B, T, d_model] at positions pos[b] + t; appends to cache; returns out [B, T, d_model]."""
    B, T = x.shape[0], x.shape[1]
    max_len = cache.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_PREFILL, B, T, pos, max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_prefill(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                              _pos_array(pos), _ptr(cache), max_len, _ptr(out), _ptr(ws), nbytes,
                              None if dbg is None else ctypes.byref(dbg), _stream(stream)))
    return out


def gdla_decode(dims, weights, x, pos, cache, out=None, ws=None, lambda_override=None,
                out_heads=None, stream=None, timer=None):
    """x [B, d_model], token b at position pos[b]; appends to cache; returns out [B, d_model]."""
    B = x.shape[0]
    max_len = cache.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_DECODE, B, 1, pos, max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_decode(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B,
                             _pos_array(pos), _ptr(cache), max_len, _ptr(out), _ptr(ws), nbytes,
                             None if dbg is None else ctypes.byref(dbg), _stream(stream)))
    return out


def gdla_prepared_weights_bytes(dims):
    return int(lib().gdla_prepared_weights_bytes(ctypes.byref(dims)))


def gdla_prepare_weights(dims, weights, prepared=None, stream=None, device="cuda"):
    """The layer's prepared (transposed) weights for gdla_prefill_prepared, in `prepared` (a
    uint8 device tensor of at least gdla_prepared_weights_bytes(dims) bytes) or a new tensor."""
    with _on(stream):
        if prepared is None:
            prepared = torch.empty(max(gdla_prepared_weights_bytes(dims), 256), dtype=torch.uint8, device=device)
    _check(lib().gdla_prepare_weights(ctypes.byref(dims), ctypes.byref(weights), _ptr(prepared),
                                      prepared.numel(), _stream(stream)))
    return prepared


def gdla_prefill_prepared(dims, weights, prepared, x, pos, cache, out=None, ws=None, lambda_override=None,
                          out_heads=None, stream=None, timer=None):
    """gdla_prefill reading the weights' transposed copies from `prepared` (gdla_prepare_weights)."""
    B, T = x.shape[0], x.shape[1]
    max_len = cache.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_PREFILL, B, T, pos, max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_prefill_prepared(ctypes.byref(dims), ctypes.byref(weights), _ptr(prepared), prepared.numel(),
                                       _ptr(x), B, T, _pos_array(pos), _ptr(cache), max_len, _ptr(out), _ptr(ws),
                                       nbytes, None if dbg is None else ctypes.byref(dbg), _stream(stream)))
    return out


def gdla_decode_noalloc(dims, weights, x, pos, cache, out, lambda_override=None, out_heads=None,
                        stream=None, timer=None):
    """gdla_decode on the library's static device scratch (no workspace argument): x [B, d_model],
    token b at position pos[b]; appends to cache; writes out [B, d_model] (caller-allocated) and
    returns it.  Calls on one GPU share the scratch: the caller orders them."""
    B = x.shape[0]
    max_len = cache.shape[1]
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_decode_noalloc(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B,
                                     _pos_array(pos), _ptr(cache), max_len, _ptr(out),
                                     None if dbg is None else ctypes.byref(dbg), _stream(stream)))
    return out


def gdla_decode_tokens(dims, weights, x, pos, cache, out=None, ws=None, lambda_override=None,
                       out_heads=None, stream=None, timer=None):
    """x [B, T, d_model], token i of sequence b at position pos[b] + i (T <= MAX_DECODE_TOKENS);
    appends to cache; returns out [B, T, d_model] (absorbed decode path)."""
    B, T = x.shape[0], x.shape[1]
    max_len = cache.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_DECODE, B, T, pos, max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_decode_tokens(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                    _pos_array(pos), _ptr(cache), max_len, _ptr(out), _ptr(ws),
                                    nbytes, None if dbg is None else ctypes.byref(dbg),
                                    _stream(stream)))
    return out


def gdla_prefill_packed(dims, weights, x, pos, doc_start, cache, out=None, ws=None,
                        lambda_override=None, out_heads=None, stream=None, timer=None):
    """gdla_prefill over packed documents: doc_start [B, T] int32 (device) holds the position of
    the first token of each token's document."""
    B, T = x.shape[0], x.shape[1]
    max_len = cache.shape[1]
    assert doc_start.dtype == torch.int32 and tuple(doc_start.shape) == (B, T)
    doc_start = doc_start.contiguous()
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_PREFILL, B, T, pos, max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_prefill_packed(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                     _pos_array(pos), _ptr(doc_start), _ptr(cache), max_len,
                                     _ptr(out), _ptr(ws), nbytes,
                                     None if dbg is None else ctypes.byref(dbg), _stream(stream)))
    return out


class PagedCache:
    """A paged latent cache: `pages` [n_pages, page_rows, d_kv_latent + d_rope] and `block_table`
    [B, max_blocks] int32 (both device tensors, owned by the caller)."""

    def __init__(self, pages, block_table):
        assert block_table.dtype == torch.int32 and block_table.dim() == 2
        self.pages, self.block_table = pages, block_table
        self.struct = GdlaPagedCache(pages.data_ptr(), block_table.data_ptr(), pages.shape[0],
                                     pages.shape[1], block_table.shape[1])

    @property
    def max_len(self):
        return self.struct.max_blocks * self.struct.page_rows


def gdla_latent_append_paged(dims, weights, x, pos, cache, ws=None, stream=None):
    """gdla_latent_append into a PagedCache."""
    B, T = x.shape[0], x.shape[1]
    with _on(stream):
        ws, nbytes = _workspace(dims, GDLA_OP_APPEND, B, T, pos, cache.max_len, ws, x.device)
    _check(lib().gdla_latent_append_paged(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                          _pos_array(pos), ctypes.byref(cache.struct), _ptr(ws),
                                          nbytes, _stream(stream)))


def gdla_prefill_paged(dims, weights, x, pos, cache, out=None, ws=None, lambda_override=None,
                       out_heads=None, stream=None, timer=None):
    """gdla_prefill over a PagedCache: x [B, T, d_model] -> out [B, T, d_model]."""
    B, T = x.shape[0], x.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_PREFILL_PAGED, B, T, pos, cache.max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_prefill_paged(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                    _pos_array(pos), ctypes.byref(cache.struct), _ptr(out),
                                    _ptr(ws), nbytes, None if dbg is None else ctypes.byref(dbg),
                                    _stream(stream)))
    return out


def gdla_decode_paged(dims, weights, x, pos, cache, out=None, ws=None, lambda_override=None,
                      out_heads=None, stream=None, timer=None):
    """Multi-token decode over a PagedCache: x [B, T, d_model] -> out [B, T, d_model]."""
    B, T = x.shape[0], x.shape[1]
    with _on(stream):
        if out is None:
            out = torch.empty_like(x)
        ws, nbytes = _workspace(dims, GDLA_OP_DECODE, B, T, pos, cache.max_len, ws, x.device)
    dbg = _debug(lambda_override, out_heads, timer)
    _check(lib().gdla_decode_paged(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                                   _pos_array(pos), ctypes.byref(cache.struct), _ptr(out), _ptr(ws),
                                   nbytes, None if dbg is None else ctypes.byref(dbg),
                                   _stream(stream)))
    return out


def gdla_backward(dims, weights, tensors, x, dout, doc_start=None, ws=None, lambda_override=None,
                  stream=None, timer=None):
    """Gradients of sum(out * dout) for training sequences x [B, T, d_model] at positions 0..T-1.
    `tensors` maps the weight names (as for make_weights) to the weight tensors, which give the
    gradient shapes.  Returns a dict of fp32 gradients (GRAD_FIELDS; the gamma gradients only for
    the gains that are set)."""
    B, T = x.shape[0], x.shape[1]
    dev = x.device
    with _on(stream):
        grads = {"dx": torch.empty((B, T, x.shape[2]), dtype=torch.float32, device=dev)}
        for name in ("w_qa", "w_qc", "w_qr", "w_dkv", "w_kr", "w_uk", "w_uv", "w_lambda", "w_gate", "w_o"):
            grads["d" + name] = torch.empty(tuple(tensors[name].shape), dtype=torch.float32, device=dev)
        for name in ("gamma_q", "gamma_kv"):
            if tensors.get(name) is not None:
                grads["d" + name] = torch.empty(tuple(tensors[name].shape), dtype=torch.float32, device=dev)
        ws, nbytes = _workspace(dims, GDLA_OP_BACKWARD, B, T, None, T, ws, dev)
    gs = GdlaGrads(*[None if grads.get(n) is None else grads[n].data_ptr() for n in GRAD_FIELDS])
    if doc_start is not None:
        assert doc_start.dtype == torch.int32 and tuple(doc_start.shape) == (B, T)
        doc_start = doc_start.contiguous()
    dbg = _debug(lambda_override, None, timer)
    _check(lib().gdla_backward(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), B, T,
                               None if doc_start is None else _ptr(doc_start), _ptr(dout),
                               ctypes.byref(gs), _ptr(ws), nbytes,
                               None if dbg is None else ctypes.byref(dbg), _stream(stream)))
    return grads
