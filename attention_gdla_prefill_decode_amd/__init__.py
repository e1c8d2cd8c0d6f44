"""GDLA (Grouped Differential Latent Attention) forward for AMD Instinct MI355X (gfx950).

The compute lives in libgdla.so (C ABI, include/gdla.h): hand-written HIP kernels for gfx950.
This package is its thin Python binding; see gdla.py.
"""

from .gdla import (EXPORTED, GDLA_BF16, GDLA_F32, GDLA_OP_APPEND, GDLA_OP_BACKWARD,  # noqa: F401
                   GDLA_OP_DECODE, GDLA_OP_PREFILL, GDLA_OP_PREFILL_PAGED, GRAD_FIELDS, GdlaGrads,
                   gdla_backward, STAGES, GdlaDebug, StageTimer, GdlaDims,
                   GdlaError, GdlaPagedCache, GdlaWeights, LIB_PATH, MAX_DECODE_TOKENS, PagedCache,
                   NOALLOC_SCRATCH_BYTES, gdla_decode, gdla_decode_noalloc, gdla_decode_paged, gdla_decode_tokens, gdla_latent_append,
                   gdla_latent_append_paged, gdla_prefill, gdla_prefill_packed, gdla_prefill_paged,
                   gdla_prepare_weights, gdla_prepared_weights_bytes, gdla_prefill_prepared,
                   gdla_workspace_bytes, lib, make_dims, make_weights)
