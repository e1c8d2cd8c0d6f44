/*
 * gdla.h -- C ABI of the GDLA (Grouped Differential Latent Attention) forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the GDLA token mixer of the Motif 3 Technical Report (picx.dev summary,
 * section 2.2, Eq.(1)-(10); paperglide reader, section "Model Architecture", Figure 1 caption):
 *
 *   c^Q  = RMSNorm(x W_qa) * gamma_q                                   Eq.(1)
 *   q^C  = c^Q W_qc,  q^R = RoPE(c^Q W_qr)            (per query head)  Eq.(2)
 *   c^KV = x W_dkv,   k^R = RoPE(x W_kr)              (one k^R/token)   Eq.(3)
 *   cbar = RMSNorm(c^KV) * gamma_kv                                     Eq.(4)
 *   K^C  = cbar W_uk, V = cbar W_uv                   (per KV head)     Eq.(5)
 *   n_N  = n_H / (g + 1), n_S = g n_N                                   Eq.(6)
 *   lambda = sigmoid(x W_lambda)                      (one per signal head and token) Eq.(7)
 *   H_h  = softmax_s(tau (q^C_h . K^C_s + q^R_h . k^R_s)) V_s          (per head)
 *   D_i  = H_i - lambda_i H_{n_S + (i mod n_N)}                         Eq.(8)
 *   G    = c^Q W_gate                                                   Eq.(9)
 *   out  = vec(sigmoid(G) * D) W_o                                      Eq.(10)
 *
 * Readings where the pages are silent (shared with the oracle and the tests):
 *   - heads 0..n_S-1 are signal heads, n_S..n_H-1 noise heads;
 *   - Repeat_g tiles: signal head i subtracts noise head (i mod n_N);
 *   - query head -> KV head: signal i -> i mod n_KV, noise j -> j mod n_KV (n_KV divides n_N);
 *   - RoPE rotates the pair (j, j + d_rope/2) by p * rope_theta^(-2j/d_rope), p = absolute
 *     0-based position of the token;
 *   - tau = softmax_scale, or 1/sqrt(d_head + d_rope) when softmax_scale is 0;
 *   - key s is visible from query p iff s <= p and (window == 0 or p - s < window).
 *
 * The latent KV cache holds, per sequence and position, one row [cbar (d_kv_latent) ; k^R
 * (d_rope)] after RMSNorm/gamma and after RoPE: the MLA property that only the latent is stored
 * and K/V are rebuilt inside attention (paperglide reader, "Model Architecture", MLA answer).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless their name ends in _host.
 *   - Tensors are dense and row-major; every tensor of one call has the dtype dims->dtype.
 *     Weights use the row-vector convention x W, so W is [in, out].
 *   - Accumulation is fp32 in every dtype.
 *   - The caller owns every buffer (inputs, weights, cache, out, workspace, debug outputs).
 *     The library allocates no device memory, keeps no per-call state, never synchronises the
 *     stream and launches only on `stream`.  Calls on different streams may run concurrently if
 *     their workspaces, outputs and written cache rows do not overlap.
 *   - All argument checks run before the first launch: on any error nothing is launched and no
 *     buffer is written.  A HIP launch failure returns GDLA_ERR_HIP (work already queued on the
 *     stream by the same call may then have run).  No C++ exception crosses this interface.
 *   - gdla_last_error() returns a short description of the last failure on the calling thread.
 *   - Size limits (GDLA_ERR_UNSUPPORTED, or a workspace size of 0): B T <= 2^30 rows per call,
 *     max_len <= 2^30, d_model and d_q_latent <= 65536, n_heads <= 1024, d_head <= 256,
 *     d_rope <= 64, d_kv_latent + d_rope <= 1024.
 *   - Numerical range of the bf16 layers: the fast paths round every matrix-core operand once, to
 *     nearest even: bf16 for the attention operands (q^C/q^R, K^C/k^R, V and P of prefill; the
 *     absorbed query, the cache and P of decode), fp16 for c^Q and Y in the projections and for
 *     every operand of the fused backward (the gradients included).  An fp16 operand beyond
 *     fp16's range (|v| > 65504) becomes +-inf and a NaN stays a NaN, so such inputs give
 *     non-finite outputs, never finite wrong ones; the library itself checks no values.  c^Q and cbar are RMS-normalised, so the range binds only through the
 *     weights' and gains' magnitudes, k^R (linear in x) and V.  A NaN in a key may also reach the
 *     outputs of the earlier queries of its 64-key tile (a masked probability of 0 times NaN).
 */
#ifndef GDLA_H_
#define GDLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDLA_OK = 0,
  GDLA_ERR_INVALID_ARG = 1,   /* null pointer, inconsistent sizes, bad alignment */
  GDLA_ERR_UNSUPPORTED = 2,   /* valid layer, but a size or dtype the library does not serve */
  GDLA_ERR_WORKSPACE = 3,     /* ws_bytes smaller than gdla_workspace_bytes(...) */
  GDLA_ERR_OUT_OF_RANGE = 4,  /* a position + T exceeds max_len, or a negative position */
  GDLA_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} gdla_status;

typedef enum { GDLA_F32 = 0, GDLA_BF16 = 1 } gdla_dtype;

typedef enum {
  GDLA_OP_PREFILL = 0,
  GDLA_OP_DECODE = 1,        /* gdla_decode, gdla_decode_tokens and gdla_decode_paged */
  GDLA_OP_APPEND = 2,        /* gdla_latent_append and gdla_latent_append_paged */
  GDLA_OP_PREFILL_PAGED = 3, /* gdla_prefill_paged (max_len = max_blocks * page_rows) */
  GDLA_OP_BACKWARD = 4       /* gdla_backward (pos_host NULL, max_len = T) */
} gdla_op;

/* Most new tokens per sequence that gdla_decode_tokens takes in one call. */
#define GDLA_MAX_DECODE_TOKENS 16

/* Size of gdla_decode_noalloc's static device scratch (96 MiB): enough for a decode step of 64
 * sequences of the 4096-wide, 80-head layer at any context length (68 MiB). */
#define GDLA_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)

/* Layer sizes (picx.dev summary section 2.2).  n_heads = n_signal + n_noise, n_signal is a
 * multiple g of n_noise (Eq.(6)), and n_kv_heads divides n_noise. */
typedef struct {
  int32_t d_model;       /* width of x and out */
  int32_t n_heads;       /* n_H: all query heads */
  int32_t n_signal;      /* n_S */
  int32_t n_noise;       /* n_N */
  int32_t n_kv_heads;    /* KV heads shared by the signal and noise paths */
  int32_t d_q_latent;    /* width of c^Q */
  int32_t d_kv_latent;   /* width of c^KV / cbar */
  int32_t d_head;        /* q^C, K^C and V width per head */
  int32_t d_rope;        /* q^R and k^R width (even) */
  int32_t window;        /* 0: full causal; W > 0: key s visible iff 0 <= p - s < W */
  float rms_eps;         /* RMSNorm epsilon (e.g. 1e-6) */
  float rope_theta;      /* RoPE base (e.g. 10000) */
  float softmax_scale;   /* 0 selects 1/sqrt(d_head + d_rope) */
  gdla_dtype dtype;      /* GDLA_F32, or GDLA_BF16 (inputs, weights, cache and out in bf16) */
} gdla_dims;

/* Layer weights, all [in, out] row-major in dims->dtype.  gamma_q / gamma_kv may be NULL (all
 * ones).  Head h of w_qc / w_qr / w_gate and KV head j of w_uk / w_uv are the column blocks h / j.
 * w_o rows follow vec(Y): row i*d_head + e belongs to signal head i, element e. */
typedef struct {
  const void *w_qa;      /* [d_model, d_q_latent]              Eq.(1) */
  const void *gamma_q;   /* [d_q_latent] or NULL                Eq.(1) */
  const void *w_qc;      /* [d_q_latent, n_heads * d_head]      Eq.(2) */
  const void *w_qr;      /* [d_q_latent, n_heads * d_rope]      Eq.(2) */
  const void *w_dkv;     /* [d_model, d_kv_latent]              Eq.(3) */
  const void *w_kr;      /* [d_model, d_rope]                   Eq.(3) */
  const void *gamma_kv;  /* [d_kv_latent] or NULL               Eq.(4) */
  const void *w_uk;      /* [d_kv_latent, n_kv_heads * d_head]  Eq.(5) */
  const void *w_uv;      /* [d_kv_latent, n_kv_heads * d_head]  Eq.(5) */
  const void *w_lambda;  /* [d_model, n_signal]                 Eq.(7) */
  const void *w_gate;    /* [d_q_latent, n_signal * d_head]     Eq.(9) */
  const void *w_o;       /* [n_signal * d_head, d_model]        Eq.(10) */
} gdla_weights;

/* Optional test and profiling hooks; pass NULL (or a struct of NULLs) in production. */
typedef struct {
  const float *lambda_override;  /* [B, T, n_signal] fp32: used instead of sigmoid(x W_lambda) */
  float *out_heads;              /* [B, T, n_heads, d_head] fp32: per-head H before Eq.(8) */
  /* Host array of 2 * GDLA_N_STAGES caller-created hipEvent_t (or NULL).  When set, the call
   * records stage_events[2k] on `stream` before stage k and stage_events[2k + 1] after it, so a
   * caller can time every kernel of the call with hipEventElapsedTime.  Stages that a call does
   * not run get both events recorded back to back.  A NULL entry skips that record (to time some
   * stages only: each record is a packet on the stream). */
  hipEvent_t *stage_events;
} gdla_debug;

/* Stages reported through gdla_debug.stage_events. */
enum {
  GDLA_STAGE_PROJ_IN = 0,    /* x [W_qa | W_dkv | W_kr | W_lambda]                  Eq.(1),(3),(7) */
  GDLA_STAGE_NORM_APPEND,    /* RMSNorm, RoPE of k^R, sigmoid, cache append         Eq.(1),(4),(7) */
  GDLA_STAGE_EXPAND_KV,      /* prefill: K^C, V of the visible keys                 Eq.(5) */
  GDLA_STAGE_PROJ_Q,         /* c^Q [W_qc | W_qr | W_gate], RoPE of q^R; decode on the bf16 MFMA
                                path also the absorbed query q~                     Eq.(2),(9) */
  GDLA_STAGE_ATTN_NOISE,     /* prefill: noise-head attention; decode: latent attention of all
                                heads over the cache (MFMA path: the split-L kernel alone) */
  GDLA_STAGE_ATTN_SIGNAL,    /* prefill: signal-head attention + Eq.(8) combine + gate;
                                decode: split merge, un-absorb, combine + gate      Eq.(8)-(10) */
  GDLA_STAGE_PROJ_OUT,       /* vec(.) W_o                                          Eq.(10) */
  GDLA_N_STAGES
};

/* Bytes of workspace that op needs for B sequences of T new tokens each (GDLA_OP_DECODE: T = 1
 * for gdla_decode, 1 .. GDLA_MAX_DECODE_TOKENS for gdla_decode_tokens).
 * pos_host (host, [B], may be NULL) gives the first new position of each sequence; with NULL the
 * size is an upper bound for any positions with pos + T <= max_len.  Returns 0 for invalid
 * dims or sizes.  The workspace must be 256-byte aligned. */
size_t gdla_workspace_bytes(const gdla_dims *dims, int32_t op, int32_t B, int32_t T,
                            const int32_t *pos_host, int32_t max_len);

/* Eq.(3)-(4) plus RoPE: writes cache rows [pos_host[b], pos_host[b] + T) of every sequence b from
 * x [B, T, d_model].  cache is [B, max_len, d_kv_latent + d_rope]; other rows are untouched. */
gdla_status gdla_latent_append(const gdla_dims *dims, const gdla_weights *w, const void *x,
                               int32_t B, int32_t T, const int32_t *pos_host, void *cache,
                               int32_t max_len, void *ws, size_t ws_bytes, hipStream_t stream);

/* Prefill / chunked prefill, Eq.(1)-(10): the T tokens of sequence b sit at positions
 * pos_host[b] .. pos_host[b] + T - 1.  Their latent rows are appended to the cache, then every
 * token attends over cache rows [0, its position] (window permitting), expanded K/V form.
 * x [B, T, d_model] -> out [B, T, d_model].  out must not alias x, the cache or the workspace. */
gdla_status gdla_prefill(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                         int32_t T, const int32_t *pos_host, void *cache, int32_t max_len,
                         void *out, void *ws, size_t ws_bytes, const gdla_debug *dbg,
                         hipStream_t stream);

/* Prepared weights for prefill: the transposed copies of the ten projection weights that the
 * prefill's large GEMMs read (K-contiguous; the weights applied to x and to the cache in bf16, those
 * applied to fp16 activations, W_qc / W_qr / W_gate / W_o, converted to fp16).  gdla_prefill makes
 * them in its workspace on every call; a caller that keeps a layer's weights resident makes them
 * once with gdla_prepare_weights and passes them to gdla_prefill_prepared instead (Eq.(1)-(5),
 * (9), (10) of picx.dev summary section 2.2 are unchanged; only where the weights' copies come
 * from differs).  gdla_prepared_weights_bytes returns the buffer size, or 0 for layers whose
 * prefill reads no transposed weights (fp32 layers, head sizes other than 128 + 64). */
size_t gdla_prepared_weights_bytes(const gdla_dims *dims);

/* Writes the prepared weights of w into `prepared` (device, 256-byte aligned, at least
 * gdla_prepared_weights_bytes(dims) bytes, owned by the caller), asynchronously on `stream`.
 * Call again whenever the weights change.  Errors: GDLA_ERR_UNSUPPORTED when the layer takes none,
 * GDLA_ERR_INVALID_ARG for NULL or misaligned pointers, GDLA_ERR_WORKSPACE when prepared_bytes is
 * too small; nothing is launched on error. */
gdla_status gdla_prepare_weights(const gdla_dims *dims, const gdla_weights *w, void *prepared,
                                 size_t prepared_bytes, hipStream_t stream);

/* gdla_prefill with prepared weights (the same arguments, plus the buffer gdla_prepare_weights
 * filled from the same w): identical results, without the per-call transposes.  w is still read
 * (gains, and the projections of calls too small for the transposed-weight GEMM).  Workspace:
 * gdla_workspace_bytes(dims, GDLA_OP_PREFILL, ...), as for gdla_prefill.  Errors as gdla_prefill,
 * plus those of the prepared buffer (as gdla_prepare_weights). */
gdla_status gdla_prefill_prepared(const gdla_dims *dims, const gdla_weights *w, const void *prepared,
                                  size_t prepared_bytes, const void *x, int32_t B, int32_t T,
                                  const int32_t *pos_host, void *cache, int32_t max_len, void *out,
                                  void *ws, size_t ws_bytes, const gdla_debug *dbg, hipStream_t stream);

/* One decode step per sequence: token b (x [B, d_model]) sits at position pos_host[b] (= number
 * of rows already cached).  Its latent row is appended, then it attends over cache rows
 * [0, pos_host[b]] in the absorbed form (queries mapped into the latent space, values mapped out
 * after the softmax average).  out [B, d_model]. */
gdla_status gdla_decode(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                        const int32_t *pos_host, void *cache, int32_t max_len, void *out,
                        void *ws, size_t ws_bytes, const gdla_debug *dbg, hipStream_t stream);

/* gdla_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace: the library uses
 * a static device array of GDLA_NOALLOC_SCRATCH_BYTES instead, one per GPU, held from the first
 * call on that GPU until the process ends.  The caller still passes x, the cache and out (as for
 * gdla_decode); the call allocates nothing and clears nothing (every scratch byte it reads it has
 * written).  All calls on one GPU share that GPU's array, so calls that overlap on one GPU (other
 * streams, other host threads) race: the caller orders them.  The stream must belong to the
 * current device.  Errors as gdla_decode, plus GDLA_ERR_WORKSPACE (nothing launched) when the
 * call needs more than GDLA_NOALLOC_SCRATCH_BYTES (gdla_workspace_bytes(dims, GDLA_OP_DECODE, B,
 * 1, pos_host, max_len) tells), and GDLA_ERR_HIP when the scratch has no address on the device. */
gdla_status gdla_decode_noalloc(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                                const int32_t *pos_host, void *cache, int32_t max_len, void *out,
                                const gdla_debug *dbg, hipStream_t stream);

/* gdla_prefill over packed documents (paperglide reader, Figure 4 (a): a training sequence that
 * holds 473 documents, drawn on the QK^T score matrix): every token attends only to keys of its own
 * document, inside the window.  doc_start is a device int32 array [B, T]: for token t of sequence
 * b, the position of the first token of its document (0 <= doc_start <= pos_host[b] + t; a
 * document may have started in an earlier chunk).  Within a sequence doc_start must not decrease
 * (documents are contiguous); the kernels clamp out-of-range values into [0, position].  All other
 * arguments, the workspace (GDLA_OP_PREFILL) and the errors are those of gdla_prefill, plus
 * GDLA_ERR_INVALID_ARG for a NULL or misaligned doc_start. */
gdla_status gdla_prefill_packed(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                int32_t B, int32_t T, const int32_t *pos_host,
                                const int32_t *doc_start, void *cache, int32_t max_len, void *out,
                                void *ws, size_t ws_bytes, const gdla_debug *dbg,
                                hipStream_t stream);

/* Several new tokens per sequence on the absorbed decode path: the verification step of
 * self-speculative decoding with a multi-token-prediction head (picx.dev summary section 2.1, the
 * MTP component; alphasignal.ai news page, "A wall of custom parts").  The T tokens of sequence b
 * (x [B, T, d_model], 0 <= T <= GDLA_MAX_DECODE_TOKENS) sit at positions pos_host[b] ..
 * pos_host[b] + T - 1.  Their latent rows are appended, then token i attends over cache rows
 * [0, pos_host[b] + i] (window permitting), so the draft tokens see each other causally.  The
 * result is that of gdla_prefill on the same arguments, computed in the absorbed form: every
 * cache row is read from HBM once per sequence for all T tokens.  out [B, T, d_model].  T = 1 is
 * gdla_decode.  Workspace: gdla_workspace_bytes(dims, GDLA_OP_DECODE, B, T, ...).  Errors as
 * gdla_decode, plus GDLA_ERR_INVALID_ARG for T outside 0 .. GDLA_MAX_DECODE_TOKENS. */
gdla_status gdla_decode_tokens(const gdla_dims *dims, const gdla_weights *w, const void *x,
                               int32_t B, int32_t T, const int32_t *pos_host, void *cache,
                               int32_t max_len, void *out, void *ws, size_t ws_bytes,
                               const gdla_debug *dbg, hipStream_t stream);

/* Paged latent cache, for serving several sequences out of one pool of fixed-size pages (the
 * multi-token decode path above is where serving systems use it).  Logical block j of sequence b
 * (positions j * page_rows .. j * page_rows + page_rows - 1) lives in physical page
 * block_table[b * max_blocks + j]; a page holds page_rows cache rows laid out as in the contiguous
 * cache.  The caller owns the pages and the table and may map any page to any block (a sliding-
 * window layer can recycle the pages of positions that have left the window).
 *   - pages: device, [n_pages, page_rows, d_kv_latent + d_rope] in dims->dtype, 16-byte aligned.
 *   - block_table: device int32 [B, max_blocks].  Every block that a call reads or writes (the
 *     visible positions of every new token, and the new positions) must map to a page in
 *     [0, n_pages); the kernels clamp other entries into that range (wrong rows, never a fault).
 *   - page_rows: a positive multiple of 32.
 * Positions run from 0 to max_blocks * page_rows - 1, which plays the role of max_len. */
typedef struct {
  void *pages;
  const int32_t *block_table;
  int32_t n_pages;
  int32_t page_rows;
  int32_t max_blocks;
} gdla_paged_cache;

/* gdla_latent_append over a paged cache. */
gdla_status gdla_latent_append_paged(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                     int32_t B, int32_t T, const int32_t *pos_host,
                                     const gdla_paged_cache *cache, void *ws, size_t ws_bytes,
                                     hipStream_t stream);

/* gdla_prefill over a paged cache: the visible rows of every sequence are gathered into the
 * workspace, the chunk runs as gdla_prefill there, and its new rows are written back to their
 * pages.  Workspace: gdla_workspace_bytes(dims, GDLA_OP_PREFILL_PAGED, B, T, pos_host,
 * max_blocks * page_rows). */
gdla_status gdla_prefill_paged(const gdla_dims *dims, const gdla_weights *w, const void *x,
                               int32_t B, int32_t T, const int32_t *pos_host,
                               const gdla_paged_cache *cache, void *out, void *ws, size_t ws_bytes,
                               const gdla_debug *dbg, hipStream_t stream);

/* gdla_decode_tokens over a paged cache: x [B, T, d_model], 0 <= T <= GDLA_MAX_DECODE_TOKENS
 * (T = 1 is one decode step).  The split-L kernel reads the cache in 32-row tiles, each inside
 * one page.  Workspace: gdla_workspace_bytes(dims, GDLA_OP_DECODE, B, T, ...). */
gdla_status gdla_decode_paged(const gdla_dims *dims, const gdla_weights *w, const void *x,
                              int32_t B, int32_t T, const int32_t *pos_host,
                              const gdla_paged_cache *cache, void *out, void *ws, size_t ws_bytes,
                              const gdla_debug *dbg, hipStream_t stream);

/* Gradient outputs of gdla_backward: fp32 device buffers shaped like the corresponding input,
 * fully overwritten (weight gradients are sums over all B * T tokens). */
typedef struct {
  float *dx;                                       /* [B, T, d_model] */
  float *dw_qa, *dw_qc, *dw_qr, *dw_dkv, *dw_kr;   /* shaped like w_qa, w_qc, w_qr, w_dkv, w_kr */
  float *dw_uk, *dw_uv, *dw_lambda, *dw_gate, *dw_o;
  float *dgamma_q, *dgamma_kv;                     /* [d_q_latent], [d_kv_latent]: required when
                                                      the weights carry gamma_q / gamma_kv, else
                                                      ignored (a fixed gain has no gradient) */
} gdla_grads;

/* Backward pass of the layer for training: B sequences of T tokens at positions 0 .. T-1 (no
 * cached prefix), with the layer's window and, optionally, packed documents (doc_start as in
 * gdla_prefill_packed, or NULL).  Given dout [B, T, d_model] (layer dtype), it writes the
 * gradients of L = sum(out (.) dout) with respect to x and every weight.  The forward is
 * recomputed inside the call (the pages train with activation recomputation: paperglide reader,
 * section "Distributed Training System"); nothing from an earlier forward is needed.
 * dbg->lambda_override, when given, fixes lambda as in the forward (then no gradient flows
 * through W_lambda).  Workspace: gdla_workspace_bytes(dims, GDLA_OP_BACKWARD, B, T, NULL, T).
 * bf16 layers with d_head 128, d_rope 64, d_model, d_q_latent and d_kv_latent multiples of 64 and
 * signal and noise head counts multiples of n_kv take the fused path when B T >= 256, T >= 32 and B times T rounded up to
 * 32 is at most 2^23 (fp16 MFMA operands, fp32 accumulation: about 3e-3 relative error per
 * gradient); the rest compute in fp32.  The fused path scales dout by a power of two computed on the device from its largest
 * magnitude (and the gradients back), so upstream gradients of any scale keep fp16 precision.  Every gradient has a single writer (no atomics), so repeated calls give identical bits.
 * Errors as gdla_prefill, plus GDLA_ERR_INVALID_ARG for a NULL gradient pointer. */
gdla_status gdla_backward(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                          int32_t T, const int32_t *doc_start, const void *dout,
                          const gdla_grads *grads, void *ws, size_t ws_bytes,
                          const gdla_debug *dbg, hipStream_t stream);

/* Static description of a status code. */
const char *gdla_status_string(gdla_status s);

/* Description of the last failure on the calling thread ("" if none). */
const char *gdla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDLA_H_ */
