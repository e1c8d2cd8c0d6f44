// Host side of the GDLA C ABI: argument validation, workspace planning and the launch sequence of
// gdla_latent_append / gdla_prefill / gdla_decode.  Every check runs before the first launch.
#include "gdla_internal.h"
#include "fast_paths.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#define GDLA_EXPORT extern "C" __attribute__((visibility("default")))

namespace gdla {
namespace {

thread_local char g_err[256] = "";

gdla_status fail(gdla_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(GDLA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t esize(gdla_dtype dt) { return dt == GDLA_F32 ? 4 : 2; }

gdla_status check_dims(const gdla_dims *d, LayerDims &ld) {
  if (!d) return fail(GDLA_ERR_INVALID_ARG, "dims is NULL");
  // (a C caller may store any int in the enum field: read it as one)
  int32_t dtype;
  static_assert(sizeof(d->dtype) == sizeof(dtype), "gdla_dtype is an int");
  memcpy(&dtype, &d->dtype, sizeof(dtype));
  if (dtype != GDLA_F32 && dtype != GDLA_BF16) return fail(GDLA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (d->d_model <= 0 || d->n_heads <= 0 || d->n_signal <= 0 || d->n_noise <= 0 ||
      d->n_kv_heads <= 0 || d->d_q_latent <= 0 || d->d_kv_latent <= 0 || d->d_head <= 0 ||
      d->d_rope <= 0 || d->window < 0)
    return fail(GDLA_ERR_INVALID_ARG, "non-positive layer size");
  if ((int64_t)d->n_signal + d->n_noise != d->n_heads)
    return fail(GDLA_ERR_INVALID_ARG, "n_signal + n_noise != n_heads");
  if (d->n_signal % d->n_noise != 0) return fail(GDLA_ERR_INVALID_ARG, "n_noise must divide n_signal");
  if (d->n_noise % d->n_kv_heads != 0) return fail(GDLA_ERR_INVALID_ARG, "n_kv_heads must divide n_noise");
  if (d->d_rope % 2 != 0) return fail(GDLA_ERR_INVALID_ARG, "d_rope must be even");
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f) || !(d->softmax_scale >= 0.f))
    return fail(GDLA_ERR_INVALID_ARG, "rms_eps, rope_theta or softmax_scale out of range");
  // Limits of the generic kernels (per-lane register arrays and LDS tables).
  if (d->d_head > 256 || d->d_rope > 64 || (int64_t)d->d_kv_latent + d->d_rope > 1024)
    return fail(GDLA_ERR_UNSUPPORTED, "d_head <= 256, d_rope <= 64, d_kv_latent + d_rope <= 1024");
  // Widths stay well inside the int32 column counts of the GEMMs (n_heads d_head <= 2^18).
  if (d->d_model > 65536 || d->d_q_latent > 65536 || d->n_heads > 1024)
    return fail(GDLA_ERR_UNSUPPORTED, "d_model <= 65536, d_q_latent <= 65536, n_heads <= 1024");
  ld.d_model = d->d_model; ld.n_heads = d->n_heads; ld.n_signal = d->n_signal;
  ld.n_noise = d->n_noise; ld.n_kv = d->n_kv_heads; ld.d_cq = d->d_q_latent;
  ld.d_c = d->d_kv_latent; ld.d_h = d->d_head; ld.d_r = d->d_rope; ld.window = d->window;
  ld.eps = d->rms_eps; ld.theta = d->rope_theta;
  ld.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)(d->d_head + d->d_rope));
  return GDLA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Most rows (B T tokens) of one call: row counts are int32 on the host and in the kernels, and
// 2^30 leaves room for padding them to whole tiles.
constexpr int64_t kMaxRows = int64_t(1) << 30;
// Most cache positions (max_len): key counts round up to whole tiles in int32.  At 2^30 positions
// one sequence's latent cache alone would exceed a GPU's memory many times over.
constexpr int32_t kMaxPositions = int32_t(1) << 30;

// ---------------------------------------------------------------------------------------------
// Workspace planning.  Every buffer starts on a 256-byte boundary.
struct Plan {
  size_t bytes = 0;
  size_t add(size_t n) {
    const size_t off = bytes;
    bytes += (n + 255) & ~size_t(255);
    return off;
  }
};

// Keys [lo_b, hi_b) of sequence b that a prefill over T tokens starting at p0 may read.
inline int32_t key_lo(int32_t p0, int32_t window) { return window > 0 ? std::max(0, p0 - window + 1) : 0; }

struct PrefillLayout {
  size_t pos, aq, ckv, krp, laml, cq, lam, qc, qrp, qr, gate, kx, vx, heads, y, total;
  size_t wt_qa, wt_dkv, wt_kr, wt_lam, wt_qc, wt_qr, wt_gate, wt_uk, wt_uv, wt_o;
  int32_t lcap;
  FastPrefillLayout fast;
  bool use_fast, use_nt;
};

// Rows from which the transposed-weight GEMM pays for transposing the weights once per call.
constexpr int32_t kNtMinRows = 256;

// Prepared weights (gdla_prepare_weights): the transposed copies the K-contiguous GEMM reads,
// x-side and expansion weights in bf16, the weights applied to fp16 activations in fp16.
struct PreparedLayout {
  size_t qa, dkv, kr, lam, qc, qr, gate, uk, uv, o, total;
};

PreparedLayout plan_prepared(const LayerDims &d) {
  PreparedLayout L{};
  Plan p;
  L.qa = p.add(2 * (size_t)d.d_model * d.d_cq);
  L.dkv = p.add(2 * (size_t)d.d_model * d.d_c);
  L.kr = p.add(2 * (size_t)d.d_model * d.d_r);
  L.lam = p.add(2 * (size_t)d.d_model * d.n_signal);
  L.qc = p.add(2 * (size_t)d.d_cq * d.n_heads * d.d_h);
  L.qr = p.add(2 * (size_t)d.d_cq * d.n_heads * d.d_r);
  L.gate = p.add(2 * (size_t)d.d_cq * d.n_signal * d.d_h);
  L.uk = p.add(2 * (size_t)d.d_c * d.n_kv * d.d_h);
  L.uv = p.add(2 * (size_t)d.d_c * d.n_kv * d.d_h);
  L.o = p.add(2 * (size_t)d.n_signal * d.d_h * d.d_model);
  L.total = p.bytes;
  return L;
}

// The 10 transposed weight copies of one layer into `dst` at the offsets of `off` (a prefill
// workspace's wt_* fields or a prepared-weight buffer's).
hipError_t transpose_layer_weights(const LayerDims &d, const gdla_weights *w, char *dst, const size_t (&off)[10],
                                   hipStream_t stream) {
  struct { const void *w; int32_t K, N; bool f16; } tw[] = {
      {w->w_qa, d.d_model, d.d_cq, false},
      {w->w_dkv, d.d_model, d.d_c, false},
      {w->w_kr, d.d_model, d.d_r, false},
      {w->w_lambda, d.d_model, d.n_signal, false},
      {w->w_qc, d.d_cq, d.n_heads * d.d_h, true},
      {w->w_qr, d.d_cq, d.n_heads * d.d_r, true},
      {w->w_gate, d.d_cq, d.n_signal * d.d_h, true},
      {w->w_uk, d.d_c, d.n_kv * d.d_h, false},
      {w->w_uv, d.d_c, d.n_kv * d.d_h, false},
      {w->w_o, d.n_signal * d.d_h, d.d_model, true},
  };
  for (int i = 0; i < 10; ++i) {
    const hipError_t e = launch_transpose_weight(tw[i].w, dst + off[i], tw[i].K, tw[i].N, tw[i].f16, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int32_t key_capacity(const LayerDims &d, int32_t B, int32_t T, const int32_t *pos, int32_t max_len) {
  int32_t lcap = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t p0 = pos ? pos[b] : max_len - T;
    const int32_t lo = pos ? key_lo(p0, d.window) : 0;
    lcap = std::max(lcap, p0 + T - lo);
  }
  return lcap;
}

PrefillLayout plan_prefill(const LayerDims &d, gdla_dtype dt, int32_t B, int32_t T,
                           const int32_t *pos, int32_t max_len) {
  PrefillLayout L{};
  const size_t es = esize(dt);
  const size_t M = (size_t)B * T;
  L.use_fast = fast_prefill_supported(d, dt);
  L.lcap = key_capacity(d, B, T, pos, max_len);
  if (L.use_fast) L.lcap = fast_prefill_lcap(L.lcap);
  Plan p;
  L.pos = p.add(sizeof(int32_t) * B);
  L.aq = p.add(4 * M * d.d_cq);
  L.ckv = p.add(4 * M * d.d_c);
  L.krp = p.add(4 * M * d.d_r);
  L.laml = p.add(4 * M * d.n_signal);
  L.cq = p.add(es * M * d.d_cq);
  L.lam = p.add(4 * M * d.n_signal);
  L.gate = p.add(4 * M * d.n_signal * d.d_h);
  L.kx = p.add(es * (size_t)B * d.n_kv * L.lcap * (L.use_fast ? fast_prefill_key_row() : d.d_h));
  L.vx = p.add(es * (size_t)B * d.n_kv * L.lcap * d.d_h);
  L.y = p.add(es * M * d.n_signal * d.d_h);
  if (L.use_fast) {
    L.fast = plan_fast_prefill(d, B, T, [&](size_t n) { return p.add(n); });
    // (the RoPE epilogue of the transposed-weight GEMM takes sequences of at least 32 tokens)
    L.use_nt = (int64_t)B * T >= kNtMinRows && T >= 32 && d.d_c % 64 == 0;
    if (L.use_nt) {
      L.wt_qa = p.add(2 * (size_t)d.d_model * d.d_cq);
      L.wt_dkv = p.add(2 * (size_t)d.d_model * d.d_c);
      L.wt_kr = p.add(2 * (size_t)d.d_model * d.d_r);
      L.wt_lam = p.add(2 * (size_t)d.d_model * d.n_signal);
      L.wt_qc = p.add(2 * (size_t)d.d_cq * d.n_heads * d.d_h);
      L.wt_qr = p.add(2 * (size_t)d.d_cq * d.n_heads * d.d_r);
      L.wt_gate = p.add(2 * (size_t)d.d_cq * d.n_signal * d.d_h);
      L.wt_uk = p.add(2 * (size_t)d.d_c * d.n_kv * d.d_h);
      L.wt_uv = p.add(2 * (size_t)d.d_c * d.n_kv * d.d_h);
      L.wt_o = p.add(2 * (size_t)d.n_signal * d.d_h * d.d_model);
    }
  } else {
    L.qc = p.add(es * M * d.n_heads * d.d_h);
    L.qrp = p.add(4 * M * d.n_heads * d.d_r);
    L.qr = p.add(es * M * d.n_heads * d.d_r);
    L.heads = p.add(4 * M * d.n_heads * d.d_h);
  }
  L.total = p.bytes;
  return L;
}

struct DecodeLayout {
  size_t pos, aq, ckv, krp, laml, cq, lam, qc, qrp, qr, gate, qabs, o, heads, y, skinny, total;
  size_t cq_lo, y_lo;   // bf16 rounding remainders of c^Q and Y (skinny projections), or 0 bytes
  size_t skinny_bytes;  // split-K partial sums of the skinny projection GEMMs (0: not used)
  FastDecodeLayout fast;
  bool use_fast;
};

// T new tokens per sequence: M = B T query rows.
DecodeLayout plan_decode(const LayerDims &d, gdla_dtype dt, int32_t B, int32_t T, int32_t max_len) {
  DecodeLayout L{};
  const size_t es = esize(dt);
  const size_t M = (size_t)B * T;
  L.use_fast = fast_decode_supported(d, dt);
  Plan p;
  L.pos = p.add(sizeof(int32_t) * B);
  L.aq = p.add(4 * M * d.d_cq);
  L.ckv = p.add(4 * M * d.d_c);
  L.krp = p.add(4 * M * d.d_r);
  L.laml = p.add(4 * M * d.n_signal);
  L.cq = p.add(es * M * d.d_cq);
  L.lam = p.add(4 * M * d.n_signal);
  L.qc = p.add(4 * M * d.n_heads * d.d_h);
  L.qrp = p.add(4 * M * d.n_heads * d.d_r);
  L.qr = p.add(4 * M * d.n_heads * d.d_r);
  L.gate = p.add(4 * M * d.n_signal * d.d_h);
  L.heads = p.add(4 * M * d.n_heads * d.d_h);
  L.y = p.add(es * M * d.n_signal * d.d_h);
  L.skinny_bytes = (dt == GDLA_BF16 && M <= 256) ? skinny_gemm_partial_bound((int32_t)M) : 0;
  L.skinny = p.add(L.skinny_bytes);
  // c^Q and Y enter the skinny projections as bf16 + bf16 remainder (about 16 bits)
  const bool two_part = L.skinny_bytes > 0;
  L.cq_lo = p.add(two_part ? 2 * M * d.d_cq : 0);
  L.y_lo = p.add(two_part ? 2 * M * d.n_signal * d.d_h : 0);
  if (L.use_fast) {
    L.fast = plan_fast_decode(d, (int32_t)M, max_len, [&](size_t n) { return p.add(n); });
  } else {
    L.qabs = p.add(4 * M * d.n_heads * (d.d_c + d.d_r));
    L.o = p.add(4 * M * d.n_heads * d.d_c);
  }
  L.total = p.bytes;
  return L;
}

struct AppendLayout {
  size_t pos, ckv, krp, total;
};

AppendLayout plan_append(const LayerDims &d, int32_t B, int32_t T) {
  AppendLayout L{};
  const size_t M = (size_t)B * T;
  Plan p;
  L.pos = p.add(sizeof(int32_t) * B);
  L.ckv = p.add(4 * M * d.d_c);
  L.krp = p.add(4 * M * d.d_r);
  L.total = p.bytes;
  return L;
}

// Workspace of a paged prefill: the contiguous prefill's (over stage_len positions), then the
// positions and the staging cache [B, stage_len, d_c + d_r] that the visible rows are gathered into.
struct PagedPrefillLayout {
  PrefillLayout pre;
  size_t pos, stage, total;
  int32_t stage_len, max_gather;
};

PagedPrefillLayout plan_prefill_paged(const LayerDims &d, gdla_dtype dt, int32_t B, int32_t T,
                                      const int32_t *pos, int32_t max_len) {
  PagedPrefillLayout L{};
  L.stage_len = pos ? 0 : max_len;
  L.max_gather = pos ? 0 : max_len - T;
  if (pos)
    for (int32_t b = 0; b < B; ++b) {
      L.stage_len = std::max(L.stage_len, pos[b] + T);
      L.max_gather = std::max(L.max_gather, pos[b] - key_lo(pos[b], d.window));
    }
  L.pre = plan_prefill(d, dt, B, T, pos, L.stage_len);
  Plan p;
  p.bytes = L.pre.total;
  L.pos = p.add(sizeof(int32_t) * B);
  L.stage = p.add(esize(dt) * (size_t)B * L.stage_len * (d.d_c + d.d_r));
  L.total = p.bytes;
  return L;
}

// Workspace of the backward: fp32 buffers of M = B T rows (fields of BwdBuffers, in order).
struct BackwardLayout {
  size_t off[34];
  size_t total;
};

BackwardLayout plan_backward(const LayerDims &d, int32_t B, int32_t T) {
  const size_t M = (size_t)B * T;
  const size_t nH = d.n_heads, nS = d.n_signal, nKV = d.n_kv;
  const size_t cols[34] = {
      (size_t)d.d_cq, (size_t)d.d_c, (size_t)d.d_r, nS, (size_t)d.d_cq, (size_t)d.d_c, (size_t)d.d_r, nS, 1, 1,
      nH * d.d_h, nH * d.d_r, nS * d.d_h, nKV * d.d_h, nKV * d.d_h, nH * d.d_h, nH,
      nS * d.d_h, nS * d.d_h, nH * d.d_h, nS * d.d_h, nS * d.d_h, nS, nH,
      nH * d.d_h, nH * d.d_r, nKV * d.d_h, nKV * d.d_h, nKV * d.d_r, (size_t)d.d_r, (size_t)d.d_c, (size_t)d.d_c,
      (size_t)d.d_cq, (size_t)d.d_cq};
  static_assert(sizeof(BwdBuffers) == 34 * sizeof(float *), "one column count per buffer");
  BackwardLayout L{};
  Plan p;
  for (int i = 0; i < 34; ++i) L.off[i] = p.add(4 * M * cols[i]);
  L.total = p.bytes;
  return L;
}

// Fast backward (bf16, the fused forward with transposed weights): the forward's workspace over T
// positions from 0, its cache, output, per-head H, log-sum-exp and key-major V, then the buffers
// of FastBwdBuffers.
struct FastBackwardLayout {
  PrefillLayout pre;
  size_t cache, out, heads, lse, vk;
  size_t fb[31];  // FastBwdBuffers fields, in order
  size_t total;
  int32_t M_pad, k8;
  bool ok;
};

FastBackwardLayout plan_backward_fast(const LayerDims &d, int32_t B, int32_t T) {
  FastBackwardLayout L{};
  // (positions 0 .. T-1 of every sequence: the bound over all positions is exact here)
  L.pre = plan_prefill(d, GDLA_BF16, B, T, nullptr, T);
  // (the dK/dV kernel addresses the dim-major copies with 32-bit offsets: at most 2^23 padded tokens)
  L.ok = L.pre.use_fast && L.pre.use_nt && fast_backward_supported(d, GDLA_BF16) &&
         (int64_t)B * ((T + 31) / 32 * 32) <= ((int64_t)1 << 23);
  if (!L.ok) return L;
  const size_t M = (size_t)B * T, nH = d.n_heads, nS = d.n_signal, nKV = d.n_kv;
  L.M_pad = (int32_t)((M + 63) / 64 * 64);
  L.k8 = (d.d_cq + d.d_c + d.d_r + d.n_signal + 63) / 64 * 64;
  const size_t Mp = L.M_pad, dm = d.d_model, dh = d.d_h, dr = d.d_r;
  const size_t k3 = 2 * nKV * dh, k6 = nH * dh + nH * dr + nS * dh, k8 = L.k8;
  Plan p;
  p.bytes = L.pre.total;
  L.cache = p.add(2 * M * (d.d_c + d.d_r));
  L.out = p.add(2 * M * dm);
  L.heads = p.add(4 * M * nH * dh);
  L.lse = p.add(4 * (M * nH + 32));  // head-major, 32 entries of padding
  L.vk = p.add(2 * (size_t)B * nKV * L.pre.lcap * dh);
  const size_t BTp = (size_t)B * ((T + 31) / 32 * 32);  // dim-major copies: B rows of T rounded to 32
  const size_t trows_a = std::max({nS * dh, (size_t)d.d_c, (size_t)d.d_cq, dm});
  const size_t trows_b = std::max({dm, k3, k6, k8});
  const size_t bytes[31] = {
      2 * nS * dh * dm, 2 * d.d_c * k3, 2 * d.d_cq * k6, 2 * dm * k8,      // wo16 w3 w6 w8
      2 * M * dm, 4 * M * nS * dh,                                          // dout16 dy
      2 * trows_a * Mp, 2 * trows_b * Mp,                                   // ta tb
      0, 4 * (kGradScaleBlocks + 2), 4 * M * nS, 4 * (M * nH + 32),         // (dheads: unused) gscale dlaml drow
      2 * M * nH * dh,                                                      // dh16
      2 * nH * (dh + dr) * BTp, 2 * nH * dh * BTp,                          // qT dhT
      0, 4 * M * nKV * (dh + dr), 4 * M * nKV * dh,                         // dq (packed by the kernel) dk dv
      2 * M * k6, 2 * M * k3, 2 * M * k8,                                   // a6 a3 a8
      4 * M * dr, 4 * M * d.d_c, 4 * M * d.d_c, 4 * M, 4 * M * d.d_cq, 4 * M * d.d_cq, 4 * M,
      4 * (M + 32), 8 * (size_t)T * (dr / 2),                             // lo rope_cs
      kSplitKBytes};                                                        // splitk
  static_assert(sizeof(FastBwdBuffers) == 31 * sizeof(void *), "one size per buffer");
  for (int i = 0; i < 31; ++i) L.fb[i] = p.add(bytes[i]);
  L.total = p.bytes;
  return L;
}

// ---------------------------------------------------------------------------------------------
gdla_status check_call(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                       int32_t T, const int32_t *pos, const void *cache, int32_t max_len,
                       const void *out, bool need_query_weights, LayerDims &ld) {
  gdla_status st = check_dims(dims, ld);
  if (st != GDLA_OK) return st;
  if (B < 0 || T < 0 || max_len <= 0) return fail(GDLA_ERR_INVALID_ARG, "negative B/T or max_len <= 0");
  if (max_len > kMaxPositions) return fail(GDLA_ERR_UNSUPPORTED, "max_len = %d above 2^30", max_len);
  if (B == 0 || T == 0) return GDLA_OK;
  if ((int64_t)B * T > kMaxRows) return fail(GDLA_ERR_UNSUPPORTED, "B T = %lld rows above 2^30", (long long)B * T);
  if (!w) return fail(GDLA_ERR_INVALID_ARG, "weights is NULL");
  if (!x || !cache || !pos) return fail(GDLA_ERR_INVALID_ARG, "x, cache or pos_host is NULL");
  if (need_query_weights && !out) return fail(GDLA_ERR_INVALID_ARG, "out is NULL");
  const void *req[] = {w->w_dkv, w->w_kr};
  for (const void *p : req)
    if (!p) return fail(GDLA_ERR_INVALID_ARG, "a required weight pointer is NULL");
  if (need_query_weights) {
    const void *req2[] = {w->w_qa, w->w_qc, w->w_qr, w->w_uk, w->w_uv, w->w_lambda, w->w_gate, w->w_o};
    for (const void *p : req2)
      if (!p) return fail(GDLA_ERR_INVALID_ARG, "a required weight pointer is NULL");
  }
  const void *al[] = {x, cache, out, w->w_qa, w->w_qc, w->w_qr, w->w_dkv, w->w_kr, w->w_uk,
                      w->w_uv, w->w_lambda, w->w_gate, w->w_o, w->gamma_q, w->gamma_kv};
  for (const void *p : al)
    if (p && !aligned16(p)) return fail(GDLA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  for (int32_t b = 0; b < B; ++b) {
    if (pos[b] < 0) return fail(GDLA_ERR_OUT_OF_RANGE, "pos_host[%d] = %d < 0", b, pos[b]);
    if ((int64_t)pos[b] + T > max_len)
      return fail(GDLA_ERR_OUT_OF_RANGE, "pos_host[%d] + T = %lld > max_len %d", b,
                  (long long)pos[b] + T, max_len);
  }
  return GDLA_OK;
}

gdla_status check_ws(const void *ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return fail(GDLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (need > 0 && !ws) return fail(GDLA_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(GDLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return GDLA_OK;
}

template <typename T> T *at(void *base, size_t off) { return (T *)((char *)base + off); }

GemmProblem gp(const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
               int32_t M, int32_t N, int32_t K, bool c_f32, int epi = EPI_NONE) {
  GemmProblem p{};
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb; p.C = C; p.ldc = ldc;
  p.M = M; p.N = N; p.K = K; p.hw = N > 0 ? N : 1; p.hs = 0; p.ho = 0;
  p.c_dt = c_f32 ? CD_F32 : CD_IN; p.a_f16 = 0; p.epi = epi;
  return p;
}

// The projections of a decode batch: problems the skinny split-K kernel serves (bf16, at most 256
// rows, columns in tiles of 64) run there, given workspace for its partial sums; the rest go to
// the general dispatch.
hipError_t launch_gemm_rows(GemmBatch &g, DT dt, void *partial, size_t partial_bytes, hipStream_t s) {
  if (dt != DT::BF16 || partial_bytes == 0) return launch_gemm(g, dt, s);
  GemmBatch sk{}, rest{};
  for (int i = 0; i < g.n; ++i) {
    if (skinny_problem_ok(g.p[i])) sk.p[sk.n++] = g.p[i];
    else rest.p[rest.n++] = g.p[i];
  }
  if (sk.n && skinny_gemm_partial_bytes(sk) <= partial_bytes) {
    const hipError_t e = launch_gemm_skinny(sk, partial, partial_bytes, s);
    if (e != hipSuccess) return e;
  } else {
    for (int i = 0; i < sk.n; ++i) rest.p[rest.n++] = sk.p[i];
  }
  return rest.n ? launch_gemm(rest, dt, s) : hipSuccess;
}

// First projection, Eq.(1), (3), (7) (x W_qa, x W_dkv, x W_kr, x W_lambda) and the row-wise
// normalisation / RoPE / cache append / sigmoid step.
gdla_status project_and_append(const LayerDims &d, DT dt, const gdla_weights *w, const void *x,
                               int32_t M, int32_t T, const int32_t *pos_dev, const CacheRef &cache,
                               float *aq, float *ckv, float *krp, float *laml,
                               void *cq, float *lam, const float *lam_override, hipStream_t s,
                               StageEvents &se, bool cq_f16 = false, const NtWeights *nt = nullptr,
                               void *partial = nullptr, size_t partial_bytes = 0, void *cq_lo = nullptr) {
  GemmBatch g{};
  // with nt, B is the transposed weight [N, K] (row stride K = d_model)
  auto wb = [&](const void *w_, const void *wt) { return nt ? wt : w_; };
  auto ldw = [&](int64_t n) { return nt ? (int64_t)d.d_model : n; };
  g.p[g.n++] = gp(x, d.d_model, wb(w->w_dkv, nt ? nt->dkv : nullptr), ldw(d.d_c), ckv, d.d_c, M, d.d_c,
                  d.d_model, true);
  g.p[g.n++] = gp(x, d.d_model, wb(w->w_kr, nt ? nt->kr : nullptr), ldw(d.d_r), krp, d.d_r, M, d.d_r,
                  d.d_model, true);
  if (cq)
    g.p[g.n++] = gp(x, d.d_model, wb(w->w_qa, nt ? nt->qa : nullptr), ldw(d.d_cq), aq, d.d_cq, M, d.d_cq,
                    d.d_model, true);
  GemmBatch plain{};  // with nt: problems whose output the transposed-weight GEMM cannot store
  if (lam && !lam_override) {
    GemmProblem pl = gp(x, d.d_model, wb(w->w_lambda, nt ? nt->lam : nullptr), ldw(d.n_signal), laml, d.n_signal,
                        M, d.n_signal, d.d_model, true);
    if (nt && !nt_gemm_problem_ok(pl))
      plain.p[plain.n++] = gp(x, d.d_model, w->w_lambda, d.n_signal, laml, d.n_signal, M, d.n_signal, d.d_model, true);
    else
      g.p[g.n++] = pl;
  }
  // with nt the caller has opened GDLA_STAGE_PROJ_IN before transposing the weights
  if (nt) {
    HIP_TRY(launch_gemm_nt(g, false, s));
    if (plain.n) HIP_TRY(launch_gemm(plain, dt, s));
  } else {
    se.begin(GDLA_STAGE_PROJ_IN);
    HIP_TRY(launch_gemm_rows(g, dt, partial, partial_bytes, s));
  }
  se.end(GDLA_STAGE_PROJ_IN);
  PrepArgs a{};
  a.aq = aq; a.ckv = ckv; a.kr = krp; a.lam_logit = laml; a.lam_override = lam_override;
  a.gamma_q = w->gamma_q; a.gamma_kv = w->gamma_kv; a.cq = cq; a.lam = lam; a.cache = cache;
  a.pos = pos_dev; a.M = M; a.T = T; a.cq_f16 = cq_f16 ? 1 : 0; a.cq_lo = cq_lo;
  se.begin(GDLA_STAGE_NORM_APPEND);
  HIP_TRY(launch_prep(a, d, dt, s));
  se.end(GDLA_STAGE_NORM_APPEND);
  return GDLA_OK;
}

}  // namespace

// GEMM dispatch shared by all entry points: bf16 problems that fit the MFMA kernel (K a multiple
// of 64, N and the row strides multiples of 8, 16-byte aligned operands) run there, the rest on
// the generic kernel.
hipError_t launch_gemm(GemmBatch &g, DT dt, hipStream_t s) {
  if (dt != DT::BF16) return launch_gemm_generic(g, dt, s);
  GemmBatch fast[2] = {}, slow{};
  for (int i = 0; i < g.n; ++i) {
    const GemmProblem &p = g.p[i];
    if (fast_gemm_problem_ok(p)) fast[p.a_f16 ? 1 : 0].p[fast[p.a_f16 ? 1 : 0].n++] = p;
    else if (p.a_f16 || p.c_dt > CD_IN || p.c_trans) return hipErrorInvalidValue;  // MFMA kernel only
    else slow.p[slow.n++] = p;
  }
  for (int k = 0; k < 2; ++k)
    if (fast[k].n) {
      const hipError_t e = launch_gemm_mfma(fast[k], s);
      if (e != hipSuccess) return e;
    }
  return slow.n ? launch_gemm_generic(slow, dt, s) : hipSuccess;
}

}  // namespace gdla

using namespace gdla;

GDLA_EXPORT const char *gdla_status_string(gdla_status s) {
  switch (s) {
    case GDLA_OK: return "GDLA_OK";
    case GDLA_ERR_INVALID_ARG: return "GDLA_ERR_INVALID_ARG";
    case GDLA_ERR_UNSUPPORTED: return "GDLA_ERR_UNSUPPORTED";
    case GDLA_ERR_WORKSPACE: return "GDLA_ERR_WORKSPACE";
    case GDLA_ERR_OUT_OF_RANGE: return "GDLA_ERR_OUT_OF_RANGE";
    case GDLA_ERR_HIP: return "GDLA_ERR_HIP";
  }
  return "unknown gdla_status";
}

GDLA_EXPORT const char *gdla_last_error(void) { return g_err; }

GDLA_EXPORT size_t gdla_workspace_bytes(const gdla_dims *dims, int32_t op, int32_t B, int32_t T,
                                        const int32_t *pos_host, int32_t max_len) {
  LayerDims d;
  if (check_dims(dims, d) != GDLA_OK) return 0;
  if (B < 0 || T < 0 || max_len <= 0 || (op == GDLA_OP_DECODE && T > GDLA_MAX_DECODE_TOKENS)) return 0;
  if (B == 0 || T == 0) return 0;
  if (T > max_len || max_len > kMaxPositions || (int64_t)B * T > kMaxRows) return 0;
  if (pos_host) {
    for (int32_t b = 0; b < B; ++b)
      if (pos_host[b] < 0 || (int64_t)pos_host[b] + T > max_len) return 0;
  }
  switch (op) {
    case GDLA_OP_PREFILL: return plan_prefill(d, dims->dtype, B, T, pos_host, max_len).total;
    case GDLA_OP_DECODE: return plan_decode(d, dims->dtype, B, T, max_len).total;
    case GDLA_OP_APPEND: return plan_append(d, B, T).total;
    case GDLA_OP_PREFILL_PAGED: return plan_prefill_paged(d, dims->dtype, B, T, pos_host, max_len).total;
    case GDLA_OP_BACKWARD: {
      if (dims->dtype == GDLA_BF16) {
        const FastBackwardLayout F = plan_backward_fast(d, B, T);
        if (F.ok) return F.total;
      }
      return plan_backward(d, B, T).total;
    }
    default: return 0;
  }
}

namespace {

// Validates a paged cache and describes it for the kernels.
gdla_status paged_ref(const gdla_paged_cache *pc, CacheRef &c) {
  if (!pc) return fail(GDLA_ERR_INVALID_ARG, "paged cache is NULL");
  if (pc->page_rows <= 0 || pc->page_rows % 32 != 0)
    return fail(GDLA_ERR_INVALID_ARG, "page_rows = %d must be a positive multiple of 32", pc->page_rows);
  if (pc->n_pages <= 0 || pc->max_blocks <= 0)
    return fail(GDLA_ERR_INVALID_ARG, "n_pages and max_blocks must be positive");
  if ((int64_t)pc->max_blocks * pc->page_rows > INT32_MAX)
    return fail(GDLA_ERR_INVALID_ARG, "max_blocks * page_rows exceeds the int32 position range");
  if (!pc->pages || !pc->block_table) return fail(GDLA_ERR_INVALID_ARG, "pages or block_table is NULL");
  if (((uintptr_t)pc->block_table & 3u) != 0) return fail(GDLA_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  c = CacheRef{};
  c.base = pc->pages;
  c.block_table = pc->block_table;
  c.max_len = pc->max_blocks * pc->page_rows;
  c.page_rows = pc->page_rows;
  c.max_blocks = pc->max_blocks;
  c.n_pages = pc->n_pages;
  return GDLA_OK;
}

gdla_status append_impl(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B, int32_t T,
                        const int32_t *pos_host, const CacheRef &cache, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  LayerDims d;
  gdla_status st = check_call(dims, w, x, B, T, pos_host, cache.base, cache.max_len, nullptr, false, d);
  if (st != GDLA_OK || B == 0 || T == 0) return st;
  const AppendLayout L = plan_append(d, B, T);
  if ((st = check_ws(ws, ws_bytes, L.total)) != GDLA_OK) return st;
  const DT dt = dims->dtype == GDLA_F32 ? DT::F32 : DT::BF16;
  int32_t *pos_dev = at<int32_t>(ws, L.pos);
  HIP_TRY(launch_set_i32(pos_dev, pos_host, B, stream));
  StageEvents se;
  return project_and_append(d, dt, w, x, B * T, T, pos_dev, cache, nullptr, at<float>(ws, L.ckv),
                            at<float>(ws, L.krp), nullptr, nullptr, nullptr, nullptr, stream, se);
}

}  // namespace

namespace gdla {
gdla_status report_error(gdla_status st, const char *msg) { return fail(st, "%s", msg); }
}  // namespace gdla

GDLA_EXPORT gdla_status gdla_latent_append(const gdla_dims *dims, const gdla_weights *w,
                                           const void *x, int32_t B, int32_t T,
                                           const int32_t *pos_host, void *cache, int32_t max_len,
                                           void *ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  return append_impl(dims, w, x, B, T, pos_host, contiguous_cache(cache, max_len), ws, ws_bytes, stream);
}

GDLA_EXPORT gdla_status gdla_latent_append_paged(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                                 int32_t B, int32_t T, const int32_t *pos_host,
                                                 const gdla_paged_cache *cache, void *ws, size_t ws_bytes,
                                                 hipStream_t stream) {
  g_err[0] = 0;
  CacheRef c;
  const gdla_status st = paged_ref(cache, c);
  if (st != GDLA_OK) return st;
  return append_impl(dims, w, x, B, T, pos_host, c, ws, ws_bytes, stream);
}

namespace {

// doc: device [B, T] first position of each token's document (packed documents), or null
// prepared: the layer's transposed weights from gdla_prepare_weights, or null (then the call
// transposes them into its workspace)
gdla_status prefill_impl(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B, int32_t T,
                         const int32_t *pos_host, void *cache, int32_t max_len, void *out, void *ws,
                         size_t ws_bytes, const gdla_debug *dbg, hipStream_t stream,
                         const int32_t *doc = nullptr, float *lse = nullptr, const void *prepared = nullptr,
                         bool attn_f16 = false) {
  LayerDims d;
  gdla_status st = check_call(dims, w, x, B, T, pos_host, cache, max_len, out, true, d);
  if (st != GDLA_OK || B == 0 || T == 0) return st;
  const PrefillLayout L = plan_prefill(d, dims->dtype, B, T, pos_host, max_len);
  if ((st = check_ws(ws, ws_bytes, L.total)) != GDLA_OK) return st;
  const DT dt = dims->dtype == GDLA_F32 ? DT::F32 : DT::BF16;
  const size_t es = esize(dims->dtype);
  const int32_t M = B * T;
  const float *lam_override = dbg ? dbg->lambda_override : nullptr;
  float *out_heads = dbg ? dbg->out_heads : nullptr;
  StageEvents se;
  se.ev = dbg ? dbg->stage_events : nullptr;
  se.s = stream;

  int32_t *pos_dev = at<int32_t>(ws, L.pos);
  HIP_TRY(launch_set_i32(pos_dev, pos_host, B, stream));
  NtWeights ntw{};
  if (L.use_nt) {
    // Transposed weights for the K-contiguous GEMM: weights applied to x and to the bf16 cache stay
    // bf16, those applied to the fp16 c^Q and Y become fp16 (the conversion the other MFMA GEMM
    // does while staging).  Prepared once by the caller, or written here into the workspace.
    se.begin(GDLA_STAGE_PROJ_IN);
    if (prepared) {
      const PreparedLayout P = plan_prepared(d);
      const char *b = (const char *)prepared;
      ntw = {b + P.qa, b + P.dkv, b + P.kr, b + P.lam, b + P.qc, b + P.qr, b + P.gate, b + P.uk, b + P.uv, b + P.o};
    } else {
      const size_t off[10] = {L.wt_qa, L.wt_dkv, L.wt_kr, L.wt_lam, L.wt_qc, L.wt_qr, L.wt_gate, L.wt_uk, L.wt_uv, L.wt_o};
      HIP_TRY(transpose_layer_weights(d, w, (char *)ws, off, stream));
      ntw = {at<void>(ws, L.wt_qa), at<void>(ws, L.wt_dkv), at<void>(ws, L.wt_kr), at<void>(ws, L.wt_lam),
             at<void>(ws, L.wt_qc), at<void>(ws, L.wt_qr), at<void>(ws, L.wt_gate), at<void>(ws, L.wt_uk),
             at<void>(ws, L.wt_uv), at<void>(ws, L.wt_o)};
    }
  }
  // Eq.(1), (3), (4), (7) and the cache append of this chunk's rows.
  st = project_and_append(d, dt, w, x, M, T, pos_dev, contiguous_cache(cache, max_len), at<float>(ws, L.aq),
                          at<float>(ws, L.ckv), at<float>(ws, L.krp), at<float>(ws, L.laml),
                          at<void>(ws, L.cq), at<float>(ws, L.lam), lam_override, stream, se,
                          L.use_fast, L.use_nt ? &ntw : nullptr);
  if (st != GDLA_OK) return st;

  // Eq.(5): expand K^C and V of every visible key, head-major [B, n_kv, lcap, *].  The MFMA path
  // keeps fp16 key rows [K^C ; k^R] of d_h + d_rope values (k^R copied from the cache into every
  // head's rows); the generic path keeps K^C rows of d_h values in the layer dtype.
  const int64_t row = d.d_c + d.d_r;
  const int64_t krow = L.use_fast ? fast_prefill_key_row() : d.d_h;
  // bf16 attention operands on the transposed-weight path, unless the caller needs fp16 ones
  const bool bf_ops = L.use_fast && L.use_nt && !attn_f16;
  const int64_t k_seq = (int64_t)d.n_kv * L.lcap * krow;
  const int64_t v_seq = (int64_t)d.n_kv * L.lcap * d.d_h;
  se.begin(GDLA_STAGE_EXPAND_KV);
  for (int32_t b0 = 0; b0 < B; b0 += kMaxGemmProblems / 2) {
    GemmBatch g{};
    for (int32_t b = b0; b < std::min(B, b0 + kMaxGemmProblems / 2); ++b) {
      const int32_t lo = key_lo(pos_host[b], d.window);
      const int32_t nk = pos_host[b] + T - lo;
      const char *a = (const char *)cache + ((int64_t)b * max_len + lo) * row * es;
      GemmProblem pk = gp(a, row, L.use_nt ? ntw.uk : w->w_uk, L.use_nt ? d.d_c : (int64_t)d.n_kv * d.d_h,
                          at<char>(ws, L.kx) + b * k_seq * es, krow, nk, d.n_kv * d.d_h, d.d_c, false);
      pk.hw = d.d_h;
      pk.hs = (int64_t)L.lcap * krow;
      if (L.use_fast) pk.c_dt = bf_ops ? CD_BF16 : CD_F16;
      GemmProblem pv = pk;
      pv.B = L.use_nt ? ntw.uv : w->w_uv;
      pv.C = at<char>(ws, L.vx) + b * v_seq * es;
      pv.ldc = d.d_h;
      pv.hs = (int64_t)L.lcap * d.d_h;
      if (L.use_fast) {  // V^T per KV head (the MFMA attention's value layout)
        pv.c_trans = 1;
        pv.ldc = L.lcap;
      }
      g.p[g.n++] = pk;
      g.p[g.n++] = pv;
    }
    if (L.use_nt) HIP_TRY(launch_gemm_nt(g, false, stream));
    else HIP_TRY(launch_gemm(g, dt, stream));
  }
  if (L.use_fast) {
    HIP_TRY(launch_kr_fill(cache, at<void>(ws, L.kx), pos_dev, B, T, L.lcap, max_len, d, bf_ops, stream));
    HIP_TRY(launch_vt_tail_zero(at<void>(ws, L.vx), pos_dev, B, T, L.lcap, d, stream));
  }
  se.end(GDLA_STAGE_EXPAND_KV);

  if (L.use_fast) {
    st = run_fast_prefill(d, w, B, T, pos_dev, pos_host, cache, max_len, at<void>(ws, L.cq),
                          at<float>(ws, L.lam), at<float>(ws, L.gate), at<void>(ws, L.kx),
                          at<void>(ws, L.vx), L.lcap, at<void>(ws, L.y), out_heads, L.fast, ws,
                          stream, se, L.use_nt ? &ntw : nullptr, doc, lse, bf_ops);
    if (st != GDLA_OK) return fail(st, "fast prefill path failed: %s", hipGetErrorString(hipGetLastError()));
  } else {
    // Eq.(2), (9): q^C, pre-RoPE q^R and gate logits.
    se.begin(GDLA_STAGE_PROJ_Q);
    GemmBatch g{};
    g.p[g.n++] = gp(at<void>(ws, L.cq), d.d_cq, w->w_qc, (int64_t)d.n_heads * d.d_h, at<void>(ws, L.qc),
                    (int64_t)d.n_heads * d.d_h, M, d.n_heads * d.d_h, d.d_cq, false);
    g.p[g.n++] = gp(at<void>(ws, L.cq), d.d_cq, w->w_qr, (int64_t)d.n_heads * d.d_r, at<float>(ws, L.qrp),
                    (int64_t)d.n_heads * d.d_r, M, d.n_heads * d.d_r, d.d_cq, true);
    g.p[g.n++] = gp(at<void>(ws, L.cq), d.d_cq, w->w_gate, (int64_t)d.n_signal * d.d_h, at<float>(ws, L.gate),
                    (int64_t)d.n_signal * d.d_h, M, d.n_signal * d.d_h, d.d_cq, true);
    HIP_TRY(launch_gemm(g, dt, stream));
    HIP_TRY(launch_rope_heads(at<float>(ws, L.qrp), at<void>(ws, L.qr), (int64_t)d.n_heads * d.d_r, d.d_r, 0,
                              M, T, d.n_heads, d.d_r, pos_dev, d.theta, dt, stream));
    se.end(GDLA_STAGE_PROJ_Q);
    AttnGenericArgs a{};
    a.qc = at<void>(ws, L.qc); a.qr = at<void>(ws, L.qr); a.kx = at<void>(ws, L.kx);
    a.vx = at<void>(ws, L.vx); a.cache = cache; a.heads = at<float>(ws, L.heads); a.pos = pos_dev; a.doc = doc;
    a.M = M; a.T = T; a.max_len = max_len; a.lcap = L.lcap;
    se.begin(GDLA_STAGE_ATTN_NOISE);
    HIP_TRY(launch_attention_generic(a, d, dt, stream));
    se.end(GDLA_STAGE_ATTN_NOISE);
    se.begin(GDLA_STAGE_ATTN_SIGNAL);
    if (out_heads)
      HIP_TRY(launch_copy_rows_f32(at<float>(ws, L.heads), (int64_t)d.n_heads * d.d_h, out_heads,
                                   (int64_t)d.n_heads * d.d_h, M, d.n_heads * d.d_h, stream));
    HIP_TRY(launch_combine(at<float>(ws, L.heads), at<float>(ws, L.lam), at<float>(ws, L.gate),
                           at<void>(ws, L.y), M, d, dt, stream));
    se.end(GDLA_STAGE_ATTN_SIGNAL);
  }
  // Eq.(10): out = Y W_o (Y is fp16 on the MFMA path).
  GemmBatch g{};
  g.p[g.n++] = gp(at<void>(ws, L.y), (int64_t)d.n_signal * d.d_h, L.use_nt ? ntw.o : w->w_o,
                  L.use_nt ? (int64_t)d.n_signal * d.d_h : d.d_model, out, d.d_model, M, d.d_model,
                  d.n_signal * d.d_h, false);
  if (L.use_fast) {
    g.p[0].a_f16 = 1;
    g.p[0].c_dt = CD_BF16;
  }
  se.begin(GDLA_STAGE_PROJ_OUT);
  if (L.use_nt) HIP_TRY(launch_gemm_nt(g, true, stream));
  else HIP_TRY(launch_gemm(g, dt, stream));
  se.end(GDLA_STAGE_PROJ_OUT);
  se.finish();
  return GDLA_OK;
}

}  // namespace

GDLA_EXPORT gdla_status gdla_prefill(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                     int32_t B, int32_t T, const int32_t *pos_host, void *cache,
                                     int32_t max_len, void *out, void *ws, size_t ws_bytes,
                                     const gdla_debug *dbg, hipStream_t stream) {
  g_err[0] = 0;
  return prefill_impl(dims, w, x, B, T, pos_host, cache, max_len, out, ws, ws_bytes, dbg, stream);
}

GDLA_EXPORT size_t gdla_prepared_weights_bytes(const gdla_dims *dims) {
  LayerDims d;
  if (check_dims(dims, d) != GDLA_OK) return 0;
  if (!fast_prefill_supported(d, dims->dtype) || d.d_c % 64 != 0) return 0;
  return plan_prepared(d).total;
}

GDLA_EXPORT gdla_status gdla_prepare_weights(const gdla_dims *dims, const gdla_weights *w, void *prepared,
                                             size_t prepared_bytes, hipStream_t stream) {
  g_err[0] = 0;
  LayerDims d;
  gdla_status st = check_dims(dims, d);
  if (st != GDLA_OK) return st;
  const size_t need = gdla_prepared_weights_bytes(dims);
  if (need == 0) return fail(GDLA_ERR_UNSUPPORTED, "this layer's prefill takes no prepared weights");
  if (!w) return fail(GDLA_ERR_INVALID_ARG, "weights is NULL");
  const void *req[] = {w->w_qa, w->w_qc, w->w_qr, w->w_dkv, w->w_kr, w->w_uk, w->w_uv, w->w_lambda, w->w_gate, w->w_o};
  for (const void *p : req) {
    if (!p) return fail(GDLA_ERR_INVALID_ARG, "a required weight pointer is NULL");
    if (!aligned16(p)) return fail(GDLA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  }
  if ((st = check_ws(prepared, prepared_bytes, need)) != GDLA_OK) return st;
  const PreparedLayout P = plan_prepared(d);
  const size_t off[10] = {P.qa, P.dkv, P.kr, P.lam, P.qc, P.qr, P.gate, P.uk, P.uv, P.o};
  HIP_TRY(transpose_layer_weights(d, w, (char *)prepared, off, stream));
  return GDLA_OK;
}

GDLA_EXPORT gdla_status gdla_prefill_prepared(const gdla_dims *dims, const gdla_weights *w, const void *prepared,
                                              size_t prepared_bytes, const void *x, int32_t B, int32_t T,
                                              const int32_t *pos_host, void *cache, int32_t max_len, void *out,
                                              void *ws, size_t ws_bytes, const gdla_debug *dbg,
                                              hipStream_t stream) {
  g_err[0] = 0;
  LayerDims d;
  const gdla_status st = check_dims(dims, d);
  if (st != GDLA_OK) return st;
  const size_t need = gdla_prepared_weights_bytes(dims);
  if (need == 0) return fail(GDLA_ERR_UNSUPPORTED, "this layer's prefill takes no prepared weights");
  if (!prepared) return fail(GDLA_ERR_INVALID_ARG, "prepared is NULL");
  if (((uintptr_t)prepared & 255u) != 0) return fail(GDLA_ERR_INVALID_ARG, "prepared must be 256-byte aligned");
  if (prepared_bytes < need)
    return fail(GDLA_ERR_WORKSPACE, "prepared weights %zu bytes < %zu needed", prepared_bytes, need);
  return prefill_impl(dims, w, x, B, T, pos_host, cache, max_len, out, ws, ws_bytes, dbg, stream, nullptr, nullptr,
                      prepared);
}

GDLA_EXPORT gdla_status gdla_prefill_packed(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                            int32_t B, int32_t T, const int32_t *pos_host,
                                            const int32_t *doc_start, void *cache, int32_t max_len, void *out,
                                            void *ws, size_t ws_bytes, const gdla_debug *dbg, hipStream_t stream) {
  g_err[0] = 0;
  if (B > 0 && T > 0 && !doc_start) return fail(GDLA_ERR_INVALID_ARG, "doc_start is NULL");
  if (((uintptr_t)doc_start & 3u) != 0) return fail(GDLA_ERR_INVALID_ARG, "doc_start must be 4-byte aligned");
  return prefill_impl(dims, w, x, B, T, pos_host, cache, max_len, out, ws, ws_bytes, dbg, stream, doc_start);
}

GDLA_EXPORT gdla_status gdla_prefill_paged(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                           int32_t B, int32_t T, const int32_t *pos_host,
                                           const gdla_paged_cache *cache, void *out, void *ws, size_t ws_bytes,
                                           const gdla_debug *dbg, hipStream_t stream) {
  g_err[0] = 0;
  CacheRef pc;
  gdla_status st = paged_ref(cache, pc);
  if (st != GDLA_OK) return st;
  LayerDims d;
  st = check_call(dims, w, x, B, T, pos_host, pc.base, pc.max_len, out, true, d);
  if (st != GDLA_OK || B == 0 || T == 0) return st;
  const PagedPrefillLayout L = plan_prefill_paged(d, dims->dtype, B, T, pos_host, pc.max_len);
  if ((st = check_ws(ws, ws_bytes, L.total)) != GDLA_OK) return st;
  const int64_t row_bytes = (int64_t)(d.d_c + d.d_r) * esize(dims->dtype);
  int32_t *pos_dev = at<int32_t>(ws, L.pos);
  const CacheRef stage = contiguous_cache(at<void>(ws, L.stage), L.stage_len);
  HIP_TRY(launch_set_i32(pos_dev, pos_host, B, stream));
  // visible rows before the chunk -> staging; the chunk as a contiguous prefill there (which
  // appends its rows to the staging cache); its new rows -> their pages
  HIP_TRY(launch_copy_cache_rows(pc, stage, pos_dev, B, L.max_gather, false, T, d.window, row_bytes, stream));
  st = prefill_impl(dims, w, x, B, T, pos_host, stage.base, L.stage_len, out, ws, L.pre.total, dbg, stream);
  if (st != GDLA_OK) return st;
  HIP_TRY(launch_copy_cache_rows(stage, pc, pos_dev, B, T, true, T, d.window, row_bytes, stream));
  return GDLA_OK;
}

namespace gdla {
namespace {

// Absorbed decode of T new tokens per sequence (row m = b T + i: token i of sequence b).
gdla_status decode_impl(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B, int32_t T,
                        const int32_t *pos_host, const CacheRef &cache, void *out, void *ws,
                        size_t ws_bytes, const gdla_debug *dbg, hipStream_t stream) {
  LayerDims d;
  gdla_status st = check_call(dims, w, x, B, T, pos_host, cache.base, cache.max_len, out, true, d);
  if (st != GDLA_OK || B == 0 || T == 0) return st;
  const DecodeLayout L = plan_decode(d, dims->dtype, B, T, cache.max_len);
  if ((st = check_ws(ws, ws_bytes, L.total)) != GDLA_OK) return st;
  const DT dt = dims->dtype == GDLA_F32 ? DT::F32 : DT::BF16;
  const int32_t M = B * T;
  const float *lam_override = dbg ? dbg->lambda_override : nullptr;
  float *out_heads = dbg ? dbg->out_heads : nullptr;
  StageEvents se;
  se.ev = dbg ? dbg->stage_events : nullptr;
  se.s = stream;

  int32_t *pos_dev = at<int32_t>(ws, L.pos);
  HIP_TRY(launch_set_i32(pos_dev, pos_host, B, stream));
  void *partial = at<void>(ws, L.skinny);
  void *cq_lo = L.skinny_bytes > 0 ? at<void>(ws, L.cq_lo) : nullptr;
  void *y_lo = L.skinny_bytes > 0 ? at<void>(ws, L.y_lo) : nullptr;
  st = project_and_append(d, dt, w, x, M, T, pos_dev, cache, at<float>(ws, L.aq),
                          at<float>(ws, L.ckv), at<float>(ws, L.krp), at<float>(ws, L.laml),
                          at<void>(ws, L.cq), at<float>(ws, L.lam), lam_override, stream, se, false, nullptr,
                          partial, L.skinny_bytes, cq_lo);
  if (st != GDLA_OK) return st;
  // Eq.(2), (9) in fp32 (decode keeps the query in fp32 until it is mapped into the latent).
  se.begin(GDLA_STAGE_PROJ_Q);
  GemmBatch g{};
  g.p[g.n++] = gp(at<void>(ws, L.cq), d.d_cq, w->w_qc, (int64_t)d.n_heads * d.d_h, at<float>(ws, L.qc),
                  (int64_t)d.n_heads * d.d_h, M, d.n_heads * d.d_h, d.d_cq, true);
  g.p[g.n++] = gp(at<void>(ws, L.cq), d.d_cq, w->w_qr, (int64_t)d.n_heads * d.d_r, at<float>(ws, L.qrp),
                  (int64_t)d.n_heads * d.d_r, M, d.n_heads * d.d_r, d.d_cq, true);
  g.p[g.n++] = gp(at<void>(ws, L.cq), d.d_cq, w->w_gate, (int64_t)d.n_signal * d.d_h, at<float>(ws, L.gate),
                  (int64_t)d.n_signal * d.d_h, M, d.n_signal * d.d_h, d.d_cq, true);
  for (int i = 0; i < g.n; ++i) g.p[i].A_lo = cq_lo;
  HIP_TRY(launch_gemm_rows(g, dt, partial, L.skinny_bytes, stream));
  if (L.use_fast) {
    // rotates q^R itself; ends GDLA_STAGE_PROJ_Q after the absorbed query; leaves
    // GDLA_STAGE_ATTN_SIGNAL open
    st = run_fast_decode(d, w, B, T, pos_dev, cache, at<float>(ws, L.qc), at<float>(ws, L.qrp),
                         at<float>(ws, L.heads), L.fast, ws, stream, se);
    if (st != GDLA_OK) return fail(st, "fast decode path failed: %s", hipGetErrorString(hipGetLastError()));
  } else {
    HIP_TRY(launch_rope_heads(at<float>(ws, L.qrp), at<float>(ws, L.qr), (int64_t)d.n_heads * d.d_r, d.d_r, 0,
                              M, T, d.n_heads, d.d_r, pos_dev, d.theta, DT::F32, stream));
    se.end(GDLA_STAGE_PROJ_Q);
    se.begin(GDLA_STAGE_ATTN_NOISE);
    HIP_TRY(launch_absorb_generic(at<float>(ws, L.qc), at<float>(ws, L.qr), w->w_uk, at<float>(ws, L.qabs),
                                  M, d, dt, stream));
    HIP_TRY(launch_latent_attention_generic(at<float>(ws, L.qabs), cache, at<float>(ws, L.o), pos_dev, B, T,
                                            d, dt, stream));
    se.end(GDLA_STAGE_ATTN_NOISE);
    se.begin(GDLA_STAGE_ATTN_SIGNAL);
    HIP_TRY(launch_unabsorb_generic(at<float>(ws, L.o), w->w_uv, at<float>(ws, L.heads), M, d, dt, stream));
  }
  if (out_heads)
    HIP_TRY(launch_copy_rows_f32(at<float>(ws, L.heads), (int64_t)d.n_heads * d.d_h, out_heads,
                                 (int64_t)d.n_heads * d.d_h, M, d.n_heads * d.d_h, stream));
  HIP_TRY(launch_combine(at<float>(ws, L.heads), at<float>(ws, L.lam), at<float>(ws, L.gate),
                         at<void>(ws, L.y), M, d, dt, stream, y_lo));
  se.end(GDLA_STAGE_ATTN_SIGNAL);
  g = GemmBatch{};
  g.p[g.n++] = gp(at<void>(ws, L.y), (int64_t)d.n_signal * d.d_h, w->w_o, d.d_model, out, d.d_model, M,
                  d.d_model, d.n_signal * d.d_h, false);
  g.p[0].A_lo = y_lo;
  se.begin(GDLA_STAGE_PROJ_OUT);
  HIP_TRY(launch_gemm_rows(g, dt, partial, L.skinny_bytes, stream));
  se.end(GDLA_STAGE_PROJ_OUT);
  se.finish();
  return GDLA_OK;
}

}  // namespace
}  // namespace gdla

namespace gdla {
gdla_status check_decode_args(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                              const int32_t *pos_host, const void *cache, int32_t max_len, const void *out) {
  g_err[0] = 0;
  LayerDims d;
  return check_call(dims, w, x, B, 1, pos_host, cache, max_len, out, true, d);
}
}  // namespace gdla

GDLA_EXPORT gdla_status gdla_decode(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                    int32_t B, const int32_t *pos_host, void *cache,
                                    int32_t max_len, void *out, void *ws, size_t ws_bytes,
                                    const gdla_debug *dbg, hipStream_t stream) {
  g_err[0] = 0;
  return decode_impl(dims, w, x, B, 1, pos_host, contiguous_cache(cache, max_len), out, ws, ws_bytes, dbg,
                     stream);
}

GDLA_EXPORT gdla_status gdla_decode_tokens(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                           int32_t B, int32_t T, const int32_t *pos_host, void *cache,
                                           int32_t max_len, void *out, void *ws, size_t ws_bytes,
                                           const gdla_debug *dbg, hipStream_t stream) {
  g_err[0] = 0;
  if (T < 0 || T > GDLA_MAX_DECODE_TOKENS)
    return fail(GDLA_ERR_INVALID_ARG, "T = %d outside 0 .. %d", T, GDLA_MAX_DECODE_TOKENS);
  return decode_impl(dims, w, x, B, T, pos_host, contiguous_cache(cache, max_len), out, ws, ws_bytes, dbg,
                     stream);
}

GDLA_EXPORT gdla_status gdla_decode_paged(const gdla_dims *dims, const gdla_weights *w, const void *x,
                                          int32_t B, int32_t T, const int32_t *pos_host,
                                          const gdla_paged_cache *cache, void *out, void *ws, size_t ws_bytes,
                                          const gdla_debug *dbg, hipStream_t stream) {
  g_err[0] = 0;
  if (T < 0 || T > GDLA_MAX_DECODE_TOKENS)
    return fail(GDLA_ERR_INVALID_ARG, "T = %d outside 0 .. %d", T, GDLA_MAX_DECODE_TOKENS);
  CacheRef c;
  const gdla_status st = paged_ref(cache, c);
  if (st != GDLA_OK) return st;
  return decode_impl(dims, w, x, B, T, pos_host, c, out, ws, ws_bytes, dbg, stream);
}

namespace gdla {
namespace {

gdla_status backward_fast(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B, int32_t T,
                          const int32_t *doc, const void *dout, const gdla_grads *grads, void *ws,
                          const gdla_debug *dbg, hipStream_t stream, const LayerDims &d, const FastBackwardLayout &F) {
  const PrefillLayout &PL = F.pre;
  const int32_t M = B * T;
  // the forward again, keeping per-head H and the log-sum-exp of every row and head
  std::vector<int32_t> zeros((size_t)B, 0);
  gdla_debug fdbg{};
  fdbg.lambda_override = dbg ? dbg->lambda_override : nullptr;
  fdbg.out_heads = at<float>(ws, F.heads);
  // fp16 attention operands: the backward kernels pair q, K and V with fp16 gradients
  gdla_status st = prefill_impl(dims, w, x, B, T, zeros.data(), at<void>(ws, F.cache), T, at<void>(ws, F.out), ws,
                                PL.total, &fdbg, stream, doc, at<float>(ws, F.lse), nullptr, true);
  if (st != GDLA_OK) return st;
  // V key-major per KV head: cbar W_uv (the forward keeps V transposed)
  {
    const int64_t row = d.d_c + d.d_r;
    GemmBatch g{};
    for (int32_t b0 = 0; b0 < B; b0 += kMaxGemmProblems) {
      g = GemmBatch{};
      for (int32_t b = b0; b < std::min(B, b0 + kMaxGemmProblems); ++b) {
        GemmProblem pv = gp(at<char>(ws, F.cache) + (int64_t)b * T * row * 2, row, at<void>(ws, PL.wt_uv), d.d_c,
                            at<char>(ws, F.vk) + (int64_t)b * d.n_kv * PL.lcap * d.d_h * 2, d.d_h, T,
                            d.n_kv * d.d_h, d.d_c, false);
        pv.hw = d.d_h;
        pv.hs = (int64_t)PL.lcap * d.d_h;
        pv.c_dt = CD_F16;
        g.p[g.n++] = pv;
      }
      HIP_TRY(launch_gemm_nt(g, false, stream));
    }
  }
  FastBwdArgs a{};
  a.x = x; a.dout = dout; a.w = w; a.doc = doc; a.grads = *grads;
  if (!w->gamma_q) a.grads.dgamma_q = nullptr;
  if (!w->gamma_kv) a.grads.dgamma_kv = nullptr;
  a.cq16 = at<f16_t>(ws, PL.cq);
  a.aq = at<float>(ws, PL.aq);
  a.ckv = at<float>(ws, PL.ckv);
  a.cache = at<bf16_t>(ws, F.cache);
  a.q16 = at<f16_t>(ws, PL.fast.q);
  a.kx = at<f16_t>(ws, PL.kx);
  a.vk = at<f16_t>(ws, F.vk);
  a.heads = at<float>(ws, F.heads);
  a.lse = at<float>(ws, F.lse);
  a.lam = at<float>(ws, PL.lam);
  a.sg16 = at<f16_t>(ws, PL.gate);
  a.y16 = at<f16_t>(ws, PL.y);
  a.lam_overridden = fdbg.lambda_override ? 1 : 0;
  void **bufs = (void **)&a.buf;
  for (int i = 0; i < 31; ++i) bufs[i] = at<void>(ws, F.fb[i]);
  a.B = B; a.T = T; a.M = M; a.M_pad = F.M_pad; a.lcap = PL.lcap; a.k8 = F.k8;
  HIP_TRY(launch_backward_fast(a, d, stream));
  return GDLA_OK;
}

}  // namespace
}  // namespace gdla

GDLA_EXPORT gdla_status gdla_backward(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                                      int32_t T, const int32_t *doc_start, const void *dout,
                                      const gdla_grads *grads, void *ws, size_t ws_bytes, const gdla_debug *dbg,
                                      hipStream_t stream) {
  g_err[0] = 0;
  LayerDims d;
  gdla_status st = check_dims(dims, d);
  if (st != GDLA_OK) return st;
  if (B < 0 || T < 0) return fail(GDLA_ERR_INVALID_ARG, "negative B or T");
  if (B == 0 || T == 0) return GDLA_OK;
  if ((int64_t)B * T > kMaxRows) return fail(GDLA_ERR_UNSUPPORTED, "B T = %lld rows above 2^30", (long long)B * T);
  if (!w || !grads) return fail(GDLA_ERR_INVALID_ARG, "weights or grads is NULL");
  if (!x || !dout) return fail(GDLA_ERR_INVALID_ARG, "x or dout is NULL");
  const void *req[] = {w->w_qa, w->w_qc, w->w_qr, w->w_dkv, w->w_kr, w->w_uk, w->w_uv, w->w_lambda, w->w_gate, w->w_o};
  for (const void *p : req)
    if (!p) return fail(GDLA_ERR_INVALID_ARG, "a required weight pointer is NULL");
  const void *al[] = {x, dout, w->w_qa, w->w_qc, w->w_qr, w->w_dkv, w->w_kr, w->w_uk, w->w_uv, w->w_lambda,
                      w->w_gate, w->w_o, w->gamma_q, w->gamma_kv};
  for (const void *p : al)
    if (p && !aligned16(p)) return fail(GDLA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const float *gp_[] = {grads->dx, grads->dw_qa, grads->dw_qc, grads->dw_qr, grads->dw_dkv, grads->dw_kr,
                        grads->dw_uk, grads->dw_uv, grads->dw_lambda, grads->dw_gate, grads->dw_o};
  for (const float *p : gp_)
    if (!p) return fail(GDLA_ERR_INVALID_ARG, "a gradient pointer is NULL");
  if ((w->gamma_q && !grads->dgamma_q) || (w->gamma_kv && !grads->dgamma_kv))
    return fail(GDLA_ERR_INVALID_ARG, "dgamma_q / dgamma_kv are required with gamma_q / gamma_kv");
  if (((uintptr_t)doc_start & 3u) != 0) return fail(GDLA_ERR_INVALID_ARG, "doc_start must be 4-byte aligned");
  if (d.d_h > 256) return fail(GDLA_ERR_UNSUPPORTED, "d_head > 256");
  if (dims->dtype == GDLA_BF16) {
    const FastBackwardLayout F = plan_backward_fast(d, B, T);
    if (F.ok) {
      if ((st = check_ws(ws, ws_bytes, F.total)) != GDLA_OK) return st;
      return backward_fast(dims, w, x, B, T, doc_start, dout, grads, ws, dbg, stream, d, F);
    }
  }
  const BackwardLayout L = plan_backward(d, B, T);
  if ((st = check_ws(ws, ws_bytes, L.total)) != GDLA_OK) return st;
  BackwardArgs a{};
  a.x = x; a.dout = dout; a.w = w; a.doc = doc_start;
  a.lam_override = dbg ? dbg->lambda_override : nullptr;
  a.grads = *grads;
  if (!w->gamma_q) a.grads.dgamma_q = nullptr;
  if (!w->gamma_kv) a.grads.dgamma_kv = nullptr;
  float **bufs = (float **)&a.buf;
  for (int i = 0; i < 34; ++i) bufs[i] = at<float>(ws, L.off[i]);
  a.M = B * T;
  a.T = T;
  HIP_TRY(launch_backward_generic(a, d, dims->dtype == GDLA_F32 ? DT::F32 : DT::BF16, stream));
  return GDLA_OK;
}
