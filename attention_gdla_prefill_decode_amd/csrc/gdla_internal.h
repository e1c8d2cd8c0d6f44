// Internal declarations of the GDLA library: problem descriptors shared by the host orchestrator
// (gdla_api.hip) and the kernel files, and the launch functions each kernel file exports.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdla.h"

namespace gdla {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

enum class DT : int32_t { F32 = 0, BF16 = 1, F16 = 2 };

// One GEMM problem: C[m, col(n)] = epi(sum_k A[m, k] * B[k, n]), fp32 accumulation.
// A is [M, K] with row stride lda, B is [K, N] with row stride ldb (both in the input dtype).
// Output column n of row m is stored at C + m * ldc + (n / hw) * hs + ho + (n % hw) (elements of
// the output dtype), which lets one launch write head-major or interleaved layouts.  With c_trans
// (MFMA kernel, fp16 output only) it is stored transposed per head instead, at
// C + (n / hw) * hs + ho + (n % hw) * ldc + vt_slot(m): the value layout of the prefill attention.
struct GemmProblem {
  const void *A;
  const void *B;
  void *C;
  int64_t lda, ldb, ldc;
  int64_t hs;
  int32_t M, N, K;
  int32_t hw, ho;
  int32_t c_dt;    // CD_*: output dtype
  int32_t a_f16;   // 1: A is fp16 and the bf16 B is converted to fp16 while staged (MFMA only)
  int32_t epi;     // EPI_*
  int32_t c_trans; // 1: transposed per-head store (see above)
  // EPI_ROPE (transposed-weight GEMM only): columns come in heads of rope_d; column j < rope_d / 2
  // and j + rope_d / 2 of a head are rotated by p * theta^(-2j / rope_d), p = rope_pos[m / rope_T]
  // + m % rope_T (rotate-half RoPE), before the store.
  const int32_t *rope_pos;
  int32_t rope_T, rope_d;
  float rope_theta;
  int32_t tile0;   // first linear tile index of this problem (filled by the launcher)
  int32_t tiles_n; // tiles along N (filled by the launcher)
  // Split-K (transposed-weight GEMM, plain fp32 outputs only): ksplit > 1 slices K into ksplit
  // equal ranges, each workgroup writes its slice's product to part[slice] ([M, N] fp32, dense) and
  // a second kernel sums the slices in order into C (deterministic).
  int32_t ksplit;
  float *part;
  // Skinny GEMM only: the bf16 rounding remainder of A (same layout and lda), or null.  A + A_lo
  // carries about 16 significant bits of an fp32 activation; the kernel adds A_lo B to the
  // product.  The other kernels ignore it.
  const void *A_lo;
};

enum { EPI_NONE = 0, EPI_SIGMOID = 1, EPI_ROPE = 2 };
// Output dtypes: fp32, the input dtype, bf16, fp16 (the generic kernel serves CD_F32 / CD_IN).
enum { CD_F32 = 0, CD_IN = 1, CD_BF16 = 2, CD_F16 = 3 };

constexpr int kMaxGemmProblems = 8;

struct GemmBatch {
  GemmProblem p[kMaxGemmProblems];
  int32_t n;
  int32_t total_tiles;
};

// Per-call layer description used by device code (all int32 sizes).
// Rotation angles p * theta^(-2j/d_r) are formed and reduced modulo 2*pi in fp64 so that large
// positions (hundreds of thousands) keep full fp32 accuracy in cos / sin.
__device__ __forceinline__ void rope_cs(int p, int j, int d_r, float theta, float &c, float &s) {
  const double freq = pow((double)theta, -2.0 * (double)j / (double)d_r);
  double a = (double)p * freq;
  const double two_pi = 6.283185307179586476925286766559;
  a -= floor(a / two_pi) * two_pi;
  sincosf((float)a, &s, &c);
}

struct LayerDims {
  int32_t d_model, n_heads, n_signal, n_noise, n_kv, d_cq, d_c, d_h, d_r, window;
  float eps, theta, scale;
};

// Where the latent cache keeps row `pos` of sequence b.  Contiguous (page_rows == 0): row
// b max_len + pos of [B, max_len, d_c + d_r].  Paged: row pos % page_rows of physical page
// block_table[b max_blocks + pos / page_rows] of [n_pages, page_rows, d_c + d_r]; a table entry
// outside [0, n_pages) is clamped into it, so a bad table gives wrong rows, never a fault.
struct CacheRef {
  void *base;
  const int32_t *block_table;  // device [B, max_blocks] (paged only)
  int32_t max_len;             // positions per sequence (paged: max_blocks * page_rows)
  int32_t page_rows, max_blocks, n_pages;
};

__host__ __device__ inline int64_t cache_row(const CacheRef &c, int b, int pos) {
  if (c.page_rows == 0) return (int64_t)b * c.max_len + pos;
  int pg = c.block_table[(int64_t)b * c.max_blocks + pos / c.page_rows];
  pg = pg < 0 ? 0 : (pg >= c.n_pages ? c.n_pages - 1 : pg);
  return (int64_t)pg * c.page_rows + pos % c.page_rows;
}

// Records `msg` as the calling thread's last error (gdla_last_error) and returns st.
gdla_status report_error(gdla_status st, const char *msg);

// The argument checks of gdla_decode alone (no workspace, nothing launched): GDLA_OK or the
// status gdla_decode would return for these arguments, with the calling thread's error text set.
gdla_status check_decode_args(const gdla_dims *dims, const gdla_weights *w, const void *x, int32_t B,
                              const int32_t *pos_host, const void *cache, int32_t max_len, const void *out);

inline CacheRef contiguous_cache(void *base, int32_t max_len) {
  CacheRef c{};
  c.base = base;
  c.max_len = max_len;
  return c;
}

__host__ __device__ inline int kv_head_of(int h, int n_signal, int n_kv) {
  return h < n_signal ? (h % n_kv) : ((h - n_signal) % n_kv);
}

// Records caller-provided stage events (gdla_debug.stage_events) around the stages of a call;
// stages a call does not run get their two events recorded back to back by finish().
struct StageEvents {
  hipEvent_t *ev = nullptr;
  hipStream_t s = nullptr;
  unsigned done = 0;
  // (a NULL entry of the caller's array skips that record)
  void begin(int k) { if (ev && ev[2 * k]) (void)hipEventRecord(ev[2 * k], s); }
  void end(int k) {
    if (!ev) return;
    if (ev[2 * k + 1]) (void)hipEventRecord(ev[2 * k + 1], s);
    done |= 1u << k;
  }
  void finish() {
    if (!ev) return;
    for (int k = 0; k < GDLA_N_STAGES; ++k)
      if (!(done & (1u << k))) { begin(k); end(k); }
  }
};

// GEMM dispatch: bf16 MFMA kernels when every problem of the batch fits them, else generic.
hipError_t launch_gemm(GemmBatch &batch, DT dt, hipStream_t s);

// ---------------- generic kernels (any sizes; fp32 or bf16 storage, fp32 math) ---------------
hipError_t launch_gemm_generic(GemmBatch &batch, DT in_dt, hipStream_t s);

// Row-wise preparation after the first projection (one row per new token):
//   c^Q = RMSNorm(aq) * gamma_q -> cq (input dtype)          [skipped when cq == nullptr]
//   cache row (b, pos[b] + t) = [RMSNorm(ckv) * gamma_kv ; RoPE(kr, pos)]
//   lam = sigmoid(lam_logit) or lam_override                 [skipped when lam == nullptr]
struct PrepArgs {
  const float *aq;        // [M, d_cq]
  const float *ckv;       // [M, d_c]
  const float *kr;        // [M, d_r]
  const float *lam_logit; // [M, n_S]
  const float *lam_override;
  const void *gamma_q, *gamma_kv;
  void *cq;               // [M, d_cq] in the input dtype, or fp16 when cq_f16
  void *cq_lo;            // bf16 layers: [M, d_cq] bf16 remainder cq_exact - cq, or null
  float *lam;             // [M, n_S]
  CacheRef cache;
  const int32_t *pos;     // [B] device
  int32_t M, T;
  int32_t cq_f16;
};
hipError_t launch_prep(const PrepArgs &a, const LayerDims &d, DT dt, hipStream_t s);

// RoPE of per-head rows: dst[m * dst_ld + h * dst_hs + dst_off + j] = RoPE(src[m, h, :], p)[j]
// with src fp32 [M, n_heads, d_r] and p = pos[m / T] + m % T.
hipError_t launch_rope_heads(const float *src, void *dst, int64_t dst_ld, int32_t dst_hs, int32_t dst_off,
                             int32_t M, int32_t T, int32_t n_heads, int32_t d_r,
                             const int32_t *pos, float theta, DT dt, hipStream_t s);

// Expanded-form attention, one wave per (query row, head).  qc [M, n_H, d_h], qr [M, n_H, d_r]
// (after RoPE), kx / vx [B, n_kv, lcap, d_h] holding keys lo_b .. lo_b + lcap - 1, k^R read from
// the cache.  Writes heads [M, n_H, d_h] fp32.
struct AttnGenericArgs {
  const void *qc, *qr, *kx, *vx, *cache;
  float *heads;
  const int32_t *pos;
  const int32_t *doc;  // [M] first position of each token's document, or null (no documents)
  int32_t M, T, max_len, lcap;
};
hipError_t launch_attention_generic(const AttnGenericArgs &a, const LayerDims &d, DT dt,
                                    hipStream_t s);

// Eq.(8)-(10) before W_o: y[m, i, e] = sigmoid(g[m, i, e]) * (H[m, i, e] - lam[m, i] *
// H[m, n_S + i mod n_N, e]) in the input dtype.
hipError_t launch_combine(const float *heads, const float *lam, const float *gate, void *y,
                          int32_t M, const LayerDims &d, DT dt, hipStream_t s, void *y_lo = nullptr);

// Absorbed decode.  The absorb / un-absorb steps work on any number of query row sets; the
// attention step takes q_len tokens per sequence, row set v = b q_len + i at position pos[b] + i.
//   qabs[b, h] = [q^C_h W_uk[:, kv(h)]^T ; q^R_h]      (fp32, [B, n_H, d_c + d_r])
hipError_t launch_absorb_generic(const float *qc, const float *qr, const void *w_uk, float *qabs,
                                 int32_t B, const LayerDims &d, DT dt, hipStream_t s);
//   o[v, h] = sum_s softmax_s(tau qabs[v, h] . cache[b, s]) cache[b, s, 0:d_c]   (fp32), s over the
//   visible keys of position pos[b] + i
hipError_t launch_latent_attention_generic(const float *qabs, const CacheRef &cache, float *o,
                                           const int32_t *pos, int32_t B, int32_t q_len,
                                           const LayerDims &d, DT dt, hipStream_t s);
//   heads[b, h] = o[b, h] W_uv[:, kv(h)]   (fp32 [B, n_H, d_h])
hipError_t launch_unabsorb_generic(const float *o, const void *w_uv, float *heads, int32_t B,
                                   const LayerDims &d, DT dt, hipStream_t s);

// Cache rows of every sequence b from src to dst (either may be paged): the visible keys before
// the new tokens [lo(pos_b), pos_b) (scatter = false; lo from the window), or the new rows
// [pos_b, pos_b + T) (scatter = true).  max_rows bounds the rows of any sequence.
hipError_t launch_copy_cache_rows(const CacheRef &src, const CacheRef &dst, const int32_t *pos_dev, int32_t B,
                                  int32_t max_rows, bool scatter, int32_t T, int32_t window, int64_t row_bytes,
                                  hipStream_t s);
// ---------------- backward (training sequences at positions 0 .. T-1) ----------------------
// fp32 work buffers of the general backward path, each [M, ...] with M = B T rows.
struct BwdBuffers {
  float *aq, *ckv, *krp, *laml, *cq, *cbar, *kr, *lam, *rq, *rkv;
  float *qc, *qr, *g, *kc, *v, *heads, *lse;
  float *dy, *y, *dheads, *dd, *dg, *dlaml, *drow;
  float *dqc, *dqr, *dkc, *dv, *dkr_part, *dkr, *dcbar, *dckv, *dcq, *daq;
};
struct BackwardArgs {
  const void *x, *dout;        // [M, d_model] in the layer dtype
  const gdla_weights *w;
  const int32_t *doc;          // [M] document starts or null
  const float *lam_override;   // [M, n_S] or null
  gdla_grads grads;
  BwdBuffers buf;
  int32_t M, T;
};
hipError_t launch_backward_generic(const BackwardArgs &a, const LayerDims &d, DT dt, hipStream_t s);

// Copies up to 128 host values into a device int32 array through kernel arguments, so that no
// host-to-device copy (and no pinned host buffer) is needed.
hipError_t launch_set_i32(int32_t *dst, const int32_t *src_host, int32_t n, hipStream_t s);
// Copies fp32 rows to another fp32 buffer with a different row stride (debug outputs).
hipError_t launch_copy_rows_f32(const float *src, int64_t src_ld, float *dst, int64_t dst_ld,
                                int32_t rows, int32_t cols, hipStream_t s);

}  // namespace gdla
