// Interfaces of the bf16 MFMA paths for gfx950 (d_head 128, d_rope 64, d_kv_latent 512).
#pragma once

#include "gdla_internal.h"

namespace gdla {

// ---- MFMA GEMM: bf16 x bf16, or fp16 A x (bf16 B converted to fp16); all problems of one
// launch share a_f16 ----
bool fast_gemm_problem_ok(const GemmProblem &p);
hipError_t launch_gemm_mfma(GemmBatch &g, hipStream_t s);

// ---- large GEMM with transposed (K-contiguous) weights: C = A[M, K] . Bt[N, K]^T, fp16 x fp16
// or bf16 x bf16 (all problems of one launch share the operand type) ----
bool nt_gemm_problem_ok(const GemmProblem &p);
hipError_t launch_gemm_nt(GemmBatch &g, bool f16, hipStream_t s);
// Wt[N, K] = W[K, N]^T of a bf16 weight, as fp16 (to_f16) or bf16.
hipError_t launch_transpose_weight(const void *w, void *wt, int32_t K, int32_t N, bool to_f16, hipStream_t s);

// ---- skinny GEMM for decode batches (M <= 256 rows, N a multiple of 64, K of 64; bf16 A and B
// with B in its stored [K, N] layout; fp32 or bf16 C).  Split along K when the column tiles do
// not fill the chip; the fp32 partial sums need skinny_gemm_partial_bytes(g) of workspace, never
// more than skinny_gemm_partial_bound(M). ----
bool skinny_problem_ok(const GemmProblem &p);
bool skinny_gemm_ok(const GemmBatch &g);  // every problem ok, one M for all
size_t skinny_gemm_partial_bytes(const GemmBatch &g);
size_t skinny_gemm_partial_bound(int32_t M);
hipError_t launch_gemm_skinny(const GemmBatch &g, void *partial, size_t partial_bytes, hipStream_t s);

// Transposed copies of the layer weights in the workspace (prefill with enough rows to amortise
// them): x-side weights stay bf16, the weights applied to fp16 activations become fp16.
struct NtWeights {
  const void *qa, *dkv, *kr, *lam, *qc, *qr, *gate, *uk, *uv, *o;
};

// ---- fused prefill attention ----
// The attention's 16-bit operands (q, expanded K and V) are bf16 when the transposed-weight GEMMs
// produce them (bf_ops) and the caller does not ask for fp16 (the fused backward's recompute,
// whose kernels pair them with fp16 gradients); fp16 otherwise.
struct FastPrefillLayout {
  size_t q;      // [M, n_H, d_h + d_r] fp16 or bf16: q^C and rotated q^R of every head, one row per head
  size_t qrp;    // [M, n_H, d_r] fp32: q^R before RoPE
  size_t hn;     // [M, n_N, d_h] fp32: normalised noise-head outputs
};

template <class Add>
FastPrefillLayout plan_fast_prefill(const LayerDims &d, int32_t B, int32_t T, Add add) {
  const size_t M = (size_t)B * T;
  FastPrefillLayout L{};
  L.q = add(2 * M * d.n_heads * (d.d_h + d.d_r));
  L.qrp = add(4 * M * d.n_heads * d.d_r);
  L.hn = add(4 * M * d.n_noise * d.d_h);
  return L;
}

// Value layout of the MFMA prefill: V^T per KV head, [n_kv][d_head][lcap] in 16-bit values, with
// the keys of every aligned group of 32 stored in the order the probability operand of the PV MFMA
// (16 x 16 x 32) takes them from the score accumulators: key 16 h + 4 g + c of a group (h < 2,
// g < 4, c < 4) at position 8 g + 4 h + c.  vt_slot maps a key to its position, vt_key back.
__host__ __device__ inline int vt_slot(int k) { return (k & ~28) | ((k & 12) << 1) | ((k & 16) >> 2); }
__host__ __device__ inline int vt_key(int p) { return (p & ~28) | ((p & 24) >> 1) | ((p & 4) << 2); }
// Key capacity of the value / key buffers on the MFMA path: whole tiles plus one spare tile, so a
// tile that starts at any 16-key boundary before the last key stays inside the buffer.
inline int32_t fast_prefill_lcap(int32_t keys) { return (keys + 63) / 64 * 64 + 64; }
// Zeroes the value positions of keys nk_b .. lcap - 1 of every sequence (never visible, but read
// as part of whole tiles, so they must hold finite values).
hipError_t launch_vt_tail_zero(void *vx, const int32_t *pos_dev, int32_t B, int32_t T, int32_t lcap,
                               const LayerDims &d, hipStream_t s);

bool fast_prefill_supported(const LayerDims &d, gdla_dtype dt);
// Elements per expanded key row on the MFMA path: [K^C (d_h) ; k^R (d_rope)] in fp16.
int32_t fast_prefill_key_row();
// Copies k^R of the visible keys from the bf16 cache (kept in bf16, or converted to fp16) into
// columns d_h .. d_h + d_rope - 1 of every KV head's expanded key rows.
hipError_t launch_kr_fill(const void *cache, void *kx, const int32_t *pos_dev, int32_t B, int32_t T,
                          int32_t lcap, int32_t max_len, const LayerDims &d, bool bf16, hipStream_t s);
gdla_status run_fast_prefill(const LayerDims &d, const gdla_weights *w, int32_t B, int32_t T,
                             const int32_t *pos_dev, const int32_t *pos_host, void *cache,
                             int32_t max_len, void *cq, float *lam, float *gate, void *kx,
                             void *vx, int32_t lcap, void *y, float *out_heads,
                             const FastPrefillLayout &L, void *ws, hipStream_t s, StageEvents &se,
                             const NtWeights *nt, const int32_t *doc, float *lse = nullptr, bool bf_ops = false);

// ---- absorbed split-L decode ----
// Sizes are per query row set: BT = B T for T new tokens per sequence.
struct FastDecodeLayout {
  size_t qabs;   // [BT, n_H, d_c + d_r] bf16
  size_t part_o; // [BT, splits, n_H, d_c] fp32
  size_t part_ml;// [BT, splits, n_H, 2] fp32
  size_t wuvt;   // [n_kv d_h, d_c] fp16: W_uv transposed (K-contiguous rows for the value MFMA)
  int32_t splits;
};

int32_t fast_decode_splits(int32_t BT, int32_t max_len);

template <class Add>
FastDecodeLayout plan_fast_decode(const LayerDims &d, int32_t B, int32_t max_len, Add add) {
  FastDecodeLayout L{};
  L.splits = fast_decode_splits(B, max_len);
  L.qabs = add(2 * (size_t)B * d.n_heads * (d.d_c + d.d_r));
  L.part_o = add(4 * (size_t)B * L.splits * d.n_heads * d.d_c);
  L.part_ml = add(4 * (size_t)B * L.splits * d.n_heads * 2);
  L.wuvt = add(2 * (size_t)d.n_kv * d.d_h * d.d_c);
  return L;
}

bool fast_decode_supported(const LayerDims &d, gdla_dtype dt);
// T new tokens per sequence (token i of sequence b at position pos_dev[b] + i, already appended);
// qc, qrp (q^R before its rotation, which the path applies itself), heads hold B T row sets of
// n_H heads.
gdla_status run_fast_decode(const LayerDims &d, const gdla_weights *w, int32_t B, int32_t T,
                            const int32_t *pos_dev, const CacheRef &cache, const float *qc,
                            const float *qrp, float *heads, const FastDecodeLayout &L, void *ws,
                            hipStream_t s, StageEvents &se);

// ---- fused backward (bf16 layer, d_head 128, d_rope 64; training sequences from position 0) ----
struct BwdAttnArgs {
  const f16_t *q;      // [M, n_H, 192]: q^C ; RoPE(q^R)
  const f16_t *k;      // [B, n_kv, lcap, 192]: K^C ; k^R of keys 0 .. lcap - 1
  const f16_t *v;      // [B, n_kv, lcap, 128]: V, key-major
  const f16_t *dh;     // [M, n_H, 128]
  // dim-major copies for the dK/dV kernel: element (token t of sequence b, head h, dim j) at
  // (h 192 + j) B Tp + b Tp + t of qT (h 128 + j of dhT); tokens T .. Tp - 1 hold zeros
  const f16_t *qT, *dhT;
  const float *lse;    // [n_H, M] (+32 padding): log2 softmax denominators of c s
  const float *drow;   // [n_H, M] (+32 padding): rowsum(dH (.) H)
  const int32_t *lo;   // [M] (+32 padding): lowest visible key of every token
  const int32_t *doc;  // [M] document starts or null
  float *dq;           // [M, n_H, 192], or (a6 non-null) not written
  // a6 non-null: dq leaves packed instead, in fp16 rows of the query-latent operand: dq^C of head
  // h at columns h d_h .., dq^R rotated back by RoPE's angle at q_off + h d_r .. (cos, sin of
  // token t and frequency j in rope_cs[t d_r / 2 + j])
  f16_t *a6;
  int64_t lda6;
  int32_t q_off;
  const float2 *rope_cs;
  float *dk;           // [B, n_kv, T, 192]: the k^R part summed over this KV group's heads only
  float *dv;           // [B, n_kv, T, 128]
  int32_t B, T, lcap, n_heads, n_signal, n_noise, n_kv, window;
  int32_t Tp;          // T rounded up to a multiple of 32
  int32_t sig_chunks;  // dq, signal heads: workgroups of 4 heads per KV head
  float c, tau;
};
bool fast_backward_supported(const LayerDims &d, gdla_dtype dt);
hipError_t launch_bwd_attention(const BwdAttnArgs &a, hipStream_t s);

// Partials of the split-K products of the fused backward (at most this many bytes per product).
constexpr size_t kSplitKBytes = (size_t)128 << 20;

constexpr int kGradScaleBlocks = 512;  // blocks of the |dout| maximum
struct FastBwdBuffers {
  f16_t *wo16, *w3, *w6, *w8;   // fp16 weights, K-concatenated: [n_S d_h, d], [d_c, k3], [d_cq, k6], [d, k8]
  f16_t *dout16;                // [M, d]
  float *dy;                    // [M, n_S d_h]
  f16_t *ta, *tb;               // transposed operands [rows, M_pad]
  float *dheads, *gscale, *dlaml, *drow;  // dheads unused (combine_row_kernel writes dH in fp16);
                                         // gscale: kGradScaleBlocks maxima of |dout|, then (s, 1/s)
  f16_t *dh16;                  // [M, n_H, d_h]
  f16_t *qT, *dhT;              // dim-major copies of q and dH (see BwdAttnArgs)
  float *dq, *dk, *dv;          // attention gradients (dq unused: the dq kernel packs into a6)
  f16_t *a6, *a3, *a8;          // gradient operands [M, k6], [M, k3], [M, k8]
  float *dkr, *dcbar, *dckv, *rkv, *dcq, *daq, *rq;
  int32_t *lo;                  // [M + 32]
  float2 *rope_cs;              // [T, d_r / 2] (cos, sin)
  float *splitk;                // kSplitKBytes: K-slice partials of the small-grid products
};
struct FastBwdArgs {
  const void *x, *dout;
  const gdla_weights *w;
  const int32_t *doc;
  gdla_grads grads;
  const f16_t *cq16;            // [M, d_cq] c^Q of the forward
  const float *aq, *ckv;        // [M, d_cq], [M, d_c] before RMSNorm
  const bf16_t *cache;          // [B, T, d_c + d_r] cache rows of the forward
  const f16_t *q16, *kx, *vk;   // forward operands (see BwdAttnArgs)
  const float *heads, *lse, *lam;  // lse: [n_H, M] (+32), from the forward
  const f16_t *sg16, *y16;      // sigmoid(G), Y of the forward [M, n_S d_h]
  int32_t lam_overridden;
  FastBwdBuffers buf;
  int32_t B, T, M, M_pad, lcap, k8;
};
hipError_t launch_backward_fast(const FastBwdArgs &a, const LayerDims &d, hipStream_t s);

}  // namespace gdla

