// Backward pass of one GDLA layer over training sequences (positions 0 .. T-1, no cached prefix):
// the gradients of L = sum(out (.) dout) with respect to x and every weight.
//
// The pages train with GDLA layers and recompute each block's forward during the backward pass
// (Motif 3 Technical Report, paperglide reader, section "Distributed Training System": activation
// recomputation).  The forward is that of picx.dev summary section 2.2, Eq.(1)-(10); the
// backward is its chain rule, taken in reverse order:
//   Eq.(10)  out = vec(Y) W_O, Y = sigmoid(G) (.) D      -> dW_O, dY, dD, dG
//   Eq.(8)   D_i = H_i - lambda_i H_(n_S + i mod n_N)    -> dH (signal and noise heads), dlambda
//   both softmax maps, per head h with KV head kv(h):
//            P = softmax(tau (q^C K^C^T + q^R k^R^T)) (masked), H = P V
//            dP = dH V^T, dS = P (.) (dP - rowsum(dH (.) H)),
//            dq^C = tau dS K^C, dq^R = tau dS k^R, dK^C += tau dS^T q^C, dk^R += tau dS^T q^R,
//            dV += P^T dH  (K^C, V summed over the heads of a KV group; k^R over all heads)
//   Eq.(5)   [K^C ; V] = cbar [W_uk | W_uv]              -> dcbar, dW_uk, dW_uv
//   Eq.(4), (1)  RMSNorm: with u = dy (.) gamma, dv = u / r - v (u . v) / (n r^3)
//   Eq.(2), (3)  RoPE: the backward rotates by the negative angle
//   Eq.(7)   lambda = sigmoid(x W_lambda)
//   Eq.(1)-(3), (7), (9)  the projections                -> dW_qa, dW_qc, dW_qr, dW_gate, dW_dkv,
//                                                           dW_kr, dW_lambda, dx
// This file is the general path: every step in fp32 (the recomputed forward included), any layer
// sizes the forward's generic path takes, fp32 or bf16 storage.
#include "fast_paths.h"

#include <math.h>

#include <algorithm>

namespace gdla {
namespace {

template <typename T> __device__ __forceinline__ float ldv(const T *p, int64_t i) { return (float)p[i]; }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------------------------------------
// C[M, N] (fp32, row stride ldc) = (beta ? C : 0) + op(A) op(B), op(A)[m, k] = A[m lda + k] or, with
// a_t, A[k lda + m]; op(B)[k, n] = B[k ldb + n] or, with b_t, B[n ldb + k].  64 x 64 tiles,
// 16-deep K slices in LDS, 4 x 4 outputs per thread.
template <typename TA, typename TB>
__global__ void __launch_bounds__(256) grad_gemm_kernel(const TA *A, int64_t lda, int a_t, const TB *B, int64_t ldb,
                                                        int b_t, float *C, int64_t ldc, int M, int N, int K, int beta,
                                                        int tiles_n) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  const int m0 = ((int)blockIdx.x / tiles_n) * 64, n0 = ((int)blockIdx.x % tiles_n) * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      // A tile: with a_t the 64 rows of op(A) are contiguous in memory, so threads run along m
      int r, c;
      if (a_t) { r = i & 63; c = i >> 6; } else { r = i >> 4; c = i & 15; }
      const int gm = m0 + r, gk = k0 + c;
      As[c][r] = (gm < M && gk < K) ? ldv(A, a_t ? (int64_t)gk * lda + gm : (int64_t)gm * lda + gk) : 0.f;
      int kr, nc;
      if (b_t) { kr = i & 15; nc = i >> 4; } else { kr = i >> 6; nc = i & 63; }
      const int bk = k0 + kr, bn = n0 + nc;
      Bs[kr][nc] = (bk < K && bn < N) ? ldv(B, b_t ? (int64_t)bn * ldb + bk : (int64_t)bk * ldb + bn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float *c = C + (int64_t)m * ldc + n;
      *c = beta ? *c + acc[i][j] : acc[i][j];
    }
  }
}

// ------------------------------------------------------------------------------------------
// Recomputed forward, row-wise: c^Q = RMSNorm(aq) gamma_q, cbar = RMSNorm(ckv) gamma_kv (and the
// inverse RMS of both rows), k^R = RoPE(krp, t), lambda = sigmoid(laml) or the override.
__device__ __forceinline__ void rope_angle(int p, int j, int d_r, float theta, float &c, float &s) {
  const double freq = pow((double)theta, -2.0 * (double)j / (double)d_r);
  double a = (double)p * freq;
  const double two_pi = 6.283185307179586476925286766559;
  a -= floor(a / two_pi) * two_pi;
  sincosf((float)a, &s, &c);
}

template <typename T>
__global__ void __launch_bounds__(64) bwd_prep_kernel(const float *aq, const float *ckv, const float *krp,
                                                      const float *laml, const float *lam_override, const T *gq,
                                                      const T *gkv, float *cq, float *cbar, float *kr, float *lam,
                                                      float *rinv_q, float *rinv_kv, int32_t T_, LayerDims d) {
  const int m = blockIdx.x, lane = threadIdx.x, t = m % T_;
  float ss = 0.f;
  for (int j = lane; j < d.d_cq; j += 64) ss += aq[(int64_t)m * d.d_cq + j] * aq[(int64_t)m * d.d_cq + j];
  const float rq = 1.0f / sqrtf(wsum(ss) / d.d_cq + d.eps);
  for (int j = lane; j < d.d_cq; j += 64)
    cq[(int64_t)m * d.d_cq + j] = aq[(int64_t)m * d.d_cq + j] * rq * (gq ? ldv(gq, j) : 1.f);
  ss = 0.f;
  for (int j = lane; j < d.d_c; j += 64) ss += ckv[(int64_t)m * d.d_c + j] * ckv[(int64_t)m * d.d_c + j];
  const float rk = 1.0f / sqrtf(wsum(ss) / d.d_c + d.eps);
  for (int j = lane; j < d.d_c; j += 64)
    cbar[(int64_t)m * d.d_c + j] = ckv[(int64_t)m * d.d_c + j] * rk * (gkv ? ldv(gkv, j) : 1.f);
  const int half = d.d_r / 2;
  for (int j = lane; j < half; j += 64) {
    float c, s;
    rope_angle(t, j, d.d_r, d.theta, c, s);
    const float u = krp[(int64_t)m * d.d_r + j], v = krp[(int64_t)m * d.d_r + j + half];
    kr[(int64_t)m * d.d_r + j] = u * c - v * s;
    kr[(int64_t)m * d.d_r + j + half] = u * s + v * c;
  }
  for (int i = lane; i < d.n_signal; i += 64)
    lam[(int64_t)m * d.n_signal + i] = lam_override ? lam_override[(int64_t)m * d.n_signal + i]
                                                    : 1.0f / (1.0f + expf(-laml[(int64_t)m * d.n_signal + i]));
  if (lane == 0) {
    rinv_q[m] = rq;
    rinv_kv[m] = rk;
  }
}

// v [M, n_heads, d_r] rotated in place by +angle (sign = 1, RoPE) or -angle (sign = -1, its
// backward); row m sits at position m % T.
__global__ void __launch_bounds__(256) bwd_rope_kernel(float *v, int32_t M, int32_t T_, int32_t n_heads, int32_t d_r,
                                                       float theta, float sign) {
  const int half = d_r / 2;
  const int64_t n = (int64_t)M * n_heads * half;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int j = (int)(i % half);
    const int64_t mh = i / half;
    const int t = (int)((mh / n_heads) % T_);
    float c, s;
    rope_angle(t, j, d_r, theta, c, s);
    s *= sign;
    float *r = v + mh * d_r;
    const float u = r[j], w = r[j + half];
    r[j] = u * c - w * s;
    r[j + half] = u * s + w * c;
  }
}

// ------------------------------------------------------------------------------------------
// Attention (fp32, one wave per query row and head).  Visible keys of token t of a sequence:
// lo(t) .. t with lo(t) = max(window start, document start).
struct BwdAttn {
  const float *qc, *qr;       // [M, n_H, d_h], [M, n_H, d_r]
  const float *kc, *v;        // [M, n_kv, d_h]
  const float *kr;            // [M, d_r]
  const int32_t *doc;         // [M] or null
  float *heads, *lse;         // [M, n_H, d_h], [M, n_H]
  const float *dheads;        // [M, n_H, d_h]
  const float *drow;          // [M, n_H]: rowsum(dH (.) H)
  float *dqc, *dqr;           // [M, n_H, d_h], [M, n_H, d_r]
  float *dkc, *dv;            // [M, n_kv, d_h]
  float *dkr_part;            // [M, n_kv, d_r]: dk^R summed over the heads of each KV group
  int32_t M, T;
};

constexpr int kMaxHd = 4;  // d_head <= 256 (chunks of 64 lanes)

__device__ __forceinline__ int vis_lo(const BwdAttn &a, const LayerDims &d, int m, int t) {
  int lo = d.window > 0 ? max(0, t - d.window + 1) : 0;
  if (a.doc) lo = max(lo, min(max(a.doc[m], 0), t));
  return lo;
}

// score of query row m (head h) against key row ms, scaled by tau
__device__ __forceinline__ float score(const BwdAttn &a, const LayerDims &d, const float (&q)[kMaxHd], float qr,
                                       int h, int ms, int lane) {
  const int kv = kv_head_of(h, d.n_signal, d.n_kv);
  const float *k = a.kc + ((int64_t)ms * d.n_kv + kv) * d.d_h;
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    if (e < d.d_h) dot = fmaf(q[i], k[e], dot);
  }
  if (lane < d.d_r) dot = fmaf(qr, a.kr[(int64_t)ms * d.d_r + lane], dot);
  return wsum(dot) * d.scale;
}

// H and the log-sum-exp of every (row, head)
__global__ void __launch_bounds__(256) bwd_attn_fwd_kernel(BwdAttn a, LayerDims d) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.M * d.n_heads) return;
  const int m = (int)(wid / d.n_heads), h = (int)(wid % d.n_heads);
  const int t = m % a.T, m0 = m - t;
  const int kv = kv_head_of(h, d.n_signal, d.n_kv);
  float q[kMaxHd], acc[kMaxHd];
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    q[i] = e < d.d_h ? a.qc[wid * d.d_h + e] : 0.f;
    acc[i] = 0.f;
  }
  const float qr = lane < d.d_r ? a.qr[wid * d.d_r + lane] : 0.f;
  float mx = -INFINITY, l = 0.f;
  for (int s = vis_lo(a, d, m, t); s <= t; ++s) {
    const float sc = score(a, d, q, qr, h, m0 + s, lane);
    const float mn = fmaxf(mx, sc);
    const float corr = expf(mx - mn), w = expf(sc - mn);
    l = l * corr + w;
    const float *vr = a.v + ((int64_t)(m0 + s) * d.n_kv + kv) * d.d_h;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i) {
      const int e = lane + 64 * i;
      if (e < d.d_h) acc[i] = acc[i] * corr + w * vr[e];
    }
    mx = mn;
  }
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    if (e < d.d_h) a.heads[wid * d.d_h + e] = acc[i] / l;
  }
  if (lane == 0) a.lse[wid] = mx + logf(l);
}

// dq^C and dq^R of every (row, head): loop over the row's visible keys
__global__ void __launch_bounds__(256) bwd_attn_dq_kernel(BwdAttn a, LayerDims d) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.M * d.n_heads) return;
  const int m = (int)(wid / d.n_heads), h = (int)(wid % d.n_heads);
  const int t = m % a.T, m0 = m - t;
  const int kv = kv_head_of(h, d.n_signal, d.n_kv);
  float q[kMaxHd], dh[kMaxHd], dq[kMaxHd];
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    q[i] = e < d.d_h ? a.qc[wid * d.d_h + e] : 0.f;
    dh[i] = e < d.d_h ? a.dheads[wid * d.d_h + e] : 0.f;
    dq[i] = 0.f;
  }
  const float qr = lane < d.d_r ? a.qr[wid * d.d_r + lane] : 0.f;
  const float lse = a.lse[wid], drow = a.drow[wid];
  float dqr = 0.f;
  for (int s = vis_lo(a, d, m, t); s <= t; ++s) {
    const int ms = m0 + s;
    const float p = expf(score(a, d, q, qr, h, ms, lane) - lse);
    const float *vr = a.v + ((int64_t)ms * d.n_kv + kv) * d.d_h;
    float dp = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i) {
      const int e = lane + 64 * i;
      if (e < d.d_h) dp = fmaf(dh[i], vr[e], dp);
    }
    const float ds = p * (wsum(dp) - drow) * d.scale;
    const float *kr = a.kc + ((int64_t)ms * d.n_kv + kv) * d.d_h;
#pragma unroll
    for (int i = 0; i < kMaxHd; ++i) {
      const int e = lane + 64 * i;
      if (e < d.d_h) dq[i] = fmaf(ds, kr[e], dq[i]);
    }
    if (lane < d.d_r) dqr = fmaf(ds, a.kr[(int64_t)ms * d.d_r + lane], dqr);
  }
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    if (e < d.d_h) a.dqc[wid * d.d_h + e] = dq[i];
  }
  if (lane < d.d_r) a.dqr[wid * d.d_r + lane] = dqr;
}

// dK^C, dV and the group's share of dk^R of every (key row, KV head): loop over the heads of the
// group and the query rows that see the key
__global__ void __launch_bounds__(256) bwd_attn_dkv_kernel(BwdAttn a, LayerDims d) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.M * d.n_kv) return;
  const int ms = (int)(wid / d.n_kv), kv = (int)(wid % d.n_kv);
  const int s = ms % a.T, m0 = ms - s;
  float k[kMaxHd], vv[kMaxHd], dk[kMaxHd], dvv[kMaxHd];
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    k[i] = e < d.d_h ? a.kc[wid * d.d_h + e] : 0.f;
    vv[i] = e < d.d_h ? a.v[wid * d.d_h + e] : 0.f;
    dk[i] = dvv[i] = 0.f;
  }
  const float kr = lane < d.d_r ? a.kr[(int64_t)ms * d.d_r + lane] : 0.f;
  float dkr = 0.f;
  const int t_end = d.window > 0 ? min(a.T - 1, s + d.window - 1) : a.T - 1;
  for (int h = 0; h < d.n_heads; ++h) {
    if (kv_head_of(h, d.n_signal, d.n_kv) != kv) continue;
    for (int t = s; t <= t_end; ++t) {
      const int m = m0 + t;
      if (a.doc && min(max(a.doc[m], 0), t) > s) break;  // later tokens' documents start later still
      const int64_t mh = (int64_t)m * d.n_heads + h;
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxHd; ++i) {
        const int e = lane + 64 * i;
        if (e < d.d_h) {
          dot = fmaf(a.qc[mh * d.d_h + e], k[i], dot);
          dp = fmaf(a.dheads[mh * d.d_h + e], vv[i], dp);
        }
      }
      if (lane < d.d_r) dot = fmaf(a.qr[mh * d.d_r + lane], kr, dot);
      const float p = expf(wsum(dot) * d.scale - a.lse[mh]);
      const float ds = p * (wsum(dp) - a.drow[mh]) * d.scale;
#pragma unroll
      for (int i = 0; i < kMaxHd; ++i) {
        const int e = lane + 64 * i;
        if (e < d.d_h) {
          dk[i] = fmaf(ds, a.qc[mh * d.d_h + e], dk[i]);
          dvv[i] = fmaf(p, a.dheads[mh * d.d_h + e], dvv[i]);
        }
      }
      if (lane < d.d_r) dkr = fmaf(ds, a.qr[mh * d.d_r + lane], dkr);
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxHd; ++i) {
    const int e = lane + 64 * i;
    if (e < d.d_h) {
      a.dkc[wid * d.d_h + e] = dk[i];
      a.dv[wid * d.d_h + e] = dvv[i];
    }
  }
  if (lane < d.d_r) a.dkr_part[wid * d.d_r + lane] = dkr;
}

// dk^R[m] = sum over KV groups of their shares
__global__ void __launch_bounds__(256) bwd_sum_groups_kernel(const float *part, float *out, int32_t M, int32_t n_kv,
                                                             int32_t d_r) {
  const int64_t n = (int64_t)M * d_r;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / d_r;
    const int j = (int)(i % d_r);
    float acc = 0.f;
    for (int g = 0; g < n_kv; ++g) acc += part[(m * n_kv + g) * d_r + j];
    out[i] = acc;
  }
}

// ------------------------------------------------------------------------------------------
// Eq.(8)-(10) forward and backward per row, element (i, e) of the signal heads:
//   sg = sigmoid(G), D = H_i - lambda_i H_(n_S + i mod n_N), Y = sg D;
//   dD = dY sg, dG = dY D sg (1 - sg), dH_i = dD.
// Y goes out in fp32 (the W_O gradient's operand); noise-head dH and dlambda are reduced below.
__global__ void __launch_bounds__(256) bwd_combine_kernel(const float *heads, const float *lam, const float *g,
                                                          const float *dy, float *y, float *dheads, float *dd,
                                                          float *dg, int32_t M, LayerDims d) {
  const int64_t n = (int64_t)M * d.n_signal * d.d_h;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int e = (int)(idx % d.d_h);
    const int64_t r = idx / d.d_h;
    const int i = (int)(r % d.n_signal);
    const int64_t m = r / d.n_signal;
    const float hs = heads[(m * d.n_heads + i) * d.d_h + e];
    const float hn = heads[(m * d.n_heads + d.n_signal + i % d.n_noise) * d.d_h + e];
    const float dval = hs - lam[m * d.n_signal + i] * hn;
    const float sg = 1.0f / (1.0f + expf(-g[idx]));
    y[idx] = sg * dval;
    const float ddv = dy[idx] * sg;
    dd[idx] = ddv;
    dg[idx] = dy[idx] * dval * sg * (1.0f - sg);
    dheads[(m * d.n_heads + i) * d.d_h + e] = ddv;
  }
}

// noise head j: dH = -sum over the signal heads i = j (mod n_N) of lambda_i dD_i; and
// dlambda_i = -sum_e dD_i,e H_(n_S + i mod n_N),e, then through the sigmoid unless overridden
__global__ void __launch_bounds__(256) bwd_noise_lambda_kernel(const float *heads, const float *lam, const float *dd,
                                                               float *dheads, float *dlam_logit, int override_lam,
                                                               int32_t M, LayerDims d) {
  const int64_t nn = (int64_t)M * d.n_noise * d.d_h;
  const int64_t nl = (int64_t)M * d.n_signal;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < nn + nl; idx += (int64_t)gridDim.x * 256) {
    if (idx < nn) {
      const int e = (int)(idx % d.d_h);
      const int64_t r = idx / d.d_h;
      const int j = (int)(r % d.n_noise);
      const int64_t m = r / d.n_noise;
      float acc = 0.f;
      for (int i = j; i < d.n_signal; i += d.n_noise)
        acc -= lam[m * d.n_signal + i] * dd[(m * d.n_signal + i) * d.d_h + e];
      dheads[(m * d.n_heads + d.n_signal + j) * d.d_h + e] = acc;
    } else {
      const int64_t r = idx - nn;
      const int i = (int)(r % d.n_signal);
      const int64_t m = r / d.n_signal;
      const float *hn = heads + (m * d.n_heads + d.n_signal + i % d.n_noise) * d.d_h;
      const float *ddi = dd + r * d.d_h;
      float acc = 0.f;
      for (int e = 0; e < d.d_h; ++e) acc -= ddi[e] * hn[e];
      const float l = lam[r];
      dlam_logit[r] = override_lam ? 0.f : acc * l * (1.0f - l);
    }
  }
}

// drow[m, h] = sum_e dH (.) H, row r = m n_H + h stored at r, or (head_major, n_heads given) at
// h M + m
__global__ void __launch_bounds__(256) bwd_drow_kernel(const float *heads, const float *dheads, float *drow,
                                                       int64_t rows, int32_t d_h, int32_t head_major_nh) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float acc = 0.f;
  for (int e = lane; e < d_h; e += 64) acc += heads[r * d_h + e] * dheads[r * d_h + e];
  acc = wsum(acc);
  if (lane == 0) {
    if (head_major_nh > 0) drow[(r % head_major_nh) * (rows / head_major_nh) + r / head_major_nh] = acc;
    else drow[r] = acc;
  }
}

// RMSNorm backward of y = v rinv (.) gamma per row: dv = rinv (u - v rinv^2 (u . v) / n), u = dy (.) gamma
template <typename T>
__global__ void __launch_bounds__(64) bwd_rms_kernel(const float *v, const float *rinv, const T *gamma, const float *dy,
                                                     float *dv, int32_t n) {
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x;
  const float r = rinv[m];
  float uv = 0.f;
  for (int j = lane; j < n; j += 64) uv += dy[m * n + j] * (gamma ? ldv(gamma, j) : 1.f) * v[m * n + j];
  uv = wsum(uv);
  for (int j = lane; j < n; j += 64) {
    const float u = dy[m * n + j] * (gamma ? ldv(gamma, j) : 1.f);
    dv[m * n + j] = r * (u - v[m * n + j] * r * r * uv / n);
  }
}

// dgamma[j] = sum over rows of dy (.) v rinv (column sums, fixed order)
__global__ void __launch_bounds__(256) bwd_dgamma_kernel(const float *v, const float *rinv, const float *dy,
                                                         float *dgamma, int32_t M, int32_t n) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float acc = 0.f;
  for (int m = 0; m < M; ++m) acc += dy[(int64_t)m * n + j] * v[(int64_t)m * n + j] * rinv[m];
  dgamma[j] = acc;
}

unsigned grid_for(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); }

template <typename TA, typename TB>
hipError_t gg(const TA *A, int64_t lda, bool a_t, const TB *B, int64_t ldb, bool b_t, float *C, int64_t ldc, int M,
              int N, int K, bool beta, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int tn = (N + 63) / 64, tm = (M + 63) / 64;
  hipLaunchKernelGGL((grad_gemm_kernel<TA, TB>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, A, lda, a_t ? 1 : 0, B,
                     ldb, b_t ? 1 : 0, C, ldc, M, N, K, beta ? 1 : 0, tn);
  return hipGetLastError();
}

#define BWD_TRY(expr)                       \
  do {                                      \
    const hipError_t e_ = (expr);           \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

template <typename T>
hipError_t backward_t(const BackwardArgs &ba, const LayerDims &d, hipStream_t s) {
  const int M = ba.M, T_ = ba.T;
  const T *x = (const T *)ba.x;
  const gdla_weights &w = *ba.w;
  const T *Wqa = (const T *)w.w_qa, *Wqc = (const T *)w.w_qc, *Wqr = (const T *)w.w_qr;
  const T *Wdkv = (const T *)w.w_dkv, *Wkr = (const T *)w.w_kr, *Wuk = (const T *)w.w_uk, *Wuv = (const T *)w.w_uv;
  const T *Wl = (const T *)w.w_lambda, *Wg = (const T *)w.w_gate, *Wo = (const T *)w.w_o;
  const T *gq = (const T *)w.gamma_q, *gkv = (const T *)w.gamma_kv;
  const int dm = d.d_model, dcq = d.d_cq, dc = d.d_c, dr = d.d_r, dh = d.d_h;
  const int nH = d.n_heads, nS = d.n_signal, nKV = d.n_kv;
  const BwdBuffers &b = ba.buf;

  // ---- recomputed forward (fp32)
  BWD_TRY(gg(x, dm, false, Wqa, dcq, false, b.aq, dcq, M, dcq, dm, false, s));
  BWD_TRY(gg(x, dm, false, Wdkv, dc, false, b.ckv, dc, M, dc, dm, false, s));
  BWD_TRY(gg(x, dm, false, Wkr, dr, false, b.krp, dr, M, dr, dm, false, s));
  BWD_TRY(gg(x, dm, false, Wl, nS, false, b.laml, nS, M, nS, dm, false, s));
  hipLaunchKernelGGL((bwd_prep_kernel<T>), dim3(M), dim3(64), 0, s, b.aq, b.ckv, b.krp, b.laml, ba.lam_override, gq,
                     gkv, b.cq, b.cbar, b.kr, b.lam, b.rq, b.rkv, T_, d);
  BWD_TRY(hipGetLastError());
  BWD_TRY(gg(b.cq, dcq, false, Wqc, (int64_t)nH * dh, false, b.qc, (int64_t)nH * dh, M, nH * dh, dcq, false, s));
  BWD_TRY(gg(b.cq, dcq, false, Wqr, (int64_t)nH * dr, false, b.qr, (int64_t)nH * dr, M, nH * dr, dcq, false, s));
  hipLaunchKernelGGL(bwd_rope_kernel, dim3(grid_for((int64_t)M * nH * dr / 2)), dim3(256), 0, s, b.qr, M, T_, nH, dr,
                     d.theta, 1.0f);
  BWD_TRY(hipGetLastError());
  BWD_TRY(gg(b.cq, dcq, false, Wg, (int64_t)nS * dh, false, b.g, (int64_t)nS * dh, M, nS * dh, dcq, false, s));
  BWD_TRY(gg(b.cbar, dc, false, Wuk, (int64_t)nKV * dh, false, b.kc, (int64_t)nKV * dh, M, nKV * dh, dc, false, s));
  BWD_TRY(gg(b.cbar, dc, false, Wuv, (int64_t)nKV * dh, false, b.v, (int64_t)nKV * dh, M, nKV * dh, dc, false, s));
  BwdAttn at{};
  at.qc = b.qc; at.qr = b.qr; at.kc = b.kc; at.v = b.v; at.kr = b.kr; at.doc = ba.doc;
  at.heads = b.heads; at.lse = b.lse; at.dheads = b.dheads; at.drow = b.drow;
  at.dqc = b.dqc; at.dqr = b.dqr; at.dkc = b.dkc; at.dv = b.dv; at.dkr_part = b.dkr_part;
  at.M = M; at.T = T_;
  const unsigned gh = (unsigned)(((int64_t)M * nH + 3) / 4);
  hipLaunchKernelGGL(bwd_attn_fwd_kernel, dim3(gh), dim3(256), 0, s, at, d);
  BWD_TRY(hipGetLastError());

  // ---- Eq.(10): dY = dout W_O^T, and dW_O = Y^T dout once Y is known
  const T *dout = (const T *)ba.dout;
  BWD_TRY(gg(dout, dm, false, Wo, dm, true, b.dy, (int64_t)nS * dh, M, nS * dh, dm, false, s));
  const int64_t nsig = (int64_t)M * nS * dh;
  hipLaunchKernelGGL(bwd_combine_kernel, dim3(grid_for(nsig)), dim3(256), 0, s, b.heads, b.lam, b.g, b.dy, b.y,
                     b.dheads, b.dd, b.dg, M, d);
  BWD_TRY(hipGetLastError());
  BWD_TRY(gg(b.y, (int64_t)nS * dh, true, dout, dm, false, ba.grads.dw_o, dm, nS * dh, dm, M, false, s));
  // ---- Eq.(8): noise-head dH and dlambda
  hipLaunchKernelGGL(bwd_noise_lambda_kernel, dim3(grid_for((int64_t)M * d.n_noise * dh + (int64_t)M * nS)), dim3(256),
                     0, s, b.heads, b.lam, b.dd, b.dheads, b.dlaml, ba.lam_override ? 1 : 0, M, d);
  BWD_TRY(hipGetLastError());
  // ---- the softmax maps
  hipLaunchKernelGGL(bwd_drow_kernel, dim3(gh), dim3(256), 0, s, b.heads, b.dheads, b.drow, (int64_t)M * nH, dh, 0);
  BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(bwd_attn_dq_kernel, dim3(gh), dim3(256), 0, s, at, d);
  BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(bwd_attn_dkv_kernel, dim3((unsigned)(((int64_t)M * nKV + 3) / 4)), dim3(256), 0, s, at, d);
  BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(bwd_sum_groups_kernel, dim3(grid_for((int64_t)M * dr)), dim3(256), 0, s, b.dkr_part, b.dkr, M,
                     nKV, dr);
  BWD_TRY(hipGetLastError());
  // RoPE backward of dq^R and dk^R (in place)
  hipLaunchKernelGGL(bwd_rope_kernel, dim3(grid_for((int64_t)M * nH * dr / 2)), dim3(256), 0, s, b.dqr, M, T_, nH, dr,
                     d.theta, -1.0f);
  BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(bwd_rope_kernel, dim3(grid_for((int64_t)M * dr / 2)), dim3(256), 0, s, b.dkr, M, T_, 1, dr,
                     d.theta, -1.0f);
  BWD_TRY(hipGetLastError());

  // ---- Eq.(5), (4): the latent
  const gdla_grads &G = ba.grads;
  BWD_TRY(gg(b.cbar, dc, true, b.dkc, (int64_t)nKV * dh, false, G.dw_uk, (int64_t)nKV * dh, dc, nKV * dh, M, false, s));
  BWD_TRY(gg(b.cbar, dc, true, b.dv, (int64_t)nKV * dh, false, G.dw_uv, (int64_t)nKV * dh, dc, nKV * dh, M, false, s));
  BWD_TRY(gg(b.dkc, (int64_t)nKV * dh, false, Wuk, (int64_t)nKV * dh, true, b.dcbar, dc, M, dc, nKV * dh, false, s));
  BWD_TRY(gg(b.dv, (int64_t)nKV * dh, false, Wuv, (int64_t)nKV * dh, true, b.dcbar, dc, M, dc, nKV * dh, true, s));
  hipLaunchKernelGGL((bwd_rms_kernel<T>), dim3(M), dim3(64), 0, s, b.ckv, b.rkv, gkv, b.dcbar, b.dckv, dc);
  BWD_TRY(hipGetLastError());
  if (G.dgamma_kv) {
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((dc + 255) / 256), dim3(256), 0, s, b.ckv, b.rkv, b.dcbar,
                       G.dgamma_kv, M, dc);
    BWD_TRY(hipGetLastError());
  }
  // ---- Eq.(2), (9), (1): the query latent
  BWD_TRY(gg(b.cq, dcq, true, b.dqc, (int64_t)nH * dh, false, G.dw_qc, (int64_t)nH * dh, dcq, nH * dh, M, false, s));
  BWD_TRY(gg(b.cq, dcq, true, b.dqr, (int64_t)nH * dr, false, G.dw_qr, (int64_t)nH * dr, dcq, nH * dr, M, false, s));
  BWD_TRY(gg(b.cq, dcq, true, b.dg, (int64_t)nS * dh, false, G.dw_gate, (int64_t)nS * dh, dcq, nS * dh, M, false, s));
  BWD_TRY(gg(b.dqc, (int64_t)nH * dh, false, Wqc, (int64_t)nH * dh, true, b.dcq, dcq, M, dcq, nH * dh, false, s));
  BWD_TRY(gg(b.dqr, (int64_t)nH * dr, false, Wqr, (int64_t)nH * dr, true, b.dcq, dcq, M, dcq, nH * dr, true, s));
  BWD_TRY(gg(b.dg, (int64_t)nS * dh, false, Wg, (int64_t)nS * dh, true, b.dcq, dcq, M, dcq, nS * dh, true, s));
  hipLaunchKernelGGL((bwd_rms_kernel<T>), dim3(M), dim3(64), 0, s, b.aq, b.rq, gq, b.dcq, b.daq, dcq);
  BWD_TRY(hipGetLastError());
  if (G.dgamma_q) {
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((dcq + 255) / 256), dim3(256), 0, s, b.aq, b.rq, b.dcq, G.dgamma_q, M,
                       dcq);
    BWD_TRY(hipGetLastError());
  }
  // ---- x and the x-side weights
  BWD_TRY(gg(x, dm, true, b.daq, dcq, false, G.dw_qa, dcq, dm, dcq, M, false, s));
  BWD_TRY(gg(x, dm, true, b.dckv, dc, false, G.dw_dkv, dc, dm, dc, M, false, s));
  BWD_TRY(gg(x, dm, true, b.dkr, dr, false, G.dw_kr, dr, dm, dr, M, false, s));
  BWD_TRY(gg(x, dm, true, b.dlaml, nS, false, G.dw_lambda, nS, dm, nS, M, false, s));
  BWD_TRY(gg(b.daq, dcq, false, Wqa, dcq, true, G.dx, dm, M, dm, dcq, false, s));
  BWD_TRY(gg(b.dckv, dc, false, Wdkv, dc, true, G.dx, dm, M, dm, dc, true, s));
  BWD_TRY(gg(b.dkr, dr, false, Wkr, dr, true, G.dx, dm, M, dm, dr, true, s));
  BWD_TRY(gg(b.dlaml, nS, false, Wl, nS, true, G.dx, dm, M, dm, nS, true, s));
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward_generic(const BackwardArgs &a, const LayerDims &d, DT dt, hipStream_t s) {
  return dt == DT::F32 ? backward_t<float>(a, d, s) : backward_t<bf16_t>(a, d, s);
}

}  // namespace gdla

// ==============================================================================================
// Fast path (bf16 layer, d_head 128, d_rope 64, after the fused forward): the attention maps run in
// bwd_attn.hip and every product on the transposed-weight MFMA GEMM with fp16 operands: data
// gradients take the stored weights [in, out] as the K-major operand directly (converted to fp16,
// and concatenated so that dc^Q and dx are one GEMM each), weight gradients take transposed
// copies of the activations and gradients (tokens as K, padded with zeros to a multiple of 64).
namespace gdla {
namespace {

__device__ __forceinline__ f16_t f16s(float v) { return (f16_t)(v); }

// dst[r, col_off + c] = fp16(src[r, c])  (r < rows, c < cols)
template <typename TS>
__global__ void __launch_bounds__(256) pack_f16_kernel(const TS *src, int64_t lds, int32_t rows, int32_t cols,
                                                       f16_t *dst, int64_t ldd, int32_t col_off, const float *scale) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const float sc = scale ? scale[0] : 1.0f;
  // runs of 4 columns when every run is aligned on both sides (the usual case), else one by one
  const bool quads = cols % 4 == 0 && lds % 4 == 0 && ldd % 4 == 0 && col_off % 4 == 0 &&
                     ((uintptr_t)src & (4 * sizeof(TS) - 1)) == 0 && ((uintptr_t)dst & 7) == 0;
  if (quads) {
    const int c4 = cols / 4;
    const int64_t n = (int64_t)rows * c4;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
      const int64_t r = i / c4;
      const int c = 4 * (int)(i % c4);
      const TS *p = src + r * lds + c;
      h4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = f16s((float)p[k] * sc);
      *(h4 *)(dst + r * ldd + col_off + c) = v;
    }
    return;
  }
  const int64_t n = (int64_t)rows * cols;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols;
    const int c = (int)(i % cols);
    dst[r * ldd + col_off + c] = f16s((float)src[r * lds + c] * sc);
  }
}

// dst[row_off + c, r] = fp16(src[r, c]) for r < R, 0 for R <= r < R_pad (64 x 64 tiles through LDS).
// Each thread moves runs of 8: 16-byte row reads of the source (when aligned and inside the
// matrix) and 16-byte column runs of the destination.
template <typename TS>
__global__ void __launch_bounds__(256) tpack_f16_kernel(const TS *src, int64_t lds, int32_t R, int32_t C, int32_t R_pad,
                                                        f16_t *dst, int64_t ldd, int32_t row_off, const float *scale) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const float sc = scale ? scale[0] : 1.0f;
  __shared__ __attribute__((aligned(16))) f16_t tile[64][72];  // row pitch 144 bytes
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int rr = i >> 3, c8 = (i & 7) * 8;
    const int r = r0 + rr, c = c0 + c8;
    h8 v;
    const TS *p = src + (int64_t)r * lds + c;
    if (r < R && c + 8 <= C && ((uintptr_t)p & 15) == 0) {
      const uint4 raw = *(const uint4 *)p;
      const TS *e = (const TS *)&raw;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = f16s((float)e[k] * sc);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (r < R && c + k < C) ? f16s((float)p[k] * sc) : (f16_t)0.f;
    }
    *(h8 *)&tile[rr][c8] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int cc = i >> 3, r8 = (i & 7) * 8;
    const int c = c0 + cc, r = r0 + r8;
    if (c >= C || r >= R_pad) continue;
    h8 v;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = tile[r8 + k][cc];
    f16_t *q = dst + (int64_t)(row_off + c) * ldd + r;
    if (r + 8 <= R_pad && ((uintptr_t)q & 15) == 0) {
      *(h8 *)q = v;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (r + k < R_pad) q[k] = v[k];
    }
  }
}

// dk [B, n_kv, T, 192], dv [B, n_kv, T, 128] -> [dK^C | dV] as the latent operand a3 [M, 2 n_kv d_h]
// (fp16) and dk^R summed over the KV groups, rotated back (fp32 [M, d_r])
__global__ void __launch_bounds__(256) pack_dkv_kernel(const float *dk, const float *dv, f16_t *a3, float *dkr,
                                                       int32_t M, int32_t T_, LayerDims d, const float2 *cs) {
  const int dqk = d.d_h + d.d_r, half = d.d_r / 2;
  const int64_t nkv = (int64_t)M * d.n_kv * d.d_h;
  const int64_t nr = (int64_t)M * half;
  const int64_t lda3 = 2ll * d.n_kv * d.d_h;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < nkv + nr; idx += (int64_t)gridDim.x * 256) {
    if (idx < nkv) {
      const int e = (int)(idx % d.d_h);
      const int64_t r = idx / d.d_h;
      const int j = (int)(r % d.n_kv);
      const int64_t m = r / d.n_kv, b = m / T_, t = m % T_;
      const int64_t src = ((b * d.n_kv + j) * T_ + t);
      a3[m * lda3 + (int64_t)j * d.d_h + e] = f16s(dk[src * dqk + e]);
      a3[m * lda3 + (int64_t)(d.n_kv + j) * d.d_h + e] = f16s(dv[src * d.d_h + e]);
    } else {
      const int64_t r = idx - nkv;
      const int jj = (int)(r % half);
      const int64_t m = r / half, b = m / T_, t = m % T_;
      float u = 0.f, w = 0.f;
      for (int g = 0; g < d.n_kv; ++g) {
        const float *s = dk + ((b * d.n_kv + g) * T_ + t) * dqk + d.d_h;
        u += s[jj];
        w += s[jj + half];
      }
      const float2 rc = cs[t * half + jj];
      const float c = rc.x, s = rc.y;
      dkr[m * d.d_r + jj] = u * c + w * s;
      dkr[m * d.d_r + jj + half] = -u * s + w * c;
    }
  }
}

// RMSNorm backward per row with the inverse RMS recomputed from v: writes dv and rinv[m]
template <typename T>
__global__ void __launch_bounds__(64) rms_bwd_kernel(const float *v, const T *gamma, const float *dy, float *dv,
                                                     float *rinv, int32_t n, float eps) {
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x;
  float ss = 0.f, uv = 0.f;
  for (int j = lane; j < n; j += 64) {
    const float x = v[m * n + j];
    ss += x * x;
    uv += dy[m * n + j] * (gamma ? (float)gamma[j] : 1.f) * x;
  }
  ss = wsum(ss);
  uv = wsum(uv);
  const float r = 1.0f / sqrtf(ss / n + eps);
  for (int j = lane; j < n; j += 64) {
    const float u = dy[m * n + j] * (gamma ? (float)gamma[j] : 1.f);
    dv[m * n + j] = r * (u - v[m * n + j] * r * r * uv / n);
  }
  if (lane == 0) rinv[m] = r;
}

// dst[r, c] = 0 for r < rows, c0 <= c < c1 (the K padding of a concatenated operand)
// Gradient scaling of the fp16 path.  The backward is linear in dout, so dout may enter the fp16
// operands multiplied by any power of two s and every fp32 gradient divided by s at the end, with
// no rounding of its own.  s puts the largest |dout| in [4, 8), where gradients of every size the
// layer produces stay inside fp16's normal range (an upstream gradient of 1e-6 would otherwise sit
// among fp16's subnormals after the first product, and a very large one overflow).
// Block maxima of |dout| (fmaxf skips a NaN, which then reaches the gradients through the data).
__global__ void __launch_bounds__(256) absmax_part_kernel(const bf16_t *v, int64_t n, float *part) {
  __shared__ float red[4];
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  // 16-byte runs of 8 values when aligned: a bf16's magnitude is its bits without the sign, as the
  // high half of an fp32 (a NaN stays a NaN, which fmaxf passes over, as in the scalar loop)
  const int64_t n8 = ((uintptr_t)v & 15) == 0 ? n / 8 : 0;
  auto take = [&](const uint4 r) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m = fmaxf(m, fmaxf(__uint_as_float((w[k] << 16) & 0x7fffffffu), __uint_as_float(w[k] & 0x7fff0000u)));
  };
  // four runs in flight per thread (the pass is bound by load latency), then the rest
  int64_t i = blockIdx.x * 256ll + threadIdx.x;
  for (; i + 3 * stride < n8; i += 4 * stride) {
    uint4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = ((const uint4 *)v)[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) take(r[u]);
  }
  for (; i < n8; i += stride) take(((const uint4 *)v)[i]);
  for (int64_t i = n8 * 8 + blockIdx.x * 256ll + threadIdx.x; i < n; i += stride) m = fmaxf(m, fabsf((float)v[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
// sc[0] = s = 2^(3 - e) for the largest |dout| = f 2^e (f in [0.5, 1)), sc[1] = 1 / s; s = 1 when
// dout is all zeros (or not finite).  The exponent is clamped so both stay normal fp32 numbers.
__global__ void __launch_bounds__(256) grad_scale_kernel(const float *part, int32_t n, float *sc) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int e = 0;
    if (m > 0.f && m <= 3.0e38f) frexpf(m, &e);
    const int k = min(max(3 - e, -100), 100);
    sc[0] = ldexpf(1.0f, k);
    sc[1] = ldexpf(1.0f, -k);
  }
}
// Every fp32 gradient of the call times 1 / s (exact: a power of two).
struct GradList {
  float *p[16];
  int64_t n[16];
};
__global__ void __launch_bounds__(256) unscale_grads_kernel(GradList g, const float *sc) {
  float *p = g.p[blockIdx.y];
  const int64_t n = g.n[blockIdx.y];
  const float inv = sc[1];
  const int64_t stride = (int64_t)gridDim.x * 256;
  // 16-byte runs when aligned, then the rest one by one
  const int64_t n4 = ((uintptr_t)p & 15) == 0 ? n / 4 : 0;
  // four runs loaded before any is stored (the pass is bound by load latency), then the rest
  int64_t i = blockIdx.x * 256ll + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = ((float4 *)p)[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u].x *= inv; v[u].y *= inv; v[u].z *= inv; v[u].w *= inv;
      ((float4 *)p)[i + u * stride] = v[u];
    }
  }
  for (; i < n4; i += stride) {
    float4 v = ((float4 *)p)[i];
    v.x *= inv; v.y *= inv; v.z *= inv; v.w *= inv;
    ((float4 *)p)[i] = v;
  }
  for (int64_t i = n4 * 4 + blockIdx.x * 256ll + threadIdx.x; i < n; i += stride) p[i] *= inv;
}

__global__ void __launch_bounds__(256) zero_cols_kernel(f16_t *dst, int64_t ldd, int32_t rows, int32_t c0, int32_t c1) {
  const int w = c1 - c0;
  const int64_t n = (int64_t)rows * w;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[(i / w) * ldd + c0 + i % w] = (f16_t)0.f;
}

// Eq.(8) backward of one row per workgroup: noise head j gets dH = -sum over the signal heads
// i = j (mod n_N) of lambda_i dD_i; dlambda_i = -sum_e dD_i,e H_(n_S + i mod n_N),e, through the
// sigmoid unless lambda is fixed.  Reads are contiguous along e.
// Eq.(10) and Eq.(8) backward of one token row m in one workgroup (d_h = 128), everything the
// attention backward and the query-latent GEMM need from the gate and the differential combine:
//   dD_i = dY_i sg_i,  dG_i = dY_i D_i sg_i (1 - sg_i) (fp16 into a6),  dH_i = dD_i,
//   dH_(n_S + j) = -sum over the signal heads i of partner j of lambda_i dD_i,
//   dlambda-logit_i = -(dD_i . H_(n_S + j)) lambda_i (1 - lambda_i)  (0 with a fixed lambda),
//   drow_h = dH_h . H_h (head-major), dH in fp16.
// Wave w takes the noise heads j = w, w + 4, ... and, for each, its signal heads i = j + n_N k;
// lane l holds dims 2 l and 2 l + 1.
__global__ void __launch_bounds__(256) combine_row_kernel(const float *heads, const float *lam, const f16_t *sg16,
                                                          const float *dy, f16_t *dh16, f16_t *a6, int64_t lda6,
                                                          int32_t g_off, float *drow, float *dlam_logit,
                                                          int override_lam, int32_t M, LayerDims d) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int64_t m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = 2 * lane;
  const int nS = d.n_signal, nN = d.n_noise, nH = d.n_heads;
  const float *hm = heads + m * nH * 128;
  for (int j = wave; j < nN; j += 4) {
    const float2 hn = *(const float2 *)(hm + (int64_t)(nS + j) * 128 + e);
    float2 dn = make_float2(0.f, 0.f);
    for (int i = j; i < nS; i += nN) {
      const int64_t yi = (m * nS + i) * 128 + e;
      const float2 hs = *(const float2 *)(hm + (int64_t)i * 128 + e);
      const float2 yv = *(const float2 *)(dy + yi);
      const h2 sgh = *(const h2 *)(sg16 + yi);
      const float l = lam[m * nS + i];
      const float s0 = (float)sgh[0], s1 = (float)sgh[1];
      const float d0 = yv.x * s0, d1 = yv.y * s1;  // dD = dH_i
      h2 g;
      g[0] = f16s(yv.x * (hs.x - l * hn.x) * s0 * (1.0f - s0));
      g[1] = f16s(yv.y * (hs.y - l * hn.y) * s1 * (1.0f - s1));
      *(h2 *)(a6 + m * lda6 + g_off + (int64_t)i * 128 + e) = g;
      h2 dh;
      dh[0] = f16s(d0);
      dh[1] = f16s(d1);
      *(h2 *)(dh16 + (m * nH + i) * 128 + e) = dh;
      dn.x -= l * d0;
      dn.y -= l * d1;
      const float rs = wsum(d0 * hs.x + d1 * hs.y);
      const float dl = wsum(d0 * hn.x + d1 * hn.y);
      if (lane == 0) {
        drow[(int64_t)i * M + m] = rs;
        dlam_logit[m * nS + i] = override_lam ? 0.f : -dl * l * (1.0f - l);
      }
    }
    h2 dh;
    dh[0] = f16s(dn.x);
    dh[1] = f16s(dn.y);
    *(h2 *)(dh16 + (m * nH + nS + j) * 128 + e) = dh;
    const float rn = wsum(dn.x * hn.x + dn.y * hn.y);
    if (lane == 0) drow[(int64_t)(nS + j) * M + m] = rn;
  }
}

// cs[t][j] = (cos, sin) of RoPE's angle for position t and pair j
__global__ void __launch_bounds__(256) rope_table_kernel(float2 *cs, int32_t T_, int32_t d_r, float theta) {
  const int half = d_r / 2;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T_ * half) return;
  float c, s;
  rope_angle(i / half, i % half, d_r, theta, c, s);
  cs[i] = make_float2(c, s);
}

// lo[m] = lowest visible key of token t = m % T (window and document start)
__global__ void __launch_bounds__(256) qlo_kernel(const int32_t *doc, int32_t *lo, int32_t M, int32_t T_, int32_t window) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const int t = m % T_;
  int v = window > 0 ? max(0, t - window + 1) : 0;
  if (doc) v = max(v, min(max(doc[m], 0), t));
  lo[m] = v;
}

template <typename TS>
hipError_t pack(const TS *src, int64_t lds, int rows, int cols, f16_t *dst, int64_t ldd, int col_off, hipStream_t s,
                const float *scale = nullptr) {
  hipLaunchKernelGGL(pack_f16_kernel<TS>, dim3(grid_for((int64_t)rows * cols)), dim3(256), 0, s, src, lds, rows, cols,
                     dst, ldd, col_off, scale);
  return hipGetLastError();
}
template <typename TS>
hipError_t tpack(const TS *src, int64_t lds, int R, int C, int R_pad, f16_t *dst, int64_t ldd, int row_off,
                 hipStream_t s, const float *scale = nullptr) {
  hipLaunchKernelGGL(tpack_f16_kernel<TS>, dim3((C + 63) / 64, (R_pad + 63) / 64), dim3(256), 0, s, src, lds, R, C,
                     R_pad, dst, ldd, row_off, scale);
  return hipGetLastError();
}

// C[M, N] (fp32, ldc) = A[M, K] Bt[N, K]^T, fp16 operands with K-contiguous rows
// C = A . Bt^T in fp32.  A product with fewer 256 x 256 tiles than the chip has CUs (the weight
// gradients reduce over all tokens: few tiles, long K) is split along K into up to 16 slices of
// at least 512, as long as the partials fit `part` (kSplitKBytes); the slices are summed in order.
hipError_t nt(const f16_t *A, int64_t lda, const f16_t *Bt, int64_t ldb, float *C, int64_t ldc, int M, int N, int K,
              hipStream_t s, float *part = nullptr) {
  GemmBatch g{};
  GemmProblem &p = g.p[g.n++];
  p.A = A; p.lda = lda; p.B = Bt; p.ldb = ldb; p.C = C; p.ldc = ldc;
  p.M = M; p.N = N; p.K = K; p.hw = N; p.hs = 0; p.ho = 0; p.c_dt = CD_F32; p.a_f16 = 1; p.epi = EPI_NONE;
  const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  int ks = 1;
  while (part && N % 4 == 0 && ks < 16 && tiles * ks < 256 && K % (64 * 2 * ks) == 0 && K / (2 * ks) >= 512 &&
         (size_t)(2 * ks) * M * N * 4 <= kSplitKBytes)
    ks *= 2;
  if (ks > 1) {
    p.ksplit = ks;
    p.part = part;
  }
  return launch_gemm_nt(g, true, s);
}

}  // namespace

hipError_t launch_backward_fast(const FastBwdArgs &a, const LayerDims &d, hipStream_t s) {
  const int M = a.M, T_ = a.T, Mp = a.M_pad;
  const int dm = d.d_model, dcq = d.d_cq, dc = d.d_c, dr = d.d_r, dh = d.d_h;
  const int nH = d.n_heads, nS = d.n_signal, nKV = d.n_kv;
  const gdla_weights &w = *a.w;
  const gdla_grads &G = a.grads;
  const FastBwdBuffers &b = a.buf;
  const int ny = nS * dh;                        // Y columns
  const int k6 = nH * dh + nH * dr + nS * dh;    // query-latent operand: [dq^C | dq^R | dG]
  const int k3 = 2 * nKV * dh;                   // latent operand: [dK^C | dV]
  const int k8 = a.k8;                           // x operand: [da^Q | dc^KV | dk^R | dlambda | 0]

  // fp16 weights, concatenated along K as the data-gradient GEMMs read them
  BWD_TRY(pack((const bf16_t *)w.w_o, dm, ny, dm, b.wo16, dm, 0, s));
  BWD_TRY(pack((const bf16_t *)w.w_uk, (int64_t)nKV * dh, dc, nKV * dh, b.w3, k3, 0, s));
  BWD_TRY(pack((const bf16_t *)w.w_uv, (int64_t)nKV * dh, dc, nKV * dh, b.w3, k3, nKV * dh, s));
  BWD_TRY(pack((const bf16_t *)w.w_qc, (int64_t)nH * dh, dcq, nH * dh, b.w6, k6, 0, s));
  BWD_TRY(pack((const bf16_t *)w.w_qr, (int64_t)nH * dr, dcq, nH * dr, b.w6, k6, nH * dh, s));
  BWD_TRY(pack((const bf16_t *)w.w_gate, (int64_t)nS * dh, dcq, nS * dh, b.w6, k6, nH * dh + nH * dr, s));
  BWD_TRY(pack((const bf16_t *)w.w_qa, dcq, dm, dcq, b.w8, k8, 0, s));
  BWD_TRY(pack((const bf16_t *)w.w_dkv, dc, dm, dc, b.w8, k8, dcq, s));
  BWD_TRY(pack((const bf16_t *)w.w_kr, dr, dm, dr, b.w8, k8, dcq + dc, s));
  BWD_TRY(pack((const bf16_t *)w.w_lambda, nS, dm, nS, b.w8, k8, dcq + dc + dr, s));
  const int k8_used = dcq + dc + dr + nS;
  if (k8 > k8_used) {
    hipLaunchKernelGGL(zero_cols_kernel, dim3(grid_for((int64_t)dm * (k8 - k8_used))), dim3(256), 0, s, b.w8,
                       (int64_t)k8, dm, k8_used, k8);
    BWD_TRY(hipGetLastError());
    hipLaunchKernelGGL(zero_cols_kernel, dim3(grid_for((int64_t)M * (k8 - k8_used))), dim3(256), 0, s, b.a8,
                       (int64_t)k8, M, k8_used, k8);
    BWD_TRY(hipGetLastError());
  }

  // ---- gradient scale s from the largest |dout| (see grad_scale_kernel); dout enters as s dout
  const float *gsc = b.gscale + kGradScaleBlocks;
  hipLaunchKernelGGL(absmax_part_kernel, dim3(kGradScaleBlocks), dim3(256), 0, s, (const bf16_t *)a.dout,
                     (int64_t)M * dm, b.gscale);
  BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(grad_scale_kernel, dim3(1), dim3(256), 0, s, b.gscale, kGradScaleBlocks, b.gscale + kGradScaleBlocks);
  BWD_TRY(hipGetLastError());

  // ---- Eq.(10): dY = dout W_O^T; dW_O = Y^T dout
  BWD_TRY(pack((const bf16_t *)a.dout, dm, M, dm, b.dout16, dm, 0, s, gsc));
  BWD_TRY(nt(b.dout16, dm, b.wo16, dm, b.dy, ny, M, ny, dm, s, b.splitk));
  BWD_TRY(tpack(a.y16, ny, M, ny, Mp, b.ta, Mp, 0, s));
  BWD_TRY(tpack((const bf16_t *)a.dout, dm, M, dm, Mp, b.tb, Mp, 0, s, gsc));
  BWD_TRY(nt(b.ta, Mp, b.tb, Mp, G.dw_o, dm, ny, dm, Mp, s, b.splitk));
  // gate and differential combine: dG, dH (fp16), noise-head dH, dlambda and the row sums, per row
  hipLaunchKernelGGL(combine_row_kernel, dim3(M), dim3(256), 0, s, a.heads, a.lam, a.sg16, b.dy, b.dh16, b.a6,
                     (int64_t)k6, nH * dh + nH * dr, b.drow, b.dlaml, a.lam_overridden ? 1 : 0, M, d);
  BWD_TRY(hipGetLastError());
  hipLaunchKernelGGL(qlo_kernel, dim3(grid_for(M)), dim3(256), 0, s, a.doc, b.lo, M, T_, d.window);
  BWD_TRY(hipGetLastError());

  // ---- the softmax maps
  BwdAttnArgs at{};
  at.q = a.q16; at.k = a.kx; at.v = a.vk; at.dh = b.dh16; at.lse = a.lse; at.drow = b.drow; at.lo = b.lo;
  at.doc = a.doc;
  at.dq = b.dq; at.dk = b.dk; at.dv = b.dv;
  at.B = a.B; at.T = T_; at.lcap = a.lcap; at.n_heads = nH; at.n_signal = nS; at.n_noise = d.n_noise;
  at.n_kv = nKV; at.window = d.window; at.c = d.scale * 1.4426950408889634f; at.tau = d.scale;
  hipLaunchKernelGGL(rope_table_kernel, dim3((T_ * (dr / 2) + 255) / 256), dim3(256), 0, s, b.rope_cs, T_, dr,
                     d.theta);
  BWD_TRY(hipGetLastError());
  // dim-major copies of q and dH for the dK/dV kernel, per sequence, tokens padded to Tp with zeros
  at.Tp = (T_ + 31) / 32 * 32;
  at.qT = b.qT; at.dhT = b.dhT;
  for (int sq = 0; sq < a.B; ++sq) {
    BWD_TRY(tpack(a.q16 + (int64_t)sq * T_ * nH * (dh + dr), (int64_t)nH * (dh + dr), T_, nH * (dh + dr), at.Tp,
                  b.qT + (int64_t)sq * at.Tp, (int64_t)a.B * at.Tp, 0, s));
    BWD_TRY(tpack((const f16_t *)(b.dh16 + (int64_t)sq * T_ * nH * dh), (int64_t)nH * dh, T_, nH * dh, at.Tp,
                  b.dhT + (int64_t)sq * at.Tp, (int64_t)a.B * at.Tp, 0, s));
  }
  // dq leaves the attention kernel already packed into a6 (dq^C, and dq^R rotated back)
  at.dq = nullptr;
  at.a6 = b.a6; at.lda6 = k6; at.q_off = nH * dh; at.rope_cs = (const float2 *)b.rope_cs;
  BWD_TRY(launch_bwd_attention(at, s));
  hipLaunchKernelGGL(pack_dkv_kernel, dim3(grid_for((int64_t)M * nKV * dh + (int64_t)M * dr / 2)), dim3(256), 0, s,
                     b.dk, b.dv, b.a3, b.dkr, M, T_, d, (const float2 *)b.rope_cs);
  BWD_TRY(hipGetLastError());

  // ---- Eq.(5), (4): dcbar = [dK^C | dV] [W_uk | W_uv]^T; dW_uk, dW_uv = cbar^T [dK^C | dV]
  BWD_TRY(nt(b.a3, k3, b.w3, k3, b.dcbar, dc, M, dc, k3, s, b.splitk));
  BWD_TRY(tpack(a.cache, (int64_t)dc + dr, M, dc, Mp, b.ta, Mp, 0, s));
  BWD_TRY(tpack(b.a3, k3, M, k3, Mp, b.tb, Mp, 0, s));
  BWD_TRY(nt(b.ta, Mp, b.tb, Mp, G.dw_uk, (int64_t)nKV * dh, dc, nKV * dh, Mp, s, b.splitk));
  BWD_TRY(nt(b.ta, Mp, b.tb + (int64_t)nKV * dh * Mp, Mp, G.dw_uv, (int64_t)nKV * dh, dc, nKV * dh, Mp, s, b.splitk));
  hipLaunchKernelGGL((rms_bwd_kernel<bf16_t>), dim3(M), dim3(64), 0, s, a.ckv, (const bf16_t *)w.gamma_kv, b.dcbar,
                     b.dckv, b.rkv, dc, d.eps);
  BWD_TRY(hipGetLastError());
  if (G.dgamma_kv) {
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((dc + 255) / 256), dim3(256), 0, s, a.ckv, b.rkv, b.dcbar, G.dgamma_kv,
                       M, dc);
    BWD_TRY(hipGetLastError());
  }

  // ---- Eq.(2), (9), (1): dc^Q = [dq^C | dq^R | dG] [W_qc | W_qr | W_gate]^T; their weight grads
  BWD_TRY(nt(b.a6, k6, b.w6, k6, b.dcq, dcq, M, dcq, k6, s, b.splitk));
  BWD_TRY(tpack(a.cq16, dcq, M, dcq, Mp, b.ta, Mp, 0, s));
  BWD_TRY(tpack(b.a6, k6, M, k6, Mp, b.tb, Mp, 0, s));
  BWD_TRY(nt(b.ta, Mp, b.tb, Mp, G.dw_qc, (int64_t)nH * dh, dcq, nH * dh, Mp, s, b.splitk));
  BWD_TRY(nt(b.ta, Mp, b.tb + (int64_t)nH * dh * Mp, Mp, G.dw_qr, (int64_t)nH * dr, dcq, nH * dr, Mp, s, b.splitk));
  BWD_TRY(nt(b.ta, Mp, b.tb + (int64_t)(nH * dh + nH * dr) * Mp, Mp, G.dw_gate, (int64_t)nS * dh, dcq, nS * dh, Mp, s, b.splitk));
  hipLaunchKernelGGL((rms_bwd_kernel<bf16_t>), dim3(M), dim3(64), 0, s, a.aq, (const bf16_t *)w.gamma_q, b.dcq, b.daq,
                     b.rq, dcq, d.eps);
  BWD_TRY(hipGetLastError());
  if (G.dgamma_q) {
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3((dcq + 255) / 256), dim3(256), 0, s, a.aq, b.rq, b.dcq, G.dgamma_q, M,
                       dcq);
    BWD_TRY(hipGetLastError());
  }

  // ---- x: dx = [da^Q | dc^KV | dk^R | dlambda] [W_qa | W_dkv | W_kr | W_lambda]^T; x-side weights
  BWD_TRY(pack(b.daq, dcq, M, dcq, b.a8, k8, 0, s));
  BWD_TRY(pack(b.dckv, dc, M, dc, b.a8, k8, dcq, s));
  BWD_TRY(pack(b.dkr, dr, M, dr, b.a8, k8, dcq + dc, s));
  BWD_TRY(pack(b.dlaml, nS, M, nS, b.a8, k8, dcq + dc + dr, s));
  BWD_TRY(nt(b.a8, k8, b.w8, k8, G.dx, dm, M, dm, k8, s, b.splitk));
  BWD_TRY(tpack((const bf16_t *)a.x, dm, M, dm, Mp, b.ta, Mp, 0, s));
  BWD_TRY(tpack(b.a8, k8, M, k8, Mp, b.tb, Mp, 0, s));
  BWD_TRY(nt(b.ta, Mp, b.tb, Mp, G.dw_qa, dcq, dm, dcq, Mp, s, b.splitk));
  BWD_TRY(nt(b.ta, Mp, b.tb + (int64_t)dcq * Mp, Mp, G.dw_dkv, dc, dm, dc, Mp, s, b.splitk));
  BWD_TRY(nt(b.ta, Mp, b.tb + (int64_t)(dcq + dc) * Mp, Mp, G.dw_kr, dr, dm, dr, Mp, s, b.splitk));
  if (nS % 8 == 0) {
    BWD_TRY(nt(b.ta, Mp, b.tb + (int64_t)(dcq + dc + dr) * Mp, Mp, G.dw_lambda, nS, dm, nS, Mp, s, b.splitk));
  } else {  // too few columns for the MFMA GEMM's 16-byte stores
    BWD_TRY(gg((const bf16_t *)a.x, dm, true, b.dlaml, nS, false, G.dw_lambda, nS, dm, nS, M, false, s));
  }

  // ---- every gradient back to dout's scale
  GradList gl{};
  int ng = 0;
  int64_t most = 0;
  auto add = [&](float *p, int64_t n) {
    if (!p || n <= 0) return;
    gl.p[ng] = p;
    gl.n[ng++] = n;
    most = std::max(most, n);
  };
  add(G.dx, (int64_t)M * dm);
  add(G.dw_qa, (int64_t)dm * dcq);
  add(G.dw_qc, (int64_t)dcq * nH * dh);
  add(G.dw_qr, (int64_t)dcq * nH * dr);
  add(G.dw_dkv, (int64_t)dm * dc);
  add(G.dw_kr, (int64_t)dm * dr);
  add(G.dw_uk, (int64_t)dc * nKV * dh);
  add(G.dw_uv, (int64_t)dc * nKV * dh);
  add(G.dw_lambda, (int64_t)dm * nS);
  add(G.dw_gate, (int64_t)dcq * ny);
  add(G.dw_o, (int64_t)ny * dm);
  add(G.dgamma_q, dcq);
  add(G.dgamma_kv, dc);
  hipLaunchKernelGGL(unscale_grads_kernel, dim3((unsigned)std::min<int64_t>((most + 255) / 256, 1024), ng), dim3(256),
                     0, s, gl, gsc);
  BWD_TRY(hipGetLastError());
  return hipSuccess;
}

}  // namespace gdla
