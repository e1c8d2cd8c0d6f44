// Generic GDLA kernels: any layer sizes, fp32 or bf16 storage, fp32 arithmetic.
//
// They serve the fp32 configuration and any bf16 sizes the MFMA kernels do not cover.  The
// equations are those of the Motif 3 Technical Report (picx.dev summary, section 2.2,
// Eq.(1)-(10)); the readings (head order, KV map, RoPE convention, window edge) are listed in
// include/gdla.h.
#include "gdla_internal.h"

#include <math.h>

#include <algorithm>

namespace gdla {

template <typename T> __device__ __forceinline__ float ld(const T *p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t *p, int64_t i) {
  return (float)p[i];
}
template <typename T> __device__ __forceinline__ void st(T *p, int64_t i, float v);
template <> __device__ __forceinline__ void st<float>(float *p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t *p, int64_t i, float v) {
  p[i] = (bf16_t)v;
}
// fp16 stores round to nearest even: a value beyond fp16's range becomes +-inf and a NaN stays a
// NaN, so an out-of-range or corrupted input surfaces as a non-finite output.
template <> __device__ __forceinline__ void st<f16_t>(f16_t *p, int64_t i, float v) {
  p[i] = (f16_t)(v);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide sum for blockDim.x == 256.
__device__ __forceinline__ float block_sum256(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// ------------------------------------------------------------------------------------------
// Grouped GEMM, 64x64 output tile, 16-deep K slices staged in LDS, 4x4 outputs per thread.
template <typename TI>
__global__ void __launch_bounds__(256) gemm_generic_kernel(GemmBatch batch) {
  __shared__ float As[16][64 + 1];
  __shared__ float Bs[16][64 + 1];
  int bid = blockIdx.x, pi = 0;
  while (pi + 1 < batch.n && bid >= batch.p[pi + 1].tile0) ++pi;
  const GemmProblem &P = batch.p[pi];
  const int tile = bid - P.tile0;
  const int m0 = (tile / P.tiles_n) * 64, n0 = (tile % P.tiles_n) * 64;
  const TI *A = (const TI *)P.A;
  const TI *B = (const TI *)P.B;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < P.K; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      int r = i >> 4, c = i & 15;  // A tile: row r, k c
      int gm = m0 + r, gk = k0 + c;
      As[c][r] = (gm < P.M && gk < P.K) ? ld<TI>(A, (int64_t)gm * P.lda + gk) : 0.f;
      int kr = i >> 6, nc = i & 63;  // B tile: k kr, col nc
      int bk = k0 + kr, bn = n0 + nc;
      Bs[kr][nc] = (bk < P.K && bn < P.N) ? ld<TI>(B, (int64_t)bk * P.ldb + bn) : 0.f;
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
    if (m >= P.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= P.N) continue;
      float v = acc[i][j];
      if (P.epi == EPI_SIGMOID) v = sigmoidf_(v);
      const int64_t off = (int64_t)m * P.ldc + (int64_t)(n / P.hw) * P.hs + P.ho + (n % P.hw);
      if (P.c_dt == CD_F32) ((float *)P.C)[off] = v;
      else st<TI>((TI *)P.C, off, v);
    }
  }
}

static void plan_tiles(GemmBatch &b, int tm, int tn) {
  int t = 0;
  for (int i = 0; i < b.n; ++i) {
    GemmProblem &p = b.p[i];
    p.tile0 = t;
    p.tiles_n = (p.N + tn - 1) / tn;
    t += ((p.M + tm - 1) / tm) * p.tiles_n;
  }
  b.total_tiles = t;
}

hipError_t launch_gemm_generic(GemmBatch &batch, DT in_dt, hipStream_t s) {
  plan_tiles(batch, 64, 64);
  if (batch.total_tiles == 0) return hipSuccess;
  if (in_dt == DT::F32)
    hipLaunchKernelGGL(gemm_generic_kernel<float>, dim3(batch.total_tiles), dim3(256), 0, s, batch);
  else
    hipLaunchKernelGGL(gemm_generic_kernel<bf16_t>, dim3(batch.total_tiles), dim3(256), 0, s, batch);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------

template <typename T>
__global__ void __launch_bounds__(256) prep_kernel(PrepArgs a, LayerDims d) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int b = m / a.T, t = m % a.T;
  const int p = a.pos[b] + t;
  const T *gq = (const T *)a.gamma_q;
  const T *gkv = (const T *)a.gamma_kv;
  if (a.cq) {
    const float *row = a.aq + (int64_t)m * d.d_cq;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d.d_cq; j += 256) ss += row[j] * row[j];
    const float r = rsqrtf(block_sum256(ss, red) / d.d_cq + d.eps);
    for (int j = threadIdx.x; j < d.d_cq; j += 256) {
      const float v = row[j] * r * (gq ? ld<T>(gq, j) : 1.f);
      if (a.cq_f16) {
        st<f16_t>((f16_t *)a.cq, (int64_t)m * d.d_cq + j, v);
      } else {
        st<T>((T *)a.cq, (int64_t)m * d.d_cq + j, v);
        if (a.cq_lo) st<bf16_t>((bf16_t *)a.cq_lo, (int64_t)m * d.d_cq + j, v - (float)(bf16_t)v);
      }
    }
  }
  T *crow = (T *)a.cache.base + cache_row(a.cache, b, p) * (d.d_c + d.d_r);
  {
    const float *row = a.ckv + (int64_t)m * d.d_c;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d.d_c; j += 256) ss += row[j] * row[j];
    const float r = rsqrtf(block_sum256(ss, red) / d.d_c + d.eps);
    for (int j = threadIdx.x; j < d.d_c; j += 256)
      st<T>(crow, j, row[j] * r * (gkv ? ld<T>(gkv, j) : 1.f));
  }
  const int half = d.d_r / 2;
  for (int j = threadIdx.x; j < half; j += 256) {
    float c, s;
    rope_cs(p, j, d.d_r, d.theta, c, s);
    const float u = a.kr[(int64_t)m * d.d_r + j], v = a.kr[(int64_t)m * d.d_r + j + half];
    st<T>(crow, d.d_c + j, u * c - v * s);
    st<T>(crow, d.d_c + j + half, u * s + v * c);
  }
  if (a.lam) {
    for (int i = threadIdx.x; i < d.n_signal; i += 256) {
      const int64_t o = (int64_t)m * d.n_signal + i;
      a.lam[o] = a.lam_override ? a.lam_override[o] : sigmoidf_(a.lam_logit[o]);
    }
  }
}

// The same step for bf16 layers of the MFMA paths' sizes (d_cq 1024, d_c 512, d_r 64): one wave per
// token row, 16-byte loads of the fp32 projections and 8-byte stores, wave reductions only (no
// block barrier).  Lane l holds elements 4 l + 256 i .. + 3 of each row.
template <int N>
__device__ __forceinline__ void rms_row(const float *row, const bf16_t *g, float eps, int lane, float (&v)[N / 64]) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < N / 256; ++i) {
    const float4 x = *(const float4 *)(row + 4 * lane + 256 * i);
    v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
    ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
  const float r = rsqrtf(wave_sum(ss) / N + eps);
#pragma unroll
  for (int i = 0; i < N / 256; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * i + e] = v[4 * i + e] * r * (g ? (float)g[4 * lane + 256 * i + e] : 1.f);
}

__global__ void __launch_bounds__(256) prep_rows_kernel(PrepArgs a, LayerDims d) {
  constexpr int DCQ = 1024, DCK = 512, DR = 64;
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.M) return;
  const int b = m / a.T, t = m % a.T;
  const int p = a.pos[b] + t;
  if (a.cq) {
    float v[DCQ / 64];
    rms_row<DCQ>(a.aq + (int64_t)m * DCQ, (const bf16_t *)a.gamma_q, d.eps, lane, v);
#pragma unroll
    for (int i = 0; i < DCQ / 256; ++i) {
      const int64_t o = (int64_t)m * DCQ + 4 * lane + 256 * i;
      if (a.cq_f16) {
        f16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (f16_t)v[4 * i + e];
        *(uint2 *)((f16_t *)a.cq + o) = *(const uint2 *)h;
      } else {
        bf16_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = (bf16_t)v[4 * i + e];
          l[e] = (bf16_t)(v[4 * i + e] - (float)h[e]);
        }
        *(uint2 *)((bf16_t *)a.cq + o) = *(const uint2 *)h;
        if (a.cq_lo) *(uint2 *)((bf16_t *)a.cq_lo + o) = *(const uint2 *)l;
      }
    }
  }
  bf16_t *crow = (bf16_t *)a.cache.base + cache_row(a.cache, b, p) * (DCK + DR);
  {
    float v[DCK / 64];
    rms_row<DCK>(a.ckv + (int64_t)m * DCK, (const bf16_t *)a.gamma_kv, d.eps, lane, v);
#pragma unroll
    for (int i = 0; i < DCK / 256; ++i) {
      bf16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (bf16_t)v[4 * i + e];
      *(uint2 *)(crow + 4 * lane + 256 * i) = *(const uint2 *)h;
    }
  }
  if (lane < DR / 2) {
    float c, s;
    rope_cs(p, lane, DR, d.theta, c, s);
    const float u = a.kr[(int64_t)m * DR + lane], v = a.kr[(int64_t)m * DR + lane + DR / 2];
    crow[DCK + lane] = (bf16_t)(u * c - v * s);
    crow[DCK + lane + DR / 2] = (bf16_t)(u * s + v * c);
  }
  if (a.lam) {
    for (int i = lane; i < d.n_signal; i += 64) {
      const int64_t o = (int64_t)m * d.n_signal + i;
      a.lam[o] = a.lam_override ? a.lam_override[o] : sigmoidf_(a.lam_logit[o]);
    }
  }
}

hipError_t launch_prep(const PrepArgs &a, const LayerDims &d, DT dt, hipStream_t s) {
  if (a.M == 0) return hipSuccess;
  // every row of the cache holds d_c + d_r = 576 bf16 (1152 B, 8-byte aligned rows)
  const bool rows = dt == DT::BF16 && d.d_cq == 1024 && d.d_c == 512 && d.d_r == 64 &&
                    ((uintptr_t)a.aq & 15) == 0 && ((uintptr_t)a.ckv & 15) == 0 && ((uintptr_t)a.cache.base & 7) == 0 &&
                    (!a.cq || ((uintptr_t)a.cq & 7) == 0) && (!a.cq_lo || ((uintptr_t)a.cq_lo & 7) == 0);
  if (rows) {
    hipLaunchKernelGGL(prep_rows_kernel, dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, s, a, d);
    return hipGetLastError();
  }
  if (dt == DT::F32) hipLaunchKernelGGL(prep_kernel<float>, dim3(a.M), dim3(256), 0, s, a, d);
  else hipLaunchKernelGGL(prep_kernel<bf16_t>, dim3(a.M), dim3(256), 0, s, a, d);
  return hipGetLastError();
}

template <typename T>
__global__ void __launch_bounds__(256) rope_heads_kernel(const float *src, T *dst, int64_t dst_ld,
                                                         int32_t dst_hs, int32_t dst_off, int32_t T_, int32_t n_heads,
                                                         int32_t d_r, const int32_t *pos,
                                                         float theta) {
  __shared__ float cs[2][128];  // d_r <= 256
  const int m = blockIdx.x;
  const int p = pos[m / T_] + m % T_;
  const int half = d_r / 2;
  for (int j = threadIdx.x; j < half; j += 256) rope_cs(p, j, d_r, theta, cs[0][j], cs[1][j]);
  __syncthreads();
  for (int i = threadIdx.x; i < n_heads * half; i += 256) {
    const int h = i / half, j = i % half;
    const float c = cs[0][j], s = cs[1][j];
    const float *r = src + ((int64_t)m * n_heads + h) * d_r;
    const float u = r[j], v = r[j + half];
    T *o = dst + (int64_t)m * dst_ld + (int64_t)h * dst_hs + dst_off;
    st<T>(o, j, u * c - v * s);
    st<T>(o, j + half, u * s + v * c);
  }
}

hipError_t launch_rope_heads(const float *src, void *dst, int64_t dst_ld, int32_t dst_hs,
                             int32_t dst_off, int32_t M, int32_t T, int32_t n_heads, int32_t d_r,
                             const int32_t *pos, float theta, DT dt, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (dt == DT::F32)
    hipLaunchKernelGGL(rope_heads_kernel<float>, dim3(M), dim3(256), 0, s, src, (float *)dst,
                       dst_ld, dst_hs, dst_off, T, n_heads, d_r, pos, theta);
  else if (dt == DT::F16)
    hipLaunchKernelGGL(rope_heads_kernel<f16_t>, dim3(M), dim3(256), 0, s, src, (f16_t *)dst,
                       dst_ld, dst_hs, dst_off, T, n_heads, d_r, pos, theta);
  else
    hipLaunchKernelGGL(rope_heads_kernel<bf16_t>, dim3(M), dim3(256), 0, s, src, (bf16_t *)dst,
                       dst_ld, dst_hs, dst_off, T, n_heads, d_r, pos, theta);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Expanded-form attention: one wave per (query row, head), online softmax over the visible keys.
constexpr int kMaxHeadChunks = 4;  // d_head <= 256

template <typename T>
__global__ void __launch_bounds__(256) attention_generic_kernel(AttnGenericArgs a, LayerDims d) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.M * d.n_heads) return;
  const int m = (int)(wid / d.n_heads), h = (int)(wid % d.n_heads);
  const int b = m / a.T, t = m % a.T;
  const int p = a.pos[b] + t;
  const int base = d.window > 0 ? max(0, a.pos[b] - d.window + 1) : 0;
  int lo = d.window > 0 ? max(0, p - d.window + 1) : 0;
  if (a.doc) lo = max(lo, min(max(a.doc[m], 0), p));  // packed documents: keys from the token's document
  const int kv = kv_head_of(h, d.n_signal, d.n_kv);
  const T *qc = (const T *)a.qc + ((int64_t)m * d.n_heads + h) * d.d_h;
  const T *qr = (const T *)a.qr + ((int64_t)m * d.n_heads + h) * d.d_r;
  const T *kx = (const T *)a.kx + ((int64_t)b * d.n_kv + kv) * a.lcap * d.d_h;
  const T *vx = (const T *)a.vx + ((int64_t)b * d.n_kv + kv) * a.lcap * d.d_h;
  const T *cache = (const T *)a.cache + (int64_t)b * a.max_len * (d.d_c + d.d_r) + d.d_c;
  float q[kMaxHeadChunks], acc[kMaxHeadChunks];
#pragma unroll
  for (int i = 0; i < kMaxHeadChunks; ++i) {
    const int e = lane + 64 * i;
    q[i] = e < d.d_h ? ld<T>(qc, e) : 0.f;
    acc[i] = 0.f;
  }
  const float qrv = lane < d.d_r ? ld<T>(qr, lane) : 0.f;
  float mx = -INFINITY, l = 0.f;
  for (int s = lo; s <= p; ++s) {
    const int64_t row = (int64_t)(s - base) * d.d_h;
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxHeadChunks; ++i) {
      const int e = lane + 64 * i;
      if (e < d.d_h) dot = fmaf(q[i], ld<T>(kx, row + e), dot);
    }
    if (lane < d.d_r) dot = fmaf(qrv, ld<T>(cache, (int64_t)s * (d.d_c + d.d_r) + lane), dot);
    const float sc = wave_sum(dot) * d.scale;
    const float mn = fmaxf(mx, sc);
    const float corr = __expf(mx - mn), w = __expf(sc - mn);
    l = l * corr + w;
#pragma unroll
    for (int i = 0; i < kMaxHeadChunks; ++i) {
      const int e = lane + 64 * i;
      if (e < d.d_h) acc[i] = acc[i] * corr + w * ld<T>(vx, row + e);
    }
    mx = mn;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < kMaxHeadChunks; ++i) {
    const int e = lane + 64 * i;
    if (e < d.d_h) a.heads[((int64_t)m * d.n_heads + h) * d.d_h + e] = acc[i] * inv;
  }
}

hipError_t launch_attention_generic(const AttnGenericArgs &a, const LayerDims &d, DT dt,
                                    hipStream_t s) {
  const int64_t waves = (int64_t)a.M * d.n_heads;
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (dt == DT::F32) hipLaunchKernelGGL(attention_generic_kernel<float>, grid, dim3(256), 0, s, a, d);
  else hipLaunchKernelGGL(attention_generic_kernel<bf16_t>, grid, dim3(256), 0, s, a, d);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// y_lo (bf16 layers, or null): the bf16 rounding remainder of each Y value, for the two-part
// output projection.
template <typename T>
__global__ void __launch_bounds__(256) combine_kernel(const float *heads, const float *lam,
                                                      const float *gate, T *y, bf16_t *y_lo, int32_t M,
                                                      LayerDims d) {
  const int64_t n = (int64_t)M * d.n_signal * d.d_h;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int e = (int)(idx % d.d_h);
    const int64_t r = idx / d.d_h;
    const int i = (int)(r % d.n_signal);
    const int64_t m = r / d.n_signal;
    const float hs = heads[(m * d.n_heads + i) * d.d_h + e];
    const float hn = heads[(m * d.n_heads + d.n_signal + i % d.n_noise) * d.d_h + e];
    const float dv = hs - lam[m * d.n_signal + i] * hn;
    const float v = sigmoidf_(gate[idx]) * dv;
    st<T>(y, idx, v);
    if (y_lo) y_lo[idx] = (bf16_t)(v - (float)(bf16_t)v);
  }
}

hipError_t launch_combine(const float *heads, const float *lam, const float *gate, void *y,
                          int32_t M, const LayerDims &d, DT dt, hipStream_t s, void *y_lo) {
  const int64_t n = (int64_t)M * d.n_signal * d.d_h;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 65536));
  if (dt == DT::F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, heads, lam, gate, (float *)y, nullptr, M, d);
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, s, heads, lam, gate, (bf16_t *)y,
                       (bf16_t *)y_lo, M, d);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Absorbed decode.
template <typename T>
__global__ void __launch_bounds__(256) absorb_kernel(const float *qc, const float *qr, const T *w_uk,
                                                     float *qabs, int32_t B, LayerDims d) {
  const int row = d.d_c + d.d_r;
  const int64_t n = (int64_t)B * d.n_heads * row;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int c = (int)(idx % row);
    const int64_t bh = idx / row;
    const int h = (int)(bh % d.n_heads);
    float v;
    if (c < d.d_c) {
      const int kv = kv_head_of(h, d.n_signal, d.n_kv);
      const float *q = qc + bh * d.d_h;
      const T *wr = w_uk + (int64_t)c * d.n_kv * d.d_h + kv * d.d_h;
      v = 0.f;
      for (int e = 0; e < d.d_h; ++e) v = fmaf(q[e], ld<T>(wr, e), v);
    } else {
      v = qr[bh * d.d_r + (c - d.d_c)];
    }
    qabs[idx] = v;
  }
}

hipError_t launch_absorb_generic(const float *qc, const float *qr, const void *w_uk, float *qabs,
                                 int32_t B, const LayerDims &d, DT dt, hipStream_t s) {
  const int64_t n = (int64_t)B * d.n_heads * (d.d_c + d.d_r);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 65536));
  if (dt == DT::F32)
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(256), 0, s, qc, qr, (const float *)w_uk, qabs, B, d);
  else
    hipLaunchKernelGGL(absorb_kernel<bf16_t>, grid, dim3(256), 0, s, qc, qr, (const bf16_t *)w_uk, qabs, B, d);
  return hipGetLastError();
}

constexpr int kMaxLatentChunks = 16;  // d_c + d_r <= 1024

template <typename T>
__global__ void __launch_bounds__(256) latent_attention_kernel(const float *qabs, CacheRef cache,
                                                               float *o, const int32_t *pos,
                                                               int32_t B, int32_t q_len, LayerDims d) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b q_len + i) n_H + h
  if (wid >= (int64_t)B * q_len * d.n_heads) return;
  const int v = (int)(wid / d.n_heads), b = v / q_len;
  const int row = d.d_c + d.d_r;
  const int p = pos[b] + v % q_len;
  const int lo = d.window > 0 ? max(0, p - d.window + 1) : 0;
  const float *q = qabs + wid * row;
  const T *c = (const T *)cache.base;
  float qv[kMaxLatentChunks], acc[kMaxLatentChunks];
#pragma unroll
  for (int i = 0; i < kMaxLatentChunks; ++i) {
    const int e = lane + 64 * i;
    qv[i] = e < row ? q[e] : 0.f;
    acc[i] = 0.f;
  }
  float mx = -INFINITY, l = 0.f;
  for (int s = lo; s <= p; ++s) {
    const T *cr = c + cache_row(cache, b, s) * row;
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxLatentChunks; ++i) {
      const int e = lane + 64 * i;
      if (e < row) dot = fmaf(qv[i], ld<T>(cr, e), dot);
    }
    const float sc = wave_sum(dot) * d.scale;
    const float mn = fmaxf(mx, sc);
    const float corr = __expf(mx - mn), w = __expf(sc - mn);
    l = l * corr + w;
#pragma unroll
    for (int i = 0; i < kMaxLatentChunks; ++i) {
      const int e = lane + 64 * i;
      if (e < d.d_c) acc[i] = acc[i] * corr + w * ld<T>(cr, e);
    }
    mx = mn;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int i = 0; i < kMaxLatentChunks; ++i) {
    const int e = lane + 64 * i;
    if (e < d.d_c) o[wid * d.d_c + e] = acc[i] * inv;
  }
}

hipError_t launch_latent_attention_generic(const float *qabs, const CacheRef &cache, float *o,
                                           const int32_t *pos, int32_t B, int32_t q_len,
                                           const LayerDims &d, DT dt, hipStream_t s) {
  const int64_t waves = (int64_t)B * q_len * d.n_heads;
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (dt == DT::F32)
    hipLaunchKernelGGL(latent_attention_kernel<float>, grid, dim3(256), 0, s, qabs, cache, o, pos, B,
                       q_len, d);
  else
    hipLaunchKernelGGL(latent_attention_kernel<bf16_t>, grid, dim3(256), 0, s, qabs, cache, o, pos, B,
                       q_len, d);
  return hipGetLastError();
}

template <typename T>
__global__ void __launch_bounds__(256) unabsorb_kernel(const float *o, const T *w_uv, float *heads,
                                                       int32_t B, LayerDims d) {
  const int64_t n = (int64_t)B * d.n_heads * d.d_h;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int e = (int)(idx % d.d_h);
    const int64_t bh = idx / d.d_h;
    const int h = (int)(bh % d.n_heads);
    const int kv = kv_head_of(h, d.n_signal, d.n_kv);
    const float *orow = o + bh * d.d_c;
    const T *wc = w_uv + kv * d.d_h + e;
    float v = 0.f;
    for (int c = 0; c < d.d_c; ++c) v = fmaf(orow[c], ld<T>(wc, (int64_t)c * d.n_kv * d.d_h), v);
    heads[idx] = v;
  }
}

hipError_t launch_unabsorb_generic(const float *o, const void *w_uv, float *heads, int32_t B,
                                   const LayerDims &d, DT dt, hipStream_t s) {
  const int64_t n = (int64_t)B * d.n_heads * d.d_h;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((n + 255) / 256, 65536));
  if (dt == DT::F32)
    hipLaunchKernelGGL(unabsorb_kernel<float>, grid, dim3(256), 0, s, o, (const float *)w_uv, heads, B, d);
  else
    hipLaunchKernelGGL(unabsorb_kernel<bf16_t>, grid, dim3(256), 0, s, o, (const bf16_t *)w_uv, heads, B, d);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
struct I32Chunk {
  int32_t v[128];
};

__global__ void set_i32_kernel(int32_t *dst, I32Chunk c, int32_t n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = c.v[i];
}

hipError_t launch_set_i32(int32_t *dst, const int32_t *src_host, int32_t n, hipStream_t s) {
  for (int32_t o = 0; o < n; o += 128) {
    I32Chunk c;
    const int32_t k = std::min<int32_t>(128, n - o);
    for (int32_t i = 0; i < k; ++i) c.v[i] = src_host[o + i];
    hipLaunchKernelGGL(set_i32_kernel, dim3(1), dim3(128), 0, s, dst + o, c, k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

__global__ void copy_rows_f32_kernel(const float *src, int64_t src_ld, float *dst, int64_t dst_ld,
                                     int32_t rows, int32_t cols) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols, c = i % cols;
    dst[r * dst_ld + c] = src[r * src_ld + c];
  }
}

hipError_t launch_copy_rows_f32(const float *src, int64_t src_ld, float *dst, int64_t dst_ld,
                                int32_t rows, int32_t cols, hipStream_t s) {
  const int64_t n = (int64_t)rows * cols;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_f32_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 65536)),
                     dim3(256), 0, s, src, src_ld, dst, dst_ld, rows, cols);
  return hipGetLastError();
}

// Rows of every sequence b copied between two caches (either may be paged): scatter = false
// copies the visible keys before the new tokens, [lo(pos_b), pos_b), with lo = pos_b - window + 1
// (at least 0) for a windowed layer and 0 otherwise; scatter = true copies the new rows
// [pos_b, pos_b + T).  Block (x, b) takes 16 rows; U is the copy unit (16, 4 or 2 bytes).
template <typename U>
__global__ void __launch_bounds__(256) copy_cache_rows_kernel(CacheRef src, CacheRef dst, const int32_t *pos,
                                                              int32_t scatter, int32_t T, int32_t window,
                                                              int32_t row_units) {
  const int b = blockIdx.y, p = pos[b];
  const int lo = scatter ? p : (window > 0 ? max(0, p - window + 1) : 0);
  const int hi = scatter ? p + T : p;
  const int r0 = lo + (int)blockIdx.x * 16;
  const int nr = min(16, hi - r0);
  for (int i = threadIdx.x; i < nr * row_units; i += 256) {
    const int r = r0 + i / row_units, u = i % row_units;
    ((U *)dst.base)[cache_row(dst, b, r) * row_units + u] = ((const U *)src.base)[cache_row(src, b, r) * row_units + u];
  }
}

hipError_t launch_copy_cache_rows(const CacheRef &src, const CacheRef &dst, const int32_t *pos_dev, int32_t B,
                                  int32_t max_rows, bool scatter, int32_t T, int32_t window, int64_t row_bytes,
                                  hipStream_t s) {
  if (B == 0 || max_rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((max_rows + 15) / 16), (unsigned)B);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(copy_cache_rows_kernel<uint4>, grid, dim3(256), 0, s, src, dst, pos_dev, scatter ? 1 : 0, T,
                       window, (int32_t)(row_bytes / 16));
  else if (row_bytes % 4 == 0)
    hipLaunchKernelGGL(copy_cache_rows_kernel<uint32_t>, grid, dim3(256), 0, s, src, dst, pos_dev, scatter ? 1 : 0,
                       T, window, (int32_t)(row_bytes / 4));
  else
    hipLaunchKernelGGL(copy_cache_rows_kernel<uint16_t>, grid, dim3(256), 0, s, src, dst, pos_dev, scatter ? 1 : 0,
                       T, window, (int32_t)(row_bytes / 2));
  return hipGetLastError();
}

}  // namespace gdla
