// Fused GDLA prefill attention for gfx950 (d_head 128, d_rope 64): fp16 MFMA operands (queries,
// expanded K^C / V, and the probabilities), k^R converted exactly from the bf16 cache, fp32
// accumulation and fp32 online softmax.
//
// Computes, per query head h and query token t at position p, the softmax attention over the
// expanded keys [K^C ; k^R] and values V of its KV head (Motif 3 Technical Report, picx.dev
// summary section 2.2, Eq.(5) feeding the signal / noise maps of Eq.(8)), then, for the signal
// heads, the grouped differential combine and the sigmoid gate of Eq.(8)-(10):
//     Y_i = sigmoid(G_i) * (H_i - lambda_i * H_{n_S + i mod n_N}).
// Two launches: the noise heads first (they write H_N in fp32), then the signal heads, whose
// epilogue reads H_N, lambda and the gate logits and writes Y in fp16 for the output projection.
//
// Work split: a workgroup is 4 waves; each wave owns 64 query rows of one head.  In the signal
// launch the 4 waves are 4 signal heads sharing one KV head and the same 64 tokens, so each K/V
// tile staged in LDS serves all of them; in the noise launch the waves are 4 consecutive 64-token
// blocks of one noise head.  Keys are processed in tiles of 64 (double-buffered in LDS):
//   S^T[key, query] = K[key, 0:192] . Q[query, 0:192]   (A = K from LDS, B = Q in registers)
//   online softmax per query (each lane owns one query column; its partner lane l^32 the other
//   half of the keys), P^T taken straight from the accumulators in bf16,
//   O^T[dim, query] += V^T[dim, key] . P^T[key, query]  (A = V^T via ds_read_tr16_b64).
// The key order inside each 16-key MFMA step is permuted identically on both operands, which lets
// the S accumulator layout serve as the P operand without any shuffle.
// Causal / sliding-window tiles are classified per wave as skipped, full or partial; only partial
// tiles evaluate the per-element mask s <= p && (W == 0 || p - s < W).
#include "fast_paths.h"

#include <algorithm>

namespace gdla {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int DH = 128, DR = 64, DQK = DH + DR;
constexpr int KT = 64;                 // keys per tile
constexpr int KS = DQK + 8;            // K tile row stride in LDS (elements)
constexpr int VS = DH + 32;            // V tile row stride in LDS (elements)
constexpr int K_STAGE = KT * KS;
constexpr int V_STAGE = KT * VS;

struct AttnArgs {
  const f16_t *q;         // [M, n_H, 192] fp16: q^C then rotated q^R of each head
  const f16_t *kx;        // [B, n_kv, lcap, 128] fp16: K^C of keys base_b .. base_b + lcap - 1
  const f16_t *vx;        // [B, n_kv, lcap, 128] fp16: V
  const bf16_t *cache;    // [B, max_len, row] bf16: k^R at columns d_c .. d_c + 63
  const int32_t *pos;     // [B] first position of the chunk
  const float *lam;       // [M, n_S]
  const float *gate;      // [M, n_S, 128] gate logits
  float *hn;              // [M, n_N, 128] normalised noise-head outputs
  f16_t *y;               // [M, n_S * 128] fp16
  float *out_heads;       // [M, n_H, 128] or null
  int32_t T, max_len, lcap, row, d_c;
  int32_t n_heads, n_signal, n_noise, n_kv, window;
  int32_t sig_per_kv, chunks, n_qblk;
  float c;                // softmax scale * log2(e)
};

__device__ __forceinline__ f16x4 tr_read(const f16_t *p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 bf16 -> 8 fp16: exact in the fp16 normal range, saturating (round toward zero) beyond it.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  auto cv = [](unsigned w) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    return __builtin_bit_cast(unsigned, h);
  };
  return make_uint4(cv(v.x), cv(v.y), cv(v.z), cv(v.w));
}

__device__ __forceinline__ f16_t to_f16(float v) { return (f16_t)fminf(fmaxf(v, -65504.f), 65504.f); }

// (own, partner) exchange between lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool SIGNAL>
__global__ void __launch_bounds__(256, 1) attn_prefill_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) f16_t Ks[2 * K_STAGE];
  __shared__ __attribute__((aligned(16))) f16_t Vs[2 * V_STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.z;
  const int qblk = a.n_qblk - 1 - (int)blockIdx.x;  // late (long) query blocks first
  int head, kvh, t0w, tlo, thi;
  if (SIGNAL) {
    kvh = blockIdx.y / a.chunks;
    const int r = (blockIdx.y % a.chunks) * 4 + wave;
    head = r < a.sig_per_kv ? kvh + a.n_kv * r : -1;
    t0w = qblk * 64;
    tlo = t0w;
    thi = min(t0w + 63, a.T - 1);
  } else {
    head = a.n_signal + blockIdx.y;
    kvh = blockIdx.y % a.n_kv;
    t0w = qblk * 256 + 64 * wave;
    tlo = qblk * 256;
    thi = min(tlo + 255, a.T - 1);
  }
  const bool active = head >= 0 && t0w < a.T;
  const int W = a.window;
  const int p0 = a.pos[b];
  const int base = W > 0 ? max(0, p0 - W + 1) : 0;
  const int klo = W > 0 ? max(0, p0 + tlo - W + 1) : 0;
  const int khi = p0 + thi + 1;
  const int ntiles = (khi - klo + KT - 1) / KT;
  const int wp_lo = p0 + t0w, wp_hi = p0 + min(t0w + 63, a.T - 1);
  const int64_t mrow0 = (int64_t)b * a.T;

  // ---- Q fragments: Qf[qb][ks] holds dims 16 ks + 8 (lane / 32) .. + 7 of query column lane % 32
  f16x8 Qf[2][12];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = t0w + qb * 32 + (lane & 31);
    const bool ok = active && t < a.T;
    const f16_t *qp = a.q + ((mrow0 + (ok ? t : 0)) * a.n_heads + (ok ? head : 0)) * DQK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      Qf[qb][ks] = ok ? *(const f16x8 *)(qp + 16 * ks) : f16x8{};
    }
  }

  // ---- global -> register staging of one key tile (K^C, k^R, V)
  const f16_t *kxh = a.kx + ((int64_t)b * a.n_kv + kvh) * a.lcap * DH;
  const f16_t *vxh = a.vx + ((int64_t)b * a.n_kv + kvh) * a.lcap * DH;
  const bf16_t *crow = a.cache + (int64_t)b * a.max_len * a.row + a.d_c;
  uint4 rk[4], rr[2], rv[4];
  auto stage = [&](int s0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int s = s0 + (c >> 4), cc = (c & 15) * 8;
      const bool ok = s < khi;
      const int64_t off = (int64_t)(ok ? s - base : 0) * DH + cc;
      rk[i] = ok ? *(const uint4 *)(kxh + off) : make_uint4(0, 0, 0, 0);
      rv[i] = ok ? *(const uint4 *)(vxh + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      const int s = s0 + (c >> 3), cc = (c & 7) * 8;
      rr[i] = s < khi ? bf16x8_to_f16x8(*(const uint4 *)(crow + (int64_t)s * a.row + cc)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
    f16_t *ks = Ks + buf * K_STAGE;
    f16_t *vs = Vs + buf * V_STAGE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *(uint4 *)(ks + (c >> 4) * KS + (c & 15) * 8) = rk[i];
      *(uint4 *)(vs + (c >> 4) * VS + (c & 15) * 8) = rv[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i;
      *(uint4 *)(ks + (c >> 3) * KS + DH + (c & 7) * 8) = rr[i];
    }
  };

  f32x16 O[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db) O[qb][db] = f32x16{};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  // transpose-read coordinates (this lane as a source of ds_read_tr16_b64)
  const int G = lane >> 4, jj = (lane & 15) >> 2, qq = lane & 3;
  const int v_key = 4 * (G >> 1) + jj, v_dim = 16 * (G & 1) + 4 * qq;
  const int hgrp = lane >> 5;  // which half of each 8-key group this lane's accumulators hold

  if (ntiles > 0) {
    stage(klo);
    store(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int s0 = klo + it * KT;
    if (it + 1 < ntiles) stage(s0 + KT);
    const bool skip = !active || s0 > wp_hi || (W > 0 && wp_lo - (s0 + KT - 1) >= W);
    if (!skip) {
      const bool full = (s0 + KT - 1 <= wp_lo) && (W == 0 || wp_hi - s0 < W);
      const f16_t *ks = Ks + buf * K_STAGE;
      const f16_t *vs = Vs + buf * V_STAGE;
      f32x16 S[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) S[kb][qb] = f32x16{};
#pragma unroll
      for (int kst = 0; kst < 12; ++kst) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const f16x8 kf = *(const f16x8 *)(ks + (kb * 32 + (lane & 31)) * KS + 16 * kst + 8 * hgrp);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            S[kb][qb] = mfma(kf, Qf[qb][kst], S[kb][qb]);
        }
      }
      f16x8 P[2][2][2];  // [kb][qb][half of the 32-key block]
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // v[16 kb + e] is the score of key s0 + 32 kb + 8 (e / 4) + 4 hgrp + e % 4
        float v[32];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) v[kb * 16 + e] = S[kb][qb][e];
        if (!full) {
          // branch-free mask: visible iff 0 <= p - s < W (W = 0: no upper bound)
          const int d0 = wp_lo + qb * 32 + (lane & 31) - s0 - 4 * hgrp;
          const unsigned wlim = W > 0 ? (unsigned)W : 0x7fffffffu;  // negative p - s wraps above it
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const int off = (i >> 4) * 32 + 8 * ((i & 15) >> 2) + (i & 3);
            v[i] = (unsigned)(d0 - off) < wlim ? v[i] : -INFINITY;
          }
        }
        float mt = v[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mt = fmaxf(mt, v[i]);
        mt = pair_max(mt);
        const float mnew = fmaxf(m[qb], mt);
        const float ms = mnew == -INFINITY ? 0.f : mnew * a.c;
        const float alpha = __builtin_amdgcn_exp2f(m[qb] * a.c - ms);
        m[qb] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          v[i] = __builtin_amdgcn_exp2f(v[i] * a.c - ms);
          rs += v[i];
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int e = 0; e < 8; ++e) P[kb][qb][h2][e] = (f16_t)v[kb * 16 + 8 * h2 + e];
        l[qb] = l[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < 4; ++db) O[qb][db] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int kst = 0; kst < 4; ++kst) {
          const f16_t *vp = vs + (16 * kst + v_key) * VS + db * 32 + v_dim;
          const f16x4 lo = tr_read(vp);
          const f16x4 hi = tr_read(vp + 8 * VS);
          const f16x8 vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            O[qb][db] = mfma(vf, P[kst >> 1][qb][kst & 1], O[qb][db]);
        }
      }
    }
    if (it + 1 < ntiles) store(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  // ---- epilogue: lane holds query column lane % 32 and dims db*32 + 8 i + 4 (lane / 32) + j
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float inv = 1.0f / pair_sum(l[qb]);
    const int t = t0w + qb * 32 + (lane & 31);
    if (t >= a.T) continue;
    const int64_t mr = mrow0 + t;
    float *oh = a.out_heads ? a.out_heads + (mr * a.n_heads + head) * DH : nullptr;
    if (!SIGNAL) {
      float *hn = a.hn + (mr * a.n_noise + (head - a.n_signal)) * DH;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dim = db * 32 + 8 * i + 4 * hgrp;
          const float4 v = make_float4(O[qb][db][4 * i] * inv, O[qb][db][4 * i + 1] * inv,
                                       O[qb][db][4 * i + 2] * inv, O[qb][db][4 * i + 3] * inv);
          *(float4 *)(hn + dim) = v;
          if (oh) *(float4 *)(oh + dim) = v;
        }
    } else {
      const float lam = a.lam[mr * a.n_signal + head];
      const float *g = a.gate + (mr * a.n_signal + head) * DH;
      const float *hn = a.hn + (mr * a.n_noise + head % a.n_noise) * DH;
      f16_t *y = a.y + mr * (int64_t)a.n_signal * DH + (int64_t)head * DH;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dim = db * 32 + 8 * i + 4 * hgrp;
          const float4 gv = *(const float4 *)(g + dim);
          const float4 nv = *(const float4 *)(hn + dim);
          const float o0 = O[qb][db][4 * i] * inv, o1 = O[qb][db][4 * i + 1] * inv;
          const float o2 = O[qb][db][4 * i + 2] * inv, o3 = O[qb][db][4 * i + 3] * inv;
          if (oh) *(float4 *)(oh + dim) = make_float4(o0, o1, o2, o3);
          f16x4 yv;
          yv[0] = to_f16((o0 - lam * nv.x) / (1.0f + __expf(-gv.x)));
          yv[1] = to_f16((o1 - lam * nv.y) / (1.0f + __expf(-gv.y)));
          yv[2] = to_f16((o2 - lam * nv.z) / (1.0f + __expf(-gv.z)));
          yv[3] = to_f16((o3 - lam * nv.w) / (1.0f + __expf(-gv.w)));
          *(f16x4 *)(y + dim) = yv;
        }
    }
  }
}

}  // namespace

bool fast_prefill_supported(const LayerDims &d, gdla_dtype dt) {
  return dt == GDLA_BF16 && d.d_h == DH && d.d_r == DR && d.d_c % 8 == 0 && d.d_cq % 64 == 0 &&
         d.d_model % 64 == 0 && (d.n_signal * DH) % 64 == 0;
}

gdla_status run_fast_prefill(const LayerDims &d, const gdla_weights *w, int32_t B, int32_t T,
                             const int32_t *pos_dev, const int32_t *pos_host, void *cache,
                             int32_t max_len, void *cq, float *lam, float *gate, void *kx,
                             void *vx, int32_t lcap, void *y, float *out_heads,
                             const FastPrefillLayout &L, void *ws, hipStream_t s, StageEvents &se) {
  (void)pos_host;
  const int32_t M = B * T;
  f16_t *q = (f16_t *)((char *)ws + L.q);
  float *qrp = (float *)((char *)ws + L.qrp);
  float *hn = (float *)((char *)ws + L.hn);
  // Eq.(2), (9): q^C straight into the per-head [q^C ; q^R] rows, q^R before RoPE, gate logits.
  GemmBatch g{};
  se.begin(GDLA_STAGE_PROJ_Q);
  // c^Q is fp16 here; the bf16 weights are converted to fp16 while the GEMM stages them.
  auto add = [&](const void *B_, int N, void *C, int64_t ldc, int c_dt, int hw, int64_t hs) {
    GemmProblem p{};
    p.A = cq; p.lda = d.d_cq; p.B = B_; p.ldb = N; p.C = C; p.ldc = ldc;
    p.M = M; p.N = N; p.K = d.d_cq; p.hw = hw; p.hs = hs; p.ho = 0; p.c_dt = c_dt; p.a_f16 = 1;
    p.epi = EPI_NONE;
    g.p[g.n++] = p;
  };
  add(w->w_qc, d.n_heads * DH, q, (int64_t)d.n_heads * DQK, CD_F16, DH, DQK);
  add(w->w_qr, d.n_heads * DR, qrp, (int64_t)d.n_heads * DR, CD_F32, d.n_heads * DR, 0);
  add(w->w_gate, d.n_signal * DH, gate, (int64_t)d.n_signal * DH, CD_F32, d.n_signal * DH, 0);
  if (launch_gemm(g, DT::BF16, s) != hipSuccess) return GDLA_ERR_HIP;
  if (launch_rope_heads(qrp, q, (int64_t)d.n_heads * DQK, DQK, DH, M, T, d.n_heads, DR, pos_dev,
                        d.theta, DT::F16, s) != hipSuccess)
    return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_PROJ_Q);

  AttnArgs a{};
  a.q = q; a.kx = (const f16_t *)kx; a.vx = (const f16_t *)vx; a.cache = (const bf16_t *)cache;
  a.pos = pos_dev; a.lam = lam; a.gate = gate; a.hn = hn; a.y = (f16_t *)y; a.out_heads = out_heads;
  a.T = T; a.max_len = max_len; a.lcap = lcap; a.row = d.d_c + d.d_r; a.d_c = d.d_c;
  a.n_heads = d.n_heads; a.n_signal = d.n_signal; a.n_noise = d.n_noise; a.n_kv = d.n_kv;
  a.window = d.window;
  a.sig_per_kv = d.n_signal / d.n_kv;
  a.chunks = (a.sig_per_kv + 3) / 4;
  a.c = d.scale * 1.4426950408889634f;
  a.n_qblk = (T + 255) / 256;
  se.begin(GDLA_STAGE_ATTN_NOISE);
  hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(a.n_qblk, d.n_noise, B), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_ATTN_NOISE);
  a.n_qblk = (T + 63) / 64;
  se.begin(GDLA_STAGE_ATTN_SIGNAL);
  hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3(a.n_qblk, d.n_kv * a.chunks, B), dim3(256), 0, s, a);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_ATTN_SIGNAL);
  return GDLA_OK;
}

}  // namespace gdla
