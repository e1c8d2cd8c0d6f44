// Fused backward of the GDLA attention maps for gfx950 (d_head 128, d_rope 64, fp16 operands, fp32
// accumulation), training sequences at positions 0 .. T-1.
//
// Per head h with KV head kv(h) (picx.dev summary section 2.2: the two softmax maps of the signal
// and noise heads, both on the KV heads of Eq.(5)), with raw scores s = q . k over [q^C ; q^R] and
// [K^C ; k^R], P = exp2(c s - lse) (c = tau log2 e, lse from the forward) on the visible keys:
//   dP = dH V^T,  dS = tau P (.) (dP - rowsum(dH (.) H)),
//   dq = dS K,    dK += dS^T q,   dV += P^T dH.
// Two kernels, so that every output has one writer and no atomics are needed:
//   bwd_dq_kernel   query-major, like the forward: a wave holds 32 queries of one head, streams
//                   the KV head's key tiles and accumulates dQ^T = K^T dS^T;
//   bwd_dkv_kernel  key-major: a wave holds 32 keys of one KV head, streams the query blocks of
//                   every head of the group and accumulates dK^T = Q^T dS and dV^T = dH^T P.
// All products run on v_mfma_f32_32x32x16_f16 (A[m = l % 32][k = 8 (l / 32) + i],
// B[k = 8 (l / 32) + i][n = l % 32], acc[j] = C[8 (j / 4) + 4 (l / 32) + j % 4][l % 32]).  Where
// an accumulator (whose rows run in that j order) feeds the next product as its B operand, the
// matching A fragments are read with ds_read_b64_tr_b16 from a row-major tile: each 4-row group of
// the transposing read covers one run of four consecutive rows in that order.
#include "fast_paths.h"

namespace gdla {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int DH = 128, DR = 64, DQK = DH + DR;
constexpr int KP = DQK + 8;  // LDS row pitch (elements) of [q ; k] rows
constexpr int VP = DH + 8;   // LDS row pitch of value / dH rows

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 tr4(const f16_t *p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
__device__ __forceinline__ f16_t h16(float v) { return (f16_t)(v); }

// A fragment of a transposed row-major tile (rows r, columns c, pitch `pitch` elements): lane l
// gets column c0 + l % 32 at the 8 rows r0 + 8 (i / 4) + 4 (l / 32) + i % 4, i = 0..7 (the row
// order of an accumulator's 16-row half).
__device__ __forceinline__ f16x8 tr_frag(const f16_t *tile, int pitch, int r0, int c0, int lane) {
  const int G = lane >> 4, s = lane & 15;
  const f16_t *p = tile + (r0 + 4 * (G >> 1) + (s >> 2)) * pitch + c0 + 16 * (G & 1) + 4 * (s & 3);
  const f16x4 lo = tr4(p), hi = tr4(p + 8 * pitch);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace



namespace {

__device__ __forceinline__ void dma16v(const void *gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_addr) : "memory");
}
__device__ __forceinline__ uint32_t lds_u32(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// lowest visible key of token t of sequence b (window and document)
__device__ __forceinline__ int qlo(const BwdAttnArgs &a, int b, int t) {
  int lo = a.window > 0 ? max(0, t - a.window + 1) : 0;
  if (a.doc) lo = max(lo, min(max(a.doc[(int64_t)b * a.T + t], 0), t));
  return lo;
}

// ------------------------------------------------------------------------------------------
// dq.  SIGNAL: workgroup (q block of 32, KV head, chunk of 4 signal heads, sequence), wave w =
// signal head kv + n_kv (4 chunk + w).  Noise: workgroup (q block of 128, noise head, sequence),
// wave w = queries 32 w ... of that head.  Key tiles of 32 rows (K at 25 slots of 16 bytes per
// row, V at 17, one slot of padding each) come by direct global -> LDS loads into three buffers
// of 24 KB, so two workgroups (two waves per SIMD, at most 256 registers each) share a CU and
// one's softmax and waits overlap the other's matrix work.
constexpr int DQ_KT = 32;                       // keys per tile
constexpr int KT_W = 6;                         // wave-instructions per wave and key tile
constexpr int KT_BYTES = 4 * KT_W * 64 * 16;    // 24 KB
constexpr int K_SLOTS = DQ_KT * 25, V_SLOTS = DQ_KT * 17;

template <bool SIGNAL>
__global__ void __launch_bounds__(256, 2) bwd_dq_kernel(BwdAttnArgs a) {
  __shared__ __attribute__((aligned(16))) char KV[3 * KT_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int QB = SIGNAL ? 32 : 128;
  const int n_qblk = (a.T + QB - 1) / QB;
  const int ny = SIGNAL ? a.n_kv * a.sig_chunks : a.n_noise;
  const int per_q = ny * a.B;
  const int qblk = n_qblk - 1 - (int)blockIdx.x / per_q;  // longest work first
  const int yy = (int)blockIdx.x % per_q % ny, b = (int)blockIdx.x % per_q / ny;
  int head, kvh, q0;
  const int q_first = qblk * QB;
  if (SIGNAL) {
    kvh = yy / a.sig_chunks;
    const int r = (yy % a.sig_chunks) * 4 + wave;
    head = r < a.n_signal / a.n_kv ? kvh + a.n_kv * r : -1;
    q0 = q_first;
  } else {
    head = a.n_signal + yy;
    kvh = yy % a.n_kv;
    q0 = q_first + 32 * wave;
  }
  const int q_last = min(q_first + QB, a.T) - 1;
  const bool active = head >= 0 && q0 < a.T;
  const int klo = qlo(a, b, q_first) & ~(DQ_KT - 1), khi = q_last + 1;
  const int ntiles = (khi - klo + DQ_KT - 1) / DQ_KT;
  const int wq_hi = min(q0 + 31, a.T - 1);
  const int wlo_min = qlo(a, b, min(q0, a.T - 1)), wlo_max = qlo(a, b, wq_hi);

  // this lane's query (column l % 32)
  const int tq = q0 + (lane & 31);
  const bool qok = active && tq < a.T;
  const int tqc = min(tq, a.T - 1);
  const int64_t mh = ((int64_t)b * a.T + tqc) * a.n_heads + (head >= 0 ? head : 0);
  const int wlim = qok ? tqc - qlo(a, b, tqc) + 1 : 0;  // key s visible iff 0 <= t - s < wlim
  const int64_t hm = (int64_t)(head >= 0 ? head : 0) * a.B * a.T + (int64_t)b * a.T + tqc;  // head-major
  const float lse = qok ? a.lse[hm] : 0.f, drow = qok ? a.drow[hm] : 0.f;
  f16x8 Qf[12], Hf[8];
#pragma unroll
  for (int k = 0; k < 12; ++k) Qf[k] = *(const f16x8 *)(a.q + mh * DQK + 16 * k + 8 * (lane >> 5));
#pragma unroll
  for (int k = 0; k < 8; ++k) Hf[k] = *(const f16x8 *)(a.dh + mh * DH + 16 * k + 8 * (lane >> 5));
  f32x16 dQ[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) dQ[i] = f32x16{};

  const f16_t *kg = a.k + ((int64_t)b * a.n_kv + kvh) * a.lcap * DQK;
  const f16_t *vg = a.v + ((int64_t)b * a.n_kv + kvh) * a.lcap * DH;
  // the query fragments have landed before any tile load is issued (the tile waits below count
  // only those loads)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // tile t into buffer t % 3; rows past the last key read the last valid row instead (finite,
  // never visible)
  const uint32_t lds0 = lds_u32(KV);
  auto issue = [&](int t) {
    const int s0 = klo + DQ_KT * t;
    const uint32_t buf = lds0 + (uint32_t)((t % 3) * KT_BYTES);
#pragma unroll
    for (int i = 0; i < KT_W; ++i) {
      const int slot = (wave + 4 * i) * 64 + lane;
      const void *src;
      if (slot < K_SLOTS) {
        const int r = slot / 25, c = min(slot % 25, 23);
        src = kg + (int64_t)min(s0 + r, a.T - 1) * DQK + 8 * c;
      } else if (slot < K_SLOTS + V_SLOTS) {
        const int s2 = slot - K_SLOTS, r = s2 / 17, c = min(s2 % 17, 15);
        src = vg + (int64_t)min(s0 + r, a.T - 1) * DH + 8 * c;
      } else {
        src = kg;
      }
      dma16v(src, __builtin_amdgcn_readfirstlane(buf + (uint32_t)((wave + 4 * i) * 64 * 16)));
    }
  };

  for (int t = 0; t < 2 && t < ntiles; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KT_W) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t has landed for every wave; every wave is done with tile t - 1
    if (t + 2 < ntiles) issue(t + 2);
    const int s0 = klo + DQ_KT * t;
    const f16_t *ks = (const f16_t *)(KV + (t % 3) * KT_BYTES);
    const f16_t *vs = (const f16_t *)(KV + (t % 3) * KT_BYTES + K_SLOTS * 16);
    const bool skip = !active || s0 > wq_hi || s0 + DQ_KT - 1 < wlo_min;
    if (!skip) {
      const bool full = s0 + DQ_KT - 1 <= q0 && s0 >= wlo_max;
#pragma unroll
      for (int kb = 0; kb < DQ_KT / 32; ++kb) {
        f32x16 S = {}, dP = {};
#pragma unroll
        for (int k = 0; k < 12; ++k)
          S = mfma(*(const f16x8 *)(ks + (32 * kb + (lane & 31)) * KP + 16 * k + 8 * (lane >> 5)), Qf[k], S);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          dP = mfma(*(const f16x8 *)(vs + (32 * kb + (lane & 31)) * VP + 16 * k + 8 * (lane >> 5)), Hf[k], dP);
        // acc[j]: key s0 + 32 kb + 8 (j / 4) + 4 (l / 32) + j % 4, query tq
        const int d0 = tq - s0 - 32 * kb - 4 * (lane >> 5);
        f16x8 dsf[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = 8 * (j >> 2) + (j & 3);
          const bool vis = full ? qok : (unsigned)(d0 - off) < (unsigned)wlim;
          const float p = vis ? __builtin_amdgcn_exp2f(S[j] * a.c - lse) : 0.f;
          dsf[j >> 3][j & 7] = h16(vis ? p * (dP[j] - drow) : 0.f);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int db = 0; db < 6; ++db)
            dQ[db] = mfma(tr_frag(ks, KP, 32 * kb + 16 * kk, 32 * db, lane), dsf[kk], dQ[db]);
      }
    }
  }
  if (!qok) return;
  // dQ[db][j] = dQ^T[dim 32 db + 8 (j / 4) + 4 (l / 32) + j % 4][query tq]
  if (a.a6) {
    // packed: dims 0..127 as they are; rope dims r and r + 32 (blocks 4 and 5, same lane and
    // index) rotated by the negative angle of token tq
    f16_t *oc = a.a6 + ((int64_t)b * a.T + tq) * a.lda6 + (int64_t)head * DH;
    f16_t *orr = a.a6 + ((int64_t)b * a.T + tq) * a.lda6 + a.q_off + (int64_t)head * DR;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = h16(dQ[db][4 * i + e] * a.tau);
        *(f16x4 *)(oc + 32 * db + 8 * i + 4 * (lane >> 5)) = v;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + 4 * (lane >> 5);
      const float4 c01 = *(const float4 *)(a.rope_cs + (int64_t)tq * (DR / 2) + r);
      const float4 c23 = *(const float4 *)(a.rope_cs + (int64_t)tq * (DR / 2) + r + 2);
      const float cs[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
      f16x4 lo4, hi4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float u = dQ[4][4 * i + e] * a.tau, w = dQ[5][4 * i + e] * a.tau;
        lo4[e] = h16(u * cs[e] + w * sn[e]);
        hi4[e] = h16(-u * sn[e] + w * cs[e]);
      }
      *(f16x4 *)(orr + r) = lo4;
      *(f16x4 *)(orr + r + 32) = hi4;
    }
    return;
  }
  float *o = a.dq + mh * DQK;
#pragma unroll
  for (int db = 0; db < 6; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4 *)(o + 32 * db + 8 * i + 4 * (lane >> 5)) =
          make_float4(dQ[db][4 * i] * a.tau, dQ[db][4 * i + 1] * a.tau, dQ[db][4 * i + 2] * a.tau,
                      dQ[db][4 * i + 3] * a.tau);
}

// ------------------------------------------------------------------------------------------
// dK, dV.  Workgroup (key block of 128, KV head, sequence); wave w holds keys 32 w .. 32 w + 31 of
// the block.  The waves walk the query blocks of 64 of every head of the group together: each
// block's Q, dH, log-sum-exp, row sum and lowest visible keys come by direct global -> LDS loads
// (M0 + 16 lane per wave-instruction, no compiler tracking) into three buffers, two blocks in
// flight while one is read.  A buffer is 44 wave-instructions of 64 slots of 16 bytes:
//   Q rows 0..63 at 25 slots per row (24 of data, one of padding), then dH rows at 17 slots per
//   row, then lse, row sum (fp32) and lowest visible key (int32) of the 64 queries, 16 slots each;
//   padding slots receive a copy of a neighbouring chunk.
constexpr int QB64 = 64;                       // queries per block
constexpr int DMA_W = 11;                      // wave-instructions per wave and block
constexpr int TB_SLOTS = 4 * DMA_W * 64;       // 2816 slots
constexpr int TB_BYTES = TB_SLOTS * 16;        // 44 KB
constexpr int Q_SLOTS = QB64 * 25, H_SLOTS = QB64 * 17;
constexpr int S_OFF = (Q_SLOTS + H_SLOTS) * 16;  // bytes: lse [64], drow [64], lo [64]

__global__ void __launch_bounds__(256, 1) bwd_dkv_kernel(BwdAttnArgs a) {
  __shared__ __attribute__((aligned(16))) char SM[3 * TB_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per_k = a.n_kv * a.B;
  const int kblk = (int)blockIdx.x / per_k;  // longest work (first keys) first
  const int kvh = (int)blockIdx.x % per_k % a.n_kv, b = (int)blockIdx.x % per_k / a.n_kv;
  const int kb0 = 128 * kblk;
  const int64_t M = (int64_t)a.B * a.T;
  // queries kb0 .. q_end - 1 can see a key of the block: lowest visible keys never decrease
  int lo_q = kb0, hi_q = a.T;
  while (lo_q < hi_q) {
    const int mid = (lo_q + hi_q) >> 1;
    if (qlo(a, b, mid) > kb0 + 127) hi_q = mid;
    else lo_q = mid + 1;
  }
  const int qb0 = kb0 / QB64, nqb = max(0, (lo_q - kb0 + QB64 - 1) / QB64);
  const int sig_g = a.n_signal / a.n_kv, n_g = a.n_heads / a.n_kv;
  const int n_it = n_g * nqb;

  // this wave's keys: K^T and V^T as B operands (B[k = dim][n = key])
  const int key = kb0 + 32 * wave + (lane & 31);
  const int keyc = min(key, a.T - 1);
  const f16_t *kg = a.k + (((int64_t)b * a.n_kv + kvh) * a.lcap + keyc) * DQK;
  const f16_t *vg = a.v + (((int64_t)b * a.n_kv + kvh) * a.lcap + keyc) * DH;
  f16x8 Kf[12], Vf[8];
#pragma unroll
  for (int k = 0; k < 12; ++k) Kf[k] = *(const f16x8 *)(kg + 16 * k + 8 * (lane >> 5));
#pragma unroll
  for (int k = 0; k < 8; ++k) Vf[k] = *(const f16x8 *)(vg + 16 * k + 8 * (lane >> 5));
  // the key fragments have landed before any block load is issued (the block waits below count
  // only those loads)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  f32x16 dK[6], dV[4];
#pragma unroll
  for (int i = 0; i < 6; ++i) dK[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i) dV[i] = f32x16{};

  auto head_of = [&](int gi) { return gi < sig_g ? kvh + a.n_kv * gi : a.n_signal + kvh + a.n_kv * (gi - sig_g); };
  // block `it` into buffer it % 3: this lane's DMA_W slots are (wave + 4 i) * 64 + lane
  const uint32_t lds0 = lds_u32(SM);
  auto issue = [&](int it) {
    const int h = head_of(it / nqb), qbase = QB64 * (qb0 + it % nqb);
    const int64_t mrow = (int64_t)b * a.T;
    const uint32_t buf = lds0 + (uint32_t)((it % 3) * TB_BYTES);
#pragma unroll
    for (int i = 0; i < DMA_W; ++i) {
      const int slot = (wave + 4 * i) * 64 + lane;
      const void *src;
      if (slot < Q_SLOTS) {
        const int r = slot / 25, c = min(slot % 25, 23);
        const int t = min(qbase + r, a.T - 1);
        src = a.q + ((mrow + t) * a.n_heads + h) * DQK + 8 * c;
      } else if (slot < Q_SLOTS + H_SLOTS) {
        const int s2 = slot - Q_SLOTS, r = s2 / 17, c = min(s2 % 17, 15);
        const int t = min(qbase + r, a.T - 1);
        src = a.dh + ((mrow + t) * a.n_heads + h) * DH + 8 * c;
      } else {
        const int s3 = min(slot - Q_SLOTS - H_SLOTS, 47), part = s3 >> 4, k4 = 4 * (s3 & 15);
        // the three arrays carry 64 entries of padding past their end
        if (part == 0) src = a.lse + (int64_t)h * M + mrow + qbase + k4;
        else if (part == 1) src = a.drow + (int64_t)h * M + mrow + qbase + k4;
        else src = a.lo + mrow + qbase + k4;
      }
      dma16v(src, __builtin_amdgcn_readfirstlane(buf + (uint32_t)((wave + 4 * i) * 64 * 16)));
    }
  };

  for (int it = 0; it < 2 && it < n_it; ++it) issue(it);
  for (int it = 0; it < n_it; ++it) {
    // at most this wave's loads of block it + 1 still in flight
    if (it + 1 < n_it) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_W) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block it has landed for every wave; every wave is done with block it - 1
    if (it + 2 < n_it) issue(it + 2);
    const int qblock = QB64 * (qb0 + it % nqb);
    const char *base = SM + (it % 3) * TB_BYTES;
    const f16_t *qs0 = (const f16_t *)base, *hs0 = (const f16_t *)(base + Q_SLOTS * 16);
    const float *ls = (const float *)(base + S_OFF);
    const int *los = (const int *)(base + S_OFF + 2 * QB64 * 4);
#pragma unroll
    for (int qh = 0; qh < QB64 / 32; ++qh) {
      const int qbase = qblock + 32 * qh;
      const f16_t *qs = qs0 + 32 * qh * KP, *hs = hs0 + 32 * qh * VP;
      f32x16 S = {}, dP = {};
#pragma unroll
      for (int k = 0; k < 12; ++k) S = mfma(*(const f16x8 *)(qs + (lane & 31) * KP + 16 * k + 8 * (lane >> 5)), Kf[k], S);
#pragma unroll
      for (int k = 0; k < 8; ++k) dP = mfma(*(const f16x8 *)(hs + (lane & 31) * VP + 16 * k + 8 * (lane >> 5)), Vf[k], dP);
      // acc[j]: query qbase + qi, qi = 8 (j / 4) + 4 (l / 32) + j % 4; key `key`.  The 16 queries
      // of a lane are four runs of four: their lse, row sums and lowest keys are 16-byte reads.
      float4 lv[4], dv4[4];
      int4 lov[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int q4 = 32 * qh + 8 * g + 4 * (lane >> 5);
        lv[g] = *(const float4 *)(ls + q4);
        dv4[g] = *(const float4 *)(ls + QB64 + q4);
        lov[g] = *(const int4 *)(los + q4);
      }
      f16x8 pf[2], dsf[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int g = j >> 2, e = j & 3;
        const int t = qbase + 8 * g + 4 * (lane >> 5) + e;
        const float lse_q = e == 0 ? lv[g].x : e == 1 ? lv[g].y : e == 2 ? lv[g].z : lv[g].w;
        const float dr_q = e == 0 ? dv4[g].x : e == 1 ? dv4[g].y : e == 2 ? dv4[g].z : dv4[g].w;
        const int lo_q = e == 0 ? lov[g].x : e == 1 ? lov[g].y : e == 2 ? lov[g].z : lov[g].w;
        const bool vis = key <= t && t < a.T && key >= lo_q;
        const float p = vis ? __builtin_amdgcn_exp2f(S[j] * a.c - lse_q) : 0.f;
        pf[j >> 3][j & 7] = h16(p);
        dsf[j >> 3][j & 7] = h16(vis ? p * (dP[j] - dr_q) : 0.f);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) dV[eb] = mfma(tr_frag(hs, VP, 16 * kk, 32 * eb, lane), pf[kk], dV[eb]);
#pragma unroll
        for (int db = 0; db < 6; ++db) dK[db] = mfma(tr_frag(qs, KP, 16 * kk, 32 * db, lane), dsf[kk], dK[db]);
      }
    }
  }
  if (key >= a.T) return;
  // dK[db][j] = dK^T[dim 32 db + 8 (j / 4) + 4 (l / 32) + j % 4][key]
  const int64_t ko = ((int64_t)b * a.n_kv + kvh) * a.T + key;
  float *dk = a.dk + ko * DQK, *dv = a.dv + ko * DH;
#pragma unroll
  for (int db = 0; db < 6; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4 *)(dk + 32 * db + 8 * i + 4 * (lane >> 5)) =
          make_float4(dK[db][4 * i] * a.tau, dK[db][4 * i + 1] * a.tau, dK[db][4 * i + 2] * a.tau,
                      dK[db][4 * i + 3] * a.tau);
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4 *)(dv + 32 * eb + 8 * i + 4 * (lane >> 5)) =
          make_float4(dV[eb][4 * i], dV[eb][4 * i + 1], dV[eb][4 * i + 2], dV[eb][4 * i + 3]);
}

}  // namespace

bool fast_backward_supported(const LayerDims &d, gdla_dtype dt) {
  return dt == GDLA_BF16 && d.d_h == DH && d.d_r == DR && d.n_noise % d.n_kv == 0 && d.n_signal % d.n_kv == 0;
}

hipError_t launch_bwd_attention(const BwdAttnArgs &a0, hipStream_t s) {
  BwdAttnArgs a = a0;
  a.sig_chunks = (a.n_signal / a.n_kv + 3) / 4;
  const int nq32 = (a.T + 31) / 32, nq128 = (a.T + 127) / 128, nk = (a.T + 127) / 128;
  hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((unsigned)(nq32 * a.n_kv * a.sig_chunks * a.B)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((unsigned)(nq128 * a.n_noise * a.B)), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)(nk * a.n_kv * a.B)), dim3(256), 0, s, a);  // 128-key blocks
  return hipGetLastError();
}

}  // namespace gdla
