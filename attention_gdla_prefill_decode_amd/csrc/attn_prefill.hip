// Fused GDLA prefill attention for gfx950 (d_head 128, d_rope 64): fp16 MFMA operands (queries,
// expanded keys [K^C ; k^R], values and probabilities), fp32 accumulation and fp32 online softmax.
//
// Computes, per query head h and query token t at position p, the softmax attention over the
// expanded keys [K^C ; k^R] and values V of its KV head (Motif 3 Technical Report, picx.dev
// summary section 2.2, Eq.(5) feeding the signal / noise maps of Eq.(8)), then, for the signal
// heads, the grouped differential combine and the sigmoid gate of Eq.(8)-(10):
//     Y_i = sigmoid(G_i) * (H_i - lambda_i * H_{n_S + i mod n_N}).
// Two launches: the noise heads first (they write H_N in fp32), then the signal heads, whose
// epilogue reads H_N, lambda and the gate (sigmoid values in fp16 from the projection's epilogue,
// or fp32 logits) and writes Y in fp16 for the output projection.
//
// Work split: a workgroup is 8 waves (2 per SIMD, so one wave's softmax overlaps the other's
// matrix work); each wave owns 32 query rows of one head.  In the signal launch the waves are 4
// signal heads sharing one KV head times 2 halves of the same 64 tokens, so each K/V tile staged
// in LDS serves all of them; in the noise launch the waves are 8 consecutive 32-token blocks of one
// noise head.  Keys are processed in tiles of 64:
//   staging: direct global -> LDS 16-byte loads (no staging registers) into three tile buffers,
//     so two tiles are in flight while one is read; rows are unpadded and XOR-swizzled per 16-byte
//     chunk so both LDS read patterns below are free of bank conflicts;
//   S^T[key, query] = K[key, 0:192] . Q[query, 0:192]   (A = K from LDS, B = Q in registers);
//   online softmax per query (each lane owns one query column; its partner lane l^32 the other
//     half of the keys), with lazy rescaling, P^T taken straight from the accumulators in fp16;
//   O^T[dim, query] += V^T[dim, key] . P^T[key, query]  (A = V^T rows, 16-byte LDS reads).
// The values arrive transposed from the expansion GEMM ([n_kv][128][keys], keys of every 16-group
// in the order vt_slot), which is the order in which the S accumulators hold the keys of P^T: the
// accumulators serve as the P operand without any shuffle and no transposing LDS read is needed.
// Causal / sliding-window / packed-document tiles are classified per wave as skipped, full or
// partial; only partial tiles evaluate the per-element mask lo(p) <= s <= p, lo(p) the first key
// of the window and of the token's document.
#include "fast_paths.h"

#include <algorithm>

namespace gdla {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int DH = 128, DR = 64, DQK = DH + DR;
constexpr int KT = 64;                 // keys per tile
constexpr int K_CH = DQK / 8;          // 16-byte chunks per key row (24)
constexpr int V_CH = DH / 8;           // 16-byte chunks per value row (16)
constexpr int K_TILE = KT * DQK;       // elements of one K tile
constexpr int V_TILE = KT * DH;        // elements of one V tile
constexpr int NBUF = 3;                // LDS tile buffers: two tiles in flight while one is read
constexpr int K_LOADS = K_TILE * 2 / 16 / 64 / 8;  // 16-byte K loads per wave per tile (3)
constexpr int V_LOADS = V_TILE * 2 / 16 / 64 / 8;  // 16-byte V^T loads per wave per tile (2)

struct AttnArgs {
  const f16_t *q;         // [M, n_H, 192] fp16: q^C then rotated q^R of each head
  const f16_t *kx;        // [B, n_kv, lcap, 192] fp16: [K^C ; k^R] of keys base_b .. base_b + lcap - 1
  const f16_t *vx;        // [B, n_kv, 128, lcap] fp16: V^T, keys in vt_slot order per 16-group
  const int32_t *pos;     // [B] first position of the chunk
  const int32_t *doc;     // [M] first position of each token's document (packed documents) or null
  const float *lam;       // [M, n_S]
  const void *gate;       // [M, n_S, 128]: sigmoid(G) in fp16 (gate_f16) or the logits G in fp32
  int32_t gate_f16;
  float *hn;              // [M, n_N, 128] normalised noise-head outputs
  f16_t *y;               // [M, n_S * 128] fp16
  float *out_heads;       // [M, n_H, 128] or null
  float *lse;             // [n_H, M] or null: log2 of the softmax denominator of the log2e-scaled scores
  int32_t T, lcap;
  int32_t n_heads, n_signal, n_noise, n_kv, window;
  int32_t sig_per_kv, chunks, n_qblk;
  int32_t ny;             // workgroups per query block and sequence (KV-head chunks or noise heads)
  int32_t nb;             // sequences
  float c;                // softmax scale * log2(e)
};

// LDS chunk slot of 16-byte chunk c of row `row`: 16 consecutive rows reading the same chunk land
// on 16 distinct 4-bank groups.  K rows are keys (24 chunks), V^T rows are dims (8 chunks = the 64
// keys of the tile).
constexpr int VT_CH = KT / 8;
__device__ __forceinline__ int kslot(int row, int c) { return row * K_CH + (c ^ ((row >> 1) & 7)); }
__device__ __forceinline__ int vslot(int row, int c) { return row * VT_CH + (c ^ ((row >> 1) & 7)); }

// 16 bytes global -> LDS (M0 + 16 lane) without the compiler's LDS-DMA tracking, so that the wait
// for a tile is explicit (s_waitcnt vmcnt before the barrier that publishes it) and can leave the
// next tile's loads in flight.  The global address is a wave-uniform base plus a 32-bit per-lane
// byte offset.  M0 is set right before the load (one wait state between them); nothing else in
// the kernel uses M0.
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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
__global__ void __launch_bounds__(512, 1) attn_prefill_kernel(AttnArgs a) {
  // NBUF buffers of one key tile each: K rows, then V^T rows
  __shared__ __attribute__((aligned(16))) f16_t KV[NBUF * (K_TILE + V_TILE)];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // 1-D grid, longest work first: late (long) query blocks of every head and sequence before any
  // earlier one.  The head index varies fastest, so with 16 KV heads each of the 8 XCDs (which
  // take workgroups round-robin) always serves the same two KV heads and their K/V stay in its L2.
  const int per_q = a.ny * a.nb;
  const int qblk = a.n_qblk - 1 - (int)blockIdx.x / per_q;
  const int yy = (int)blockIdx.x % per_q % a.ny;
  const int b = (int)blockIdx.x % per_q / a.ny;
  int head, kvh, t0w, tlo, thi;
  if (SIGNAL) {
    kvh = yy / a.chunks;
    const int r = (yy % a.chunks) * 4 + (wave >> 1);
    head = r < a.sig_per_kv ? kvh + a.n_kv * r : -1;
    tlo = qblk * 64;
    t0w = tlo + 32 * (wave & 1);
    thi = min(tlo + 63, a.T - 1);
  } else {
    head = a.n_signal + yy;
    kvh = yy % a.n_kv;
    tlo = qblk * 256;
    t0w = tlo + 32 * wave;
    thi = min(tlo + 255, a.T - 1);
  }
  const bool active = head >= 0 && t0w < a.T;
  const int W = a.window;
  const int p0 = a.pos[b];
  const int base = W > 0 ? max(0, p0 - W + 1) : 0;
  const int64_t mrow0 = (int64_t)b * a.T;
  // lowest visible key of query t: the window's and (packed documents) its document's first key
  auto qlo = [&](int t) {
    int lo = W > 0 ? max(0, p0 + t - W + 1) : 0;
    if (a.doc) lo = max(lo, min(max(a.doc[mrow0 + t], 0), p0 + t));
    return lo;
  };
  // first key tile: from the block's first query (document starts never decrease along a packed
  // sequence), aligned to 16 keys past `base` (the value layout's key groups); the extra keys in
  // front are masked
  const int klo = base + ((qlo(tlo) - base) & ~15);
  const int khi = p0 + thi + 1;
  const int ntiles = (khi - klo + KT - 1) / KT;
  const int wp_lo = p0 + t0w, wp_hi = p0 + min(t0w + 31, a.T - 1);
  // this lane's query (column lane % 32 of the score tiles): key s is visible iff
  // 0 <= p - s < wlim; wlo_min / wlo_max: lowest visible key over the wave's queries
  int wlim, wlo_min, wlo_max;
  {
    const int tq = min(t0w + (lane & 31), a.T - 1);
    const int lo = qlo(tq);
    wlim = p0 + tq - lo + 1;
    int mn = lo, mx = lo;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      mn = min(mn, __shfl_xor(mn, o, 64));
      mx = max(mx, __shfl_xor(mx, o, 64));
    }
    wlo_min = __builtin_amdgcn_readfirstlane(mn);
    wlo_max = __builtin_amdgcn_readfirstlane(mx);
  }

  // ---- Q fragments: Qf[ks] holds dims 16 ks + 8 (lane / 32) .. + 7 of query column lane % 32
  f16x8 Qf[12];
  {
    const int t = t0w + (lane & 31);
    const bool ok = active && t < a.T;
    const f16_t *qp = a.q + ((mrow0 + (ok ? t : 0)) * a.n_heads + (ok ? head : 0)) * DQK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) Qf[ks] = ok ? *(const f16x8 *)(qp + 16 * ks) : f16x8{};
    // Q has landed before any tile load is issued: the compiler does not see the tile loads, and
    // a vmcnt(0) it placed for Q inside the loop would also wait for the tiles in flight.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }

  // ---- direct global -> LDS staging of one key tile.  The last tile may run up to 63 keys past
  // khi: the buffers hold lcap >= (keys rounded up to 64) + 64 rows, those keys are masked for
  // every valid query (any value, NaN included, is replaced), and their values are the
  // expansion's zeroed tail.
  const f16_t *kxh = a.kx + ((int64_t)b * a.n_kv + kvh) * a.lcap * DQK;
  const f16_t *vth = a.vx + ((int64_t)b * a.n_kv + kvh) * DH * a.lcap;
  // per-lane byte offsets of this wave's K and V^T loads within a tile (rows swizzled per chunk)
  uint32_t koff[K_LOADS], voff[V_LOADS];
#pragma unroll
  for (int j = 0; j < K_LOADS; ++j) {  // K: 24 wave-instructions of 64 chunks
    const int slot = (wave * K_LOADS + j) * 64 + lane;
    const int row = slot / K_CH, cpos = slot % K_CH;
    koff[j] = (uint32_t)(row * DQK + (cpos ^ ((row >> 1) & 7)) * 8) * 2;
  }
#pragma unroll
  for (int j = 0; j < V_LOADS; ++j) {  // V^T: 128 dims x 8 chunks = 16 wave-instructions
    const int slot = (wave * V_LOADS + j) * 64 + lane;
    const int row = slot / VT_CH, cpos = slot % VT_CH;
    voff[j] = (uint32_t)(row * a.lcap + (cpos ^ ((row >> 1) & 7)) * 8) * 2;
  }
  auto issue = [&](int t) {
    const int s0 = klo + t * KT;
    f16_t *buf = KV + (t % NBUF) * (K_TILE + V_TILE);
    const uint32_t kl = lds_u32(buf), vl = lds_u32(buf + K_TILE);
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) dma16(kxh + (int64_t)(s0 - base) * DQK, koff[j], kl + (wave * K_LOADS + j) * 1024);
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) dma16(vth + (s0 - base), voff[j], vl + (wave * V_LOADS + j) * 1024);
  };

  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int hgrp = lane >> 5;  // which half of each 8-key group this lane's accumulators hold
  const int krow = lane & 31;
  // Lane-dependent byte offsets of the LDS fragment reads; the rest of each address is an
  // immediate.  K fragment (kb, kst): row 32 kb + krow, chunk 2 kst + hgrp; the row swizzle is
  // (krow >> 1) & 7 for both kb and only touches the low 3 bits of the chunk, so the lane part
  // depends on kst & 3 only.  V^T fragment (db, kst): row 32 db + krow, chunk 2 kst + hgrp.
  int offK[4], offV[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    offK[q] = krow * (K_CH * 16) + (((2 * q + hgrp) ^ ((krow >> 1) & 7)) * 16);
    offV[q] = krow * (VT_CH * 16) + (((2 * q + hgrp) ^ ((krow >> 1) & 7)) * 16);
  }

  auto compute = [&](const f16_t *ks, const f16_t *vs, int s0) {
    const bool skip = !active || s0 > wp_hi || s0 + KT - 1 < wlo_min;
    if (skip) return;
    const bool full = s0 + KT - 1 <= wp_lo && s0 >= wlo_max;
    const char *kb8 = (const char *)ks;
    const char *vb8 = (const char *)vs;
    // S phase, software-pipelined one k-step ahead: [reads of step kst + 1][MFMAs of step kst]
    f32x16 S[2];
    f16x8 kf[2][2];
    auto ldK = [&](f16x8 (&f)[2], int kst) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        f[kb] = *(const f16x8 *)(kb8 + offK[kst & 3] + kb * 32 * K_CH * 16 + (kst >> 2) * 128);
    };
    ldK(kf[0], 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int kst = 0; kst < 12; ++kst) {
      if (kst + 1 < 12) ldK(kf[(kst + 1) & 1], kst + 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) S[kb] = mfma(kf[kst & 1][kb], Qf[kst], kst == 0 ? f32x16{} : S[kb]);
      if (kst + 1 < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // v[16 kb + e] is the score of key s0 + 32 kb + 8 (e / 4) + 4 hgrp + e % 4
    float v[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) v[kb * 16 + e] = S[kb][e];
    if (!full) {
      // branch-free mask: visible iff 0 <= p - s < wlim (negative p - s wraps above it)
      const int d0 = wp_lo + (lane & 31) - s0 - 4 * hgrp;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int off = (i >> 4) * 32 + 8 * ((i & 15) >> 2) + (i & 3);
        v[i] = (unsigned)(d0 - off) < (unsigned)wlim ? v[i] : -INFINITY;
      }
    }
    float mt = v[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mt = fmaxf(mt, v[i]);
    mt = pair_max(mt);
    // Lazy rescaling: the reference max m moves (and O, l are rescaled) only when some row's tile
    // max exceeds it by more than 2^8 in the exp2 domain, so P <= 256 (fine in fp16) and the O
    // rescale runs on few tiles.
    if (__any((mt - m) * a.c > 8.0f)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m - mnew) * a.c);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db] *= alpha;
    }
    const float ms = m == -INFINITY ? 0.f : m * a.c;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = __builtin_amdgcn_exp2f(v[i] * a.c - ms);
      rs += v[i];
    }
    f16x8 P[4];  // P[kst]: keys 16 kst .. 16 kst + 15 of the tile, in accumulator order
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int e = 0; e < 8; ++e) P[k4][e] = (f16_t)v[8 * k4 + e];
    l += rs;
    // PV phase, pipelined one dim block ahead: [reads of block db + 1][MFMAs of block db]
    f16x8 vf[2][4];
    auto ldV = [&](f16x8 (&f)[4], int db) {
#pragma unroll
      for (int kst = 0; kst < 4; ++kst) f[kst] = *(const f16x8 *)(vb8 + offV[kst] + db * 32 * VT_CH * 16);
    };
    ldV(vf[0], 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      if (db + 1 < 4) ldV(vf[(db + 1) & 1], db + 1);
#pragma unroll
      for (int kst = 0; kst < 4; ++kst) O[db] = mfma(vf[db & 1][kst], P[kst], O[db]);
      if (db + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };

  // Triple buffering: tiles t + 1 and t + 2 are in flight while tile t is read.
  for (int t = 0; t < NBUF - 1 && t < ntiles; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    // vmcnt(n): at most n of this wave's loads still in flight (those of tile t + 1)
    if (t + 1 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K_LOADS + V_LOADS) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t has landed for every wave; every wave is done with tile t - 1
    if (t + NBUF - 1 < ntiles) issue(t + NBUF - 1);
    const f16_t *kv = KV + (t % NBUF) * (K_TILE + V_TILE);
    compute(kv, kv + K_TILE, klo + t * KT);
  }

  if (!active) return;
  // ---- epilogue: lane holds query column lane % 32 and dims db*32 + 8 i + 4 (lane / 32) + j
  const float lsum = pair_sum(l);
  const float inv = 1.0f / lsum;
  const int t = t0w + (lane & 31);
  if (t >= a.T) return;
  const int64_t mr = mrow0 + t;
  // the probabilities are exp2(c s - lse) for raw scores s (what a backward pass recomputes)
  if (a.lse && hgrp == 0) a.lse[(int64_t)head * a.nb * a.T + mr] = m * a.c + __log2f(lsum);  // head-major
  float *oh = a.out_heads ? a.out_heads + (mr * a.n_heads + head) * DH : nullptr;
  if (!SIGNAL) {
    float *hn = a.hn + (mr * a.n_noise + (head - a.n_signal)) * DH;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = db * 32 + 8 * i + 4 * hgrp;
        const float4 v = make_float4(O[db][4 * i] * inv, O[db][4 * i + 1] * inv, O[db][4 * i + 2] * inv,
                                     O[db][4 * i + 3] * inv);
        *(float4 *)(hn + dim) = v;
        if (oh) *(float4 *)(oh + dim) = v;
      }
  } else {
    const float lam = a.lam[mr * a.n_signal + head];
    const int64_t goff = (mr * a.n_signal + head) * DH;
    const float *hn = a.hn + (mr * a.n_noise + head % a.n_noise) * DH;
    f16_t *y = a.y + mr * (int64_t)a.n_signal * DH + (int64_t)head * DH;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = db * 32 + 8 * i + 4 * hgrp;
        float sg[4];
        if (a.gate_f16) {
          const f16x4 gh = *(const f16x4 *)((const f16_t *)a.gate + goff + dim);
#pragma unroll
          for (int e = 0; e < 4; ++e) sg[e] = (float)gh[e];
        } else {
          const float4 gv = *(const float4 *)((const float *)a.gate + goff + dim);
          sg[0] = 1.0f / (1.0f + __expf(-gv.x));
          sg[1] = 1.0f / (1.0f + __expf(-gv.y));
          sg[2] = 1.0f / (1.0f + __expf(-gv.z));
          sg[3] = 1.0f / (1.0f + __expf(-gv.w));
        }
        const float4 nv = *(const float4 *)(hn + dim);
        const float o0 = O[db][4 * i] * inv, o1 = O[db][4 * i + 1] * inv;
        const float o2 = O[db][4 * i + 2] * inv, o3 = O[db][4 * i + 3] * inv;
        if (oh) *(float4 *)(oh + dim) = make_float4(o0, o1, o2, o3);
        f16x4 yv;
        yv[0] = to_f16((o0 - lam * nv.x) * sg[0]);
        yv[1] = to_f16((o1 - lam * nv.y) * sg[1]);
        yv[2] = to_f16((o2 - lam * nv.z) * sg[2]);
        yv[3] = to_f16((o3 - lam * nv.w) * sg[3]);
        *(f16x4 *)(y + dim) = yv;
      }
  }
}

// k^R of keys lo_b .. lo_b + nk_b - 1, converted from the bf16 cache to fp16 (exact in the fp16
// normal range, saturating beyond it), into columns 128 .. 191 of every KV head's key rows.
__global__ void __launch_bounds__(256) kr_fill_kernel(const bf16_t *cache, f16_t *kx, const int32_t *pos,
                                                      int32_t T, int32_t window, int32_t max_len,
                                                      int32_t row, int32_t d_c, int32_t n_kv, int32_t lcap) {
  const int b = blockIdx.y;
  const int p0 = pos[b];
  const int lo = window > 0 ? max(0, p0 - window + 1) : 0;
  const int nk = p0 + T - lo;
  const int i = blockIdx.x * 256 + threadIdx.x;  // (key, chunk of 8) index
  if (i >= nk * (DR / 8)) return;
  const int r = i / (DR / 8), ch = i % (DR / 8);
  const uint4 v = *(const uint4 *)(cache + ((int64_t)b * max_len + lo + r) * row + d_c + ch * 8);
  auto cv = [](unsigned w) {
    const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
    return __builtin_bit_cast(unsigned, h);
  };
  const uint4 o = make_uint4(cv(v.x), cv(v.y), cv(v.z), cv(v.w));
  for (int h = 0; h < n_kv; ++h)
    *(uint4 *)(kx + (((int64_t)b * n_kv + h) * lcap + r) * DQK + DH + ch * 8) = o;
}

// Zeroes V^T positions of keys nk .. lcap - 1 (one block of 64 threads per (dim row, sequence)).
__global__ void __launch_bounds__(64) vt_tail_zero_kernel(f16_t *vx, const int32_t *pos, int32_t T,
                                                          int32_t window, int32_t rows, int32_t lcap) {
  const int b = blockIdx.y;
  const int p0 = pos[b];
  const int lo = window > 0 ? max(0, p0 - window + 1) : 0;
  const int nk = p0 + T - lo;
  f16_t *r = vx + ((int64_t)b * rows + blockIdx.x) * lcap;
  for (int i = (nk & ~15) + threadIdx.x; i < lcap; i += 64)
    if (vt_slot(i) >= nk) r[i] = (f16_t)0.0f;
}

}  // namespace

hipError_t launch_vt_tail_zero(void *vx, const int32_t *pos_dev, int32_t B, int32_t T, int32_t lcap,
                               const LayerDims &d, hipStream_t s) {
  hipLaunchKernelGGL(vt_tail_zero_kernel, dim3(d.n_kv * DH, B), dim3(64), 0, s, (f16_t *)vx, pos_dev, T,
                     d.window, d.n_kv * DH, lcap);
  return hipGetLastError();
}

bool fast_prefill_supported(const LayerDims &d, gdla_dtype dt) {
  return dt == GDLA_BF16 && d.d_h == DH && d.d_r == DR && d.d_c % 8 == 0 && d.d_cq % 64 == 0 &&
         d.d_model % 64 == 0 && (d.n_signal * DH) % 64 == 0;
}

int32_t fast_prefill_key_row() { return DQK; }

hipError_t launch_kr_fill(const void *cache, void *kx, const int32_t *pos_dev, int32_t B, int32_t T,
                          int32_t lcap, int32_t max_len, const LayerDims &d, hipStream_t s) {
  const dim3 grid((lcap * (DR / 8) + 255) / 256, B);
  hipLaunchKernelGGL(kr_fill_kernel, grid, dim3(256), 0, s, (const bf16_t *)cache, (f16_t *)kx, pos_dev,
                     T, d.window, max_len, d.d_c + d.d_r, d.d_c, d.n_kv, lcap);
  return hipGetLastError();
}

gdla_status run_fast_prefill(const LayerDims &d, const gdla_weights *w, int32_t B, int32_t T,
                             const int32_t *pos_dev, const int32_t *pos_host, void *cache,
                             int32_t max_len, void *cq, float *lam, float *gate, void *kx,
                             void *vx, int32_t lcap, void *y, float *out_heads,
                             const FastPrefillLayout &L, void *ws, hipStream_t s, StageEvents &se,
                             const NtWeights *nt, const int32_t *doc, float *lse) {
  (void)pos_host;
  (void)cache;
  (void)max_len;
  const int32_t M = B * T;
  f16_t *q = (f16_t *)((char *)ws + L.q);
  float *qrp = (float *)((char *)ws + L.qrp);
  float *hn = (float *)((char *)ws + L.hn);
  // Eq.(2), (9): q^C straight into the per-head [q^C ; q^R] rows, q^R before RoPE, gate logits.
  se.begin(GDLA_STAGE_PROJ_Q);
  // c^Q is fp16 here; the bf16 weights are converted to fp16 while the GEMM stages them.
  // with nt, B is the transposed fp16 weight [N, d_cq]
  GemmBatch g{};
  auto add = [&](const void *B_, int N, void *C, int64_t ldc, int c_dt, int hw, int64_t hs) {
    GemmProblem p{};
    p.A = cq; p.lda = d.d_cq; p.B = B_; p.ldb = nt ? d.d_cq : N; p.C = C; p.ldc = ldc;
    p.M = M; p.N = N; p.K = d.d_cq; p.hw = hw; p.hs = hs; p.ho = 0; p.c_dt = c_dt; p.a_f16 = 1;
    p.epi = EPI_NONE;
    g.p[g.n++] = p;
  };
  add(nt ? nt->qc : w->w_qc, d.n_heads * DH, q, (int64_t)d.n_heads * DQK, CD_F16, DH, DQK);
  if (nt) {
    // q^R rotated in the GEMM epilogue, straight into columns 128 .. 191 of every head's q row
    add(nt->qr, d.n_heads * DR, q, (int64_t)d.n_heads * DQK, CD_F16, DR, DQK);
    GemmProblem &pr = g.p[g.n - 1];
    pr.ho = DH;
    pr.epi = EPI_ROPE;
    pr.rope_pos = pos_dev;
    pr.rope_T = T;
    pr.rope_d = DR;
    pr.rope_theta = d.theta;
  } else {
    add(w->w_qr, d.n_heads * DR, qrp, (int64_t)d.n_heads * DR, CD_F32, d.n_heads * DR, 0);
  }
  // with nt the gate leaves the GEMM as sigmoid(G) in fp16, else as fp32 logits
  add(nt ? nt->gate : w->w_gate, d.n_signal * DH, gate, (int64_t)d.n_signal * DH, nt ? CD_F16 : CD_F32,
      d.n_signal * DH, 0);
  if (nt) g.p[g.n - 1].epi = EPI_SIGMOID;
  if ((nt ? launch_gemm_nt(g, true, s) : launch_gemm(g, DT::BF16, s)) != hipSuccess) return GDLA_ERR_HIP;
  if (!nt && launch_rope_heads(qrp, q, (int64_t)d.n_heads * DQK, DQK, DH, M, T, d.n_heads, DR, pos_dev,
                               d.theta, DT::F16, s) != hipSuccess)
    return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_PROJ_Q);

  AttnArgs a{};
  a.q = q; a.kx = (const f16_t *)kx; a.vx = (const f16_t *)vx;
  a.pos = pos_dev; a.doc = doc; a.lse = lse; a.lam = lam; a.gate = gate; a.gate_f16 = nt ? 1 : 0; a.hn = hn; a.y = (f16_t *)y; a.out_heads = out_heads;
  a.T = T; a.lcap = lcap;
  a.n_heads = d.n_heads; a.n_signal = d.n_signal; a.n_noise = d.n_noise; a.n_kv = d.n_kv;
  a.window = d.window;
  a.sig_per_kv = d.n_signal / d.n_kv;
  a.chunks = (a.sig_per_kv + 3) / 4;
  a.c = d.scale * 1.4426950408889634f;
  a.n_qblk = (T + 255) / 256;
  a.ny = d.n_noise;
  se.begin(GDLA_STAGE_ATTN_NOISE);
  a.nb = B;
  hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(a.n_qblk * a.ny * B), dim3(512), 0, s, a);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_ATTN_NOISE);
  a.n_qblk = (T + 63) / 64;
  a.ny = d.n_kv * a.chunks;
  se.begin(GDLA_STAGE_ATTN_SIGNAL);
  hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3(a.n_qblk * a.ny * B), dim3(512), 0, s, a);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_ATTN_SIGNAL);
  return GDLA_OK;
}

}  // namespace gdla
