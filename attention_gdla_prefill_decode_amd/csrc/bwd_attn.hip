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
//   bwd_dkv_kernel  key-major: a workgroup holds 128 keys of one KV head, streams the queries of
//                   every head of the group and accumulates dK^T = Q^T dS and dV^T = dH^T P
//                   (one wave per 32 keys and product: see the kernel).
// All products run on v_mfma_f32_32x32x16_f16 (A[m = l % 32][k = 8 (l / 32) + i],
// B[k = 8 (l / 32) + i][n = l % 32], acc[j] = C[8 (j / 4) + 4 (l / 32) + j % 4][l % 32]).  Where
// an accumulator (whose rows run in that j order) feeds the next product as its B operand, the dq
// kernel reads the matching A fragments with ds_read_b64_tr_b16 from a row-major tile: each 4-row
// group of the transposing read covers one run of four consecutive rows in that order.  The dK/dV
// kernel stages a second, dim-major copy of its operands instead.
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
// The same with a wave-uniform base and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16s(const void *base, uint32_t voff, uint32_t lds_addr) {
  // readfirstlane returns int: each half goes through uint32_t (no sign extension into the high half)
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint64_t sbase = (uint64_t)hi << 32 | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
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
constexpr int KT_W = 6;                         // wave-instructions per wave and key tile (at most)
constexpr int KT_BYTES = 4 * KT_W * 64 * 16;    // 24 KB
// K rows in chunks 0..12 of 64 slots (800 slots used), V rows in chunks 13..21 (544 used)
constexpr int VC0 = 13, KT_CHUNKS = 22;
static_assert(DQ_KT * 25 <= VC0 * 64 && DQ_KT * 17 <= (KT_CHUNKS - VC0) * 64, "tile regions");

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
  // Tile t into buffer t % 3: instruction i of this wave fills chunk c = wave + 4 i (a
  // wave-uniform region; waves 2 and 3 have no sixth chunk), lane l unit 64 c' + l of its region.
  // Each load is a wave-uniform base (the tile's first key) plus the lane's fixed byte offset; in
  // the last tile, rows past the last key read the last key's row instead (finite, never visible).
  // (The offsets are recomputed at each tile, a few integer operations: kept in registers they
  // would be spilled, and each reload would wait for every load in flight.)
  const uint32_t lds0 = lds_u32(KV);
  auto issue = [&](int t) {
    const int s0 = klo + DQ_KT * t;
    const uint32_t buf = lds0 + (uint32_t)((t % 3) * KT_BYTES);
    const int rmax = min(DQ_KT - 1, a.T - 1 - s0);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keeps the offsets below inside the loop
#pragma unroll
    for (int i = 0; i < KT_W; ++i) {
      const int c = wave + 4 * i;
      if (c >= KT_CHUNKS) continue;
      uint32_t off;
      if (c < VC0) {
        const int s = 64 * c + ln;
        off = (uint32_t)min(s / 25, rmax) * (DQK * 2) + 16u * (uint32_t)min(s % 25, 23);
      } else {
        const int s = 64 * (c - VC0) + ln;
        off = (uint32_t)min(s / 17, rmax) * (DH * 2) + 16u * (uint32_t)min(s % 17, 15);
      }
      dma16s(c < VC0 ? (const void *)(kg + (int64_t)s0 * DQK) : (const void *)(vg + (int64_t)s0 * DH), off,
             __builtin_amdgcn_readfirstlane(buf + (uint32_t)(c * 64 * 16)));
    }
  };

  for (int t = 0; t < 2 && t < ntiles; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    // at most this wave's loads of tile t + 1 still in flight (6 per tile, 5 for waves 2 and 3)
    if (t + 1 < ntiles) {
      if (wave < 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KT_W) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KT_W - 1) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();  // tile t has landed for every wave; every wave is done with tile t - 1
    if (t + 2 < ntiles) issue(t + 2);
    const int s0 = klo + DQ_KT * t;
    const f16_t *ks = (const f16_t *)(KV + (t % 3) * KT_BYTES);
    const f16_t *vs = (const f16_t *)(KV + (t % 3) * KT_BYTES + VC0 * 64 * 16);
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
// dK, dV.  Workgroup (key block of 128, KV head, sequence): 8 waves in two roles on the four key
// blocks kb of 32 keys, one wave of each role per SIMD:
//   P wave (w = kb):      S = Q K^T, P = exp2(c S - lse) on the visible pairs, dV^T += dH^T P;
//                         hands P (fp16) through LDS to
//   dS wave (w = 4 + kb): dP = dH V^T, dS = P (.) (dP - rowsum), dK^T += Q^T dS,
// one step behind: in iteration j the P waves take step j and the dS waves step j - 1, so the
// two streams of a SIMD are independent between the one barrier per iteration, and one's softmax
// or dS arithmetic runs beside the other's matrix products.
// A step is 32 queries of one head: every head of the group, over the queries that can see the
// key block, last query block first.  Each role stages its own operands of a step, by direct
// global -> LDS loads, in its own ring of three slots of 24 chunks of 64 x 16 bytes (two steps in
// flight while one is read):
//   P ring:  Q query-major (rows of 25 slots, one of padding), the 32 queries' lse and lowest
//            visible keys, dH dim-major (from the transposed copy dH^T: rows of 5 slots);
//   dS ring: dH query-major (rows of 17 slots), the 32 row sums, Q dim-major (from q^T).
// So every LDS read is a plain 16-byte read: the products summed over the queries (dK, dV) take
// their query-contiguous A fragments from the dim-major copies instead of transposing reads, which
// cost about three times as much per byte.  The query-major A fragments of S and dP read row R(m)
// (bits 2 and 3 of m swapped) for accumulator row m, which makes each lane's 8 values of an
// accumulator half 8 consecutive queries: the k order of the dim-major fragments and of P.
constexpr int QS = 32;                     // queries per step
constexpr int TP = 5 * 8;                  // dim-major row pitch (elements)
constexpr int KV_DMA = 6;                  // wave-instructions per wave and step
constexpr int RING_SLOT = 24 * 64 * 16;    // bytes of one ring slot (24 chunks)
// P slot (in 16-byte units): Q rows 0..799, lse 800..807, lowest keys 808..815, dH^T from 832
// (chunks 13..22; chunk 23 repeats chunk 22).  dS slot: dH rows 0..543, row sums 544..551, Q^T
// from 576 (chunks 9..23).
constexpr int P_ST = QS * 25, P_HT = 13 * 64, S_ST = QS * 17, S_QT = 9 * 64;
static_assert(P_ST + 16 <= P_HT && P_HT + DH * 5 == 23 * 64 && S_ST + 8 <= S_QT && S_QT + DQK * 5 == 24 * 64,
              "regions fit their slots");
constexpr int KV_LDS = 6 * RING_SLOT;      // then the P exchange: [2 steps][4 key blocks][2][64 lanes] f16x8

struct DkvUnit {
  int b, kvh, kb0, qb0, nqb, n_it, sig_g;
};

template <bool PW>
__device__ __forceinline__ void dkv_body(const BwdAttnArgs &a, const DkvUnit &u, char *SM, f16x8 (*PX)[4][2][64],
                                         int wave, int lane) {
  const int kb = wave & 3, h2 = lane >> 5;
  const int key = u.kb0 + 32 * kb + (lane & 31);
  const int keyc = min(key, a.T - 1);
  const int rq = (lane & 19) | ((lane & 4) << 1) | ((lane & 8) >> 1);  // R(lane % 32)
  const int64_t kvrow = ((int64_t)u.b * a.n_kv + u.kvh) * a.lcap + keyc;
  // this wave's keys as B operands (B[k = dim][n = key]): K^T for a P wave, V^T for a dS wave
  constexpr int NF = PW ? 12 : 8;
  f16x8 F[NF];
  const f16_t *fg = PW ? a.k + kvrow * DQK : a.v + kvrow * DH;
#pragma unroll
  for (int k = 0; k < NF; ++k) F[k] = *(const f16x8 *)(fg + 16 * k + 8 * h2);
  // the key fragments have landed before any step load is issued (the waits below count only those)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  constexpr int NACC = PW ? 4 : 6;  // dV^T: 4 dim blocks of 32; dK^T: 6
  f32x16 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = f32x16{};

  auto head_of = [&](int gi) {
    return gi < u.sig_g ? u.kvh + a.n_kv * gi : a.n_signal + u.kvh + a.n_kv * (gi - u.sig_g);
  };
  const int n_g = a.n_heads / a.n_kv, qlast = u.qb0 + u.nqb - 1;
  const int64_t ldt = (int64_t)a.B * a.Tp, bT = (int64_t)u.b * a.T, bTp = (int64_t)u.b * a.Tp, M = (int64_t)a.B * a.T;
  const uint32_t ring = lds_u32(SM) + (PW ? 0u : 3u * RING_SLOT);
  // Staging loads: instruction i fills chunk c = kb + 4 i of the role's slot (wave-uniform region);
  // lane l takes unit 64 c + l of it.  Most are a wave-uniform base (head, query block) plus the
  // lane's byte offset, fixed for every step but a sequence's last block, whose rows past the last
  // token read the last token's row instead (finite, never visible).  (The offsets stay below
  // 2^32: the fused path takes at most 2^23 padded tokens.)  The chunk that mixes the last rows
  // with the statistics takes full per-lane addresses.  Padding units copy a unit of the step.
  const uint32_t rowq = (uint32_t)a.n_heads * DQK * 2, rowh = (uint32_t)a.n_heads * DH * 2, ldtb = (uint32_t)(ldt * 2);
  auto lane_off = [&](int c, int rmax) -> uint32_t {
    if (PW && c < 13) {
      const int s = 64 * c + lane;
      return (uint32_t)min(s / 25, rmax) * rowq + 16u * (uint32_t)min(s % 25, 23);
    }
    if (PW) {
      const int s = 64 * (min(c, 22) - 13) + lane;
      return (uint32_t)(s / 5) * ldtb + 16u * (uint32_t)min(s % 5, 3);
    }
    if (c < 9) {
      const int s = 64 * c + lane;
      return (uint32_t)min(s / 17, rmax) * rowh + 16u * (uint32_t)min(s % 17, 15);
    }
    const int s = 64 * (c - 9) + lane;
    return (uint32_t)(s / 5) * ldtb + 16u * (uint32_t)min(s % 5, 3);
  };
  uint32_t off[KV_DMA];
#pragma unroll
  for (int i = 0; i < KV_DMA; ++i) off[i] = lane_off(kb + 4 * i, QS - 1);
  auto issue = [&](int st) {  // step st into slot st % 3
    const int h = head_of(st % n_g), qbase = QS * (qlast - st / n_g);
    const uint32_t slot = ring + (uint32_t)((st % 3) * RING_SLOT);
    const int rmax = min(QS - 1, a.T - 1 - qbase);
#pragma unroll
    for (int i = 0; i < KV_DMA; ++i) {
      const int c = kb + 4 * i;
      const uint32_t lds = __builtin_amdgcn_readfirstlane(slot + (uint32_t)(c * 64 * 16));
      if (c == (PW ? 12 : 8)) {  // last rows, then the statistics (their arrays carry 32 entries of padding)
        const int s = 64 * c + lane;
        const void *src;
        if (PW && s < P_ST) {
          src = a.q + ((bT + qbase + min(s / 25, rmax)) * a.n_heads + h) * DQK + 8 * min(s % 25, 23);
        } else if (!PW && s < S_ST) {
          src = a.dh + ((bT + qbase + min(s / 17, rmax)) * a.n_heads + h) * DH + 8 * min(s % 17, 15);
        } else {
          const int e = min(s - (PW ? P_ST : S_ST), PW ? 15 : 7);  // lse 0..7, lowest keys 8..15; row sums 0..7
          src = PW ? (e < 8 ? (const void *)(a.lse + h * M + bT + qbase + 4 * e) : (const void *)(a.lo + bT + qbase + 4 * (e - 8)))
                   : (const void *)(a.drow + h * M + bT + qbase + 4 * e);
        }
        dma16v(src, lds);
        continue;
      }
      const f16_t *base;
      if (PW && c < 13) base = a.q + ((bT + qbase) * a.n_heads + h) * DQK;
      else if (PW) base = a.dhT + (int64_t)h * DH * ldt + bTp + qbase;
      else if (c < 9) base = a.dh + ((bT + qbase) * a.n_heads + h) * DH;
      else base = a.qT + (int64_t)h * DQK * ldt + bTp + qbase;
      dma16s(base, rmax < QS - 1 ? lane_off(c, rmax) : off[i], lds);
    }
  };

  // P waves: step j in iteration j (two steps in flight); dS waves: step j - 1 (issued one
  // iteration later, also two in flight).  One more iteration than steps.
  const int lag = PW ? 0 : 1;
  for (int st = 0; st < 2 - lag && st < u.n_it; ++st) issue(st);
  for (int j = 0; j <= u.n_it; ++j) {
    const int st = j - lag;  // this wave's step
    // at most this wave's loads of step st + 1 still in flight
    if (st + 1 < u.n_it) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KV_DMA) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // steps j and j - 1 have landed for every wave; every wave is done with their previous steps
    __syncthreads();
    if (st + 2 < u.n_it) issue(st + 2);
    if (st < 0 || st >= u.n_it) continue;
    const int qbase = QS * (qlast - st / n_g);
    const char *base = SM + (PW ? 0 : 3 * RING_SLOT) + (st % 3) * RING_SLOT;
    // query-major product over the dims (S or dP): row m = query R(m), column = this lane's key.
    // The 16 values of a lane are queries qbase + 16 kk + 8 h2 + i at index 8 kk + i.
    const f16_t *rows = (const f16_t *)base + rq * (PW ? KP : VP) + 8 * h2;
    // (at most 8 fragments in registers: the P wave reads its last four after the first products)
    f16x8 A[NF];
#pragma unroll
    for (int k = 0; k < 8; ++k) A[k] = *(const f16x8 *)(rows + 16 * k);
    f32x16 X = {};
#pragma unroll
    for (int k = 0; k < NF - 4; ++k) X = mfma(A[k], F[k], X);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 8; k < NF; ++k) A[k] = *(const f16x8 *)(rows + 16 * k);
#pragma unroll
    for (int k = NF - 4; k < NF; ++k) X = mfma(A[k], F[k], X);
    __builtin_amdgcn_sched_barrier(0);  // the second product's fragments stay below (registers)
    f16x8 pf[2];
    const float *stt = (const float *)(base + 16 * (PW ? P_ST : S_ST));
    if constexpr (PW) {
      const int *los = (const int *)(stt + QS);
      // every pair of the step visible (wave-uniform): all queries at or after the wave's last key
      // and inside the sequence, and the last query's lowest visible key (lowest keys never
      // decrease) at or before the wave's first key
      const int kfirst = u.kb0 + 32 * kb;
      const bool full = qbase >= kfirst + 31 && qbase + QS <= a.T &&
                        __builtin_amdgcn_readfirstlane(los[QS - 1]) <= kfirst;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int q8 = 16 * kk + 8 * h2;
        const float4 l0 = *(const float4 *)(stt + q8), l1 = *(const float4 *)(stt + q8 + 4);
        const float lse8[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        if (full) {
#pragma unroll
          for (int i = 0; i < 8; ++i) pf[kk][i] = h16(__builtin_amdgcn_exp2f(X[8 * kk + i] * a.c - lse8[i]));
        } else {
          const int4 o0 = *(const int4 *)(los + q8), o1 = *(const int4 *)(los + q8 + 4);
          const int lo8[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int t = qbase + q8 + i;
            const bool vis = key <= t && t < a.T && key >= lo8[i];
            pf[kk][i] = h16(vis ? __builtin_amdgcn_exp2f(X[8 * kk + i] * a.c - lse8[i]) : 0.f);
          }
        }
        PX[st & 1][kb][kk][lane] = pf[kk];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int q8 = 16 * kk + 8 * h2;
        const float4 d0 = *(const float4 *)(stt + q8), d1 = *(const float4 *)(stt + q8 + 4);
        const float dr8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        const f16x8 p8 = PX[st & 1][kb][kk][lane];  // written by this SIMD's P wave last iteration
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = (float)p8[i];
          pf[kk][i] = h16(p != 0.f ? p * (X[8 * kk + i] - dr8[i]) : 0.f);  // dS
        }
      }
    }
    // the product over the queries (dV or dK): dim-major A fragments, row = dim 32 blk + l % 32,
    // queries 16 kk + 8 h2 ..
    const f16_t *cols = (const f16_t *)(base + 16 * (PW ? P_HT : S_QT)) + (lane & 31) * TP + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int blk = 0; blk < NACC; ++blk) acc[blk] = mfma(*(const f16x8 *)(cols + 32 * blk * TP + 16 * kk), pf[kk], acc[blk]);
  }
  if (key >= a.T) return;
  // acc[blk][j] = (dK^T or dV^T)[dim 32 blk + 8 (j / 4) + 4 (l / 32) + j % 4][key]
  const int64_t ko = ((int64_t)u.b * a.n_kv + u.kvh) * a.T + key;
  const float sc = PW ? 1.f : a.tau;
  float *o = PW ? a.dv + ko * DH : a.dk + ko * DQK;
#pragma unroll
  for (int blk = 0; blk < NACC; ++blk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(float4 *)(o + 32 * blk + 8 * i + 4 * h2) =
          make_float4(acc[blk][4 * i] * sc, acc[blk][4 * i + 1] * sc, acc[blk][4 * i + 2] * sc, acc[blk][4 * i + 3] * sc);
}

__global__ void __launch_bounds__(512, 1) bwd_dkv_kernel(BwdAttnArgs a) {
  __shared__ __attribute__((aligned(16))) char SM[KV_LDS];
  __shared__ __attribute__((aligned(16))) f16x8 PX[2][4][2][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int per_k = a.n_kv * a.B;
  DkvUnit u;
  const int kblk = (int)blockIdx.x / per_k;  // longest work (first keys) first
  u.kvh = (int)blockIdx.x % per_k % a.n_kv;
  u.b = (int)blockIdx.x % per_k / a.n_kv;
  u.kb0 = 128 * kblk;
  // queries kb0 .. lo_q - 1 can see a key of the block: lowest visible keys never decrease
  int lo_q = u.kb0, hi_q = a.T;
  while (lo_q < hi_q) {
    const int mid = (lo_q + hi_q) >> 1;
    if (qlo(a, u.b, mid) > u.kb0 + 127) hi_q = mid;
    else lo_q = mid + 1;
  }
  u.qb0 = u.kb0 / QS;
  u.nqb = max(0, (lo_q - u.kb0 + QS - 1) / QS);
  u.sig_g = a.n_signal / a.n_kv;
  u.n_it = (a.n_heads / a.n_kv) * u.nqb;
  if (wave < 4) dkv_body<true>(a, u, SM, PX, wave, lane);  // wave-uniform: each wave runs its role
  else dkv_body<false>(a, u, SM, PX, wave, lane);
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
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)(nk * a.n_kv * a.B)), dim3(512), 0, s, a);  // 128-key blocks
  return hipGetLastError();
}

}  // namespace gdla
