// Absorbed-weight GDLA decode for gfx950 (d_kv_latent 512, d_rope 64): split-L attention of every
// query head directly over the bf16 latent cache, then the LSE merge of the splits.
//
// The MLA property the Motif 3 Technical Report relies on (paperglide reader, section "Model
// Architecture", MLA answer; picx.dev summary section 2.2, Eq.(5)) is that only the latent is
// cached and K/V are rebuilt inside attention.  With q~_h = [q^C_h W_uk[:, kv(h)]^T ; q^R_h]:
//     score_s = tau q~_h . cache_s,    o_h = sum_s softmax(score)_s cbar_s,    H_h = o_h W_uv[:, kv(h)]
// which is exactly the expanded form, re-associated.  Every cached row is read once per sequence
// and serves all query heads.
//
// Kernel layout: one workgroup per (sequence, key split), one wave per SIMD.  Query heads come in
// blocks of 16 (the N side of v_mfma_f32_16x16x32_bf16).
//   Scores: wave w computes the scores of block w and, when there are five blocks (65..80 heads),
//   also those of block 4 (every wave, from the fragments it already reads), so q~ of two blocks
//   (2 x 72 registers) stays in registers.
//   Values: wave w accumulates output dims 128 w .. 128 w + 127 of every head block (160 registers),
//   so each wave transposes only its quarter of the tile (the transposing LDS reads are about 3x
//   slower per byte than plain ones).  The probabilities of blocks 0..3 go through a 4 KB LDS
//   buffer; block 4's are identical in every wave.
// Cache tiles of 32 rows (576 bf16 = 72 chunks of 16 bytes each) stream through a 4-slot LDS ring
// by direct global -> LDS 16-byte loads; every tile serves all heads.  Per tile and wave:
//   S^T[key, head] = cache[key, 0:576] . q~[head, 0:576]   (A = cache rows, B = q~ from registers)
//   softmax against a fixed reference (see SoftmaxState), P^T -> LDS, barrier,
//   O^T[dim, head] += cbar^T[dim, key] . P^T[key, head]    (A = cbar^T by ds_read_b64_tr_b16,
//                                                           B = P^T of each head block)
// Rows are unpadded; chunk c of row r sits at c ^ (r mod 8).  With it the hardware counter reads no
// LDS bank conflicts for the 16-byte row reads (16 consecutive rows, one chunk) or the transposing
// reads (4 consecutive rows, an aligned pair of chunks).
// Each split writes its unnormalised O, its reference m (log2 units) and sum l; merge_splits
// combines them.
#include "fast_paths.h"

#include <algorithm>

namespace gdla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int DC = 512, DR = 64, ROW = DC + DR;
constexpr int RB = ROW * 2;        // bytes per cache row
constexpr int RCH = ROW / 8;       // 72 chunks per cache row
constexpr int KT = 32;             // keys per tile
constexpr int NBUF = 4;            // LDS ring of tiles: three in flight while one is consumed
constexpr int TILE = KT * ROW;     // elements per tile
constexpr int TILE_CH = KT * RCH;  // chunks per tile (2304 = 36 wave-instructions)
constexpr int NKST = ROW / 32;     // 18 k-steps of 32 in S
constexpr int NDB = DC / 16;       // 32 dim blocks of 16 in O^T
constexpr int MAX_WAVES = 4;      // always launched: one wave per SIMD
constexpr int DMA_PER_WAVE = TILE_CH / 64 / MAX_WAVES;  // 16-byte loads per lane and tile (9)
constexpr int MAX_HEADS = 16 * (MAX_WAVES + 1);
constexpr int WDB = NDB / MAX_WAVES;    // dim blocks of 16 owned by each wave (8)
constexpr int NHB = MAX_WAVES + 1;      // head blocks of 16 (at most)
constexpr int PG_CAP = 1024;            // pages of a split's block-table slice kept in LDS

// Queries are indexed by v = b q_len + i: token i of sequence b, at position pos[b] + i.
struct DecodeArgs {
  const bf16_t *qabs;  // [B q_len, n_H, 576] bf16
  CacheRef cache;      // bf16 rows of 576 (contiguous or paged in pages of a multiple of 32 rows)
  const int32_t *pos;  // [B] position of the first new token (token i sees keys 0 .. pos + i)
  float *part_o;       // [B q_len, splits, n_H, 512]
  float *part_ml;      // [B q_len, splits, n_H, 2]
  int32_t B, q_len, n_heads, window, splits;
  float c;             // softmax scale * log2(e)
};

// Workgroup -> (sequence b, token i, split sp).  The units u = b splits + sp come in groups of 8,
// one per XCD (the XCDs take workgroups round-robin); within a group the q_len tokens of a unit are
// 8 workgroups apart, so they run on the same XCD at the same time and read the unit's cache tiles
// once from HBM and then from that XCD's L2.  Returns false for the padding of the last group.
__device__ __forceinline__ bool decode_unit(const DecodeArgs &a, int &b, int &tok, int &sp) {
  const int id = blockIdx.x, q = a.q_len;
  const int u = id / (8 * q) * 8 + id % 8;
  tok = id / 8 % q;
  b = u / a.splits;
  sp = u % a.splits;
  return b < a.B;
}

int decode_grid(int B, int q_len, int splits) { return (B * splits + 7) / 8 * 8 * q_len; }

__host__ __device__ constexpr int swz(int r) { return r & 7; }

__device__ __forceinline__ bf16x4 tr_read(const char *p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ _Float16 sat16(float v) { return (_Float16)fminf(fmaxf(v, -65504.f), 65504.f); }
// 8 fp32 -> hi = fp16(v) (saturating), lo = fp16(v - hi): hi + lo carries about 21 bits of v
__device__ __forceinline__ void split16(const float *v, f16x8 &hi, f16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hi[i] = sat16(v[i]);
    lo[i] = (_Float16)(v[i] - (float)hi[i]);
  }
}
// 8 bf16 (16 bytes) -> fp16: exact in the fp16 normal range, saturating beyond it
__device__ __forceinline__ f16x8 bf16_to_f16x8(uint4 w) {
  const unsigned u[4] = {w.x, w.y, w.z, w.w};
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)fminf(fmaxf(__uint_as_float(u[i] << 16), -65504.f), 65504.f);
    r[2 * i + 1] = (_Float16)fminf(fmaxf(__uint_as_float(u[i] & 0xffff0000u), -65504.f), 65504.f);
  }
  return r;
}

__device__ __forceinline__ float head_max(float v) {  // over lanes l, l^16, l^32, l^48
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float head_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// Softmax state of one 16-head block in one wave.  The probabilities of a split are taken against a
// fixed reference mref = 0 (scores in log2 units), so the accumulators are never rescaled and the
// tile loop needs no cross-lane reduction.  A score more than 64 above the reference (overflow
// risk), or a split whose maximum stays more than 64 below it (underflow risk), raises `redo`, and
// the split is then computed again against its exact maximum, so neither can happen.  mrun and l
// are kept per lane (each lane sees a quarter of the keys of its head) and reduced over the 4 lanes
// of a head at the end.
struct SoftmaxState {
  float mref = 0.f, mrun = -INFINITY, l = 0.f;
  bool redo = false;
};

// Scores -> probabilities for one tile (score of key s0 + 16 kb + 4 g + j in S[kb][j]); `lim` =
// k_end - s0 - 4 g masks the keys past the split and, with LOWER (paged cache with a window: the
// first tile, aligned to the pages, may start below it), `llim` = lo - s0 - 4 g those before it.  Returns P^T as the B operand of the 32-key
// step (slot e <-> key 16 (e / 4) + 4 g + e % 4).  Branch-free, so it stays in the MFMA block.
template <bool LOWER>
__device__ __forceinline__ void softmax_tile(f32x4 (&S)[2], SoftmaxState &st, int llim, int lim, float c,
                                             bf16x8 &P) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kidx = 16 * (i >> 2) + (i & 3);
    v[i] = kidx < lim && (!LOWER || kidx >= llim) ? S[i >> 2][i & 3] * c : -INFINITY;
  }
  float mt = v[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, v[i]);
  st.mrun = fmaxf(st.mrun, mt);
  st.redo |= mt - st.mref > 64.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = __builtin_amdgcn_exp2f(v[i] - st.mref);
    st.l += v[i];
    P[i] = (bf16_t)v[i];
  }
}

// 16 bytes global -> LDS (M0 + 16 lane) without the compiler's LDS-DMA tracking: the waits for
// these loads are explicit (s_waitcnt vmcnt before the barrier that publishes a tile).  M0 is set
// right before the load (one wait state between them); nothing else in the kernel uses M0.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Shared head block (heads 64..79): its 36 score MFMAs per tile are split over the waves, wave
// ROLE taking key block ROLE / 2 and k-steps 9 (ROLE % 2) .. + 8 with the fragments it reads for its
// own block anyway; the partial sums meet in LDS and every wave then takes the same softmax of the
// whole block (so its P^T needs no further exchange).
constexpr int K4N = NKST / 2;  // k-steps of the shared block per wave (9)

template <bool SHARED, bool PAGED, bool LOWER, int ROLE>
__device__ __forceinline__ void decode_body(const DecodeArgs &a, bf16_t *CB, bf16x8 (*PB)[64], f32x4 (*S4B)[64],
                                            int32_t *PG, int wave) {
  constexpr int KB4 = ROLE >> 1, K4LO = (ROLE & 1) * K4N;
  const int lane = threadIdx.x & 63;
  int b, tok, sp;
  decode_unit(a, b, tok, sp);
  const int v = b * a.q_len + tok;  // query row set
  const int p = a.pos[b] + tok;
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  // PAGED: tiles start on multiples of KT (so a tile never crosses a page) and the keys below lo
  // of the first tile are masked; contiguous: tiles start at lo
  const int kbase = PAGED ? lo & ~(KT - 1) : lo;
  const int span = p + 1 - kbase;
  const int kps = ((span + a.splits - 1) / a.splits + KT - 1) / KT * KT;  // keys per split
  const int k_begin = kbase + sp * kps, k_end = min(p + 1, k_begin + kps);
  const int ntiles = k_end > k_begin ? (k_end - k_begin + KT - 1) / KT : 0;
  const int col = lane & 15, g = lane >> 4;
  const int head = 16 * wave + col, head4 = 16 * MAX_WAVES + col;
  const bool head_ok = head < a.n_heads, head4_ok = SHARED && head4 < a.n_heads;

  // q~ fragments (B operand): Qf[kst] = dims 32 kst + 8 g .. + 7 of head `head`; Q4[k] those of
  // head `head4` at k-step K4LO + k
  bf16x8 Qf[NKST], Q4[SHARED ? K4N : 1];
  {
    const bf16_t *qb = a.qabs + (int64_t)v * a.n_heads * ROW + 8 * g;
    const bf16_t *qp = qb + (int64_t)(head_ok ? head : 0) * ROW;
#pragma unroll
    for (int k = 0; k < NKST; ++k) {
      Qf[k] = *(const bf16x8 *)(qp + 32 * k);
      if (!head_ok) Qf[k] = bf16x8{};
    }
    if (SHARED) {
      const bf16_t *q4 = qb + (int64_t)(head4_ok ? head4 : 0) * ROW;
#pragma unroll
      for (int k = 0; k < K4N; ++k) {
        Q4[k] = *(const bf16x8 *)(q4 + 32 * (K4LO + k));
        if (!head4_ok) Q4[k] = bf16x8{};
      }
    }
  }

  // PAGED: the physical pages of the split's blocks are copied to LDS once (when there are at
  // most PG_CAP of them), so a tile's page costs an LDS read, not a scalar memory load (whose wait
  // the compiler would merge with the next LDS wait of the tile loop).
  const CacheRef &cr = a.cache;
  const bf16_t *cb = (const bf16_t *)cr.base + (PAGED ? 0 : (int64_t)b * cr.max_len * ROW);
  int blk0 = 0;
  bool pg_lds = false;
  if (PAGED) {
    blk0 = k_begin / cr.page_rows;
    const int nblk = ntiles > 0 ? (k_begin + ntiles * KT - 1) / cr.page_rows - blk0 + 1 : 0;
    pg_lds = nblk > 0 && nblk <= PG_CAP;
    if (pg_lds) {
      const int32_t *bt = cr.block_table + (int64_t)b * cr.max_blocks + blk0;
      for (int i = threadIdx.x; i < nblk; i += 64 * MAX_WAVES) PG[i] = min(max(bt[i], 0), cr.n_pages - 1);
    }
    __syncthreads();
  }
  // first cache row (relative to cb) of the tile at s0; paged, the tiles are visited in order
  // and (blk, off) = (s0 / page_rows, s0 % page_rows) is advanced without a division
  int blk = blk0, off = PAGED ? k_begin - blk0 * cr.page_rows : 0;
  auto tile_row = [&](int s0) -> int64_t {
    if (!PAGED) return s0;
    const int64_t r = pg_lds ? (int64_t)PG[blk - blk0] * cr.page_rows + off : cache_row(cr, b, s0);
    off += KT;
    if (off == cr.page_rows) {
      off = 0;
      ++blk;
    }
    return r;
  };
  // Tile t goes to ring slot t % NBUF; wave w issues wave-instructions w, w + 4, ... of the tile
  // (DMA_PER_WAVE of them).  rowoff[i] is this lane's source offset (bytes) inside the tile.
  // Keys past k_end (and, paged, before lo) are read from row k_end - 1 (lo) instead: masked later,
  // and never a row outside the visible range, which a paged cache may no longer map.
  const uint32_t ring = lds_u32(CB);
  int rowoff[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int sl = (wave + MAX_WAVES * i) * 64 + lane;
    const int row = sl / RCH;
    rowoff[i] = row * RB + (((sl % RCH) ^ swz(row)) * 16);
  }
  // first cache row of the next tile to issue (one block-table lookup ahead when paged)
  int64_t row_next = 0;
  auto issue = [&](int t) {
    const int s0 = k_begin + t * KT;
    const uint32_t base = ring + (uint32_t)((t % NBUF) * TILE * 2) + wave * 1024;
    const char *src = (const char *)(cb + (PAGED ? row_next : (int64_t)s0) * ROW);
    if (PAGED && t + 1 < ntiles) row_next = tile_row(s0 + KT);
    if ((!PAGED || s0 >= lo) && s0 + KT <= k_end) {
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i)
        dma16(src + rowoff[i], __builtin_amdgcn_readfirstlane(base + i * MAX_WAVES * 1024));
    } else {
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int row = rowoff[i] / RB;
        const int off = rowoff[i] - row * RB + (min(PAGED ? max(s0 + row, lo) : s0 + row, k_end - 1) - s0) * RB;
        dma16(src + off, __builtin_amdgcn_readfirstlane(base + i * MAX_WAVES * 1024));
      }
    }
  };

  // O[hb][dd] = O^T[dims 16 (WDB wave + dd) + 4 g + j][heads 16 hb + col]
  constexpr int HB = SHARED ? NHB : MAX_WAVES;
  f32x4 O[HB][WDB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int d = 0; d < WDB; ++d) O[hb][d] = f32x4{};
  SoftmaxState st, st4;
  int pass = 0;

  // Lane-dependent byte offsets of the LDS reads; everything else is an immediate.
  // S phase: row 16 kb + col, logical chunk 4 kst + g; swz(row) = swz(col) for every kb.
  int offS[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) offS[q] = col * RB + (((4 * q + g) ^ swz(col)) * 16);
  // PV phase: lane (g, jj, qq) of a transposing read addresses row 16 hi + 4 g + jj and dims
  // 16 d + 4 qq .. + 3 with d = WDB wave + dd, i.e. logical chunk 16 wave + 2 dd + (qq >> 1), half
  // qq & 1; swz(row) = swz(4 g + jj) and the XOR only touches the low 3 bits of the chunk.
  const int jj = (lane & 15) >> 2, qq = lane & 3;
  int offP[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 4 * g + jj;
    offP[q] = r * RB + wave * (2 * WDB * 16) + (((2 * q + (qq >> 1)) ^ swz(r)) * 16) + (qq & 1) * 8;
  }

  auto compute = [&](const bf16_t *cs, int s0) {
    const char *cbyte = (const char *)cs;
    f32x4 S[2], S4p;
    // S phase, key block by key block, software-pipelined two k-steps ahead:
    // [reads of step n + 2][MFMAs of step n]; the own block and this wave's part of the shared
    // block use the same fragment
    bf16x8 af[3];
    auto ldA = [&](bf16x8 &f, int n) {  // n = 18 kb + kst
      const int kb = n / NKST, kst = n % NKST;
      f = *(const bf16x8 *)(cbyte + offS[kst & 1] + kb * 16 * RB + (kst >> 1) * 128);
    };
    ldA(af[0], 0);
    ldA(af[1], 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int n = 0; n < 2 * NKST; ++n) {
      const int kb = n / NKST, kst = n % NKST;
      if (n + 2 < 2 * NKST) ldA(af[(n + 2) % 3], n + 2);
      const bool part4 = SHARED && kb == KB4 && kst >= K4LO && kst < K4LO + K4N;
      S[kb] = mfma16(af[n % 3], Qf[kst], kst == 0 ? f32x4{} : S[kb]);
      if (part4) S4p = mfma16(af[n % 3], Q4[kst - K4LO], kst == K4LO ? f32x4{} : S4p);
      if (n + 2 < 2 * NKST) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (part4) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    bf16x8 P;
    const int lim = k_end - s0 - 4 * g, llim = lo - s0 - 4 * g;
    softmax_tile<LOWER>(S, st, llim, lim, a.c, P);
    if (SHARED) S4B[wave][lane] = S4p;
    PB[wave][lane] = P;
    __syncthreads();  // P^T of blocks 0..3 and the shared block's partial scores visible to every wave
    bf16x8 PH[HB];
#pragma unroll
    for (int hb = 0; hb < MAX_WAVES; ++hb) PH[hb] = PB[hb][lane];
    if (SHARED) {
      f32x4 S4[2];
      S4[0] = S4B[0][lane] + S4B[1][lane];
      S4[1] = S4B[2][lane] + S4B[3][lane];
      softmax_tile<LOWER>(S4, st4, llim, lim, a.c, PH[HB - 1]);
    }
    // PV phase over this wave's dim blocks, pipelined two ahead: [reads of dd + 2][MFMAs of dd]
    bf16x8 vf[3];
    auto ldV = [&](bf16x8 &f, int dd) {
      const char *p0 = cbyte + offP[dd & 3] + (dd >> 2) * 128;
      const bf16x4 lo4 = tr_read(p0);
      const bf16x4 hi4 = tr_read(p0 + 16 * RB);
      f = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    ldV(vf[0], 0);
    ldV(vf[1], 1);
#pragma unroll
    for (int dd = 0; dd < WDB; ++dd) {
      if (dd + 2 < WDB) ldV(vf[(dd + 2) % 3], dd + 2);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) O[hb][dd] = mfma16(vf[dd % 3], PH[hb], O[hb][dd]);
    }
  };

  // vmcnt(n): at most n of this wave's loads still in flight (n = 0, one tile, two tiles)
  auto wait_tiles_after = [&](int n_after) {
    if (n_after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMA_PER_WAVE) : "memory");
    else if (n_after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_WAVE) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  for (;;) {
    if (PAGED && ntiles > 0) {
      blk = blk0;
      off = k_begin - blk0 * cr.page_rows;
      row_next = tile_row(k_begin);
    }
    for (int t = 0; t < NBUF - 1 && t < ntiles; ++t) issue(t);
    for (int t = 0; t < ntiles; ++t) {
      wait_tiles_after(min(ntiles - 1 - t, NBUF - 2));
      __syncthreads();  // tile t has landed for every wave; every wave is done with tile t - 1
      if (t + NBUF - 1 < ntiles) issue(t + NBUF - 1);
      compute(CB + (t % NBUF) * TILE, k_begin + t * KT);
    }
    __syncthreads();
    // reduce the per-lane maxima over the 4 lanes of each head; check for underflow
    st.mrun = head_max(st.mrun);
    st.redo |= ntiles > 0 && st.mrun - st.mref < -64.0f;
    if (SHARED) {
      st4.mrun = head_max(st4.mrun);
      st4.redo |= ntiles > 0 && st4.mrun - st4.mref < -64.0f;
    }
    if (pass == 1 || !__syncthreads_or(st.redo || st4.redo)) break;
    // second pass against the exact maximum
    pass = 1;
    st.mref = st.mrun;
    st.l = 0.f;
    st4.mref = st4.mrun;
    st4.l = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int d = 0; d < WDB; ++d) O[hb][d] = f32x4{};
  }

  // (m, l) of head block hb come from the wave that owns its scores (wave 0 for block 4)
  const float lt = head_sum(st.l);
  if (head_ok && g == 0) {
    const int64_t ph = ((int64_t)v * a.splits + sp) * a.n_heads + head;
    a.part_ml[ph * 2] = ntiles > 0 ? st.mref : -INFINITY;
    a.part_ml[ph * 2 + 1] = lt;
  }
  if (SHARED) {
    const float lt4 = head_sum(st4.l);
    if (head4_ok && wave == 0 && g == 0) {
      const int64_t ph = ((int64_t)v * a.splits + sp) * a.n_heads + head4;
      a.part_ml[ph * 2] = ntiles > 0 ? st4.mref : -INFINITY;
      a.part_ml[ph * 2 + 1] = lt4;
    }
  }
  // this wave's dims of every head: O[hb][dd][j] = O^T[dim 16 (WDB wave + dd) + 4 g + j][16 hb + col]
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int h = 16 * hb + col;
    if (h >= a.n_heads) continue;
    float *po = a.part_o + (((int64_t)v * a.splits + sp) * a.n_heads + h) * DC + 16 * WDB * wave + 4 * g;
#pragma unroll
    for (int dd = 0; dd < WDB; ++dd)
      *(float4 *)(po + 16 * dd) = make_float4(O[hb][dd][0], O[hb][dd][1], O[hb][dd][2], O[hb][dd][3]);
  }
}

// PAGED: paged cache; LOWER: with a window (paged tiles may then start below it)
template <bool SHARED, bool PAGED, bool LOWER>
__global__ void __launch_bounds__(256, 1) latent_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t CB[NBUF * TILE];
  __shared__ __attribute__((aligned(16))) bf16x8 PB[MAX_WAVES][64];   // P^T of head blocks 0..3
  __shared__ __attribute__((aligned(16))) f32x4 S4B[MAX_WAVES][64];   // partial scores, shared block
  __shared__ int32_t PG[PAGED ? PG_CAP : 1];                           // physical pages of the split
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    int b, tok, sp;
    if (!decode_unit(a, b, tok, sp)) return;  // uniform over the workgroup, before any barrier
  }
  if (!SHARED) {
    decode_body<false, PAGED, LOWER, 0>(a, CB, PB, S4B, PG, wave);
  } else {
    switch (wave) {  // wave-uniform: each wave runs the code of its part of the shared block
      case 0: decode_body<true, PAGED, LOWER, 0>(a, CB, PB, S4B, PG, 0); break;
      case 1: decode_body<true, PAGED, LOWER, 1>(a, CB, PB, S4B, PG, 1); break;
      case 2: decode_body<true, PAGED, LOWER, 2>(a, CB, PB, S4B, PG, 2); break;
      default: decode_body<true, PAGED, LOWER, 3>(a, CB, PB, S4B, PG, 3); break;
    }
  }
}

// o[b, h] = sum_sp 2^(m_sp - M) o_sp / sum_sp 2^(m_sp - M) l_sp, M = max_sp m_sp (each split's
// reference in log2 units; -inf marks an empty split).
__global__ void __launch_bounds__(128) merge_splits_kernel(const float *part_o, const float *part_ml, float *o,
                                                         int32_t n_heads, int32_t splits) {
  const int bh = blockIdx.x;  // b * n_heads + h
  const int b = bh / n_heads, h = bh % n_heads;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[(((int64_t)b * splits + s) * n_heads + h) * 2]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < splits; ++s) {
    const int64_t ph = ((int64_t)b * splits + s) * n_heads + h;
    const float ms = part_ml[ph * 2];
    if (ms == -INFINITY) continue;  // empty split
    const float w = __builtin_amdgcn_exp2f(ms - M);
    L += w * part_ml[ph * 2 + 1];
    const float4 v = *(const float4 *)(part_o + ph * DC + 4 * threadIdx.x);
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  const float inv = 1.0f / L;
  *(float4 *)(o + (int64_t)bh * DC + 4 * threadIdx.x) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// Query rows that share one KV head.  Block (i, kv) takes rows i R .. i R + R - 1 of the list
// (b, k) -> b * hk + k over sequences b and the hk heads k of kv (signal heads first).
constexpr int R = 16;

__device__ __forceinline__ int kv_heads(int kv, const LayerDims &d, int &ns) {
  ns = kv < d.n_signal ? (d.n_signal - kv + d.n_kv - 1) / d.n_kv : 0;
  const int nn = kv < d.n_noise ? (d.n_noise - kv + d.n_kv - 1) / d.n_kv : 0;
  return ns + nn;
}
__device__ __forceinline__ int kv_head(int kv, int k, int ns, const LayerDims &d) {
  return k < ns ? kv + d.n_kv * k : d.n_signal + kv + d.n_kv * (k - ns);
}

// q~ = [q^C_h W_uk[:, kv(h)]^T ; q^R_h] in bf16.  Each thread keeps one W_uk row slice (d_h values
// of latent dimension c) in registers and applies it to the block's R query rows.
__global__ void __launch_bounds__(256) absorb_kernel(const float *qc, const float *qr, const bf16_t *w_uk,
                                                     bf16_t *qabs, int32_t B, LayerDims d) {
  __shared__ __attribute__((aligned(16))) float qs[R][128];
  __shared__ int64_t rowq[R];
  const int kv = blockIdx.y, tid = threadIdx.x;
  int ns;
  const int hk = kv_heads(kv, d, ns);
  const int r0 = blockIdx.x * R, nr = min(R, B * hk - r0);
  if (nr <= 0) return;
  if (tid < nr) {
    const int L = r0 + tid, b = L / hk;
    rowq[tid] = (int64_t)b * d.n_heads + kv_head(kv, L % hk, ns, d);
  }
  __syncthreads();
  for (int i = tid; i < nr * 32; i += 256) {
    const int r = i >> 5, e = (i & 31) * 4;
    *(float4 *)&qs[r][e] = *(const float4 *)(qc + rowq[r] * 128 + e);
  }
  for (int i = tid; i < nr * DR; i += 256) {
    const int r = i / DR, e = i % DR;
    qabs[rowq[r] * ROW + DC + e] = (bf16_t)qr[rowq[r] * DR + e];
  }
  for (int i = nr * 32 + tid; i < R * 32; i += 256) {  // rows past the list: zeros
    const int r = i >> 5, e = (i & 31) * 4;
    *(float4 *)&qs[r][e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  // q~[r][c] = sum_e q^C[r][e] W_uk[c][128 kv + e] on v_mfma_f32_16x16x32_f16 (A[m = r][k = e],
  // B[k = e][n = c], acc[j] = C[4 (l / 16) + j][l % 16]); wave w takes c = 128 w .. 128 w + 127
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  const int64_t ldw = (int64_t)d.n_kv * 128;
  // q^C as the sum of two fp16 parts (hi + lo carry about 21 bits), so the product keeps the
  // fp32 query's precision; the weights are exact in fp16
  f16x8 qa[4], ql[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) split16(&qs[l16][32 * k + 8 * g], qa[k], ql[k]);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int c = 128 * wave + 16 * nb + l16;
    const bf16_t *wr = w_uk + (int64_t)c * ldw + kv * 128 + 8 * g;
    f32x4 acc = {};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x8 wb = bf16_to_f16x8(*(const uint4 *)(wr + 32 * k));
      acc = mfma16h(qa[k], wb, acc);
      acc = mfma16h(ql[k], wb, acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * g + j;
      if (r < nr) qabs[rowq[r] * ROW + c] = (bf16_t)acc[j];
    }
  }
}

// H_h = o_h W_uv[:, kv(h)] in fp32, for the block's R rows.  Thread (half, e) sums latent
// dimensions half * 256 .. + 255 for output column e; the two halves are added through LDS.
__global__ void __launch_bounds__(256) unabsorb_kernel(const float *o, const f16_t *wuvt, float *heads,
                                                       int32_t B, LayerDims d) {
  __shared__ __attribute__((aligned(16))) float os[R][DC];
  __shared__ int64_t rowq[R];
  const int kv = blockIdx.y, tid = threadIdx.x;
  int ns;
  const int hk = kv_heads(kv, d, ns);
  const int r0 = blockIdx.x * R, nr = min(R, B * hk - r0);
  if (nr <= 0) return;
  if (tid < nr) {
    const int L = r0 + tid, b = L / hk;
    rowq[tid] = (int64_t)b * d.n_heads + kv_head(kv, L % hk, ns, d);
  }
  __syncthreads();
  for (int i = tid; i < nr * (DC / 4); i += 256) {
    const int r = i / (DC / 4), c = (i % (DC / 4)) * 4;
    *(float4 *)&os[r][c] = *(const float4 *)(o + rowq[r] * DC + c);
  }
  for (int i = nr * (DC / 4) + tid; i < R * (DC / 4); i += 256) {
    const int r = i / (DC / 4), c = (i % (DC / 4)) * 4;
    *(float4 *)&os[r][c] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  // H[r][e] = sum_c o[r][c] W_uv[c][128 kv + e] on v_mfma_f32_16x16x32_f16 (A[m = r][k = c],
  // B[k = c][n = e]); wave w takes e = 32 w .. 32 w + 31 (two blocks of 16), K = 512 in 16 steps
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g = lane >> 4;
  f32x4 acc[2] = {};
#pragma unroll 4
  for (int k = 0; k < DC / 32; ++k) {
    const int c0 = 32 * k + 8 * g;
    f16x8 oa, ol;  // o as hi + lo fp16 parts
    split16(&os[l16][c0], oa, ol);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      // W_uv^T row 128 kv + e, latent dims c0 .. c0 + 7
      const f16x8 wb = *(const f16x8 *)(wuvt + (int64_t)(kv * 128 + 32 * wave + 16 * nb + l16) * DC + c0);
      acc[nb] = mfma16h(oa, wb, acc[nb]);
      acc[nb] = mfma16h(ol, wb, acc[nb]);
    }
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * g + j;
      if (r < nr) heads[rowq[r] * 128 + 32 * wave + 16 * nb + l16] = acc[nb][j];
    }
}

}  // namespace

bool fast_decode_supported(const LayerDims &d, gdla_dtype dt) {
  return dt == GDLA_BF16 && d.d_c == DC && d.d_r == DR && d.d_h == 128 && d.n_heads <= MAX_HEADS;
}

int32_t fast_decode_splits(int32_t B, int32_t max_len) {
  // about one workgroup per CU (256 CUs), at least 1024 keys per split
  const int32_t by_cu = (256 + B - 1) / B;
  const int32_t by_len = std::max(1, max_len / 1024);
  return std::max(1, std::min(by_cu, by_len));
}

gdla_status run_fast_decode(const LayerDims &d, const gdla_weights *w, int32_t B, int32_t T,
                            const int32_t *pos_dev, const CacheRef &cache, const float *qc,
                            const float *qr, float *heads, const FastDecodeLayout &L, void *ws, hipStream_t s,
                            StageEvents &se) {
  const int32_t BT = B * T;  // query rows sets: token i of sequence b is row set b T + i
  bf16_t *qabs = (bf16_t *)((char *)ws + L.qabs);
  float *part_o = (float *)((char *)ws + L.part_o);
  float *part_ml = (float *)((char *)ws + L.part_ml);
  float *o = (float *)((char *)ws + L.o);
  const int hk_max = (d.n_signal + d.n_kv - 1) / d.n_kv + (d.n_noise + d.n_kv - 1) / d.n_kv;
  const dim3 gk((unsigned)((BT * hk_max + R - 1) / R), (unsigned)d.n_kv);
  hipLaunchKernelGGL(absorb_kernel, gk, dim3(256), 0, s, qc, qr, (const bf16_t *)w->w_uk, qabs, BT, d);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_PROJ_Q);
  DecodeArgs a{};
  a.qabs = qabs; a.cache = cache; a.pos = pos_dev; a.part_o = part_o; a.part_ml = part_ml;
  const int nblk = (d.n_heads + 15) / 16;
  a.B = B; a.q_len = T;
  a.n_heads = d.n_heads; a.window = d.window; a.splits = L.splits;
  a.c = d.scale * 1.4426950408889634f;
  se.begin(GDLA_STAGE_ATTN_NOISE);
  const dim3 grid((unsigned)decode_grid(B, T, L.splits));
  const bool shared = nblk > MAX_WAVES, paged = cache.page_rows > 0, lower = paged && d.window > 0;
  const dim3 block(64 * MAX_WAVES);
  if (shared && lower) hipLaunchKernelGGL((latent_decode_kernel<true, true, true>), grid, block, 0, s, a);
  else if (shared && paged) hipLaunchKernelGGL((latent_decode_kernel<true, true, false>), grid, block, 0, s, a);
  else if (shared) hipLaunchKernelGGL((latent_decode_kernel<true, false, false>), grid, block, 0, s, a);
  else if (lower) hipLaunchKernelGGL((latent_decode_kernel<false, true, true>), grid, block, 0, s, a);
  else if (paged) hipLaunchKernelGGL((latent_decode_kernel<false, true, false>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((latent_decode_kernel<false, false, false>), grid, block, 0, s, a);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  se.end(GDLA_STAGE_ATTN_NOISE);
  se.begin(GDLA_STAGE_ATTN_SIGNAL);
  hipLaunchKernelGGL(merge_splits_kernel, dim3(BT * d.n_heads), dim3(128), 0, s, part_o, part_ml, o, d.n_heads,
                     L.splits);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  f16_t *wuvt = (f16_t *)((char *)ws + L.wuvt);
  if (launch_transpose_weight(w->w_uv, wuvt, DC, d.n_kv * 128, true, s) != hipSuccess) return GDLA_ERR_HIP;
  hipLaunchKernelGGL(unabsorb_kernel, gk, dim3(256), 0, s, o, (const f16_t *)wuvt, heads, BT, d);
  if (hipGetLastError() != hipSuccess) return GDLA_ERR_HIP;
  return GDLA_OK;
}

}  // namespace gdla
