// Large GEMM for the prefill projections on gfx950: C = A[M, K] . Bt[N, K]^T, both operands
// K-contiguous (the weights arrive transposed, see transpose_weights below), fp16 x fp16 or
// bf16 x bf16, fp32 accumulation, the epilogue options of GemmProblem.
//
// Used for the projections of the GDLA layer (Motif 3 Technical Report, picx.dev summary, section
// 2.2: Eq.(1), (3), (7) input projections, Eq.(2), (9) query / gate projections, Eq.(5) expansion,
// Eq.(10) output projection) when the problem is large enough to fill the chip.
//
// Block tile 256 x 256, K slices of 64 staged in LDS by direct global -> LDS 16-byte loads (two
// stages of 64 KB; one in flight while the other is consumed).  8 waves in a 2 x 4 grid, each
// computing 128 x 64 as 8 x 4 v_mfma_f32_16x16x32 blocks (at the chip's power limit the 16 x 16
// blocks sustain a higher rate than 32 x 32 ones for the same operand traffic: the wave tile, not
// the block shape, sets the LDS reads per flop).  Both operands are read from LDS with 16-byte
// reads (8 consecutive k of one row): with K-contiguous operands no transposing read is needed,
// and the XOR swizzle (chunk c of row r at c ^ ((r >> 1) & 7)) keeps 16 consecutive rows reading
// one chunk on distinct banks.  Tiles are spread so that each XCD gets a contiguous range, and
// ordered in groups of row tiles within it.
#include "fast_paths.h"

#include <type_traits>

namespace gdla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int ROWB = BK * 2;                  // bytes per staged row (128 = 8 chunks)
constexpr int A_BYTES = BM * ROWB;            // 32 KB
constexpr int STAGE_BYTES = (BM + BN) * ROWB; // 64 KB
constexpr int WAVES = 8;
constexpr int GROUP_M = 4;                    // row tiles per group of the tile order
constexpr int DMA_PER_WAVE = STAGE_BYTES / 1024 / WAVES;  // 16-byte loads per lane per stage (8)

template <typename T> struct V8;
template <> struct V8<bf16_t> { typedef bf16x8 t; };
template <> struct V8<f16_t> { typedef f16x8 t; };

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16 bytes global -> LDS (M0 + 16 lane) outside the compiler's LDS-DMA tracking; the wait is the
// explicit s_waitcnt vmcnt(0) before the barrier that publishes a stage.  M0 is set right before
// the load (one wait state between them); nothing else in the kernel uses M0.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds_addr)
               : "memory");
}

__device__ __forceinline__ int remap_xcd(int bid, int total) {
  if (total < 8) return bid;
  const int q = total / 8, r = total % 8, x = bid % 8, i = bid / 8;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// The wave tile is held as 8 x 4 blocks of 16 x 16:
// acc[mb][nb][i] = C[r0 + 16 mb + 4 (lane / 16) + i][c0 + 16 nb + lane % 16].

// Transposed per-head store of the wave's 128 x 64 block of the value expansion (V^T, keys in
// vt_slot order), 4 consecutive keys per 8-byte store; E is the 16-bit output type.
template <typename E>
__device__ __forceinline__ void trans_store(const GemmProblem &P, const f32x4 (&acc)[8][4], int r0, int c0, int lane) {
  typedef E e4 __attribute__((ext_vector_type(4)));
  const int c16 = lane & 15, q4 = lane >> 4;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = c0 + nb * 16 + c16;
    if (n >= P.N) continue;
    E *base = (E *)P.C + (int64_t)(n / P.hw) * P.hs + P.ho + (int64_t)(n % P.hw) * P.ldc;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int m = r0 + mb * 16 + 4 * q4;
      if (m >= P.M) continue;
      e4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (E)(acc[mb][nb][e]);
      if (m + 3 < P.M) {
        *(e4 *)(base + vt_slot(m)) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (m + e < P.M) base[vt_slot(m + e)] = v[e];
      }
    }
  }
}

// Epilogue through LDS: the wave stages 32 rows x its 64 columns at a time (after the epilogue
// function, in the output type: KIND 0 fp32, 1 fp16, 2 bf16) in its own area `wt` and writes them
// back as 16-byte row segments, which lie inside one head since head widths are multiples of 8.
// Staged rows are padded so that the rows a staging store touches fall on other banks.
template <int KIND>
__device__ __forceinline__ void staged_epilogue(const GemmProblem &P, const f32x4 (&acc)[8][4], unsigned char *wt,
                                                  int r0, int c0, int lane) {
  constexpr int ESZ = KIND == 0 ? 4 : 2, EPS = 16 / ESZ, SPR = 64 / EPS;
  constexpr int PITCH = KIND == 0 ? 272 : 144;
  const int c16 = lane & 15, q4 = lane >> 4;
  // RoPE: column j of the wave's head (j < 32) pairs with column j + 32; this lane holds the pairs
  // j = c16 and j = 16 + c16 (blocks nb and nb + 2), rotated by p * rope_theta^(-2 j / 64)
  double rev[2] = {0.0, 0.0};
  if (P.epi == EPI_ROPE) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      rev[nb] = pow((double)P.rope_theta, -2.0 * (double)(16 * nb + c16) / (double)P.rope_d) * 0.15915494309189533577;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // rows 32 q .. 32 q + 31 of the wave tile: blocks mb = 2 q, 2 q + 1
    const int mrow0 = r0 + q * 32;
    float v[2][4][4];  // [mb - 2 q][nb][i]
    if (KIND != 0 && P.epi == EPI_ROPE) {
      // row m is token m % T of sequence m / T; 32 rows span at most two sequences (T >= 32)
      const int sb = min(mrow0, P.M - 1) / P.rope_T;
      const int sb_end = (sb + 1) * P.rope_T;
      const int pos0 = P.rope_pos[sb], pos1 = sb_end < P.M ? P.rope_pos[sb + 1] : 0;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = min(mrow0 + 16 * h2 + 4 * q4 + i, P.M - 1);
          const int pp = m < sb_end ? pos0 + (m - sb * P.rope_T) : pos1 + (m - sb_end);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            double turns = (double)pp * rev[nb];
            turns -= floor(turns);  // angle / 2 pi, reduced to [0, 1)
            const float sn = __builtin_amdgcn_sinf((float)turns), cs = __builtin_amdgcn_cosf((float)turns);
            const float u = acc[2 * q + h2][nb][i], w = acc[2 * q + h2][nb + 2][i];
            v[h2][nb][i] = u * cs - w * sn;
            v[h2][nb + 2][i] = u * sn + w * cs;
          }
        }
    } else if (P.epi == EPI_SIGMOID) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[h2][nb][i] = __builtin_amdgcn_rcpf(1.0f + __expf(-acc[2 * q + h2][nb][i]));
    } else {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[h2][nb][i] = acc[2 * q + h2][nb][i];
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned char *a = wt + (16 * h2 + 4 * q4 + i) * PITCH + (16 * nb + c16) * ESZ;
          if constexpr (KIND == 0) *(float *)a = v[h2][nb][i];
          else if constexpr (KIND == 1) *(f16_t *)a = (f16_t)(v[h2][nb][i]);
          else *(bf16_t *)a = (bf16_t)v[h2][nb][i];
        }
    // 32 rows x SPR segments, 64 per instruction
#pragma unroll
    for (int it = 0; it < 32 * SPR / 64; ++it) {
      const int seg = it * 64 + lane;
      const int row = seg / SPR, cs = seg % SPR;
      const int m = mrow0 + row, n = c0 + cs * EPS;
      const uint4 val = *(const uint4 *)(wt + row * PITCH + cs * 16);
      if (m < P.M && n < P.N) {
        const int64_t o = (int64_t)m * P.ldc + (int64_t)(n / P.hw) * P.hs + P.ho + (n % P.hw);
        *(uint4 *)((unsigned char *)P.C + o * ESZ) = val;
      }
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(512, 1) gemm_nt_kernel(GemmBatch batch) {
  typedef typename V8<T>::t v8;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE_BYTES];

  const int bid = remap_xcd(blockIdx.x, batch.total_tiles);
  int pi = 0;
  while (pi + 1 < batch.n && bid >= batch.p[pi + 1].tile0) ++pi;
  const GemmProblem &P = batch.p[pi];
  int tile = bid - P.tile0, kc = 0;
  if (P.ksplit > 1) {  // slice kc of K; the tiles of one slice are consecutive
    const int per_slice = ((P.M + BM - 1) / BM) * P.tiles_n;
    kc = tile / per_slice;
    tile -= kc * per_slice;
  }
  const int kbeg = P.ksplit > 1 ? kc * (P.K / P.ksplit) : 0;
  // Grouped order: each run of GROUP_M row tiles walks the column tiles together, so the tiles an
  // XCD holds at once (consecutive indices) read a few row blocks of A and a few column blocks of
  // Bt instead of one row block and as many column blocks as there are tiles.
  int m0, n0;
  {
    const int tiles_m = (P.M + BM - 1) / BM;
    const int g = tile / (GROUP_M * P.tiles_n), r = tile - g * (GROUP_M * P.tiles_n);
    const int gm = min(GROUP_M, tiles_m - g * GROUP_M);
    m0 = (g * GROUP_M + r % gm) * BM;
    n0 = (r / gm) * BN;
  }
  const T *A = (const T *)P.A;
  const T *Bt = (const T *)P.B;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // wave tile rows 128 wm, cols 64 wn

  // Global source offsets of this lane's DMA_PER_WAVE loads per stage (k0 added per stage): wave
  // instruction j = wave + 8 i covers 64 chunks; j < 32 stage A rows, the rest Bt rows.  Rows
  // past M / N are clamped to the last row (their results are never stored).
  const T *src[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int j = wave + WAVES * i;
    const int jj = j & 31;
    const int sl = jj * 64 + lane;
    const int row = sl >> 3, c = (sl & 7) ^ ((row >> 1) & 7);
    if (j < 32) src[i] = A + (int64_t)min(m0 + row, P.M - 1) * P.lda + kbeg + c * 8;
    else src[i] = Bt + (int64_t)min(n0 + row, P.N - 1) * P.ldb + kbeg + c * 8;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)smem;
  auto issue = [&](int stage, int k0) {
    const uint32_t base = lds0 + stage * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int j = wave + WAVES * i;
      dma16(src[i] + k0, __builtin_amdgcn_readfirstlane(base + j * 1024));
    }
  };

  // Fragment reads: A block mb rows 128 wm + 16 mb + (lane % 16), Bt block nb rows
  // 64 wn + 16 nb + (lane % 16); k-step kk (32 k) reads chunk 4 kk + lane / 16.  The row swizzle
  // depends on lane % 16 only, so the lane part of the offset depends on kk only.
  const int r16 = lane & 15, q4 = lane >> 4;
  int off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) off[kk] = r16 * ROWB + (((4 * kk + q4) ^ ((r16 >> 1) & 7)) * 16);
  const int a_base = wm * 128 * ROWB, b_base = A_BYTES + wn * 64 * ROWB;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};

  auto compute = [&](int stage) {
    const unsigned char *sb = smem + stage * STAGE_BYTES;
    v8 af[2][8], bfr[2][4];
    auto ld = [&](int kk, v8 (&a)[8], v8 (&b)[4]) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) a[mb] = *(const v8 *)(sb + a_base + mb * 16 * ROWB + off[kk]);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) b[nb] = *(const v8 *)(sb + b_base + nb * 16 * ROWB + off[kk]);
    };
    ld(0, af[0], bfr[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      if (kk + 1 < 2) ld(kk + 1, af[1], bfr[1]);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma(af[kk][mb], bfr[kk][nb], acc[mb][nb]);
      if (kk + 1 < 2) __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
    }
  };

  const int nk = (P.ksplit > 1 ? P.K / P.ksplit : P.K) / BK;
  issue(0, 0);
  for (int ks = 0; ks < nk; ++ks) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // stage ks % 2 has landed for every wave; stage (ks + 1) % 2 is free
    if (ks + 1 < nk) issue((ks + 1) & 1, (ks + 1) * BK);
    compute(ks & 1);
  }

  // epilogue: acc[mb][nb][i] holds row 16 mb + 4 (lane / 16) + i, column 16 nb + lane % 16
  // output kinds of the staged epilogue: 0 fp32, 1 fp16, 2 bf16
  const int okind = P.c_dt == CD_F32 ? 0 : (P.c_dt == CD_F16 || (P.c_dt == CD_IN && __is_same(T, f16_t))) ? 1 : 2;
  if (P.ksplit > 1) {  // this slice's partial product, dense fp32 [M, N]
    __syncthreads();  // every wave is done with the stage buffers
    GemmProblem Q = P;
    Q.C = P.part + (int64_t)kc * P.M * P.N;
    Q.ldc = P.N; Q.hw = P.N; Q.hs = 0; Q.ho = 0; Q.epi = EPI_NONE;
    staged_epilogue<0>(Q, acc, smem + wave * 32 * 272, m0 + wm * 128, n0 + wn * 64, lane);
    return;
  }
  if (!P.c_trans) {  // row-major outputs: 16-byte storable (nt_gemm_problem_ok)
    __syncthreads();  // every wave is done with the stage buffers
    unsigned char *wt = smem + wave * 32 * 272;
    if (okind == 0) staged_epilogue<0>(P, acc, wt, m0 + wm * 128, n0 + wn * 64, lane);
    else if (okind == 1) staged_epilogue<1>(P, acc, wt, m0 + wm * 128, n0 + wn * 64, lane);
    else staged_epilogue<2>(P, acc, wt, m0 + wm * 128, n0 + wn * 64, lane);
    return;
  }
  // transposed per-head store of the value expansion (V^T, keys in vt_slot order): 8-byte stores
  // along the rows, in fp16 or bf16
  if (P.c_dt == CD_BF16) trans_store<bf16_t>(P, acc, m0 + wm * 128, n0 + wn * 64, lane);
  else trans_store<f16_t>(P, acc, m0 + wm * 128, n0 + wn * 64, lane);
}

// C[m][n] = sum over the K slices s = 0 .. ks - 1 (in that order) of part[s][m][n]; four columns
// per thread.
__global__ void __launch_bounds__(256) splitk_sum_kernel(const float *part, int32_t ks, int32_t M, int32_t N, float *C,
                                                         int64_t ldc) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)M * (N / 4)) return;
  const int64_t m = q / (N / 4), n = 4 * (q % (N / 4));
  const int64_t slice = (int64_t)M * N;
  float4 acc = *(const float4 *)(part + m * N + n);
  for (int s = 1; s < ks; ++s) {
    const float4 v = *(const float4 *)(part + s * slice + m * N + n);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  float *c = C + m * ldc + n;
  c[0] = acc.x; c[1] = acc.y; c[2] = acc.z; c[3] = acc.w;
}

// Wt[n][k] = W[k][n] for a [K, N] bf16 weight, converted to fp16 (exact in the fp16 normal range,
// round-to-nearest below it, +-inf above) or kept in bf16.  64 x 64 tiles through LDS with
// 16-byte global loads and stores (K and N multiples of 8; the scalar kernel serves the rest).
template <typename TO>
__global__ void __launch_bounds__(256) transpose16_kernel(const bf16_t *W, TO *Wt, int32_t K, int32_t N) {
  __shared__ bf16_t t[64][72];  // row stride 144 B: consecutive rows of a column read hit distinct banks
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int r = q >> 3, c = (q & 7) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k0 + r < K && n0 + c < N) v = *(const uint4 *)(W + (int64_t)(k0 + r) * N + n0 + c);
    *(uint4 *)&t[r][c] = v;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = threadIdx.x + 256 * i;
    const int rn = q >> 3, kc = (q & 7) * 8;
    if (n0 + rn >= N || k0 + kc >= K) continue;
    TO o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)t[kc + e][rn];
      if constexpr (__is_same(TO, f16_t)) o[e] = (f16_t)(v);
      else o[e] = (bf16_t)v;
    }
    *(uint4 *)(Wt + (int64_t)(n0 + rn) * K + k0 + kc) = *(const uint4 *)o;
  }
}

template <typename TO>
__global__ void __launch_bounds__(256) transpose_kernel(const bf16_t *W, TO *Wt, int32_t K, int32_t N) {
  __shared__ float t[64][65];
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int k = k0 + r, n = n0 + tx;
    t[r][tx] = (k < K && n < N) ? (float)W[(int64_t)k * N + n] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int n = n0 + r, k = k0 + tx;
    if (n < N && k < K) {
      const float v = t[tx][r];
      if constexpr (__is_same(TO, f16_t)) Wt[(int64_t)n * K + k] = (f16_t)(v);
      else Wt[(int64_t)n * K + k] = (bf16_t)v;
    }
  }
}

}  // namespace

bool nt_gemm_problem_ok(const GemmProblem &p) {
  return p.K % BK == 0 && p.K > 0 && p.M > 0 && p.N > 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
         ((uintptr_t)p.A & 15) == 0 && ((uintptr_t)p.B & 15) == 0 && p.hw > 0 &&
         (p.epi != EPI_ROPE || (p.rope_d == 64 && p.hw % 64 == 0 && p.N % 64 == 0 &&
                                (p.c_dt == CD_F16 || p.c_dt == CD_BF16) && p.rope_pos && p.rope_T >= 32)) &&
         (!p.c_trans || ((p.c_dt == CD_F16 || p.c_dt == CD_BF16) && p.ldc % 4 == 0 && (p.hs + p.ho) % 4 == 0 &&
                         ((uintptr_t)p.C & 7) == 0)) &&
         // row-major outputs leave as 16-byte row segments inside one head
         (p.c_trans || (p.N % 8 == 0 && p.hw % 8 == 0 && ((uintptr_t)p.C & 15) == 0 &&
                        p.ldc % (p.c_dt == CD_F32 ? 4 : 8) == 0 && p.hs % (p.c_dt == CD_F32 ? 4 : 8) == 0 &&
                        p.ho % (p.c_dt == CD_F32 ? 4 : 8) == 0));
}

hipError_t launch_gemm_nt(GemmBatch &g, bool f16, hipStream_t s) {
  int t = 0;
  for (int i = 0; i < g.n; ++i) {
    GemmProblem &p = g.p[i];
    if (!nt_gemm_problem_ok(p)) return hipErrorInvalidValue;
    if (p.ksplit > 1 && (p.c_dt != CD_F32 || p.epi != EPI_NONE || p.c_trans || !p.part || p.N % 4 != 0 ||
                         p.K % (BK * p.ksplit) != 0))
      return hipErrorInvalidValue;
    p.tile0 = t;
    p.tiles_n = (p.N + BN - 1) / BN;
    t += ((p.M + BM - 1) / BM) * p.tiles_n * (p.ksplit > 1 ? p.ksplit : 1);
  }
  g.total_tiles = t;
  if (t == 0) return hipSuccess;
  if (f16) hipLaunchKernelGGL(gemm_nt_kernel<f16_t>, dim3(t), dim3(64 * WAVES), 0, s, g);
  else hipLaunchKernelGGL(gemm_nt_kernel<bf16_t>, dim3(t), dim3(64 * WAVES), 0, s, g);
  hipError_t e = hipGetLastError();
  for (int i = 0; i < g.n && e == hipSuccess; ++i) {
    const GemmProblem &p = g.p[i];
    if (p.ksplit <= 1) continue;
    const int64_t quads = (int64_t)p.M * (p.N / 4);
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, p.part, p.ksplit,
                       p.M, p.N, (float *)p.C, p.ldc);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_transpose_weight(const void *w, void *wt, int32_t K, int32_t N, bool to_f16, hipStream_t s) {
  const dim3 grid((N + 63) / 64, (K + 63) / 64);
  const bool vec = K % 8 == 0 && N % 8 == 0 && ((uintptr_t)w & 15) == 0 && ((uintptr_t)wt & 15) == 0;
  if (vec && to_f16)
    hipLaunchKernelGGL(transpose16_kernel<f16_t>, grid, dim3(256), 0, s, (const bf16_t *)w, (f16_t *)wt, K, N);
  else if (vec)
    hipLaunchKernelGGL(transpose16_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t *)w, (bf16_t *)wt, K, N);
  else if (to_f16)
    hipLaunchKernelGGL(transpose_kernel<f16_t>, grid, dim3(256), 0, s, (const bf16_t *)w, (f16_t *)wt, K, N);
  else
    hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t *)w, (bf16_t *)wt, K, N);
  return hipGetLastError();
}

}  // namespace gdla
