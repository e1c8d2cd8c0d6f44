// Skinny bf16 GEMM for decode-sized batches (at most 256 rows): C[M, N] = A[M, K] . B[K, N] with
// the weights B in their stored [K, N] layout, for the projections of one decode step (Motif 3
// Technical Report, picx.dev summary section 2.2: Eq.(1)-(3), (7), (9) and the output projection
// of Eq.(10)).  With so few rows the product is bound by streaming the weights once from HBM, so
// the work is cut into many workgroups: 64 columns each, and, when the column tiles alone do not
// fill the chip, split along K into `splits` slices whose fp32 partial sums a second kernel adds
// in a fixed order (deterministic).  More than 64 rows take up to 4 row blocks of 64; the row
// blocks of one weight tile are neighbouring workgroups, so they stream that tile at about the
// same time.
//
// One workgroup = 4 waves; per 64-deep k-step it stages the weight tile B[k0:+64, n0:+64] and the
// activation tile A[0:64, k0:+64] (8 KB each) by direct global -> LDS 16-byte loads into a 4-stage
// ring (three k-steps in flight).  Wave w owns columns n0 + 16 w .. + 15 and all 64 rows:
//   C^T[n, m] += B^T[n, k] . A^T[k, m]   with v_mfma_f32_16x16x32_bf16,
// With a two-part activation (A_lo: the bf16 rounding remainder of an fp32 activation) the stage
// also holds the A_lo tile, the ring has 3 stages (two in flight, 72 KB, still two workgroups per
// CU) and every weight fragment meets both parts, so the product keeps about 16 bits of A.
// the B^T fragments read by the transposing ds_read_b64_tr_b16 from the row-major weight tile,
// the A^T fragments by 16-byte reads of activation rows.  Both tiles are XOR-swizzled so the reads
// are free of bank conflicts.  Rows past M read row M - 1 (always inside A) and are not stored.
#include "fast_paths.h"

namespace gdla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int SM = 64;          // rows (M) per workgroup
constexpr int MAX_MB = 4;       // row blocks: at most 256 rows
constexpr int SN = 64;          // columns per workgroup
constexpr int SK = 64;          // k per stage
constexpr int NST = 4;          // ring stages
constexpr int TILE_B = SK * SN; // elements of a weight tile
constexpr int TILE_A = SM * SK; // elements of an activation tile
constexpr int LOADS = 4;        // 16-byte loads per lane and stage (16 KB / 256 lanes / 16 B)

__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

__device__ __forceinline__ bf16x4 tr_read(const char *p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}

// 16-byte chunk positions: weight row r (128 bytes = 4 segments of 32) keeps chunk c in segment
// (c / 2) ^ (r % 4); activation row m keeps chunk c at c ^ (m % 8).  Each map is its own inverse.
__device__ __forceinline__ int wslot(int r, int c) { return 2 * ((c >> 1) ^ (r & 3)) + (c & 1); }
__device__ __forceinline__ int aslot(int m, int c) { return c ^ (m & 7); }

struct SkinnyArgs {
  GemmBatch g;
  float *partial;   // [splits, M, n_total] fp32 when splits > 1
  int32_t splits, n_total, mblocks;
  int32_t col0[kMaxGemmProblems];  // column offset of each problem in the partial rows
};

template <bool SPLIT>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(const SkinnyArgs a) {
  constexpr int NS = SPLIT ? 3 : NST;                           // ring stages
  constexpr int NL = SPLIT ? LOADS + 2 : LOADS;                 // 16-byte loads per lane and stage
  constexpr int STAGE = TILE_B + (SPLIT ? 2 : 1) * TILE_A;      // elements per stage
  __shared__ __attribute__((aligned(16))) bf16_t ring[NS * STAGE];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = (int)blockIdx.x / a.mblocks;
  int pi = 0;
#pragma unroll 1
  for (int i = 1; i < a.g.n; ++i)
    if (tile >= a.g.p[i].tile0) pi = i;
  const GemmProblem &P = a.g.p[pi];
  const int n0 = (tile - P.tile0) * SN;
  const int m0 = ((int)blockIdx.x % a.mblocks) * SM;
  const int ks = P.K / a.splits;
  const int kbeg = (int)blockIdx.y * ks;
  const int nsteps = ks / SK;
  const bf16_t *Ab = (const bf16_t *)P.A;
  const bf16_t *Al = (const bf16_t *)P.A_lo;
  const bf16_t *Bb = (const bf16_t *)P.B;

  // this lane's source offsets (bytes) for its loads of a stage: loads 0..7 of the workgroup fill
  // weight rows 8 q .. 8 q + 7, loads 8..15 activation rows 8 (q - 8) .., and (SPLIT) loads 16..23
  // the same rows of A_lo; wave w issues loads w, w + 4, w + 8, ...  Load q lands at 1 KB q of the
  // stage (weight tile, then A, then A_lo).
  uint32_t soff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int q = wave + 4 * i;
    const int r = (q & 7) * 8 + (lane >> 3), cp = lane & 7;
    if (q < 8) {
      soff[i] = (uint32_t)(((int64_t)r * P.ldb + 8 * wslot(r, cp)) * 2);
    } else {
      const int m = min(m0 + r, P.M - 1);
      soff[i] = (uint32_t)(((int64_t)m * P.lda + 8 * aslot(r, cp)) * 2);
    }
  }
  const uint32_t rbase = lds_u32(ring);
  auto issue = [&](int st) {
    const int k0 = kbeg + st * SK;
    const uint32_t slot = rbase + (uint32_t)((st % NS) * STAGE * 2);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = wave + 4 * i;
      if (q < 8) dma16(Bb + (int64_t)k0 * P.ldb + n0, soff[i], slot + q * 1024);
      else if (q < 16) dma16(Ab + k0, soff[i], slot + q * 1024);
      else dma16(Al + k0, soff[i], slot + q * 1024);
    }
  };

  // fragment read offsets (bytes within a stage)
  const int g = lane >> 4, j = lane & 15;
  int offW[2], offA[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int r = 32 * kk + 8 * g + (j >> 2);  // low rows; the high rows are r + 4 (same r % 4)
    offW[kk] = r * 128 + 32 * (wave ^ (r & 3)) + 8 * (j & 3);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = 16 * mb + j;
      offA[kk][mb] = TILE_B * 2 + m * 128 + 16 * aslot(m, 4 * kk + g);
    }
  }

  f32x4 acc[4] = {};
  for (int st = 0; st < NS - 1 && st < nsteps; ++st) issue(st);
  for (int st = 0; st < nsteps; ++st) {
    const int ahead = min(nsteps - 1 - st, NS - 2);
    if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");
    else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // stage st has landed for every wave; every wave is done with stage st - 1
    if (st + NS - 1 < nsteps) issue(st + NS - 1);
    const char *sb = (const char *)(ring + (st % NS) * STAGE);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x4 lo = tr_read(sb + offW[kk]);
      const bf16x4 hi = tr_read(sb + offW[kk] + 4 * 128);
      const bf16x8 wf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 af = *(const bf16x8 *)(sb + offA[kk][mb]);
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, af, acc[mb], 0, 0, 0);
        if (SPLIT) {
          const bf16x8 al = *(const bf16x8 *)(sb + offA[kk][mb] + TILE_A * 2);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, al, acc[mb], 0, 0, 0);
        }
      }
    }
  }

  // acc[mb][r] = C[m = m0 + 16 mb + j][n = n0 + 16 wave + 4 g + r]
  const int n = n0 + 16 * wave + 4 * g;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + 16 * mb + j;
    if (m >= P.M) continue;
    if (a.splits > 1) {
      float *d = a.partial + ((int64_t)blockIdx.y * P.M + m) * a.n_total + a.col0[pi] + n;
      *(float4 *)d = make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
    } else if (P.c_dt == CD_F32) {
      *(float4 *)((float *)P.C + (int64_t)m * P.ldc + n) = make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
    } else {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16_t)acc[mb][r];
      *(bf16x4 *)((bf16_t *)P.C + (int64_t)m * P.ldc + n) = v;
    }
  }
}

// C[m, n] = sum over splits of the partial rows (in split order), for every problem.
__global__ void __launch_bounds__(256) skinny_reduce_kernel(const SkinnyArgs a) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // element of [M, n_total]
  const GemmProblem &P0 = a.g.p[0];
  const int M = P0.M;
  if (i >= (int64_t)M * a.n_total) return;
  const int m = (int)(i / a.n_total), col = (int)(i % a.n_total);
  int pi = 0;
  for (int k = 1; k < a.g.n; ++k)
    if (col >= a.col0[k]) pi = k;
  const GemmProblem &P = a.g.p[pi];
  const int n = col - a.col0[pi];
  float4 s = *(const float4 *)(a.partial + (int64_t)m * a.n_total + col);
  for (int sp = 1; sp < a.splits; ++sp) {
    const float4 v = *(const float4 *)(a.partial + ((int64_t)sp * M + m) * a.n_total + col);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (P.c_dt == CD_F32) {
    *(float4 *)((float *)P.C + (int64_t)m * P.ldc + n) = s;
  } else {
    bf16x4 v;
    v[0] = (bf16_t)s.x; v[1] = (bf16_t)s.y; v[2] = (bf16_t)s.z; v[3] = (bf16_t)s.w;
    *(bf16x4 *)((bf16_t *)P.C + (int64_t)m * P.ldc + n) = v;
  }
}

// split count: double while the workgroups do not cover the chip (256 compute units), every K
// splits into whole stages and the slices stay at least 4 stages deep.  So splits * tiles * row
// blocks < 512, which bounds the partial sums (skinny_gemm_partial_bound).
int choose_splits(const GemmBatch &g) {
  int tiles = 0;
  for (int i = 0; i < g.n; ++i) tiles += g.p[i].N / SN;
  const int mb = (g.p[0].M + SM - 1) / SM;
  int s = 1;
  for (;;) {
    bool ok = tiles * mb * s < 256;
    for (int i = 0; i < g.n && ok; ++i) ok = g.p[i].K % (2 * s * SK) == 0 && g.p[i].K / (2 * s) >= 4 * SK;
    if (!ok) return s;
    s *= 2;
  }
}

}  // namespace

bool skinny_problem_ok(const GemmProblem &p) {
  return p.M >= 1 && p.M <= SM * MAX_MB && p.N % SN == 0 && p.K % SK == 0 && p.K >= SK && p.a_f16 == 0 &&
         p.epi == EPI_NONE && !p.c_trans && (p.c_dt == CD_F32 || p.c_dt == CD_IN) && p.lda % 8 == 0 &&
         p.ldb % 8 == 0 && p.ldc % 4 == 0 && ((uintptr_t)p.A & 15) == 0 && ((uintptr_t)p.B & 15) == 0 &&
         ((uintptr_t)p.C & 15) == 0 && ((uintptr_t)p.A_lo & 15) == 0 && p.hw == p.N && p.hs == 0 && p.ho == 0 &&
         (int64_t)(p.M - 1) * p.lda + p.K < (int64_t)1 << 30 && (int64_t)63 * p.ldb + 64 < (int64_t)1 << 30;
}

bool skinny_gemm_ok(const GemmBatch &g) {
  if (g.n < 1) return false;
  for (int i = 0; i < g.n; ++i)
    if (!skinny_problem_ok(g.p[i]) || g.p[i].M != g.p[0].M || (g.p[i].A_lo == nullptr) != (g.p[0].A_lo == nullptr))
      return false;
  return true;
}

size_t skinny_gemm_partial_bound(int32_t M) { return (size_t)M * 512 * SN * 4; }

size_t skinny_gemm_partial_bytes(const GemmBatch &g) {
  if (!skinny_gemm_ok(g)) return 0;
  const int s = choose_splits(g);
  if (s == 1) return 0;
  int64_t n_total = 0;
  for (int i = 0; i < g.n; ++i) n_total += g.p[i].N;
  return (size_t)s * g.p[0].M * n_total * 4;
}

hipError_t launch_gemm_skinny(const GemmBatch &g, void *partial, size_t partial_bytes, hipStream_t s) {
  if (!skinny_gemm_ok(g)) return hipErrorInvalidValue;
  SkinnyArgs a{};
  a.g = g;
  a.splits = choose_splits(g);
  int tiles = 0, cols = 0;
  for (int i = 0; i < g.n; ++i) {
    a.g.p[i].tile0 = tiles;
    a.col0[i] = cols;
    tiles += g.p[i].N / SN;
    cols += g.p[i].N;
  }
  a.n_total = cols;
  a.mblocks = (g.p[0].M + SM - 1) / SM;
  if (a.splits > 1) {
    if (!partial || partial_bytes < (size_t)a.splits * g.p[0].M * cols * 4) return hipErrorInvalidValue;
    a.partial = (float *)partial;
  }
  if (g.p[0].A_lo)
    hipLaunchKernelGGL(gemm_skinny_kernel<true>, dim3(tiles * a.mblocks, a.splits, 1), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_skinny_kernel<false>, dim3(tiles * a.mblocks, a.splits, 1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t quads = (int64_t)g.p[0].M * cols / 4;
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdla
