// Grouped GEMM on gfx950 matrix cores: C = A[M, K] B[K, N], fp32 accumulation.  Two operand
// modes: bf16 x bf16, or fp16 A x bf16 B, where B is converted to fp16 while it is staged (bf16
// values convert exactly unless they fall outside the fp16 range, where they become +-inf; NaN
// stays NaN).  Outputs are fp32, bf16 or fp16 (round to nearest even, +-inf beyond fp16's range).
//
// Used for every projection of the GDLA layer (Motif 3 Technical Report, picx.dev summary,
// section 2.2: x W^Q_a, x W^KV_a, x W^lambda in Eq.(1), (3), (7); c^Q W^Q_b, c^Q W^G in Eq.(2),
// (9); cbar W^KV_b in Eq.(5); vec(.) W^O in Eq.(10)).
//
// Block tile 128 x 128, K slices of 32 staged in LDS (double buffered, one barrier per slice),
// 4 waves of 64 x 64, each a 2 x 2 grid of v_mfma_f32_32x32x16 (bf16 or fp16).  A fragments (8
// consecutive k of one row) come from ds_read_b128; B is stored [k][n] in LDS and its fragments (8
// consecutive k of one column) come from two ds_read_tr16_b64.  Row paddings keep both reads free
// of bank conflicts.  The short K slice keeps LDS at 40 KB and registers at about 123, so 4
// workgroups (16 waves) share a CU and hide each other's load latency.  Tiles are spread so that
// each XCD gets a contiguous range of tiles.
#include "fast_paths.h"

namespace gdla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDA_S = BK + 8;    // A row stride in LDS (elements)
constexpr int LDB_S = BN + 32;   // B row stride in LDS (elements)
constexpr int A_STAGE = BM * LDA_S;
constexpr int B_STAGE = BK * LDB_S;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <typename T> struct Frag;
template <> struct Frag<bf16_t> { typedef bf16x8 v8; typedef bf16x4 v4; };
template <> struct Frag<f16_t> { typedef f16x8 v8; typedef f16x4 v4; };

template <typename T>
__device__ __forceinline__ typename Frag<T>::v4 tr_read(const T *p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
  return __builtin_bit_cast(typename Frag<T>::v4, v);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 8 bf16 -> 8 fp16 (exact in the fp16 normal range, +-inf beyond it, NaN kept).
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  auto cv = [](unsigned w) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xffff0000u)};
    return __builtin_bit_cast(unsigned, h);
  };
  return make_uint4(cv(v.x), cv(v.y), cv(v.z), cv(v.w));
}

__device__ __forceinline__ int remap_xcd(int bid, int total) {
  if (total < 8) return bid;
  const int q = total / 8, r = total % 8, x = bid % 8, i = bid / 8;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <typename TA>  // bf16_t: bf16 x bf16; f16_t: fp16 A x converted B
__global__ void __launch_bounds__(256, 4) gemm_mfma_kernel(GemmBatch batch) {
  typedef typename Frag<TA>::v8 v8;
  typedef typename Frag<TA>::v4 v4;
  constexpr bool CONVERT_B = __is_same(TA, f16_t);
  __shared__ __attribute__((aligned(16))) TA As[2 * A_STAGE];
  __shared__ __attribute__((aligned(16))) TA Bs[2 * B_STAGE];

  const int bid = remap_xcd(blockIdx.x, batch.total_tiles);
  int pi = 0;
  while (pi + 1 < batch.n && bid >= batch.p[pi + 1].tile0) ++pi;
  const GemmProblem &P = batch.p[pi];
  const int tile = bid - P.tile0;
  const int m0 = (tile / P.tiles_n) * BM, n0 = (tile % P.tiles_n) * BN;
  const TA *A = (const TA *)P.A;
  const bf16_t *B = (const bf16_t *)P.B;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: NCH A chunks and NCH B chunks of 8 elements per thread
  constexpr int NCH = BK / 16;  // chunks of each operand per thread
  uint4 ra[NCH], rb[NCH];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int gm = m0 + r;
      ra[i] = gm < P.M ? *(const uint4 *)(A + (int64_t)gm * P.lda + k0 + kc) : make_uint4(0, 0, 0, 0);
      const int kr = c >> 4, nc = (c & 15) * 8;
      const int gn = n0 + nc;
      rb[i] = gn < P.N ? *(const uint4 *)(B + (int64_t)(k0 + kr) * P.ldb + gn) : make_uint4(0, 0, 0, 0);
      if (CONVERT_B) rb[i] = bf16x8_to_f16x8(rb[i]);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + 256 * i;
      *(uint4 *)(As + buf * A_STAGE + (c / (BK / 8)) * LDA_S + (c % (BK / 8)) * 8) = ra[i];
      *(uint4 *)(Bs + buf * B_STAGE + (c >> 4) * LDB_S + (c & 15) * 8) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // per-lane fragment coordinates
  const int a_row = lane & 31, a_k = (lane >> 5) * 8;
  const int G = lane >> 4, jj = (lane & 15) >> 2, qq = lane & 3;
  const int b_k = 8 * (G >> 1) + jj, b_n = 16 * (G & 1) + 4 * qq;

  const int nk = P.K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * BK);
    const TA *as = As + buf * A_STAGE + (wm * 64) * LDA_S;
    const TA *bs = Bs + buf * B_STAGE + wn * 64;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      v8 af[2], bfr[2];
#pragma unroll
      for (int r = 0; r < 2; ++r)
        af[r] = *(const v8 *)(as + (r * 32 + a_row) * LDA_S + kk + a_k);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const TA *p = bs + (kk + b_k) * LDB_S + c * 32 + b_n;
        const v4 lo = tr_read<TA>(p);
        const v4 hi = tr_read<TA>(p + 4 * LDB_S);
        bfr[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[r][c] = mfma(af[r], bfr[c], acc[r][c]);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(j/4) + 4*(lane/32) + j%4 of each block
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int n = n0 + wn * 64 + c * 32 + (lane & 31);
      if (n >= P.N) continue;
      if (P.c_trans) {
        // 4 consecutive rows m .. m + 3 land on 4 consecutive positions of column n's row
        f16_t *base = (f16_t *)P.C + (int64_t)(n / P.hw) * P.hs + P.ho + (int64_t)(n % P.hw) * P.ldc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + wm * 64 + r * 32 + 8 * q + 4 * (lane >> 5);
          if (m >= P.M) continue;
          f16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (f16_t)(acc[r][c][4 * q + e]);
          if (m + 3 < P.M) {
            *(f16x4 *)(base + vt_slot(m)) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (m + e < P.M) base[vt_slot(m + e)] = v[e];
          }
        }
        continue;
      }
      const int64_t coff = (int64_t)(n / P.hw) * P.hs + P.ho + (n % P.hw);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = m0 + wm * 64 + r * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
        if (m >= P.M) continue;
        float v = acc[r][c][j];
        if (P.epi == EPI_SIGMOID) v = 1.0f / (1.0f + __expf(-v));
        const int64_t off = (int64_t)m * P.ldc + coff;
        if (P.c_dt == CD_F32) ((float *)P.C)[off] = v;
        else if (P.c_dt == CD_F16 || (P.c_dt == CD_IN && CONVERT_B))
          ((f16_t *)P.C)[off] = (f16_t)(v);
        else ((bf16_t *)P.C)[off] = (bf16_t)v;
      }
    }
  }
}

}  // namespace

bool fast_gemm_problem_ok(const GemmProblem &p) {
  return p.K % BK == 0 && p.K > 0 && p.N % 8 == 0 && p.lda % 8 == 0 && p.ldb % 8 == 0 &&
         ((uintptr_t)p.A & 15) == 0 && ((uintptr_t)p.B & 15) == 0 && p.hw > 0 &&
         (!p.c_trans || (p.c_dt == CD_F16 && p.ldc % 4 == 0 && (p.hs + p.ho) % 4 == 0 &&
                         ((uintptr_t)p.C & 7) == 0));
}

hipError_t launch_gemm_mfma(GemmBatch &g, hipStream_t s) {
  int t = 0;
  for (int i = 0; i < g.n; ++i) {
    GemmProblem &p = g.p[i];
    p.tile0 = t;
    p.tiles_n = (p.N + BN - 1) / BN;
    t += ((p.M + BM - 1) / BM) * p.tiles_n;
  }
  g.total_tiles = t;
  if (t == 0) return hipSuccess;
  if (g.p[0].a_f16) hipLaunchKernelGGL(gemm_mfma_kernel<f16_t>, dim3(t), dim3(256), 0, s, g);
  else hipLaunchKernelGGL(gemm_mfma_kernel<bf16_t>, dim3(t), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace gdla
