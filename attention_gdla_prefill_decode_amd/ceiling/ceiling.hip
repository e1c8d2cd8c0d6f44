// Measured ceilings of one MI355X for the roofline fractions the benchmark reports next to the
// published peaks: the bf16 matrix-core rate with random operands, on the instruction the prefill
// attention runs (the chip's clock under that load, not the nominal 2.4 GHz, sets what any MFMA
// kernel can reach) and the HBM read rate of a streaming kernel.  Not part of the GDLA library:
// bench.py loads libgdla_ceiling.so.
//
//   int ceiling_mfma(float *out, int blocks, int iters, hipStream_t s)
//     blocks x 512 threads, each wave issuing iters x 8 independent v_mfma_f32_16x16x32_bf16 on
//     pseudo-random bf16 operands; FLOP = blocks * 8 * iters * 8 * 16384.  out: blocks * 512 floats.
//   int ceiling_read(const void *p, int64_t bytes, float *out, int blocks, hipStream_t s)
//     reads `bytes` (a multiple of blocks * 32 KiB) once: each of `blocks` workgroups (one per CU:
//     256) streams its contiguous share through a 4-slot LDS ring of 32 KiB slots with direct
//     global -> LDS 16-byte loads, three slots in flight, a barrier per slot (the way the decode
//     kernel streams its cache; loads into registers reach less); out: 1 float.
// Both return 0, or the HIP error of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CHAINS = 8;  // independent accumulators per wave
constexpr int RING = 4;    // LDS slots of the read probe
constexpr int IPW = 8;     // 1 KiB wave-loads per wave and slot
constexpr int SLOT = 4 * IPW * 1024;

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  return x ^ (x >> 16);
}

__global__ void __launch_bounds__(512) mfma_kernel(float *out, int iters) {
  const uint32_t tid = blockIdx.x * 512 + threadIdx.x;
  bf16x8 a[CHAINS], b[CHAINS];
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // uniform in [-1, 1): every bit of the operands toggles like real data
      a[j][e] = (__bf16)((float)(mix(tid * 128 + j * 8 + e) >> 8) * (2.0f / 16777216.0f) - 1.0f);
      b[j][e] = (__bf16)((float)(mix(tid * 128 + 64 + j * 8 + e) >> 8) * (2.0f / 16777216.0f) - 1.0f);
    }
  f32x4 acc[CHAINS] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < CHAINS; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < CHAINS; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[j][e];
  out[tid] = s;
}

// 16 bytes global (wave-uniform base + 32-bit lane offset) -> LDS at M0 + 16 lane; the wait is
// explicit (s_waitcnt vmcnt) before the barrier that publishes a slot.
__device__ __forceinline__ void dma16(const char *base, uint32_t voff, uint32_t lds_addr) {
  const uint64_t q = (uint64_t)(uintptr_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(q >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)q);
  const uint64_t sbase = (uint64_t)hi << 32 | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
}

__global__ void __launch_bounds__(256, 1) read_kernel(const char *p, int64_t per_wg, float *out) {
  __shared__ __attribute__((aligned(16))) char ring[RING * SLOT];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const char *base = p + blockIdx.x * per_wg;
  const int n = (int)(per_wg / SLOT);
  const uint32_t r0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)ring;
  auto issue = [&](int t) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int ins = wave + 4 * i;
      dma16(base + (int64_t)t * SLOT, ins * 1024 + lane * 16,
            __builtin_amdgcn_readfirstlane(r0 + (t % RING) * SLOT + ins * 1024));
    }
  };
  for (int t = 0; t < RING - 1 && t < n; ++t) issue(t);
  float acc = 0.f;
  for (int t = 0; t < n; ++t) {
    const int after = min(n - 1 - t, RING - 2);  // this wave's slots issued after slot t
    if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * IPW) : "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // slot t landed; every wave is done with slot t - 1
    if (t + RING - 1 < n) issue(t + RING - 1);
    acc += *(const float *)(ring + (t % RING) * SLOT + wave * 1024 + lane * 16);  // this wave's own load
  }
  if (acc == 1234.5f) out[0] = acc;  // keeps the loop; practically never taken
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int ceiling_mfma(float *out, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(512), 0, s, out, iters);
  return (int)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int ceiling_read(const void *p, int64_t bytes, float *out, int blocks,
                                                                  hipStream_t s) {
  if (blocks <= 0 || bytes <= 0 || bytes % ((int64_t)blocks * SLOT) != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, s, (const char *)p, bytes / blocks, out);
  return (int)hipGetLastError();
}
