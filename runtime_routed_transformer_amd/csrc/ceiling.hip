// Measurement only: the bf16 matrix-core rate this GPU sustains, and its
// shader clock while doing so, for each bf16 MFMA shape the kernels issue.
//
// The datasheet peak of MI355X (2.5 PFLOP/s dense bf16) assumes every
// matrix core busy at 2.4 GHz.  The clock the chip holds depends on its
// power draw, and the draw of a matrix instruction depends on its data:
// identical operands in every instruction toggle few multiplier bits, random
// operands (as in a real GEMM) toggle many.  This kernel issues nothing but
// one MFMA shape on operands held in registers (no memory traffic in the
// loop), two waves per SIMD: v_mfma_f32_32x32x16_bf16 with eight
// independent accumulators per wave, or v_mfma_f32_16x16x32_bf16 with
// sixteen (the same MACs per iteration).  It stamps the shader clock
// (s_memtime) against the 100 MHz reference clock (s_memrealtime).  The GEMM
// roofline fractions are reported against the datasheet peak; this gives
// the ceiling the hardware actually reaches beside it.
#include <stdint.h>

#include "lol_internal.h"

namespace lol {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kCeilThreads = 512;   // 8 waves: two per SIMD
constexpr int kCeilAcc = 8;

// A 32-bit mixing hash (the finaliser of MurmurHash3) of (block, lane, slot),
// for operand bits that differ from lane to lane and instruction to
// instruction.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// A bf16 pair with a random sign and mantissa and an exponent in [2^-4, 2^2)
// (values of the size GEMM operands have), or a fixed pair.
__device__ __forceinline__ uint32_t operand_pair(uint32_t h, bool random) {
  if (!random) return 0x3f803f80u;   // (1.0, 1.0)
  const uint32_t lo = 0x3d80u + (h & 0x2ffu) + ((h >> 10) & 1u) * 0x8000u;
  const uint32_t hi = 0x3d80u + ((h >> 11) & 0x2ffu) + ((h >> 21) & 1u) * 0x8000u;
  return lo | (hi << 16);
}

template <int SHAPE>
__global__ void __launch_bounds__(kCeilThreads, 1)
    k_mfma_ceiling(float *__restrict__ out, long long *__restrict__ clk, int iters, int random) {
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const uint32_t seed = (blockIdx.x * kCeilThreads + threadIdx.x) * 64u;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wa[j] = operand_pair(mix32(seed + q * 8 + j), random != 0);
      wb[j] = operand_pair(mix32(seed + 32 + q * 8 + j), random != 0);
    }
    a[q] = __builtin_bit_cast(bf16x8, make_uint4(wa[0], wa[1], wa[2], wa[3]));
    b[q] = __builtin_bit_cast(bf16x8, make_uint4(wb[0], wb[1], wb[2], wb[3]));
  }
  float s = 0.f;
  // two instruction blocks per iteration, with different B operands (the
  // operand arrays are indexed with constants only, so they stay in
  // registers)
  if constexpr (SHAPE == 32) {
    f32x16 acc[kCeilAcc];
#pragma unroll
    for (int i = 0; i < kCeilAcc; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
      for (int i = 0; i < kCeilAcc; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[i >> 2], acc[i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < kCeilAcc; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[2 + (i >> 2)], acc[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kCeilAcc; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) s += acc[i][j];
  } else {
    // half the MACs per instruction: twice the instructions per block
    f32x4 acc[2 * kCeilAcc];
#pragma unroll
    for (int i = 0; i < 2 * kCeilAcc; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
      for (int i = 0; i < 2 * kCeilAcc; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 3], b[(i >> 2) & 1], acc[i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 2 * kCeilAcc; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 3], b[2 + ((i >> 2) & 1)], acc[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * kCeilAcc; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) s += acc[i][j];
  }
  out[blockIdx.x * kCeilThreads + threadIdx.x] = s;   // keeps the arithmetic alive
  // the end stamp after every wave of the block is done: the two waves of a
  // SIMD do not progress evenly (the older one is favoured), so the first
  // wave alone can finish at half the block's time
  __syncthreads();
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

size_t mfma_ceiling_scratch_bytes(int blocks) {
  return (size_t)blocks * kCeilThreads * sizeof(float) + (size_t)blocks * 2 * sizeof(long long);
}

hipError_t launch_mfma_ceiling(int shape, int blocks, int iters, int random, void *scratch,
                               hipStream_t st) {
  float *out = static_cast<float *>(scratch);
  long long *clk = reinterpret_cast<long long *>(out + (size_t)blocks * kCeilThreads);
  if (shape == 32)
    lol_launch(k_mfma_ceiling<32>, dim3(blocks), dim3(kCeilThreads), 0, st, out, clk, iters, random);
  else
    lol_launch(k_mfma_ceiling<16>, dim3(blocks), dim3(kCeilThreads), 0, st, out, clk, iters, random);
  return hipGetLastError();
}

double mfma_ceiling_flops_per_block(int iters) {
  // 8 waves x iters (rounded up to even) x 8 instructions x 2 * 32 * 32 * 16
  // flops (the 16 x 16 x 32 loop: twice the instructions, half the flops each)
  return (double)(kCeilThreads / 64) * ((iters + 1) / 2 * 2) * kCeilAcc * 2.0 * 32 * 32 * 16;
}

}  // namespace lol
