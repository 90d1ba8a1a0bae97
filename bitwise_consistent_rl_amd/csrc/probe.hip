// The chip's sustained dense bf16 MFMA rate, measured: every SIMD issues
// v_mfma_f32_16x16x32_bf16 back to back (16 independent accumulator chains per
// wave, two waves per SIMD, operands resident in registers, no memory traffic in
// the loop).  With pseudo-random operands the MFMA arrays switch about as many bits
// as in a GEMM on random data, so the rate includes the power-limited clock; with
// all-zero operands it shows the clock the chip holds when little switches.  This
// is the denominator a GEMM's fraction can be read against besides the datasheet's.
#include "common.h"
#include "kernels.h"

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PROBE_THREADS = 512;  // 8 waves: two per SIMD
constexpr int PROBE_CHAINS = 16;

__global__ __launch_bounds__(PROBE_THREADS, 1) void mfma_rate_kernel(float* __restrict__ out, int iters,
                                                                      int random) {
  const uint32_t gid = blockIdx.x * PROBE_THREADS + threadIdx.x;
  // 4 A and 4 B fragments of pseudo-random bf16 values in [-2, 2) (xorshift32 bits,
  // exponent held to 126..127 so no value overflows the accumulators), or zeros
  bf16x8_t fa[4], fb[4];
  uint32_t x = gid * 2654435761u + 12345u;
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        const uint32_t b = random ? ((x & 0x807Fu) | (126u + ((x >> 8) & 1u)) << 7) : 0u;
        v |= b << (16 * h);
      }
      w[i] = v;
    }
    if (f < 4) fa[f] = __builtin_bit_cast(bf16x8_t, w);
    else fb[f - 4] = __builtin_bit_cast(bf16x8_t, w);
  }
  f32x4_t acc[PROBE_CHAINS];
#pragma unroll
  for (int k = 0; k < PROBE_CHAINS; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < PROBE_CHAINS; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[k & 3], fb[(k >> 2) & 3], acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < PROBE_CHAINS; ++k) s = s + acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[gid] = s;  // keeps the chains live
}

hipError_t launch_mfma_rate(float* out, int blocks, int iters, int random, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(PROBE_THREADS), 0, s, out, iters, random);
  return hipGetLastError();
}

}  // namespace bci
