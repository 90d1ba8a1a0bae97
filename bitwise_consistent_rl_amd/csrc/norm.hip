// Fused residual add + RMSNorm, embedding gather and row gather.
//
// RMSNorm with an added residual is one of the fused inference ops the
// training forward imports unchanged (page "No More Train-Inference
// Mismatch", section "方法细节").  One workgroup of 256 threads owns one row
// for every row count, so a row's reduction tree never depends on the batch:
// thread t sums the squares of its 8-element slices t, t+256, ... in
// ascending order, a fixed xor butterfly combines the 64 lanes of each wave,
// and wave 0..3 partials are added in that order.
#include "common.h"
#include "kernels.h"

namespace bci {

constexpr int NORM_THREADS = 256;
constexpr int NORM_MAX_SLICES = 4;  // cols <= 256 * 8 * 4 = 8192

__global__ __launch_bounds__(NORM_THREADS) void add_rmsnorm_kernel(
    const bf16_t* __restrict__ a, const bf16_t* r_in, bf16_t* r_out, bf16_t* __restrict__ h,
    const bf16_t* __restrict__ g, const int32_t* __restrict__ ids, const bf16_t* __restrict__ E,
    int cols, float eps) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ float wsum[NORM_THREADS / WAVE];

  const bf16_t* src = ids ? E + (size_t)ids[row] * cols : r_in + (size_t)row * cols;
  // the norm weight is loaded with the row, so that its latency is not paid after the
  // reduction (columns past the row repeat its last 8)
  uint4 gv[NORM_MAX_SLICES];
#pragma unroll
  for (int sl = 0; sl < NORM_MAX_SLICES; ++sl)
    gv[sl] = *reinterpret_cast<const uint4*>(g + min((sl * NORM_THREADS + tid) * 8, cols - 8));
  float x[NORM_MAX_SLICES][8];
  float ss = 0.0f;
#pragma unroll
  for (int sl = 0; sl < NORM_MAX_SLICES; ++sl) {
    const int c0 = (sl * NORM_THREADS + tid) * 8;
    if (c0 < cols) {
      uint4 rv = *reinterpret_cast<const uint4*>(src + c0);
      const bf16_t* rp = reinterpret_cast<const bf16_t*>(&rv);
      bf16_t rr[8];
      if (a) {
        uint4 av = *reinterpret_cast<const uint4*>(a + (size_t)row * cols + c0);
        const bf16_t* ap = reinterpret_cast<const bf16_t*>(&av);
#pragma unroll
        for (int i = 0; i < 8; ++i) rr[i] = f2bf(bf2f(ap[i]) + bf2f(rp[i]));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) rr[i] = rp[i];
      }
      uint4 ov;
      uint32_t* op = reinterpret_cast<uint32_t*>(&ov);
#pragma unroll
      for (int i = 0; i < 4; ++i) op[i] = pack_bf2(rr[2 * i], rr[2 * i + 1]);
      if (a || ids) *reinterpret_cast<uint4*>(r_out + (size_t)row * cols + c0) = ov;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[sl][i] = bf2f(rr[i]);
        ss = ss + x[sl][i] * x[sl][i];
      }
    }
  }
  ss = wave_sum(ss);
  if ((tid & (WAVE - 1)) == 0) wsum[tid / WAVE] = ss;
  __syncthreads();
  float tot = wsum[0];
#pragma unroll
  for (int w = 1; w < NORM_THREADS / WAVE; ++w) tot = tot + wsum[w];
  const float inv = 1.0f / sqrtf(tot / (float)cols + eps);
#pragma unroll
  for (int sl = 0; sl < NORM_MAX_SLICES; ++sl) {
    const int c0 = (sl * NORM_THREADS + tid) * 8;
    if (c0 < cols) {
      const bf16_t* gp = reinterpret_cast<const bf16_t*>(&gv[sl]);
      uint4 ov;
      uint32_t* op = reinterpret_cast<uint32_t*>(&ov);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float h0 = (x[sl][2 * i] * inv) * bf2f(gp[2 * i]);
        const float h1 = (x[sl][2 * i + 1] * inv) * bf2f(gp[2 * i + 1]);
        op[i] = pack_bf2(f2bf(h0), f2bf(h1));
      }
      *reinterpret_cast<uint4*>(h + (size_t)row * cols + c0) = ov;
    }
  }
}

hipError_t launch_add_rmsnorm(const void* a, const void* r_in, void* r_out, void* h,
                              const void* g, const int32_t* ids, const void* E, int rows,
                              int cols, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(rows), dim3(NORM_THREADS), 0, s,
                     (const bf16_t*)a, (const bf16_t*)r_in, (bf16_t*)r_out, (bf16_t*)h,
                     (const bf16_t*)g, ids, (const bf16_t*)E, cols, eps);
  return hipGetLastError();
}

// dst[i] = src[rows ? rows[i] : i], 16-byte vectors; one workgroup per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t* __restrict__ src,
                                                          const int32_t* __restrict__ rows,
                                                          bf16_t* __restrict__ dst, int cols) {
  const int i = blockIdx.x;
  const size_t sr = (size_t)rows[i];
  for (int c = threadIdx.x * 8; c < cols; c += 256 * 8)
    *reinterpret_cast<uint4*>(dst + (size_t)i * cols + c) =
        *reinterpret_cast<const uint4*>(src + sr * cols + c);
}

hipError_t launch_embed(const int32_t* ids, const void* E, void* out, int rows, int cols,
                        hipStream_t s) {
  return launch_gather_rows(E, ids, out, rows, cols, s);
}

hipError_t launch_gather_rows(const void* src, const int32_t* rows, void* dst, int n_rows,
                              int cols, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n_rows), dim3(256), 0, s, (const bf16_t*)src, rows,
                     (bf16_t*)dst, cols);
  return hipGetLastError();
}

}  // namespace bci
