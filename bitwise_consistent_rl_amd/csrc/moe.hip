// MoE routing and combine: router top-K with a fixed tie rule, a stable
// permutation of (token, slot) pairs by expert, the per-expert tile plan for
// the grouped GEMMs, and the FP32 combine in fixed slot order.
//
// The DeepSeek recipe unifies MoE rounding, computes row by row and combines
// expert outputs in FP32 in a fixed slot order after they return to the
// token's GPU, instead of recording and replaying routes (page "Finish RL
// Training Faster" digest, section "让训练前向使用推理的数值"); Top-K ties are
// broken by a fixed rule because a discrete choice turns a tiny numeric
// difference into a different expert set (same page, section
// "零差异需要一个精确的比较对象").
//
// Invariance: a token's expert set depends only on its own logits; each
// (token, expert) output row comes out of the row-invariant grouped GEMM; the
// combine adds the k slot outputs in slot order with one fp32 FMA chain and
// then the shared expert.  Nothing depends on how many tokens share an expert.
#include "common.h"
#include "kernels.h"

namespace bci {

// fp32 -> uint32 whose unsigned order is the float order (finite values).
__device__ __forceinline__ uint32_t orderable(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per token, lane e holds logit e (E <= 64).  Slot s takes the
// largest remaining key (logit descending, then expert index ascending).
// Weights: softmax over the k selected logits, summed in slot order.
__global__ __launch_bounds__(256) void moe_topk_kernel(const float* __restrict__ z, int T, int E,
                                                       int k, int32_t* __restrict__ ids,
                                                       float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  const float v = lane < E ? z[(size_t)t * E + lane] : 0.0f;
  uint64_t key = lane < E ? ((uint64_t)orderable(v) << 32) | (uint32_t)(63 - lane) : 0;
  float sel[MOE_MAX_K];
  int sid[MOE_MAX_K];
#pragma unroll
  for (int s = 0; s < MOE_MAX_K; ++s) {
    if (s < k) {
      uint64_t best = key;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t other = __shfl_xor(best, o, WAVE);
        best = other > best ? other : best;
      }
      const int e = 63 - (int)(best & 0xffffffffu);
      sid[s] = e;
      sel[s] = __shfl(v, e, WAVE);
      if (lane == e) key = 0;
    }
  }
  if (lane == 0) {
    float sum = 0.0f;
    float ex[MOE_MAX_K];
#pragma unroll
    for (int s = 0; s < MOE_MAX_K; ++s)
      if (s < k) {
        ex[s] = fexp(sel[s] - sel[0]);
        sum = sum + ex[s];
      }
#pragma unroll
    for (int s = 0; s < MOE_MAX_K; ++s)
      if (s < k) {
        ids[(size_t)t * k + s] = sid[s];
        w[(size_t)t * k + s] = ex[s] / sum;
      }
  }
}

hipError_t launch_moe_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// Block-wide exclusive scan of one flag per thread (256 threads) in thread
// order; returns this thread's rank and writes the block total.
__device__ __forceinline__ int block_rank(bool flag, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + in_wave;
}

// Pass 1 (one workgroup): per-expert counts of the (token, slot) pairs by integer
// LDS atomics (exact in any order), then the expert offsets and the tile list of
// the grouped GEMMs: tile = (expert, first row, rows), rows <= 256, in expert order.
constexpr int MOE_PLAN_THREADS = 1024;

__global__ __launch_bounds__(MOE_PLAN_THREADS) void moe_plan_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ tiles,
                                                                    int32_t* __restrict__ n_tiles) {
  __shared__ int hist[64];
  if (threadIdx.x < 64) hist[threadIdx.x] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += MOE_PLAN_THREADS) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (threadIdx.x < E) counts[threadIdx.x] = hist[threadIdx.x];
  if (threadIdx.x != 0) return;
  int off = 0, nt = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = off;
    for (int r = 0; r < hist[e]; r += GEMM_BM) {
      tiles[3 * nt] = e;
      tiles[3 * nt + 1] = off + r;
      tiles[3 * nt + 2] = min(GEMM_BM, hist[e] - r);
      ++nt;
    }
    off += hist[e];
  }
  offsets[E] = off;
  *n_tiles = nt;
}

// Pass 3: one workgroup per expert writes its pairs in (token, slot) order:
// perm[pos] = pair, inv[pair] = pos.  Stable by construction.
__global__ __launch_bounds__(256) void moe_scatter_kernel(const int32_t* __restrict__ ids, int P,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  __shared__ int wsum[4];
  const int e = blockIdx.x;
  int pos = offsets[e];
  for (int base = 0; base < P; base += 256) {
    const int p = base + threadIdx.x;
    const bool f = p < P && ids[p] == e;
    int tot;
    const int r = block_rank(f, wsum, tot);
    if (f) {
      perm[pos + r] = p;
      inv[p] = pos + r;
    }
    pos += tot;
  }
}

hipError_t launch_moe_sort(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* n_tiles,
                           hipStream_t s) {
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(MOE_PLAN_THREADS), 0, s, ids, P, E, counts, offsets, tiles,
                     n_tiles);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(E), dim3(256), 0, s, ids, P, offsets, perm, inv);
  return hipGetLastError();
}

// out[t] = bf( fma-chain over s = 0..k-1 of w[t,s] * y[inv[t*k+s]] , then + y_shared[t] ).
// A slot whose expert id is outside [0, E) poisons the row with NaN instead of
// reading an unset position.  Each thread owns 8 consecutive columns (16-byte loads of
// every slot's row); every element is the same chain whatever thread computes it.
constexpr int COMBINE_THREADS = 256;

__global__ __launch_bounds__(COMBINE_THREADS) void moe_combine_kernel(const bf16_t* __restrict__ y,
                                                                      const bf16_t* __restrict__ ys,
                                                                      const int32_t* __restrict__ ids,
                                                                      const float* __restrict__ w,
                                                                      const int32_t* __restrict__ inv, int k,
                                                                      int E, int H, bf16_t* __restrict__ out) {
  const int t = blockIdx.x;
  bool ok = true;
  float ws[MOE_MAX_K];
  size_t rows[MOE_MAX_K];
#pragma unroll
  for (int s = 0; s < MOE_MAX_K; ++s) {
    if (s < k) {
      const int e = ids[(size_t)t * k + s];
      ok = ok && e >= 0 && e < E;
      ws[s] = w[(size_t)t * k + s];
      rows[s] = (size_t)inv[(size_t)t * k + s];
    }
  }
  for (int c0 = threadIdx.x * 8; c0 < H; c0 += COMBINE_THREADS * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    if (ok) {
#pragma unroll
      for (int s = 0; s < MOE_MAX_K; ++s) {
        if (s < k) {
          const uint4 v = *reinterpret_cast<const uint4*>(y + rows[s] * H + c0);
          const bf16_t* vp = reinterpret_cast<const bf16_t*>(&v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(ws[s], bf2f(vp[i]), acc[i]);
        }
      }
      if (ys) {
        const uint4 v = *reinterpret_cast<const uint4*>(ys + (size_t)t * H + c0);
        const bf16_t* vp = reinterpret_cast<const bf16_t*>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + bf2f(vp[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __uint_as_float(0x7fc00000u);
    }
    uint4 o;
    uint32_t* op = reinterpret_cast<uint32_t*>(&o);
#pragma unroll
    for (int i = 0; i < 4; ++i) op[i] = pack_bf2(f2bf(acc[2 * i]), f2bf(acc[2 * i + 1]));
    *reinterpret_cast<uint4*>(out + (size_t)t * H + c0) = o;
  }
}

hipError_t launch_moe_combine(const void* y, const void* ys, const int32_t* ids, const float* w,
                              const int32_t* inv, int T, int k, int E, int H, void* out,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (H % 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(T), dim3(COMBINE_THREADS), 0, s, (const bf16_t*)y,
                     (const bf16_t*)ys, ids, w, inv, k, E, H, (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace bci
