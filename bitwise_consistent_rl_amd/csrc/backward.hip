// Backward kernels of the invariant forward.
//
// The trainer keeps the inference forward and adds its own backward, whose
// gradients must be checked separately (page "Finish RL Training Faster" digest,
// section "让训练前向使用推理的数值").  Every GEMM of the backward (dX = dY . W,
// dW = dY^T . X, the logits of the lm_head) runs on the invariant forward GEMM with
// transposed operands, so each output element is one ascending fp32 MFMA chain over
// its contraction, the same for any batch; the kernels here are the pieces around
// those GEMMs.  The forward's roundings are taken as the identity (straight-through)
// and the backward is evaluated at the forward's stored bf16 values.  Activation
// gradients are stored in bf16, weight and gain gradients in fp32.
//   transpose_bf16        dst[c][r] = src[r][c], zero for r >= R (pads a GEMM's K)
//   rmsnorm_backward      per row: s = 1/sqrt(mean(r^2)+eps) (the forward's expression),
//                         dr = (g dh) s - r (s^3 sum_k g_k dh_k r_k / H) + dr_in
//   rmsnorm_dg            dg = sum over rows, ascending, of dh r s: partial sums over
//                         blocks of 64 rows, then the partials in block order
//   silu_mul_backward     d gate = dact u silu'(gate), d up = dact silu(gate)
//   logprob_dz            per row: (m, S) = (max z, sum exp(z - m)) folded per thread and
//                         merged by a fixed tree; dz = g ((j == id) - exp(z - m) / S)
#include "common.h"
#include "kernels.h"

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- transpose

constexpr int TT = 64;
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ src,
                                                             bf16_t* __restrict__ dst, int R, int C,
                                                             int ldd) {
  __shared__ bf16_t tile[TT][TT + 2];
  const int r0 = blockIdx.x * TT, c0 = blockIdx.y * TT;
  const int tid = threadIdx.x;
  // load: 64 rows x 8 pieces of 8 columns
  for (int u = tid; u < TT * (TT / 8); u += 256) {
    const int rr = u / (TT / 8), pc = u % (TT / 8);
    const int r = r0 + rr, c = c0 + 8 * pc;
    u32x4_t v = u32x4_t{0, 0, 0, 0};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4_t*>(src + (size_t)r * C + c);
    const bf16_t* e = reinterpret_cast<const bf16_t*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[rr][8 * pc + i] = e[i];
  }
  __syncthreads();
  // store: 64 destination rows (columns of src) x 8 pieces of 8 source rows
  for (int u = tid; u < TT * (TT / 8); u += 256) {
    const int cc = u / (TT / 8), pr = u % (TT / 8);
    const int c = c0 + cc, r = r0 + 8 * pr;
    if (c >= C || r >= ldd) continue;
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf2(tile[8 * pr + 2 * i][cc], tile[8 * pr + 2 * i + 1][cc]);
    *reinterpret_cast<u32x4_t*>(dst + (size_t)c * ldd + r) = v;
  }
}

hipError_t launch_transpose_bf16(const void* src, void* dst, int R, int C, int ldd, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((ldd + TT - 1) / TT, (C + TT - 1) / TT), dim3(256), 0,
                     s, (const bf16_t*)src, (bf16_t*)dst, R, C, ldd);
  return hipGetLastError();
}

// ------------------------------------------------------------- add+RMSNorm backward

constexpr int BW_THREADS = 256;

// sum over the workgroup: each wave by a fixed xor tree, then the wave sums in order
__device__ __forceinline__ float block_sum_fixed(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < BW_THREADS / WAVE; ++w) t = t + red[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(BW_THREADS) void rmsnorm_backward_kernel(
    const bf16_t* __restrict__ r, const bf16_t* __restrict__ g, const bf16_t* __restrict__ dh,
    const bf16_t* __restrict__ dr_in, bf16_t* __restrict__ dr, float* __restrict__ rstd, int cols,
    float eps) {
  __shared__ float red[BW_THREADS / WAVE];
  const size_t row = blockIdx.x;
  const bf16_t* rr = r + row * cols;
  const bf16_t* dd = dh + row * cols;
  float ss = 0.0f, dot = 0.0f;
  for (int k = threadIdx.x; k < cols; k += BW_THREADS) {
    const float x = bf2f(rr[k]);
    ss = ss + x * x;
    dot = dot + (bf2f(g[k]) * bf2f(dd[k])) * x;
  }
  const float tot = block_sum_fixed(ss, red);
  const float dt = block_sum_fixed(dot, red);
  const float s = 1.0f / sqrtf(tot / (float)cols + eps);
  const float c = ((s * s) * s) * (dt / (float)cols);
  for (int k = threadIdx.x; k < cols; k += BW_THREADS) {
    float v = (bf2f(g[k]) * bf2f(dd[k])) * s - bf2f(rr[k]) * c;
    if (dr_in) v = v + bf2f(dr_in[row * cols + k]);
    dr[row * cols + k] = f2bf(v);
  }
  if (threadIdx.x == 0) rstd[row] = s;
}

constexpr int DG_ROWS = BW_DG_ROWS;
// partial[b][k] = sum over rows 64b .. 64b+63 (ascending) of dh r s
__global__ __launch_bounds__(BW_THREADS) void rmsnorm_dg_partial_kernel(
    const bf16_t* __restrict__ r, const bf16_t* __restrict__ dh, const float* __restrict__ rstd,
    float* __restrict__ part, int rows, int cols) {
  const int k = blockIdx.x * BW_THREADS + threadIdx.x;
  const int b = blockIdx.y;
  if (k >= cols) return;
  const int i1 = min(rows, (b + 1) * DG_ROWS);
  float acc = 0.0f;
  for (int i = b * DG_ROWS; i < i1; ++i)
    acc = acc + (bf2f(dh[(size_t)i * cols + k]) * bf2f(r[(size_t)i * cols + k])) * rstd[i];
  part[(size_t)b * cols + k] = acc;
}
__global__ __launch_bounds__(BW_THREADS) void rmsnorm_dg_final_kernel(const float* __restrict__ part,
                                                                      float* __restrict__ dg, int nb,
                                                                      int cols) {
  const int k = blockIdx.x * BW_THREADS + threadIdx.x;
  if (k >= cols) return;
  float acc = 0.0f;
  for (int b = 0; b < nb; ++b) acc = acc + part[(size_t)b * cols + k];
  dg[k] = acc;
}

hipError_t launch_rmsnorm_backward(const void* r, const void* g, const void* dh, const void* dr_in,
                                   void* dr, float* rstd, float* dg, float* part, int rows, int cols,
                                   float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_backward_kernel, dim3(rows), dim3(BW_THREADS), 0, s, (const bf16_t*)r,
                     (const bf16_t*)g, (const bf16_t*)dh, (const bf16_t*)dr_in, (bf16_t*)dr, rstd, cols,
                     eps);
  const int nb = (rows + DG_ROWS - 1) / DG_ROWS;
  const int cb = (cols + BW_THREADS - 1) / BW_THREADS;
  hipLaunchKernelGGL(rmsnorm_dg_partial_kernel, dim3(cb, nb), dim3(BW_THREADS), 0, s, (const bf16_t*)r,
                     (const bf16_t*)dh, rstd, part, rows, cols);
  hipLaunchKernelGGL(rmsnorm_dg_final_kernel, dim3(cb), dim3(BW_THREADS), 0, s, part, dg, nb, cols);
  return hipGetLastError();
}

// ------------------------------------------------------------- SiLU * up backward

__global__ __launch_bounds__(BW_THREADS) void silu_mul_backward_kernel(
    const bf16_t* __restrict__ gu, const bf16_t* __restrict__ dact, bf16_t* __restrict__ dgu, int rows,
    int inter) {
  const size_t idx = (size_t)blockIdx.x * BW_THREADS + threadIdx.x;
  if (idx >= (size_t)rows * inter) return;
  const size_t i = idx / inter, k = idx % inter;
  const float gt = bf2f(gu[i * 2 * inter + k]);
  const float up = bf2f(gu[i * 2 * inter + inter + k]);
  const float da = bf2f(dact[idx]);
  const float sig = 1.0f / (1.0f + fexp(-gt));
  dgu[i * 2 * inter + k] = f2bf((da * up) * (sig * (1.0f + gt * (1.0f - sig))));
  dgu[i * 2 * inter + inter + k] = f2bf(da * silu_f32(gt));
}

hipError_t launch_silu_mul_backward(const void* gu, const void* dact, void* dgu, int rows, int inter,
                                    hipStream_t s) {
  const size_t n = (size_t)rows * inter;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_backward_kernel, dim3((unsigned)((n + BW_THREADS - 1) / BW_THREADS)),
                     dim3(BW_THREADS), 0, s, (const bf16_t*)gu, (const bf16_t*)dact, (bf16_t*)dgu, rows,
                     inter);
  return hipGetLastError();
}

// ------------------------------------------------------------- logprob backward

constexpr int LP_THREADS = 1024;

// (m, s) <- (m, s) merged with (m2, s2): the running max and the sum of exp(x - max)
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * fexp(m - mn) + s2 * fexp(m2 - mn);
  m = mn;
}

// One workgroup per row: each thread folds its columns (16-byte loads, strided by the
// workgroup) into a running (max, sum exp) pair, the pairs are merged by a fixed xor
// tree in each wave and then wave by wave in order; a second pass writes dz.
__global__ __launch_bounds__(LP_THREADS) void logprob_dz_kernel(const float* __restrict__ z,
                                                                const int32_t* __restrict__ ids,
                                                                const float* __restrict__ gout,
                                                                bf16_t* __restrict__ dz, int V) {
  __shared__ float wm[LP_THREADS / WAVE], ws[LP_THREADS / WAVE];
  const size_t row = blockIdx.x;
  const float* zr = z + row * V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V4 = (V & 3) == 0 ? V / 4 : 0;   // rows of a multiple of 4 columns: 16-byte loads
  float m = -INFINITY, s = 0.0f;
  if (V4) {
    for (int j = tid; j < V4; j += LP_THREADS) {
      const f32x4_t v = reinterpret_cast<const f32x4_t*>(zr)[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) ms_merge(m, s, v[i], 1.0f);
    }
  } else {
    for (int j = tid; j < V; j += LP_THREADS) ms_merge(m, s, zr[j], 1.0f);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    ms_merge(m, s, m2, s2);
  }
  if (lane == 0) {
    wm[wave] = m;
    ws[wave] = s;
  }
  __syncthreads();
  m = wm[0];
  s = ws[0];
  for (int w = 1; w < LP_THREADS / WAVE; ++w) ms_merge(m, s, wm[w], ws[w]);
  const int id = ids[row];
  const float g = gout[row];
  const bool bad = id < 0 || id >= V;
  const float nan = __uint_as_float(0x7fc00000u);
  bf16_t* dr = dz + row * V;
  if (V4) {
    for (int j = tid; j < V4; j += LP_THREADS) {
      const f32x4_t v = reinterpret_cast<const f32x4_t*>(zr)[j];
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fexp(v[i] - m) / s;
        o[i] = bad ? nan : g * ((4 * j + i == id ? 1.0f : 0.0f) - p);
      }
      *reinterpret_cast<uint2*>(dr + 4 * j) = make_uint2(pack_f2bf2(o[0], o[1]), pack_f2bf2(o[2], o[3]));
    }
  } else {
    for (int j = tid; j < V; j += LP_THREADS) {
      const float p = fexp(zr[j] - m) / s;
      dr[j] = f2bf(bad ? nan : g * ((j == id ? 1.0f : 0.0f) - p));
    }
  }
}

hipError_t launch_logprob_dz(const float* z, const int32_t* ids, const float* gout, void* dz, int M, int V,
                             hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(logprob_dz_kernel, dim3(M), dim3(LP_THREADS), 0, s, z, ids, gout, (bf16_t*)dz, V);
  return hipGetLastError();
}



// ---------------------------------------------------------------- RoPE backward
// The rotation's transpose at each token's position, with the forward's fp32 table:
// for the pair (x1, x2) = (e, d/2 + e) of a q or k head,
//   dx1 = dr1 c + dr2 s,  dx2 = dr2 c - dr1 s   (fp32, rounded to bf16 once),
// and the v heads' gradient passes through.  Output row t is dqkv [t] laid out as
// the forward's qkv row (q heads, k heads, v heads).  One workgroup per token; a
// thread owns 8 consecutive pairs of one head (16-byte loads and stores).
__global__ __launch_bounds__(256) void rope_backward_kernel(
    const bf16_t* __restrict__ dq, const bf16_t* __restrict__ dk, const bf16_t* __restrict__ dv,
    bf16_t* __restrict__ dqkv, const int32_t* __restrict__ tok_pos, const float* __restrict__ rcos,
    const float* __restrict__ rsin, int nq, int nkv, int d) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int t = blockIdx.x;
  const int half = d >> 1, upr = d >> 4;
  const int pos = tok_pos[t];
  const int n_heads = nq + 2 * nkv;
  for (int u = threadIdx.x; u < n_heads * upr; u += blockDim.x) {
    const int hd = u / upr, e0 = 8 * (u % upr);
    const bf16_t* src;
    if (hd < nq) src = dq + ((size_t)t * nq + hd) * d;
    else if (hd < nq + nkv) src = dk + ((size_t)t * nkv + hd - nq) * d;
    else src = dv + ((size_t)t * nkv + hd - nq - nkv) * d;
    u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src + e0);
    u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + half + e0);
    if (hd < nq + nkv) {
      const bf16_t* rl = reinterpret_cast<const bf16_t*>(&lo);
      const bf16_t* rh = reinterpret_cast<const bf16_t*>(&hi);
      float y1[8], y2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float c = rcos[(size_t)pos * half + e0 + i], sn = rsin[(size_t)pos * half + e0 + i];
        const float r1 = bf2f(rl[i]), r2 = bf2f(rh[i]);
        const float a1 = r1 * c, b1 = r2 * sn;
        const float a2 = r2 * c, b2 = r1 * sn;
        y1[i] = a1 + b1;
        y2[i] = a2 - b2;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = pack_f2bf2(y1[2 * i], y1[2 * i + 1]);
        hi[i] = pack_f2bf2(y2[2 * i], y2[2 * i + 1]);
      }
    }
    bf16_t* dst = dqkv + ((size_t)t * n_heads + hd) * d;
    *reinterpret_cast<u32x4_t*>(dst + e0) = lo;
    *reinterpret_cast<u32x4_t*>(dst + half + e0) = hi;
  }
}

hipError_t launch_rope_backward(const void* dq, const void* dk, const void* dv, void* dqkv,
                                const int32_t* tok_pos, const float* rcos, const float* rsin, int T, int nq,
                                int nkv, int d, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_backward_kernel, dim3(T), dim3(256), 0, s, static_cast<const bf16_t*>(dq),
                     static_cast<const bf16_t*>(dk), static_cast<const bf16_t*>(dv), static_cast<bf16_t*>(dqkv),
                     tok_pos, rcos, rsin, nq, nkv, d);
  return hipGetLastError();
}

}  // namespace bci
