// RoPE on q and k, KV-cache write (bf16 or FP8 e4m3), and the standalone
// gather + dequantise of a sequence's cache.
//
// FP8 KV: the cache stays in FP8; prefill, decode and the training
// recompute all read it back by gathering and converting to BF16 before the
// one attention operator, and the recompute writes its private cache copy
// through the same FP8 round trip (page "Finish RL Training Faster" digest,
// section "让训练前向使用推理的数值", FP8 KV paragraph and figure caption).
// Every phase therefore writes the cache through launch_rope_kv_write and
// reads it through kv_decode (common.h), here and inside the attention kernel.
//
// Cache layout per layer: [n_blocks][n_kv][64][d] (codes or bf16) and
// [n_blocks][n_kv][64] fp32 scales, so one (block, kv head) chunk of 64 keys
// is contiguous for the attention kernel's loads.
#include "common.h"
#include "kernels.h"

namespace bci {

// One workgroup per token.  Work unit u = (head u / (d/16), chunk j = u % (d/16)):
// one thread owns the 8 rotation pairs (8j + i, d/2 + 8j + i), i = 0..7, so
// every load and store moves 16 bytes; the d/16 units of a head are
// consecutive lanes of one wave.  Scale rule: amax over the head's d rounded
// values (an exact max, so the reduction order is immaterial), s = amax / 448.
__global__ __launch_bounds__(256) void rope_kv_write_kernel(
    const bf16_t* __restrict__ qkv, bf16_t* __restrict__ q_out, const int32_t* __restrict__ tok_pos,
    const int32_t* __restrict__ tok_slot, const float* __restrict__ rcos,
    const float* __restrict__ rsin, KvLayer kv, int nq, int nkv, int d, int fp8) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4v_t __attribute__((ext_vector_type(4)));
  const int t = blockIdx.x;
  const int half = d >> 1;
  const int upr = d >> 4;  // units (threads) per head
  const int pos = tok_pos[t];
  const int slot = tok_slot[t];
  const int blk = slot >> 6, off = slot & 63;
  const int n_heads = nq + 2 * nkv;
  const bf16_t* x = qkv + (size_t)t * n_heads * d;
  for (int u = threadIdx.x; u < n_heads * upr; u += blockDim.x) {
    const int hd = u / upr, j = u % upr;
    const int e0 = 8 * j;  // first element of the pair's low half
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(x + hd * d + e0);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(x + hd * d + half + e0);
    const bf16_t* xl = reinterpret_cast<const bf16_t*>(&lo);
    const bf16_t* xh = reinterpret_cast<const bf16_t*>(&hi);
    float y1[8], y2[8];
    if (hd < nq + nkv) {  // q and k heads are rotated
      const f32x4v_t c0 = *reinterpret_cast<const f32x4v_t*>(rcos + (size_t)pos * half + e0);
      const f32x4v_t c1 = *reinterpret_cast<const f32x4v_t*>(rcos + (size_t)pos * half + e0 + 4);
      const f32x4v_t s0 = *reinterpret_cast<const f32x4v_t*>(rsin + (size_t)pos * half + e0);
      const f32x4v_t s1 = *reinterpret_cast<const f32x4v_t*>(rsin + (size_t)pos * half + e0 + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float c = i < 4 ? c0[i] : c1[i - 4];
        const float sn = i < 4 ? s0[i] : s1[i - 4];
        const float x1 = bf2f(xl[i]), x2 = bf2f(xh[i]);
        const float a1 = x1 * c, b1 = x2 * sn;
        const float a2 = x2 * c, b2 = x1 * sn;
        y1[i] = bf2f(f2bf(a1 - b1));
        y2[i] = bf2f(f2bf(a2 + b2));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        y1[i] = bf2f(xl[i]);
        y2[i] = bf2f(xh[i]);
      }
    }
    if (hd < nq || !fp8) {
      u32x4_t wl, wh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wl[i] = pack_f2bf2(y1[2 * i], y1[2 * i + 1]);
        wh[i] = pack_f2bf2(y2[2 * i], y2[2 * i + 1]);
      }
      bf16_t* dst;
      if (hd < nq) {
        dst = q_out + (size_t)t * nq * d + hd * d;
      } else {
        const bool is_k = hd < nq + nkv;
        const int g = is_k ? hd - nq : hd - nq - nkv;
        const size_t row = ((size_t)blk * nkv + g) * 64 + off;  // cache row of (block, head, slot)
        dst = reinterpret_cast<bf16_t*>(is_k ? kv.k : kv.v) + row * d;
      }
      *reinterpret_cast<u32x4_t*>(dst + e0) = wl;
      *reinterpret_cast<u32x4_t*>(dst + half + e0) = wh;
    } else {
      const bool is_k = hd < nq + nkv;
      const int g = is_k ? hd - nq : hd - nq - nkv;
      const size_t row = ((size_t)blk * nkv + g) * 64 + off;
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(y1[i]), fabsf(y2[i])));
      for (int o = 1; o < upr; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
      const float sc = kv_scale_from_amax(amax);
      uint32_t c1[2] = {0, 0}, c2[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c1[i >> 2] |= kv_encode(y1[i], sc) << (8 * (i & 3));
        c2[i >> 2] |= kv_encode(y2[i], sc) << (8 * (i & 3));
      }
      uint8_t* dst = reinterpret_cast<uint8_t*>(is_k ? kv.k : kv.v) + row * d;
      *reinterpret_cast<uint2*>(dst + e0) = make_uint2(c1[0], c1[1]);
      *reinterpret_cast<uint2*>(dst + half + e0) = make_uint2(c2[0], c2[1]);
      if (j == 0) (is_k ? kv.ks : kv.vs)[row] = sc;
    }
  }
}

hipError_t launch_rope_kv_write(const void* qkv, void* q_out, const int32_t* tok_pos,
                                const int32_t* tok_slot, const float* rope_cos,
                                const float* rope_sin, KvLayer kv, int T, int nq, int nkv, int d,
                                bool fp8, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int units = (nq + 2 * nkv) * (d / 16);
  const int threads = units >= 256 ? 256 : (units + 63) / 64 * 64;
  hipLaunchKernelGGL(rope_kv_write_kernel, dim3(T), dim3(threads), 0, s, (const bf16_t*)qkv,
                     (bf16_t*)q_out, tok_pos, tok_slot, rope_cos, rope_sin, kv, nq, nkv, d,
                     (int)fp8);
  return hipGetLastError();
}

// k_out/v_out [n_pos, nkv, d] bf16 for positions 0..n_pos-1 of one sequence
// whose block row (block ids of positions 64j..64j+63) is block_row.
__global__ __launch_bounds__(256) void kv_gather_kernel(KvLayer kv, const int32_t* __restrict__ block_row,
                                                        int n_pos, int nkv, int d, int fp8,
                                                        bf16_t* __restrict__ k_out,
                                                        bf16_t* __restrict__ v_out) {
  const int p = blockIdx.x;
  const int blk = block_row[p >> 6], off = p & 63;
  for (int e = threadIdx.x; e < nkv * d; e += 256) {
    const int g = e / d, i = e % d;
    const size_t row = ((size_t)blk * nkv + g) * 64 + off;
    bf16_t kk, vv;
    if (fp8) {
      kk = kv_decode(reinterpret_cast<const uint8_t*>(kv.k)[row * d + i], kv.ks[row]);
      vv = kv_decode(reinterpret_cast<const uint8_t*>(kv.v)[row * d + i], kv.vs[row]);
    } else {
      kk = reinterpret_cast<const bf16_t*>(kv.k)[row * d + i];
      vv = reinterpret_cast<const bf16_t*>(kv.v)[row * d + i];
    }
    k_out[(size_t)p * nkv * d + e] = kk;
    v_out[(size_t)p * nkv * d + e] = vv;
  }
}

hipError_t launch_kv_gather(KvLayer kv, const int32_t* block_row, int n_pos, int nkv, int d,
                            bool fp8, void* k_out, void* v_out, hipStream_t s) {
  if (n_pos == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_gather_kernel, dim3(n_pos), dim3(256), 0, s, kv, block_row, n_pos, nkv,
                     d, (int)fp8, (bf16_t*)k_out, (bf16_t*)v_out);
  return hipGetLastError();
}

}  // namespace bci
