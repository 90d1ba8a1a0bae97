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

// One workgroup per token, one wave per head (heads strided over the 4
// waves); lane i owns the rotation pair (i, i + d/2).  Scale rule: amax over
// the head's d rounded values (an exact max), s = amax / 448.
__global__ __launch_bounds__(256) void rope_kv_write_kernel(
    const bf16_t* __restrict__ qkv, bf16_t* __restrict__ q_out, const int32_t* __restrict__ tok_pos,
    const int32_t* __restrict__ tok_slot, const float* __restrict__ rcos,
    const float* __restrict__ rsin, KvLayer kv, int nq, int nkv, int d, int fp8) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = d >> 1;
  const int pos = tok_pos[t];
  const int slot = tok_slot[t];
  const int blk = slot >> 6, off = slot & 63;
  const int width = (nq + 2 * nkv) * d;
  const bf16_t* x = qkv + (size_t)t * width;
  const bool active = lane < half;
  const float c = active ? rcos[(size_t)pos * half + lane] : 0.0f;
  const float s = active ? rsin[(size_t)pos * half + lane] : 0.0f;

  for (int hd = wave; hd < nq + 2 * nkv; hd += 4) {
    bf16_t y1 = 0, y2 = 0;
    if (active) {
      const float x1 = bf2f(x[hd * d + lane]);
      const float x2 = bf2f(x[hd * d + lane + half]);
      if (hd < nq + nkv) {  // q and k heads are rotated
        const float a1 = x1 * c, b1 = x2 * s;
        const float a2 = x2 * c, b2 = x1 * s;
        y1 = f2bf(a1 - b1);
        y2 = f2bf(a2 + b2);
      } else {
        y1 = f2bf(x1);
        y2 = f2bf(x2);
      }
    }
    if (hd < nq) {
      if (active) {
        q_out[(size_t)t * nq * d + hd * d + lane] = y1;
        q_out[(size_t)t * nq * d + hd * d + lane + half] = y2;
      }
      continue;
    }
    const bool is_k = hd < nq + nkv;
    const int g = is_k ? hd - nq : hd - nq - nkv;
    const size_t row = ((size_t)blk * nkv + g) * 64 + off;  // cache row of (block, head, slot)
    if (!fp8) {
      bf16_t* dst = reinterpret_cast<bf16_t*>(is_k ? kv.k : kv.v) + row * d;
      if (active) {
        dst[lane] = y1;
        dst[lane + half] = y2;
      }
    } else {
      const float f1 = bf2f(y1), f2 = bf2f(y2);
      const float amax = wave_max(active ? fmaxf(fabsf(f1), fabsf(f2)) : 0.0f);
      const float sc = kv_scale_from_amax(amax);
      uint8_t* dst = reinterpret_cast<uint8_t*>(is_k ? kv.k : kv.v) + row * d;
      if (active) {
        dst[lane] = (uint8_t)kv_encode(f1, sc);
        dst[lane + half] = (uint8_t)kv_encode(f2, sc);
      }
      if (lane == 0) (is_k ? kv.ks : kv.vs)[row] = sc;
    }
  }
}

hipError_t launch_rope_kv_write(const void* qkv, void* q_out, const int32_t* tok_pos,
                                const int32_t* tok_slot, const float* rope_cos,
                                const float* rope_sin, KvLayer kv, int T, int nq, int nkv, int d,
                                bool fp8, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kv_write_kernel, dim3(T), dim3(256), 0, s, (const bf16_t*)qkv,
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
