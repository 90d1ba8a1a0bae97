// Device-side helpers shared by the gfx950 kernels of libbci.
//
// Every kernel that touches the same quantity uses the same helper, so the
// same inputs give the same bits in every phase: one bf16 rounding, one e4m3
// encoder/decoder, one exp/exp2/log, one reduction tree per shape.  The
// library is compiled with -ffp-contract=off, so a*b+c is never fused
// behind our back; an FMA appears only where written as __builtin_fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bci {

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (v_cvt_pk_bf16_f32): for every non-NaN fp32 input,
// denormals and infinities included, it gives the bits of the integer rule
// u + 0x7fff + ((u >> 16) & 1) >> 16, checked exhaustively over all 2^32
// patterns on gfx950; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf2(bf16_t lo, bf16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// two roundings packed into one word (lo in bits 0..15), one instruction
__device__ __forceinline__ uint32_t pack_f2bf2(float lo, float hi) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, bf2_t));
}

// ------------------------------------------------------ e4m3fn (OCP FP8)
// 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; S.1111.111 is
// NaN; largest finite 448.

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if ((c & 0x7fu) == 0x7fu) {
    v = __uint_as_float(0x7fc00000u);
  } else if (e == 0) {
    v = (float)m * 0.001953125f;  // m/8 * 2^-6, exact
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return (c & 0x80u) ? -v : v;
}

// x already clamped to [-448, 448] (NaN passes through to 0x7F).  Round to
// nearest even.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return 0x7fu;
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 8 -> 0x08 == 2^-6, consistent
  } else {
    const uint32_t ua = __float_as_uint(a);
    uint32_t e = (ua >> 23) - 127u + 7u;     // biased e4m3 exponent (>= 1 here)
    uint32_t m = (ua >> 20) & 7u;
    const uint32_t rem = ua & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) {
      if (++m == 8u) { m = 0; ++e; }
    }
    code = (e << 3) | m;
  }
  return code | sign;
}

// The one quantisation rule of the FP8 KV cache: per (token, head) row of d
// values with amax a: s = a / 448 (fp32, correctly rounded), 1 when a == 0.
__device__ __forceinline__ float kv_scale_from_amax(float amax) {
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}
__device__ __forceinline__ uint32_t kv_encode(float x, float s) {
  float q = x / s;
  q = fminf(fmaxf(q, -448.0f), 448.0f);
  return f32_to_e4m3(q);
}
// ... and the one dequantisation: bf(fp32(code) * s).
// e4m3fn -> fp32 of the four codes of a word by v_cvt_pk_f32_fp8 (byte i -> element i).
// On gfx950 this conversion is OCP e4m3fn; it equals e4m3_to_f32 above for all 256
// codes (NaN for NaN), checked on the GPU.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = a[0];
  f[1] = a[1];
  f[2] = b[0];
  f[3] = b[1];
}
__device__ __forceinline__ bf16_t kv_decode(uint32_t code, float s) {
  float f[4];
  e4m3x4_to_f32(code & 0xffu, f);
  return f2bf(f[0] * s);
}
// sixteen codes (one 16-byte load) -> sixteen products fp32(code) * s, not yet rounded
__device__ __forceinline__ void kv_decode16_f32(const uint32_t* w, float s, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e4m3x4_to_f32(w[i], x + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[4 * i + j] = x[4 * i + j] * s;
  }
}

// ------------------------------------------------------------ math

__device__ __forceinline__ float fexp(float x) { return expf(x); }
// v_exp_f32.  Compared with the library exp2f on all 2^32 inputs on gfx950: equal for
// every x >= -126; only results below 2^-126 (denormal range) differ.  exp2(0) = 1 and
// exp2(-inf) = 0 exactly, which the attention's no-op chunks rely on.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog(float x) { return logf(x); }
// SiLU g * sigma(g) = g * rcp(1 + 2^(-g log2 e)) on v_exp_f32 and v_rcp_f32 (about 1 ulp
// each), the activation of every forward schedule (tiled, skinny and split-K epilogues).
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * LOG2E));
}

// Attention output o = bf(ACC / L) evaluated as ACC * rcp(L) (v_rcp_f32, about 1 ulp):
// one reciprocal per row instead of a division per element, in every attention
// schedule (tiled, split + merge, sparse) alike.  L >= 1: the row's largest score
// contributes 2^0.
__device__ __forceinline__ float attn_inv_l(float L) { return __builtin_amdgcn_rcpf(L); }

// ------------------------------------------------- online-softmax rescaling
// x * f, except that a factor of exactly 1 returns x itself.  Every rescale and merge
// of online-softmax states (m, l, acc) in this library goes through this rule, so a
// kernel that skips a multiply by 1 for a whole wave and one that tests each value
// give the same bits, including where a multiply would quiet a NaN or flush a
// denormal.  In a merge max(M, m) is one of the two maxima, so one of the two
// factors 2^(M - max), 2^(m - max) is exactly 2^0 = 1.
__device__ __forceinline__ float mul_unless_one(float x, float f) { return f == 1.0f ? x : x * f; }

// x[i][r] <- mul_unless_one(x[i][r], f) with f per lane, as a branch: lanes with f == 1
// are masked off (their x untouched, no temporaries), and a wave in which no lane
// needs the multiply skips it.
template <int N>
__device__ __forceinline__ void scale_unless_one(f32x4_t (&x)[N], float f) {
  if (f != 1.0f) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[i][r] = x[i][r] * f;
  }
}

// ------------------------------------------------------ wave reductions
// Fixed xor butterflies over the 64 lanes (or a lane group).  For + the two
// partners add the same two values in either order, which IEEE addition
// makes bit-identical, so every lane ends with the same bits.

// Reductions over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the same position in each
// 16-lane row), every lane getting the result.  v_permlane16/32_swap leave each lane
// holding its own value and its partner's (order depends on the lane); max and fp32
// addition are commutative, so every lane computes (v_l (+) v_l^16) (+) (same for l^32).
__device__ __forceinline__ float xrow_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xrow_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The value of lane l ^ O, without a trip through LDS addressing where the hardware
// has a lane pattern for it: DPP quad permutes (O = 1, 2) and row rotate by 8 (O = 8),
// swizzle in bitmask mode (O = 4, 16) and the gfx950 half-wave swap (O = 32).  The bits
// are moved, not computed, so a butterfly built on it adds the same values in the same
// pairs as one built on __shfl_xor.
template <int O>
__device__ __forceinline__ float lane_xor(float v) {
  const int u = __float_as_int(v);
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
    return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
  } else if constexpr (O == 16) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(u, 0x401F));
  } else if constexpr (O == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(u, 0x128, 0xF, 0xF, true));
  } else if constexpr (O == 4) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(u, 0x101F));
  } else if constexpr (O == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(u, 0x4E, 0xF, 0xF, true));
  } else {
    static_assert(O == 1, "xor distance");
    return __int_as_float(__builtin_amdgcn_mov_dpp(u, 0xB1, 0xF, 0xF, true));
  }
}

// xor butterflies over all 64 lanes, distances 32, 16, 8, 4, 2, 1
__device__ __forceinline__ float wave_sum(float v) {
  v = v + lane_xor<32>(v);
  v = v + lane_xor<16>(v);
  v = v + lane_xor<8>(v);
  v = v + lane_xor<4>(v);
  v = v + lane_xor<2>(v);
  v = v + lane_xor<1>(v);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, lane_xor<32>(v));
  v = fmaxf(v, lane_xor<16>(v));
  v = fmaxf(v, lane_xor<8>(v));
  v = fmaxf(v, lane_xor<4>(v));
  v = fmaxf(v, lane_xor<2>(v));
  v = fmaxf(v, lane_xor<1>(v));
  return v;
}

}  // namespace bci
