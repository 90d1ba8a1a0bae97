// Backward of the causal GQA attention, deterministic (no atomics).
//
// The trainer adds its own backward to the inference forward and checks it against
// an independent reference (page "Finish RL Training Faster" digest, section
// "让训练前向使用推理的数值"); for the FP8 KV cache of the same section the keys and
// values the forward attended to are the dequantised ones, and the quantiser's
// gradient is taken as the identity (straight-through), so dK and dV below are also
// the gradients of the keys and values before quantisation.
//
// One sequence at positions 0..L-1; rows are (token, query head of the kv head's
// group) pairs as in the forward's tiles.  With t = (q . k) log2(e)/sqrt(d):
//   pass 1 (per 128-row query tile, 8 waves x 16 rows):
//     lse2 = log2-sum-exp2 of t over keys <= the row's position (online, per 64-key
//            chunk, the forward's expressions), D = sum_d dO o (fixed tree);
//     P = 2^(t - lse2), dP = dO . v, dS = P (dP - D),
//     dQ = (sum over 64-key chunks, ascending, of dS . K) / sqrt(d)
//   pass 2 (per 128-key tile, one wave per 16 keys; rows ascending in 64-row chunks):
//     dV = sum_rows P^T dO,  dK = (sum_rows dS^T Q) / sqrt(d)
//     With a part buffer and many rows, the rows are cut into P <= 4 fixed parts (by
//     row index, the same for every key tile); a tile's part writes its fp32 sums and a
//     third kernel adds the parts in ascending order, so the first key tiles (which see
//     every row) no longer set the pass's length.  One part gives the unsplit bits.
// Products on v_mfma_f32_16x16x32_bf16 with P and dS rounded to bf16 as operands (as P
// in the forward).  Each output element accumulates in one fixed order, so the result
// is deterministic; rows of dQ do not depend on other sequences.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int AB_CH = 64;             // keys per chunk / rows per chunk
constexpr int AB_TS = AB_CH + 4;      // stride of transposed tiles (bf16): 34 dwords, few bank conflicts

template <int D>
__device__ __forceinline__ int rswz(int row, int ch) {  // 16-byte chunk ch of a D-wide row
  if constexpr (D == 128)
    return row * (D / 8) + (ch ^ (row & 15));
  else
    return row * (D / 8) + (ch ^ ((row >> 1) & 7));
}

// 64 rows of D bf16 (row i from src_row(i), or zeros) -> rows (swizzled) and/or the
// transpose [D][AB_TS]; a unit is two consecutive rows x 8 columns, so the transpose
// is written as 4-byte pairs.  Consecutive lanes take consecutive row pairs (32 per
// column chunk): their transposed writes land on consecutive banks (lanes along a row's
// chunks would put 8 of them on each bank, the stride of 8 columns being 288 dwords).
template <int D, int NT, typename RowPtr>
__device__ __forceinline__ void stage(RowPtr src_row, int n_valid, u32x4_t* rows, bf16_t* tr, int tid) {
  for (int u = tid; u < (AB_CH / 2) * (D / 8); u += NT) {
    const int ip = u % (AB_CH / 2), pc = u / (AB_CH / 2);
    const int i0 = 2 * ip;
    u32x4_t va = u32x4_t{0, 0, 0, 0}, vb = va;
    if (i0 < n_valid) va = *reinterpret_cast<const u32x4_t*>(src_row(i0) + 8 * pc);
    if (i0 + 1 < n_valid) vb = *reinterpret_cast<const u32x4_t*>(src_row(i0 + 1) + 8 * pc);
    if (rows) {
      rows[rswz<D>(i0, pc)] = va;
      rows[rswz<D>(i0 + 1, pc)] = vb;
    }
    if (tr) {
      const bf16_t* ea = reinterpret_cast<const bf16_t*>(&va);
      const bf16_t* eb = reinterpret_cast<const bf16_t*>(&vb);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        *reinterpret_cast<uint32_t*>(tr + (8 * pc + k) * AB_TS + i0) = pack_bf2(ea[k], eb[k]);
    }
  }
}

// B operand (or A operand) of a 32-wide step made of the transposed tile: for column
// c, entries 32 k2 + 4 lg + 0..3 and 32 k2 + 16 + 4 lg + 0..3 (the P^T layout)
__device__ __forceinline__ bf16x8_t tr_frag(const bf16_t* tr, int c, int k2, int lg) {
  const bf16_t* r = tr + c * AB_TS + k2 * 32 + 4 * lg;
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(r);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(r + 16);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ bf16x8_t pack_frag(const float (&x)[4][4], int k2) {
  u32x4_t w;
  w[0] = pack_f2bf2(x[2 * k2][0], x[2 * k2][1]);
  w[1] = pack_f2bf2(x[2 * k2][2], x[2 * k2][3]);
  w[2] = pack_f2bf2(x[2 * k2 + 1][0], x[2 * k2 + 1][1]);
  w[3] = pack_f2bf2(x[2 * k2 + 1][2], x[2 * k2 + 1][3]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// ------------------------------------------------------------- pass 1: stats, dQ
constexpr int AB_WAVES = 8;                 // waves per workgroup (16 rows or keys each)
constexpr int AB_THREADS = AB_WAVES * 64;
constexpr int AB_TILE = AB_WAVES * 16;      // query rows (pass 1) or keys (pass 2) per workgroup

template <int D>
__global__ __launch_bounds__(AB_THREADS) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) u32x4_t Kr[AB_CH * D / 8];
  __shared__ __attribute__((aligned(16))) u32x4_t Vr[AB_CH * D / 8];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[D * AB_TS];
  const int tile = gridDim.x - 1 - blockIdx.x, g = blockIdx.y;  // longest (latest) tiles first
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int group = a.nq / a.nkv;
  const int row = tile * AB_TILE + wave * 16 + lc;
  const int tk = row / group, hq = g * group + row % group;
  const bool row_ok = tk < a.L;
  const int kmax = min(a.L - 1, (tile * AB_TILE + AB_TILE - 1) / group);  // last key any row needs
  const bf16_t* qrow = a.q + ((size_t)tk * a.nq + hq) * D;
  const bf16_t* dorow = a.dout + ((size_t)tk * a.nq + hq) * D;
  const bf16_t* orow = a.o + ((size_t)tk * a.nq + hq) * D;

  bf16x8_t qf[D / 32], dof[D / 32];
  float dpart = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4_t vq = u32x4_t{0, 0, 0, 0}, vd = vq, vo = vq;
    if (row_ok) {
      vq = *reinterpret_cast<const u32x4_t*>(qrow + ks * 32 + 8 * lg);
      vd = *reinterpret_cast<const u32x4_t*>(dorow + ks * 32 + 8 * lg);
      vo = *reinterpret_cast<const u32x4_t*>(orow + ks * 32 + 8 * lg);
    }
    qf[ks] = __builtin_bit_cast(bf16x8_t, vq);
    dof[ks] = __builtin_bit_cast(bf16x8_t, vd);
    const bf16_t* ed = reinterpret_cast<const bf16_t*>(&vd);
    const bf16_t* eo = reinterpret_cast<const bf16_t*>(&vo);
#pragma unroll
    for (int i = 0; i < 8; ++i) dpart = dpart + bf2f(ed[i]) * bf2f(eo[i]);
  }
  const float Drow = xrow_sum(dpart);

  auto krow = [&](int i) { return a.k + ((size_t)(i) * a.nkv + g) * D; };
  auto vrow = [&](int i) { return a.v + ((size_t)(i) * a.nkv + g) * D; };
  const int nchunks = kmax / AB_CH + 1;

  // pass 1a: (m, l) of the row over its keys
  float m = -INFINITY, l = 0.0f;
  for (int c = 0; c < nchunks; ++c) {
    if (c > 0) __syncthreads();
    const int base = c * AB_CH;
    stage<D, AB_THREADS>([&](int i) { return krow(base + i); }, min(AB_CH, a.L - base), Kr, nullptr, tid);
    __syncthreads();
    float t[4][4], mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Kr[rswz<D>(kt * 16 + lc, ks * 4 + lg)]),
                                                    qf[ks], s, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = base + kt * 16 + 4 * lg + r;
        t[kt][r] = (key <= tk) ? s[r] * a.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, t[kt][r]);
      }
    }
    mloc = xrow_max(mloc);
    const float mn = fmaxf(m, mloc);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    float rs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) rs = rs + fexp2(t[kt][r] - mu);
    rs = xrow_sum(rs);
    l = l * fexp2(m - mu) + rs;
    m = mn;
  }
  const float lse2 = m + __log2f(l);
  if (row_ok && lg == 0) {
    a.lse[(size_t)tk * a.nq + hq] = lse2;
    a.dsum[(size_t)tk * a.nq + hq] = Drow;
  }

  // pass 1b: dQ^T = sum over chunks of K^T . dS^T
  f32x4_t acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
    const int base = c * AB_CH;
    const int nv = min(AB_CH, a.L - base);
    stage<D, AB_THREADS>([&](int i) { return krow(base + i); }, nv, Kr, Kt, tid);
    stage<D, AB_THREADS>([&](int i) { return vrow(base + i); }, nv, Vr, nullptr, tid);
    __syncthreads();
    float ds[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f}, dp = s;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Kr[rswz<D>(kt * 16 + lc, ks * 4 + lg)]),
                                                    qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Vr[rswz<D>(kt * 16 + lc, ks * 4 + lg)]),
                                                     dof[ks], dp, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = base + kt * 16 + 4 * lg + r;
        const float p = (key <= tk && row_ok) ? fexp2(s[r] * a.scale_log2 - lse2) : 0.0f;
        ds[kt][r] = p * (dp[r] - Drow);
      }
    }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const bf16x8_t dsf = pack_frag(ds, k2);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag(Kt, dt * 16 + lc, k2, lg), dsf, acc[dt], 0, 0, 0);
    }
  }
  if (row_ok) {
    bf16_t* dq = a.dq + ((size_t)tk * a.nq + hq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2_t w = u32x2_t{pack_f2bf2(acc[dt][0] * a.scale, acc[dt][1] * a.scale),
                                pack_f2bf2(acc[dt][2] * a.scale, acc[dt][3] * a.scale)};
      *reinterpret_cast<u32x2_t*>(dq + dt * 16 + 4 * lg) = w;
    }
  }
}

// ------------------------------------------------------------- pass 2: dK, dV
template <int D>
__global__ __launch_bounds__(AB_THREADS) void attn_bwd_dkdv_kernel(AttnBwdArgs a, int n_parts, int part_rows) {
  __shared__ __attribute__((aligned(16))) u32x4_t Qr[AB_CH * D / 8];
  __shared__ __attribute__((aligned(16))) u32x4_t Or[AB_CH * D / 8];   // dO rows
  __shared__ __attribute__((aligned(16))) bf16_t Qt[D * AB_TS];
  __shared__ __attribute__((aligned(16))) bf16_t Ot[D * AB_TS];        // dO^T
  __shared__ float lse_s[AB_CH], dsum_s[AB_CH];
  __shared__ int tok_s[AB_CH];
  const int ktile = blockIdx.x / n_parts, part = blockIdx.x % n_parts, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int group = a.nq / a.nkv;
  const int key = ktile * AB_TILE + wave * 16 + lc;  // this lane's key (MFMA column)
  const bool key_ok = key < a.L;

  bf16x8_t kf[D / 32], vf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4_t vk = u32x4_t{0, 0, 0, 0}, vv = vk;
    if (key_ok) {
      vk = *reinterpret_cast<const u32x4_t*>(a.k + ((size_t)key * a.nkv + g) * D + ks * 32 + 8 * lg);
      vv = *reinterpret_cast<const u32x4_t*>(a.v + ((size_t)key * a.nkv + g) * D + ks * 32 + 8 * lg);
    }
    kf[ks] = __builtin_bit_cast(bf16x8_t, vk);
    vf[ks] = __builtin_bit_cast(bf16x8_t, vv);
  }
  f32x4_t dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    dk[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int n_rows_all = a.L * group;
  // rows of this (tile, part): from the first row whose token can see the tile, within the part
  const int row0 = max((ktile * AB_TILE) * group, part * part_rows);
  const int n_rows = min(n_rows_all, (part + 1) * part_rows);
  if (row0 >= n_rows) return;  // the whole workgroup: no row of this part sees the tile
  for (int rb = row0; rb < n_rows; rb += AB_CH) {
    if (rb > row0) __syncthreads();
    const int nv = min(AB_CH, n_rows - rb);
    auto qrow = [&](int i) {
      const int R = rb + i;
      return a.q + ((size_t)(R / group) * a.nq + g * group + R % group) * D;
    };
    auto drow = [&](int i) {
      const int R = rb + i;
      return a.dout + ((size_t)(R / group) * a.nq + g * group + R % group) * D;
    };
    stage<D, AB_THREADS>(qrow, nv, Qr, Qt, tid);
    stage<D, AB_THREADS>(drow, nv, Or, Ot, tid);
    if (tid < AB_CH) {
      const int R = rb + tid;
      const bool ok = tid < nv;
      const size_t idx = ok ? (size_t)(R / group) * a.nq + g * group + R % group : 0;
      lse_s[tid] = ok ? a.lse[idx] : 0.0f;
      dsum_s[tid] = ok ? a.dsum[idx] : 0.0f;
      tok_s[tid] = ok ? R / group : -1;
    }
    __syncthreads();
    // S[row][key] = Q . K^T and dP = dO . V^T, rows 16 rt + 4 lg + r of the chunk
    float p[4][4], ds[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f}, dp = s;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Qr[rswz<D>(rt * 16 + lc, ks * 4 + lg)]),
                                                    kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, Or[rswz<D>(rt * 16 + lc, ks * 4 + lg)]),
                                                     vf[ks], dp, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rt * 16 + 4 * lg + r;
        const int tq = tok_s[i];
        const float pv = (key_ok && tq >= key) ? fexp2(s[r] * a.scale_log2 - lse_s[i]) : 0.0f;
        p[rt][r] = pv;
        ds[rt][r] = pv * (dp[r] - dsum_s[i]);
      }
    }
    // dV^T += dO^T . P, dK^T += Q^T . dS (contraction over the chunk's rows)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const bf16x8_t pf = pack_frag(p, k2), dsf = pack_frag(ds, k2);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        dv[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag(Ot, dt * 16 + lc, k2, lg), pf, dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_frag(Qt, dt * 16 + lc, k2, lg), dsf, dk[dt], 0, 0, 0);
      }
    }
  }
  if (key_ok && n_parts > 1) {  // fp32 sums of this part
    float* pk = a.part + (((size_t)part * a.L + key) * a.nkv + g) * D;
    float* pv = pk + (size_t)AB_MAX_PARTS * a.L * a.nkv * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      *reinterpret_cast<f32x4_t*>(pk + dt * 16 + 4 * lg) = dk[dt];
      *reinterpret_cast<f32x4_t*>(pv + dt * 16 + 4 * lg) = dv[dt];
    }
  } else if (key_ok) {
    bf16_t* dkr = a.dk + ((size_t)key * a.nkv + g) * D;
    bf16_t* dvr = a.dv + ((size_t)key * a.nkv + g) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      *reinterpret_cast<u32x2_t*>(dkr + dt * 16 + 4 * lg) =
          u32x2_t{pack_f2bf2(dk[dt][0] * a.scale, dk[dt][1] * a.scale), pack_f2bf2(dk[dt][2] * a.scale, dk[dt][3] * a.scale)};
      *reinterpret_cast<u32x2_t*>(dvr + dt * 16 + 4 * lg) =
          u32x2_t{pack_f2bf2(dv[dt][0], dv[dt][1]), pack_f2bf2(dv[dt][2], dv[dt][3])};
    }
  }
}

// dK, dV = the parts' fp32 sums in ascending part order (only the parts that saw the
// key's tile), then bf16 (dK times 1/sqrt(d) first, as in the unsplit pass).  One thread
// per 4 consecutive elements of a (key, kv head) row.
__global__ __launch_bounds__(256) void attn_bwd_part_sum_kernel(AttnBwdArgs a, int n_parts, int part_rows) {
  const int group = a.nq / a.nkv;
  const size_t n4 = (size_t)a.L * a.nkv * a.d / 4;
  const size_t pstride = (size_t)a.L * a.nkv * a.d;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = 4 * i;
    const int key = (int)(e / ((size_t)a.nkv * a.d));
    const int p0 = ((key / AB_TILE) * AB_TILE * group) / part_rows;
    f32x4_t sk = *reinterpret_cast<const f32x4_t*>(a.part + p0 * pstride + e);
    f32x4_t sv = *reinterpret_cast<const f32x4_t*>(a.part + (AB_MAX_PARTS + p0) * pstride + e);
    for (int p = p0 + 1; p < n_parts; ++p) {
      const f32x4_t xk = *reinterpret_cast<const f32x4_t*>(a.part + p * pstride + e);
      const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(a.part + (AB_MAX_PARTS + p) * pstride + e);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sk[r] = sk[r] + xk[r];
        sv[r] = sv[r] + xv[r];
      }
    }
    *reinterpret_cast<u32x2_t*>(a.dk + e) =
        u32x2_t{pack_f2bf2(sk[0] * a.scale, sk[1] * a.scale), pack_f2bf2(sk[2] * a.scale, sk[3] * a.scale)};
    *reinterpret_cast<u32x2_t*>(a.dv + e) = u32x2_t{pack_f2bf2(sv[0], sv[1]), pack_f2bf2(sv[2], sv[3])};
  }
}

template <int D>
static void launch_ab(const AttnBwdArgs& a, hipStream_t s) {
  const int group = a.nq / a.nkv;
  const int n_rows = a.L * group;
  int n_parts = 1, part_rows = n_rows;
  if (a.part) {
    n_parts = std::min(AB_MAX_PARTS, std::max(1, n_rows / AB_PART_MIN_ROWS));
    part_rows = ((n_rows + n_parts - 1) / n_parts + AB_CH - 1) / AB_CH * AB_CH;
    n_parts = (n_rows + part_rows - 1) / part_rows;
  }
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), dim3((a.L * group + AB_TILE - 1) / AB_TILE, a.nkv),
                     dim3(AB_THREADS), 0, s, a);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), dim3((a.L + AB_TILE - 1) / AB_TILE * n_parts, a.nkv),
                     dim3(AB_THREADS), 0, s, a, n_parts, part_rows);
  if (n_parts > 1) {
    const size_t n4 = (size_t)a.L * a.nkv * a.d / 4;
    hipLaunchKernelGGL(attn_bwd_part_sum_kernel, dim3((unsigned)std::min<size_t>((n4 + 255) / 256, 8192)),
                       dim3(256), 0, s, a, n_parts, part_rows);
  }
}

hipError_t launch_attention_backward(const AttnBwdArgs& a, hipStream_t s) {
  if (a.L == 0) return hipSuccess;
  if (a.d == 128)
    launch_ab<128>(a, s);
  else if (a.d == 64)
    launch_ab<64>(a, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bci
