// Sparse attention over a Top-K selected key set, on the FP8 KV path.
//
// The DeepSeek-V4-Flash recipe fixes the tie rule of its sparse-attention
// Top-K, lists the selected set in a fixed position order so that the same
// set is always summed in the same order, and feeds every phase the FP8
// cache gathered and dequantised to BF16 before one sparse attention
// operator (page "Finish RL Training Faster" digest, section
// "让训练前向使用推理的数值" and its figure caption).  The pages name no
// scoring function; the index score here is the indexer of DeepSeek's sparse
// attention, score(t, s) = sum_h w[t,h] * relu(q_I[t,h] . k_I[s]), with the
// index keys kept in the FP8 cache format and read back through the same
// dequantiser as K and V.
//
// Four kernels, each giving a token the same bits in any batch and phase:
//   index_key_write   one index key per token into the paged FP8 index cache
//                     (the KV cache's quantisation rule: per-token amax / 448)
//   index_scores      for every key s <= pos(t), on MFMA:
//                       dot_h = q_I[t,h] . bf(code * scale)   (ascending 32-wide d
//                               steps of v_mfma_f32_16x16x32_bf16)
//                       lane chain over its 16 heads h = 16ht + 4g + r (ht major):
//                               v = fma(w_h, max(dot_h, 0), v) from v = 0
//                       then the four lane groups g added by xrow_sum.
//                     Two schedules (keys straight from memory for decode-like
//                     calls, keys staged once in LDS for four query tokens of a
//                     sequence otherwise) run this same chain per (t, s).
//   sparse_topk       radix select of the K-th largest order key, then the
//                     selected positions written in ascending order; ties go
//                     to the lower position.  Integer work: exact.
//   sparse_attention  per (token, kv head): the list cut into segments of 256
//                     entries (one wave each), 64-entry chunks in list order
//                     with the dense operator's online-softmax expressions,
//                     segments merged in ascending order.  With every key
//                     selected this is, expression for expression, the dense
//                     kernel with 256-key segments.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int SCHUNK = 64;           // entries (keys) per chunk
constexpr int SSEG = 256;            // list entries per segment (one wave)
constexpr int SVT_STRIDE = SCHUNK + 8;

// eight e4m3 codes (one 8-byte word pair) -> eight bf(fp32(code) * s)
__device__ __forceinline__ bf16x8_t dequant8(u32x2_t w, float s) {
  float f[8];
  e4m3x4_to_f32(w[0], f);
  e4m3x4_to_f32(w[1], f + 4);
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_f2bf2(f[2 * i] * s, f[2 * i + 1] * s);
  return __builtin_bit_cast(bf16x8_t, o);
}

// ------------------------------------------------------------ index keys

template <int DI>
__global__ __launch_bounds__(256) void index_key_write_kernel(const bf16_t* kidx,
                                                              const int32_t* tok_slot,
                                                              uint8_t* codes, float* scales, int T) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  constexpr int PER = DI / 64;
  const bf16_t* row = kidx + (size_t)t * DI;
  float x[PER];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    x[i] = bf2f(row[PER * lane + i]);
    amax = fmaxf(amax, fabsf(x[i]));
  }
  amax = wave_max(amax);
  const float s = kv_scale_from_amax(amax);
  const size_t slot = (size_t)tok_slot[t];
  if constexpr (PER == 2) {
    const uint32_t c = kv_encode(x[0], s) | (kv_encode(x[1], s) << 8);
    reinterpret_cast<uint16_t*>(codes + slot * DI)[lane] = (uint16_t)c;
  } else {
    codes[slot * DI + lane] = (uint8_t)kv_encode(x[0], s);
  }
  if (lane == 0) scales[slot] = s;
}

hipError_t launch_index_key_write(const void* kidx, const int32_t* tok_slot, void* codes,
                                  float* scales, int T, int DI, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + 3) / 4);
  if (DI == 128)
    hipLaunchKernelGGL(index_key_write_kernel<128>, grid, dim3(256), 0, s,
                       (const bf16_t*)kidx, tok_slot, (uint8_t*)codes, scales, T);
  else if (DI == 64)
    hipLaunchKernelGGL(index_key_write_kernel<64>, grid, dim3(256), 0, s,
                       (const bf16_t*)kidx, tok_slot, (uint8_t*)codes, scales, T);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------ index scores

// The per-(token, key) chain shared by both schedules: MFMA dot products of the
// wave's token's index heads (A operand, rows) with 64 keys (B operand,
// columns: key 16kt + lc of the block), relu, weighted head sum.  Lane group lg
// returns the scores of keys 16 lg + lc.
template <int NHT, int DI, typename Fetch>
__device__ __forceinline__ float index_chain(const bf16x8_t (&qa)[NHT][DI / 32], Fetch fetch,
                                             const float (&wv)[NHT][4], int lg) {
  float out = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    bf16x8_t kb[DI / 32];
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks) kb[ks] = fetch(kt, ks);
    float v = 0.0f;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x4_t d = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DI / 32; ++ks)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][ks], kb[ks], d, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) v = __builtin_fmaf(wv[ht][r], fmaxf(d[r], 0.0f), v);
    }
    v = xrow_sum(v);
    if (lg == kt) out = v;
  }
  return out;
}

template <int NHT, int DI>
__device__ __forceinline__ void index_load_query(const IdxArgs& a, int t, bool ok, int lg, int lc,
                                                 bf16x8_t (&qa)[NHT][DI / 32],
                                                 float (&wv)[NHT][4]) {
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) {
    const bf16_t* qrow = a.q + ((size_t)t * a.heads + 16 * ht + lc) * DI;
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks) {
      u32x4_t v = u32x4_t{0, 0, 0, 0};
      if (ok) v = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks + 8 * lg);
      qa[ht][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[ht][r] = ok ? a.w[(size_t)t * a.heads + 16 * ht + 4 * lg + r] : 0.0f;
  }
}

template <int DI>
__device__ __forceinline__ int iswz(int key, int ch) {
  if constexpr (DI == 128)
    return key * (DI / 8) + (ch ^ (key & 15));
  else
    return key * (DI / 8) + (ch ^ ((key >> 1) & 7));
}

// Decode-like schedule: one token per workgroup row of the grid; wave w of
// workgroup x takes key blocks x*4 + w, then + 4*gridDim.x, ... (64 keys each),
// reading the codes straight into the B operand (dequantised in registers).  A
// prefetch of the next block's codes was measured slower (more registers, fewer
// waves per SIMD) and is not used.
template <int DI>
struct RawKeys {
  u32x2_t c[4][DI / 32];
  float sc[4];
};

template <int DI>
__device__ __forceinline__ void raw_keys_load(const IdxArgs& a, const int* btab, int s0, int pos,
                                              int lg, int lc, RawKeys<DI>& r) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int s = min(s0 + 16 * kt + lc, pos);
    const size_t slot = (size_t)btab[s >> 6] * SCHUNK + (s & 63);
    r.sc[kt] = a.scales[slot];
    const uint8_t* crow = a.codes + slot * DI;
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks)
      r.c[kt][ks] = *reinterpret_cast<const u32x2_t*>(crow + 32 * ks + 8 * lg);
  }
}

template <int NHT, int DI>
__global__ __launch_bounds__(256) void index_scores_direct(IdxArgs a) {
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int pos = a.tok_pos[t];
  const int nblk = pos / SCHUNK + 1;
  const int step = 4 * gridDim.x;
  int b = blockIdx.x * 4 + wave;
  if (b >= nblk) return;
  const int* btab = a.block_table + (size_t)a.tok_seq[t] * a.max_blocks;

  RawKeys<DI> cur;
  raw_keys_load<DI>(a, btab, b * SCHUNK, pos, lg, lc, cur);
  bf16x8_t qa[NHT][DI / 32];
  float wv[NHT][4];
  index_load_query<NHT, DI>(a, t, true, lg, lc, qa, wv);
  float* srow = a.scores + (size_t)t * a.stride;

  while (true) {
    const int bn = b + step;
    const float v = index_chain<NHT, DI>(
        qa, [&](int kt, int ks) { return dequant8(cur.c[kt][ks], cur.sc[kt]); }, wv, lg);
    const int s = b * SCHUNK + 16 * lg + lc;
    if (s <= pos) srow[s] = v;
    if (bn >= nblk) break;
    b = bn;
    raw_keys_load<DI>(a, btab, bn * SCHUNK, pos, lg, lc, cur);
  }
}

// Prefill-like schedule: a tile of up to four consecutive tokens of one
// sequence (one wave each) shares each 64-key block, dequantised once into LDS.
constexpr int IDX_STAGE_KEYS = 256;  // keys per workgroup

template <int NHT, int DI>
__global__ __launch_bounds__(256) void index_scores_staged(IdxArgs a) {
  __shared__ __attribute__((aligned(16))) u32x4_t Ks[SCHUNK * DI / 8];
  const int tile = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int seq = a.tiles[4 * tile + 0];
  const int tok_begin = a.tiles[4 * tile + 1];
  const int n_tok = a.tiles[4 * tile + 2];
  const int pos_begin = a.tiles[4 * tile + 3];
  const int kmax = pos_begin + n_tok - 1;
  const int s_begin = blockIdx.x * IDX_STAGE_KEYS;
  if (s_begin > kmax) return;
  const int* btab = a.block_table + (size_t)seq * a.max_blocks;
  const bool ok = wave < n_tok;
  const int t = tok_begin + wave;
  const int pos = pos_begin + wave;

  bf16x8_t qa[NHT][DI / 32];
  float wv[NHT][4];
  index_load_query<NHT, DI>(a, t, ok, lg, lc, qa, wv);

  constexpr int CPK = DI / 32;  // 32-code pieces per key row (2 or 4 threads per key)
  for (int it = 0; it < IDX_STAGE_KEYS / SCHUNK; ++it) {
    const int s0 = s_begin + it * SCHUNK;
    if (s0 > kmax) break;
    if (it > 0) __syncthreads();  // the previous block's LDS reads are done
    for (int u = tid; u < SCHUNK * CPK; u += 256) {
      const int key = u / CPK, pc = u % CPK;
      const int s = min(s0 + key, kmax);
      const size_t slot = (size_t)btab[s >> 6] * SCHUNK + (s & 63);
      const float sc = a.scales[slot];
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.codes + slot * DI + 32 * pc);
      const u32x4_t lo = src[0], hi = src[1];
      Ks[iswz<DI>(key, 4 * pc + 0)] = __builtin_bit_cast(u32x4_t, dequant8(u32x2_t{lo[0], lo[1]}, sc));
      Ks[iswz<DI>(key, 4 * pc + 1)] = __builtin_bit_cast(u32x4_t, dequant8(u32x2_t{lo[2], lo[3]}, sc));
      Ks[iswz<DI>(key, 4 * pc + 2)] = __builtin_bit_cast(u32x4_t, dequant8(u32x2_t{hi[0], hi[1]}, sc));
      Ks[iswz<DI>(key, 4 * pc + 3)] = __builtin_bit_cast(u32x4_t, dequant8(u32x2_t{hi[2], hi[3]}, sc));
    }
    __syncthreads();
    if (ok && s0 <= pos) {
      const float v = index_chain<NHT, DI>(
          qa,
          [&](int kt, int ks) {
            return __builtin_bit_cast(bf16x8_t, Ks[iswz<DI>(16 * kt + lc, 4 * ks + lg)]);
          },
          wv, lg);
      const int s = s0 + 16 * lg + lc;
      if (s <= pos) a.scores[(size_t)t * a.stride + s] = v;
    }
  }
}

template <int NHT, int DI>
static void launch_scores_t(const IdxArgs& a, bool staged, hipStream_t s) {
  if (staged)
    hipLaunchKernelGGL((index_scores_staged<NHT, DI>),
                       dim3((a.max_pos + IDX_STAGE_KEYS) / IDX_STAGE_KEYS, a.n_tiles), dim3(256), 0,
                       s, a);
  else {
    // blocks per wave: enough workgroups to fill the chip, then longer runs per wave
    // so that the token's index query is loaded once per several key blocks
    const int max_blk = a.max_pos / SCHUNK + 1;
    const long long waves = (long long)a.T * max_blk;
    const int per_wave = (int)std::min<long long>(8, std::max<long long>(1, waves / 8192));
    const int gx = (max_blk + 4 * per_wave - 1) / (4 * per_wave);
    hipLaunchKernelGGL((index_scores_direct<NHT, DI>), dim3(gx, a.T), dim3(256), 0, s, a);
  }
}

hipError_t launch_index_scores(const IdxArgs& a, bool staged, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nht = a.heads / 16;
  if (a.dim == 128) {
    switch (nht) {
      case 1: launch_scores_t<1, 128>(a, staged, s); break;
      case 2: launch_scores_t<2, 128>(a, staged, s); break;
      case 4: launch_scores_t<4, 128>(a, staged, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if (a.dim == 64) {
    switch (nht) {
      case 1: launch_scores_t<1, 64>(a, staged, s); break;
      case 2: launch_scores_t<2, 64>(a, staged, s); break;
      case 4: launch_scores_t<4, 64>(a, staged, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ Top-K

// Order key of an fp32 score: a larger score gives a larger unsigned key.
// NaN ranks above every number; -0 and +0 are the same score.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0x7fc00000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_EPT = 64;      // positions per thread held in registers: rows up to 65536
constexpr int TK_BINS = 4096;   // first digit: up to 12 bits below the row's common prefix
constexpr int TK_CAP = 4096;    // keys of the chosen first-digit bin kept in LDS

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, WAVE);
    if (lane >= o) v += y;
  }
  return v;
}

struct TopkShared {
  uint32_t hist[TK_BINS + 1];  // + a spare bin that takes the placeholder keys' adds
  uint32_t cand[TK_CAP];
  uint32_t wg[TK_WAVES], we[TK_WAVES];
  uint32_t digit, above, ncand, kmin, kmax;
};

// Exclusive prefix over the workgroup (thread order) of two counters; also
// returns the totals.
__device__ __forceinline__ void topk_block_scan(TopkShared& sh, uint32_t cg, uint32_t ce, int tid,
                                                uint32_t& pg, uint32_t& pe, uint32_t& tg,
                                                uint32_t& te) {
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t ig = wave_incl_scan(cg, lane), ie = wave_incl_scan(ce, lane);
  if (lane == 63) {
    sh.wg[wave] = ig;
    sh.we[wave] = ie;
  }
  __syncthreads();
  pg = ig - cg;
  pe = ie - ce;
  tg = 0;
  te = 0;
  for (int w = 0; w < TK_WAVES; ++w) {
    const uint32_t a = sh.wg[w], b = sh.we[w];
    if (w < wave) {
      pg += a;
      pe += b;
    }
    tg += a;
    te += b;
  }
  __syncthreads();  // wg/we may be rewritten after this
}

// After a histogram of nb bins (all threads call): sh.digit = the bin holding the
// kk-th largest counted key, sh.above = the count in higher bins.  Thread tid owns
// bins nb-1-tid*bpt down to nb-(tid+1)*bpt (descending order = thread order).
__device__ __forceinline__ void topk_pick(TopkShared& sh, int nb, uint32_t kk, int tid) {
  const int bpt = nb > TK_THREADS ? nb / TK_THREADS : 1;
  const int hi = nb - 1 - tid * bpt;
  uint32_t c[TK_BINS / TK_THREADS], sum = 0;
#pragma unroll
  for (int j = 0; j < TK_BINS / TK_THREADS; ++j) {
    c[j] = (j < bpt && hi - j >= 0) ? sh.hist[hi - j] : 0u;
    sum += c[j];
  }
  uint32_t above, dummy, t0, t1;
  topk_block_scan(sh, sum, 0u, tid, above, dummy, t0, t1);
#pragma unroll
  for (int j = 0; j < TK_BINS / TK_THREADS; ++j) {
    if (above < kk && kk <= above + c[j]) {
      sh.digit = (uint32_t)(hi - j);
      sh.above = above;
    }
    above += c[j];
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o, WAVE));
  return v;
}

// Rows of up to TK_THREADS * TK_EPT positions.  Thread tid holds positions
// [tid * ept, tid * ept + ept) as order keys in registers (the row is read once);
// slots past the row hold 0, below every real key (the smallest, that of -inf, is
// 0x007fffff).  The K-th largest key tau is found in up to three steps:
//   1. the row's smallest and largest keys: the bits above their highest
//      differing bit are common to every key;
//   2. a histogram of the next (up to) 12 bits picks the bin holding the K-th
//      largest key -- these bits vary across the row, so the LDS adds spread;
//   3. the keys of that bin (usually few) are copied to LDS and the remaining
//      bits are resolved there, 10 at a time; a bin too full for LDS is resolved
//      in the registers instead, 8 bits at a time.
// tau and kk (how many keys equal to tau are taken) are exact integer results,
// independent of the order of the LDS adds.
__device__ __forceinline__ void topk_registers(TopkShared& sh, const float* row, int n, int K,
                                               int32_t* out, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int ept = (((n + TK_THREADS - 1) / TK_THREADS) + 3) & ~3;  // workgroup-uniform
  const int p0 = tid * ept;
  const int nv = max(0, min(ept, n - p0));
  // one 16-byte load per group of four; a group that starts inside the row may run
  // past its end, but never past the row's stride (a multiple of 4): those slots,
  // and whole groups past the row (read from the row start instead), become 0
  uint32_t key[TK_EPT];
#pragma unroll
  for (int j = 0; j < TK_EPT / 4; ++j) {
    if (4 * j >= ept) continue;
    const int off = 4 * j < nv ? p0 + 4 * j : 0;
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + off);
#pragma unroll
    for (int c = 0; c < 4; ++c) key[4 * j + c] = (4 * j + c < nv) ? order_key(v[c]) : 0u;
  }
  // 1. min and max over the real keys
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < TK_EPT; ++e) {
    if (e >= ept) continue;
    mn = min(mn, key[e] != 0u ? key[e] : 0xffffffffu);
    mx = max(mx, key[e]);
  }
  mn = wave_umin(mn);
  mx = wave_umax(mx);
  if (lane == 0) {
    sh.wg[wave] = mn;
    sh.we[wave] = mx;
  }
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
  for (int w = 0; w < TK_WAVES; ++w) {
    mn = min(mn, sh.wg[w]);
    mx = max(mx, sh.we[w]);
  }
  __syncthreads();
  uint32_t tau, kk = (uint32_t)K;
  if (mn == mx) {
    tau = mn;  // every key equal: the first K positions
  } else {
    const int rb = 32 - __clz(mn ^ mx);            // bits below the common prefix
    const uint32_t common = rb == 32 ? 0u : (mx >> rb) << rb;
    const int wa = min(rb, 12), sha = rb - wa;
    const int nba = 1 << wa;
    // 2. first digit
    for (int i = tid; i <= TK_BINS; i += TK_THREADS) sh.hist[i] = 0;
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < TK_EPT; ++e) {
      if (e >= ept) continue;
      const uint32_t bin = key[e] >= mn ? (key[e] >> sha) & (uint32_t)(nba - 1) : (uint32_t)TK_BINS;
      atomicAdd(&sh.hist[bin], 1u);
    }
    __syncthreads();
    topk_pick(sh, nba, kk, tid);
    const uint32_t da = sh.digit;
    kk -= sh.above;
    const uint32_t c_eq = sh.hist[da];
    __syncthreads();  // every thread has read the bin count before hist is cleared again
    uint32_t prefix = common | (da << sha);
    if (sha == 0) {
      tau = prefix;
    } else if (c_eq <= (uint32_t)TK_CAP) {
      // 3a. the bin's keys into LDS (their low bits), resolved there
      const uint32_t low_mask = (1u << sha) - 1u;
#pragma unroll
      for (int e = 0; e < TK_EPT; ++e) {
        if (e >= ept) continue;
        if (key[e] >= mn && (key[e] >> sha) == (prefix >> sha))
          sh.cand[atomicAdd(&sh.ncand, 1u)] = key[e] & low_mask;
      }
      __syncthreads();
      uint32_t low = 0;
      int left = sha;
      while (left > 0) {
        const int w = min(10, left), shb = left - w;
        for (int i = tid; i < (1 << w); i += TK_THREADS) sh.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < (int)c_eq; i += TK_THREADS) {
          const uint32_t v = sh.cand[i];
          if ((v >> left) == (low >> left)) atomicAdd(&sh.hist[(v >> shb) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        topk_pick(sh, 1 << w, kk, tid);
        low |= sh.digit << shb;
        kk -= sh.above;
        left = shb;
      }
      tau = prefix | low;
    } else {
      // 3b. a crowded bin: the remaining bits in the registers, 8 at a time
      int left = sha;
      while (left > 0) {
        const int w = min(8, left), shb = left - w;
        const uint32_t pm = ~((1u << left) - 1u);
        for (int i = tid; i <= TK_BINS; i += TK_THREADS) sh.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < TK_EPT; ++e) {
          if (e >= ept) continue;
          const bool m = key[e] >= mn && (key[e] & pm) == prefix;
          atomicAdd(&sh.hist[m ? (key[e] >> shb) & ((1u << w) - 1u) : (uint32_t)TK_BINS], 1u);
        }
        __syncthreads();
        topk_pick(sh, 1 << w, kk, tid);
        prefix |= sh.digit << shb;
        kk -= sh.above;
        left = shb;
      }
      tau = prefix;
    }
  }
  // the selection in position order: every key above tau, and the first kk keys
  // equal to it (tau > 0, so placeholders never qualify)
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int e = 0; e < TK_EPT; ++e) {
    if (e >= ept) continue;
    cg += key[e] > tau ? 1u : 0u;
    ce += key[e] == tau ? 1u : 0u;
  }
  uint32_t gb, eb, tg, te;
  topk_block_scan(sh, cg, ce, tid, gb, eb, tg, te);
#pragma unroll
  for (int e = 0; e < TK_EPT; ++e) {
    if (e >= ept) continue;
    const bool gt = key[e] > tau, eq = key[e] == tau;
    const uint32_t slot = gb + min(eb, kk);  // < K by the selection invariant
    if ((gt || (eq && eb < kk)) && slot < (uint32_t)K) out[slot] = p0 + e;
    gb += gt ? 1u : 0u;
    eb += eq ? 1u : 0u;
  }
}

// Longer rows: radix select 8 bits at a time from the top, the row read from
// memory in every pass.
__device__ __forceinline__ void topk_streaming(TopkShared& sh, const float* row, int n, int K,
                                               int32_t* out, int tid) {
  const int n4 = n & ~3;
  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    for (int i = 4 * tid; i < n4; i += 4 * TK_THREADS) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = order_key(v[j]);
        if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1u);
      }
    }
    for (int i = n4 + tid; i < n; i += TK_THREADS) {
      const uint32_t u = order_key(row[i]);
      if ((u & pmask) == prefix) atomicAdd(&sh.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    topk_pick(sh, 256, kk, tid);
    prefix |= sh.digit << shift;
    pmask |= 255u << shift;
    kk -= sh.above;
  }
  const uint32_t tau = prefix;
  uint32_t base_gt = 0, base_eq = 0;
  for (int i0 = 0; i0 < n; i0 += 4 * TK_THREADS) {
    const int i = i0 + 4 * tid;
    uint32_t u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (i + j < n) ? order_key(row[i + j]) : 0u;
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = i + j < n;
      cg += (valid && u[j] > tau) ? 1u : 0u;
      ce += (valid && u[j] == tau) ? 1u : 0u;
    }
    uint32_t gb, eb, tg, te;
    topk_block_scan(sh, cg, ce, tid, gb, eb, tg, te);
    gb += base_gt;
    eb += base_eq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (i + j < n) {
        const bool gt = u[j] > tau, eq = u[j] == tau;
        const uint32_t slot = gb + min(eb, kk);  // < K by the selection invariant
        if ((gt || (eq && eb < kk)) && slot < (uint32_t)K) out[slot] = i + j;
        gb += gt ? 1u : 0u;
        eb += eq ? 1u : 0u;
      }
    }
    base_gt += tg;
    base_eq += te;
  }
}

// The K largest order keys of a row, ties to the lower position, written in
// ascending position order.
__global__ __launch_bounds__(TK_THREADS) void sparse_topk_kernel(const float* scores, size_t stride,
                                                                 const int32_t* tok_pos, int K,
                                                                 int32_t* sel) {
  __shared__ TopkShared sh;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = tok_pos[t] + 1;
  int32_t* out = sel + (size_t)t * K;
  if (n <= K) {
    for (int i = tid; i < K; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + (size_t)t * stride;
  if (n <= TK_THREADS * TK_EPT)
    topk_registers(sh, row, n, K, out, tid);
  else
    topk_streaming(sh, row, n, K, out, tid);
}

hipError_t launch_sparse_topk(const float* scores, size_t stride, const int32_t* tok_pos, int T,
                              int K, int32_t* sel, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(sparse_topk_kernel, dim3(T), dim3(TK_THREADS), 0, s, scores, stride, tok_pos,
                     K, sel);
  return hipGetLastError();
}

// -------------------------------------------------------- sparse attention

// LDS fence inside one wave: every LDS access issued before it has completed
// (the wave's own V^T buffer is rewritten chunk after chunk).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ __launch_bounds__(512, 1) void sparse_attention_kernel(SparseAttnArgs p) {
  constexpr int NW = 8;
  __shared__ __attribute__((aligned(16))) bf16_t Vt[NW][D * SVT_STRIDE];
  __shared__ float MLs[NW][2][16];
  __shared__ int used[NW];
  const int t = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int pos = p.tok_pos[t];
  const int* btab = p.block_table + (size_t)p.tok_seq[t] * p.max_blocks;
  const int group = p.nq / p.nkv;
  const bool col_ok = lc < group;
  const int hq = g * group + lc;
  const size_t qstride = (size_t)p.nq * D;
  const int32_t* srow = p.sel + (size_t)t * p.K;
  const int e_seg = wave * SSEG;
  const int n_chunks = max(0, min(SSEG, p.K - e_seg)) / SCHUNK;
  bf16_t* V = Vt[wave];

  bf16x8_t qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4_t v = u32x4_t{0, 0, 0, 0};
    if (col_ok)
      v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const bf16_t*>(p.q) +
                                            (size_t)t * qstride + hq * D + ks * 32 + 8 * lg);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }

  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool first = true;
  const size_t kvrow0 = (size_t)g * SCHUNK;  // head g's row offset inside a cache block

  // the cache rows of all of this wave's entries first (entry e_seg + 64c + lane:
  // row of kv head g, -1 when not a valid position), so each chunk then waits on
  // one round of K/V loads only
  constexpr int CPS = SSEG / SCHUNK;
  int slots[CPS];
  {
    int sp[CPS];
#pragma unroll
    for (int c = 0; c < CPS; ++c) sp[c] = c < n_chunks ? srow[e_seg + c * SCHUNK + lane] : -1;
#pragma unroll
    for (int c = 0; c < CPS; ++c) {
      const bool valid = sp[c] >= 0 && sp[c] <= pos;
      slots[c] = valid ? (btab[sp[c] >> 6] * p.nkv * SCHUNK + (int)kvrow0 + (sp[c] & 63)) : -1;
    }
  }

#pragma unroll
  for (int c = 0; c < CPS; ++c) {
    if (c >= n_chunks) break;
    const int slot = slots[c];
    const bool valid = slot >= 0;
    const uint64_t any = __ballot(valid);
    if (any == 0) continue;
    // K: the A operand rows, key 16kt + lc of the chunk, dims 32ks + 8lg .. +7
    bf16x8_t kf[4][D / 32];
    bool kval[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int ks_slot = __shfl(slot, 16 * kt + lc, WAVE);
      kval[kt] = ks_slot >= 0;
      const float sc = kval[kt] ? p.kv.ks[ks_slot] : 0.0f;
      const uint8_t* krow = reinterpret_cast<const uint8_t*>(p.kv.k) + (size_t)max(ks_slot, 0) * D;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        u32x2_t w = u32x2_t{0, 0};
        if (kval[kt]) w = *reinterpret_cast<const u32x2_t*>(krow + ks * 32 + 8 * lg);
        kf[kt][ks] = dequant8(w, sc);
      }
    }
    // V: units of (entry pair kp, 16 dims), written transposed into this wave's LDS
    constexpr int CH16 = D / 16;
    constexpr int VU = (SCHUNK / 2) * CH16 / WAVE;  // units per lane
    u32x4_t va[VU], vb[VU];
    float vsa[VU], vsb[VU];
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = j * WAVE + lane;
      const int kp = u % 32, c16 = u / 32;
      const int sa = __shfl(slot, 2 * kp, WAVE), sb = __shfl(slot, 2 * kp + 1, WAVE);
      va[j] = u32x4_t{0, 0, 0, 0};
      vb[j] = u32x4_t{0, 0, 0, 0};
      vsa[j] = 0.0f;
      vsb[j] = 0.0f;
      if (sa >= 0) {
        va[j] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(p.kv.v) +
                                                  (size_t)sa * D + c16 * 16);
        vsa[j] = p.kv.vs[sa];
      }
      if (sb >= 0) {
        vb[j] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(p.kv.v) +
                                                  (size_t)sb * D + c16 * 16);
        vsb[j] = p.kv.vs[sb];
      }
    }
    // S^T = K . Q^T
    f32x4_t sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt][ks], qf[ks], sacc[kt], 0, 0, 0);
    }
    // lane holds entries 16kt + 4lg + r of column lc; invalid entries score -inf
    float tt[4][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ent = 16 * kt + 4 * lg + r;
        const bool ok = (any >> ent) & 1ull;
        const float v = sacc[kt][r] * p.scale_log2;
        tt[kt][r] = ok ? v : -INFINITY;
        mloc = fmaxf(mloc, tt[kt][r]);
      }
    mloc = xrow_max(mloc);
    const float mn = fmaxf(m, mloc);
    const float mu = (mn == -INFINITY) ? 0.0f : mn;
    float rs = 0.0f;
    float pr[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[kt][r] = fexp2(tt[kt][r] - mu);
        rs = rs + pr[kt][r];
      }
    rs = xrow_sum(rs);
    if (first) {
      l = rs;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else {
      const float alpha = fexp2(m - mu);
      l = mul_unless_one(l, alpha) + rs;
      scale_unless_one(acc, alpha);
    }
    m = mn;
    first = false;

    // V^T into LDS (the previous chunk's reads of this buffer are complete)
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = j * WAVE + lane;
      const int kp = u % 32, c16 = u / 32;
      const int k0 = 2 * kp;
      float xa[16], xb[16];
      kv_decode16_f32(reinterpret_cast<const uint32_t*>(&va[j]), vsa[j], xa);
      kv_decode16_f32(reinterpret_cast<const uint32_t*>(&vb[j]), vsb[j], xb);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        *reinterpret_cast<uint32_t*>(V + (c16 * 16 + i) * SVT_STRIDE + k0) = pack_f2bf2(xa[i], xb[i]);
    }
    wave_lds_fence();

    // O^T += V^T . P^T over two 32-entry steps
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      u32x4_t pw;
      pw[0] = pack_f2bf2(pr[2 * k2][0], pr[2 * k2][1]);
      pw[1] = pack_f2bf2(pr[2 * k2][2], pr[2 * k2][3]);
      pw[2] = pack_f2bf2(pr[2 * k2 + 1][0], pr[2 * k2 + 1][1]);
      pw[3] = pack_f2bf2(pr[2 * k2 + 1][2], pr[2 * k2 + 1][3]);
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
      const int ko = k2 * 32 + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const bf16_t* vr = V + (dt * 16 + lc) * SVT_STRIDE;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr + ko);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + ko + 16);
        const u32x4_t vw = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vw), pf,
                                                          acc[dt], 0, 0, 0);
      }
    }
  }

  // segments -> LDS (each wave's own V^T buffer holds its acc), merged ascending
  __syncthreads();
  float* A = reinterpret_cast<float*>(V);  // [16 columns][D]
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) A[lc * D + dt * 16 + 4 * lg + r] = acc[dt][r];
  if (lg == 0) {
    MLs[wave][0][lc] = m;
    MLs[wave][1][lc] = l;
  }
  if (lane == 0) used[wave] = first ? 0 : 1;
  __syncthreads();
  for (int idx = tid; idx < group * D; idx += NW * WAVE) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY, L = 0.0f, ACC = 0.0f;
    for (int w = 0; w < NW; ++w) {
      if (!used[w]) continue;
      const float mw = MLs[w][0][h], lw = MLs[w][1][h];
      const float aw = reinterpret_cast<const float*>(Vt[w])[h * D + d];
      const float Mn = fmaxf(M, mw);
      const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
      const float a = fexp2(M - Mu), b = fexp2(mw - Mu);
      L = mul_unless_one(L, a) + mul_unless_one(lw, b);
      ACC = mul_unless_one(ACC, a) + mul_unless_one(aw, b);
      M = Mn;
    }
    reinterpret_cast<bf16_t*>(p.o)[(size_t)t * qstride + (size_t)(g * group + h) * D + d] =
        f2bf(ACC * attn_inv_l(L));
  }
}

hipError_t launch_sparse_attention(const SparseAttnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.d == 128)
    hipLaunchKernelGGL(sparse_attention_kernel<128>, dim3(a.T, a.nkv), dim3(512), 0, s, a);
  else if (a.d == 64)
    hipLaunchKernelGGL(sparse_attention_kernel<64>, dim3(a.T, a.nkv), dim3(512), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bci
