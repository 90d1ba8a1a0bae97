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
template <int NHT, int DI>
__device__ __forceinline__ float index_chain(const bf16x8_t (&qa)[NHT][DI / 32],
                                             const bf16x8_t (&kb)[4][DI / 32],
                                             const float (&wv)[NHT][4], int lg) {
  float out = 0.0f;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    float v = 0.0f;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      f32x4_t d = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DI / 32; ++ks)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][ks], kb[kt][ks], d, 0, 0, 0);
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

// Decode-like schedule: one token per workgroup, each wave one 64-key block,
// key codes read straight into the B operand and dequantised in registers.
template <int NHT, int DI>
__global__ __launch_bounds__(256) void index_scores_direct(IdxArgs a) {
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lg = lane >> 4, lc = lane & 15;
  const int pos = a.tok_pos[t];
  const int s0 = (blockIdx.x * 4 + wave) * SCHUNK;
  if (s0 > pos) return;
  const int* btab = a.block_table + (size_t)a.tok_seq[t] * a.max_blocks;

  bf16x8_t kb[4][DI / 32];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int s = min(s0 + 16 * kt + lc, pos);
    const size_t slot = (size_t)btab[s >> 6] * SCHUNK + (s & 63);
    const float sc = a.scales[slot];
    const uint8_t* crow = a.codes + slot * DI;
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks)
      kb[kt][ks] = dequant8(*reinterpret_cast<const u32x2_t*>(crow + 32 * ks + 8 * lg), sc);
  }
  bf16x8_t qa[NHT][DI / 32];
  float wv[NHT][4];
  index_load_query<NHT, DI>(a, t, true, lg, lc, qa, wv);

  const float v = index_chain<NHT, DI>(qa, kb, wv, lg);
  const int s = s0 + 16 * lg + lc;
  if (s <= pos) a.scores[(size_t)t * a.stride + s] = v;
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
      bf16x8_t kb[4][DI / 32];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int ks = 0; ks < DI / 32; ++ks)
          kb[kt][ks] = __builtin_bit_cast(bf16x8_t, Ks[iswz<DI>(16 * kt + lc, 4 * ks + lg)]);
      const float v = index_chain<NHT, DI>(qa, kb, wv, lg);
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
  else
    hipLaunchKernelGGL((index_scores_direct<NHT, DI>),
                       dim3((a.max_pos + 4 * SCHUNK) / (4 * SCHUNK), a.T), dim3(256), 0, s, a);
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

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o, WAVE);
    if (lane >= o) v += y;
  }
  return v;
}

__global__ __launch_bounds__(TK_THREADS) void sparse_topk_kernel(const float* scores, size_t stride,
                                                                 const int32_t* tok_pos, int K,
                                                                 int32_t* sel) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_above;
  __shared__ uint32_t wgt[TK_WAVES], weq[TK_WAVES];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = tok_pos[t] + 1;
  int32_t* out = sel + (size_t)t * K;
  if (n <= K) {
    for (int i = tid; i < K; i += TK_THREADS) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + (size_t)t * stride;
  const int n4 = n & ~3;

  // radix select of the K-th largest key, eight bits at a time from the top
  uint32_t prefix = 0, pmask = 0;
  uint32_t kk = (uint32_t)K;  // rank still to find among keys matching the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = 4 * tid; i < n4; i += 4 * TK_THREADS) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = order_key(v[j]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
    }
    for (int i = n4 + tid; i < n; i += TK_THREADS) {
      const uint32_t u = order_key(row[i]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds bins 255-4l .. 252-4l, i.e. the bins in descending order
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = hist[255 - 4 * lane - j];
        sum += c[j];
      }
      uint32_t above = wave_incl_scan(sum, lane) - sum;  // keys in higher bins
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < kk && kk <= above + c[j]) {
          s_digit = 255u - 4u * lane - j;
          s_above = above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    kk -= s_above;
  }
  // prefix is the K-th largest key; the selection is every key above it and the
  // first kk keys equal to it in position order.  Written in position order.
  const uint32_t tau = prefix;
  uint32_t base_gt = 0, base_eq = 0;
  for (int i0 = 0; i0 < n; i0 += 4 * TK_THREADS) {
    const int i = i0 + 4 * tid;
    uint32_t u[4];
    if (i + 3 < n) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(row + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = order_key(v[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = (i + j < n) ? order_key(row[i + j]) : 0u;
    }
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool valid = i + j < n;
      cg += (valid && u[j] > tau) ? 1u : 0u;
      ce += (valid && u[j] == tau) ? 1u : 0u;
    }
    const uint32_t ig = wave_incl_scan(cg, lane), ie = wave_incl_scan(ce, lane);
    if (lane == 63) {
      wgt[wave] = ig;
      weq[wave] = ie;
    }
    __syncthreads();
    uint32_t pg = 0, pe = 0, tg = 0, te = 0;
    for (int w = 0; w < TK_WAVES; ++w) {
      const uint32_t a = wgt[w], b = weq[w];
      if (w < wave) {
        pg += a;
        pe += b;
      }
      tg += a;
      te += b;
    }
    uint32_t g_before = base_gt + pg + ig - cg, e_before = base_eq + pe + ie - ce;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (i + j >= n) break;
      const bool gt = u[j] > tau, eq = u[j] == tau;
      const uint32_t slot = g_before + min(e_before, kk);  // < K by the radix invariant
      if ((gt || (eq && e_before < kk)) && slot < (uint32_t)K) out[slot] = i + j;
      g_before += gt ? 1u : 0u;
      e_before += eq ? 1u : 0u;
    }
    base_gt += tg;
    base_eq += te;
    __syncthreads();  // wgt/weq are rewritten by the next tile
  }
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

  for (int c = 0; c < n_chunks; ++c) {
    // entry e0 + lane: its cache row (kv head g), -1 when not a valid position
    const int e = e_seg + c * SCHUNK + lane;
    const int sp = srow[e];
    const bool valid = sp >= 0 && sp <= pos;
    const int slot = valid ? (btab[sp >> 6] * p.nkv * SCHUNK + (int)kvrow0 + (sp & 63)) : -1;
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
      l = l * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[dt][r] = acc[dt][r] * alpha;
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
      L = L * a + lw * b;
      ACC = ACC * a + aw * b;
      M = Mn;
    }
    reinterpret_cast<bf16_t*>(p.o)[(size_t)t * qstride + (size_t)(g * group + h) * D + d] =
        f2bf(ACC / L);
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
