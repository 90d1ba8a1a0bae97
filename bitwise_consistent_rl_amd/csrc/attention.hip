// Causal GQA attention over the paged KV cache; one kernel for prefill,
// chunked prefill, decode and the training recompute.
//
// The pages trace train/inference mismatch partly to prefill and decode
// running different attention algorithms, and require one attention
// operator fed by the same gathered, dequantised KV in every phase (page
// "Finish RL Training Faster" digest, sections "零差异需要一个精确的比较对象"
// and "让训练前向使用推理的数值").
//
// Per query row (a token x a query head of the kv head's group) the kernel
// performs exactly this sequence, whatever tile or phase the row is in:
//   for segment s = 0, 1, ... (S keys each, S a multiple of 64):
//     (m, l, acc) = (-inf, 0, 0)
//     for chunk c of the segment (64 keys at absolute positions 64c..64c+63):
//       t_j = (q . k_j) * (log2(e)/sqrt(d))   [MFMA, fp32]; t_j = -inf if j > pos
//       m' = max(m, max_j t_j); a = 2^(m - m'); p_j = 2^(t_j - m')
//       l = l * a + sum_j p_j   [fixed tree];  acc = acc * a + P.V  [MFMA, P in bf16]
//     merge (m, l, acc) into (M, L, ACC) with the same exp2 rule
//   (every "x * a" above is mul_unless_one: x itself when a is exactly 1)
//   o = bf(ACC * rcp(L))
// A chunk or segment that lies wholly after the row's position is an exact
// no-op (a = 2^0 = 1, p = 0, and keys past the tile's last position are
// zeroed on load, so no 0 * NaN from unwritten cache slots), so a row gives the
// same bits whether its tile stops at its own position (decode) or runs on
// (prefill).  MFMA outputs depend only on their own operand row and column,
// so the row's slot in the tile does not matter either.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16, lane l, g = l >> 4, c = l & 15):
//   scores are computed transposed, S^T = K . Q^T, so lane l holds keys
//   16kt + 4g + r of query row c; after exp2 these are exactly the values the
//   P^T operand of O^T = V^T . P^T needs in lane l (keys 4g..4g+3 and
//   16+4g..16+4g+3 of each 32-key step), so P never leaves registers.  V is
//   stored transposed in LDS (V^T[d][key]) so the V^T operand is two 8-byte
//   reads.  O^T lands with query row c in lane l again, so the softmax
//   statistics never move between lanes.
#include "common.h"
#include "kernels.h"

#include <climits>
#include <type_traits>

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int ATHREADS = 256;
constexpr int CHUNK = 64;
constexpr int VT_STRIDE = CHUNK + 4;  // bf16 per V^T row: 34 dwords, so the 8-byte fragment
                                      // reads of 16 rows and the pair writes spread over the banks

template <int D>
__device__ __forceinline__ int kswz(int key, int ch) {
  if constexpr (D == 128)
    return key * (D / 8) + (ch ^ (key & 15));
  else
    return key * (D / 8) + (ch ^ ((key >> 1) & 7));
}

// ---- chunk loads, software-pipelined: chunk c+1 is fetched into registers
// while chunk c is multiplied, and written to the second of two LDS buffers
// after it.  K rows past the tile's last position are written as loaded:
// their scores are replaced by -inf for every row before use, and an MFMA
// output element depends only on its own K row.  V rows past the last position
// are zeroed, so a never-written cache slot cannot put 0 * NaN into the
// accumulator.  V is stored transposed for the MFMA; FP8 K and V are
// dequantised on the way into LDS.
template <int D, bool FP8>
struct ChunkLoader {
  static constexpr int CH = D / 8;                  // 16-byte bf16 chunks per key row
  static constexpr int CH16 = D / 16;               // 16-code FP8 chunks per key row
  static constexpr int KBF = CHUNK * CH / ATHREADS;  // bf16 K: 16-byte loads per thread
  static constexpr int VUN = FP8 ? (CHUNK / 2) * CH16 : (CHUNK / 2) * CH;  // V units (2 keys)
  static constexpr int VPT = (VUN + ATHREADS - 1) / ATHREADS;
  static constexpr int KUN = CHUNK * CH16;          // FP8 K units (1 key, 16 codes)
  static constexpr int KPT = FP8 ? (KUN + ATHREADS - 1) / ATHREADS : 0;
  // every thread owns a whole number of units: no per-unit bound test (a branch around
  // a load makes the compiler's wait before each later use cover the path without it)
  static constexpr bool V_EVEN = VUN % ATHREADS == 0;
  static constexpr bool K_EVEN = KUN % ATHREADS == 0;

  // registers in flight
  u32x4_t va[VPT], vb[VPT];
  float vsa[VPT], vsb[VPT];
  u32x4_t kr[FP8 ? (KPT > 0 ? KPT : 1) : KBF];
  float ksc[KPT > 0 ? KPT : 1];

  // V unit u -> (key pair, column chunk): consecutive lanes take consecutive key
  // pairs (32 per chunk), so the transposed 4-byte LDS writes of one instruction fall
  // on distinct banks.
  __device__ static void vunit(int u, int& kp, int& ch) {
    kp = u % 32;
    ch = u / 32;
  }

  __device__ void issue(const AttnArgs& p, int blk, int g, int tid) {
    const size_t base = ((size_t)blk * p.nkv + g) * CHUNK;  // first cache row of the chunk
    if constexpr (!FP8) {
      // K unit u: key u / CH, 16-byte chunk u % CH (a wave reads 4 whole key rows)
      const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.kv.k) + base * D;
#pragma unroll
      for (int i = 0; i < KBF; ++i) {
        const int u = i * ATHREADS + tid;
        kr[i] = *reinterpret_cast<const u32x4_t*>(kg + (u / CH) * D + (u % CH) * 8);
      }
      const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.kv.v) + base * D;
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int u = j * ATHREADS + tid;
        if (V_EVEN || u < VUN) {
          int kp, ch;
          vunit(u, kp, ch);
          va[j] = *reinterpret_cast<const u32x4_t*>(vg + (2 * kp) * D + ch * 8);
          vb[j] = *reinterpret_cast<const u32x4_t*>(vg + (2 * kp + 1) * D + ch * 8);
        }
      }
    } else {
      const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.kv.k) + base * D;
      const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.kv.v) + base * D;
      const float* ksg = p.kv.ks + base;
      const float* vsg = p.kv.vs + base;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int u = j * ATHREADS + tid;
        if (K_EVEN || u < KUN) {
          const int key = u / CH16, c16 = u % CH16;
          kr[j] = *reinterpret_cast<const u32x4_t*>(kg + key * D + c16 * 16);
          ksc[j] = ksg[key];
        }
      }
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int u = j * ATHREADS + tid;
        if (V_EVEN || u < VUN) {
          int kp, c16;
          vunit(u, kp, c16);
          va[j] = *reinterpret_cast<const u32x4_t*>(vg + (2 * kp) * D + c16 * 16);
          vb[j] = *reinterpret_cast<const u32x4_t*>(vg + (2 * kp + 1) * D + c16 * 16);
          vsa[j] = vsg[2 * kp];
          vsb[j] = vsg[2 * kp + 1];
        }
      }
    }
  }

  // registers -> LDS (FP8 K dequantised; V transposed, zeroed past key_lim)
  __device__ void store(int key_lim, u32x4_t* Ks, bf16_t* Vt, int tid) {
    if constexpr (!FP8) {
#pragma unroll
      for (int i = 0; i < KBF; ++i) {
        const int u = i * ATHREADS + tid;
        Ks[kswz<D>(u / CH, u % CH)] = kr[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int u = j * ATHREADS + tid;
        if (K_EVEN || u < KUN) {
          const int key = u / CH16, c16 = u % CH16;
          float x[16];
          kv_decode16_f32(reinterpret_cast<const uint32_t*>(&kr[j]), ksc[j], x);
          u32x4_t lo, hi;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lo[i] = pack_f2bf2(x[2 * i], x[2 * i + 1]);
            hi[i] = pack_f2bf2(x[8 + 2 * i], x[8 + 2 * i + 1]);
          }
          Ks[kswz<D>(key, 2 * c16)] = lo;
          Ks[kswz<D>(key, 2 * c16 + 1)] = hi;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int u = j * ATHREADS + tid;
      if (V_EVEN || u < VUN) {
        int kp, ch;
        vunit(u, kp, ch);
        const int k0 = 2 * kp;
        const bool za = k0 > key_lim, zb = k0 + 1 > key_lim;
        if constexpr (!FP8) {
          u32x4_t a = va[j], bv = vb[j];
          if (key_lim < CHUNK - 1) {  // only the chunk holding the tile's last position
            if (za) a = u32x4_t{0, 0, 0, 0};
            if (zb) bv = u32x4_t{0, 0, 0, 0};
          }
          const bf16_t* pa = reinterpret_cast<const bf16_t*>(&a);
          const bf16_t* pb = reinterpret_cast<const bf16_t*>(&bv);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint32_t*>(Vt + (ch * 8 + i) * VT_STRIDE + k0) = pack_bf2(pa[i], pb[i]);
        } else {
          float xa[16], xb[16];
          kv_decode16_f32(reinterpret_cast<const uint32_t*>(&va[j]), vsa[j], xa);
          kv_decode16_f32(reinterpret_cast<const uint32_t*>(&vb[j]), vsb[j], xb);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t w = pack_f2bf2(xa[i], xb[i]);
            *reinterpret_cast<uint32_t*>(Vt + (ch * 16 + i) * VT_STRIDE + k0) =
                (za ? 0u : (w & 0xffffu)) | (zb ? 0u : (w & 0xffff0000u));
          }
        }
      }
    }
  }
};

// Synchronous chunk load for the single-buffer schedule: each unit is loaded,
// converted and stored in turn, which keeps few registers live.
template <int D, bool FP8>
__device__ __forceinline__ void load_chunk_sync(const AttnArgs& p, int blk, int g, int key_lim,
                                           u32x4_t* Ks, bf16_t* Vt, int tid) {
  const size_t base = ((size_t)blk * p.nkv + g) * CHUNK;  // first cache row of the chunk
  if constexpr (!FP8) {
    const bf16_t* kg = reinterpret_cast<const bf16_t*>(p.kv.k) + base * D;
    const bf16_t* vg = reinterpret_cast<const bf16_t*>(p.kv.v) + base * D;
    constexpr int CH = D / 8;  // 16-byte chunks per key row
    // K: straight copy, swizzled
#pragma unroll
    for (int u = tid; u < CHUNK * CH; u += ATHREADS) {
      const int key = u / CH, ch = u % CH;
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(kg + key * D + ch * 8);
      if (key > key_lim) v = u32x4_t{0, 0, 0, 0};
      Ks[kswz<D>(key, ch)] = v;
    }
    // V: two consecutive keys per unit, written transposed as 4-byte pairs
#pragma unroll
    for (int u = tid; u < (CHUNK / 2) * CH; u += ATHREADS) {
      const int kp = u % (CHUNK / 2), ch = u / (CHUNK / 2);  // lanes along key pairs (banks)
      const int k0 = 2 * kp;
      u32x4_t a = *reinterpret_cast<const u32x4_t*>(vg + k0 * D + ch * 8);
      u32x4_t b = *reinterpret_cast<const u32x4_t*>(vg + (k0 + 1) * D + ch * 8);
      if (k0 > key_lim) a = u32x4_t{0, 0, 0, 0};
      if (k0 + 1 > key_lim) b = u32x4_t{0, 0, 0, 0};
      const bf16_t* pa = reinterpret_cast<const bf16_t*>(&a);
      const bf16_t* pb = reinterpret_cast<const bf16_t*>(&b);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t*>(Vt + (ch * 8 + i) * VT_STRIDE + k0) = pack_bf2(pa[i], pb[i]);
    }
  } else {
    const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.kv.k) + base * D;
    const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.kv.v) + base * D;
    const float* ksg = p.kv.ks + base;
    const float* vsg = p.kv.vs + base;
    constexpr int CH16 = D / 16;  // 16-code chunks per key row
#pragma unroll
    for (int u = tid; u < CHUNK * CH16; u += ATHREADS) {
      const int key = u / CH16, c16 = u % CH16;
      const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(kg + key * D + c16 * 16);
      const float sc = ksg[key];
      float x[16];
      kv_decode16_f32(reinterpret_cast<const uint32_t*>(&raw), sc, x);
      u32x4_t lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo[i] = pack_f2bf2(x[2 * i], x[2 * i + 1]);
        hi[i] = pack_f2bf2(x[8 + 2 * i], x[8 + 2 * i + 1]);
      }
      if (key > key_lim) {
        lo = u32x4_t{0, 0, 0, 0};
        hi = u32x4_t{0, 0, 0, 0};
      }
      Ks[kswz<D>(key, 2 * c16)] = lo;
      Ks[kswz<D>(key, 2 * c16 + 1)] = hi;
    }
#pragma unroll
    for (int u = tid; u < (CHUNK / 2) * CH16; u += ATHREADS) {
      const int kp = u % (CHUNK / 2), c16 = u / (CHUNK / 2);  // lanes along key pairs (banks)
      const int k0 = 2 * kp;
      const u32x4_t ra = *reinterpret_cast<const u32x4_t*>(vg + k0 * D + c16 * 16);
      const u32x4_t rb = *reinterpret_cast<const u32x4_t*>(vg + (k0 + 1) * D + c16 * 16);
      const float sa = vsg[k0], sb = vsg[k0 + 1];
      const bool za = k0 > key_lim, zb = k0 + 1 > key_lim;
      float xa[16], xb[16];
      kv_decode16_f32(reinterpret_cast<const uint32_t*>(&ra), sa, xa);
      kv_decode16_f32(reinterpret_cast<const uint32_t*>(&rb), sb, xb);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w = pack_f2bf2(xa[i], xb[i]);
        *reinterpret_cast<uint32_t*>(Vt + (c16 * 16 + i) * VT_STRIDE + k0) =
            (za ? 0u : (w & 0xffffu)) | (zb ? 0u : (w & 0xffff0000u));
      }
    }
  }
}

// Two schedules of the same per-row arithmetic.  PIPE (tiles of many rows:
// prefill, recompute): two LDS buffers, chunk c+1 in flight while chunk c is
// multiplied.  !PIPE (the split schedule, used for decode-like calls with few
// rows per tile): one LDS buffer and short register lifetimes, so twice as
// many workgroups fit on a CU to hide the load latency.
// PF2 (PIPE, tiles of at most 16 rows: decode): two chunks in flight instead of one.
// A decode tile's chunk costs one memory latency per chunk when only the next chunk is
// fetched, while its arithmetic is a small fraction of that; with the loads of chunks
// c + 1 and c + 2 outstanding while chunk c is multiplied, and the issues unconditional
// (a chunk index past the last is clamped, its copy never used), the wait before
// storing chunk c + 1 leaves chunk c + 2's loads in flight.
// DS (decode tiles, at most 16 rows; implied by PF2): the four waves split the PV work.
// ONESEG (PIPE, calls whose every position lies in the first segment): the running state
// of finished segments (M, L, ACC) is never needed; the one merge, into the empty state, is
// (0 + l, 0 + acc), which the epilogue computes directly.  With those 32 registers fewer the
// schedule keeps one LDS buffer (the next chunk waits in registers until every wave has
// finished reading the current one: two barriers per chunk) and three workgroups fit on a
// CU instead of two.
template <int D, bool FP8, bool SPLIT, bool PF2 = false, bool DS = PF2, bool ONESEG = false>
__global__ __launch_bounds__(ATHREADS, SPLIT ? 4 : (ONESEG ? 3 : 2)) void attention_kernel(AttnArgs p) {
  constexpr bool PIPE = !SPLIT;
  static_assert(!(PF2 && SPLIT), "two chunks in flight: pipelined schedule only");
  static_assert(!(ONESEG && SPLIT), "one segment: unsplit schedules only");
  constexpr int NBUF = (PIPE && !ONESEG) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) u32x4_t Ks[NBUF][CHUNK * D / 8];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[NBUF][D * VT_STRIDE];

  // Workgroups are handed to the 8 XCDs round-robin; renumber them so each XCD
  // gets a contiguous run of (kv head, tile) pairs, i.e. consecutive tiles of
  // the same sequence and head, which read the same K/V chunks through its L2.
  int tile = blockIdx.x, g = blockIdx.y;
  if constexpr (!SPLIT) {
    const int total = gridDim.x * gridDim.y;
    const int id = blockIdx.y * gridDim.x + blockIdx.x;
    const int xcd = id & 7, lo = total >> 3, rem = total & 7;
    const int w = xcd * lo + min(xcd, rem) + (id >> 3);
    g = w / gridDim.x;
    tile = w % gridDim.x;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lg = lane >> 4, lc = lane & 15;
  const int* trec = p.tiles + (size_t)tile * ATTN_TILE_WORDS;
  const int seq = trec[0];
  const int tok_begin = trec[1];
  const int n_tok = trec[2];
  const int pos_begin = trec[3];
  // physical blocks of chunks 0 and 1, from the tile record itself: the first loads of
  // an unsplit tile do not wait for the block table (a second dependent memory latency)
  const int blk_c0 = trec[4], blk_c1 = trec[5];
  const int group = p.nq / p.nkv;
  const int kmax = pos_begin + n_tok - 1;  // last key position any row of the tile needs
  const int* btab = p.block_table + (size_t)seq * p.max_blocks;
  const size_t qstride = (size_t)p.nq * D;

  // this lane's query row (B operand of S^T and column of O^T).  DS (tiles of at most
  // 16 rows): every wave takes rows 0-15, computes the same scores and softmax
  // statistics, and owns D/64 of the D/16 head-dimension blocks of P.V, the rescales
  // and the output, so the four waves split the chunk's PV work instead of three idling
  constexpr int DT = D / 16;                    // 16-wide head-dimension blocks
  constexpr int DPW = DS ? DT / 4 : DT;         // blocks this wave accumulates
  const int rw = DS ? 0 : wave;
  const int dt0 = DS ? wave * DPW : 0;
  const int row = rw * 16 + lc;
  const int tk = row / group;
  const int hq = g * group + row % group;
  const bool row_ok = tk < n_tok;
  const int qpos = row_ok ? pos_begin + tk : -1;
  // smallest position among this wave's valid rows (rows are token-major)
  const int wave_tk0 = (rw * 16) / group;
  const int wave_qpos_min = wave_tk0 < n_tok ? pos_begin + wave_tk0 : INT_MAX;
  // a wave without a valid row (decode tiles fill one wave of 16 rows) only loads
  const bool wave_active = wave_tk0 < n_tok;

  const int last_chunk = kmax / CHUNK;
  const int seg_chunks = p.seg_keys / CHUNK;
  int c_first = 0, c_stop = last_chunk;
  if constexpr (SPLIT) {
    // this workgroup computes one segment only; its partial goes to the workspace
    c_first = blockIdx.z * seg_chunks;
    if (c_first > last_chunk) return;
    c_stop = min(c_first + seg_chunks - 1, last_chunk);
  }

  ChunkLoader<D, FP8> ld, ld2;
  // PIPE schedules start at chunk 0 (c_first = 0)
  if constexpr (PIPE) ld.issue(p, blk_c0, g, tid);
  if constexpr (PF2) ld2.issue(p, c_stop >= 1 ? blk_c1 : blk_c0, g, tid);

  bf16x8_t qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4_t v = u32x4_t{0, 0, 0, 0};
    if (row_ok)
      v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const bf16_t*>(p.q) +
                                            (size_t)(tok_begin + tk) * qstride + hq * D + ks * 32 +
                                            8 * lg);
    qf[ks] = __builtin_bit_cast(bf16x8_t, v);
  }

  float M = -INFINITY, L = 0.0f;
  f32x4_t ACC[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) ACC[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;
  f32x4_t acc[DPW];

  if constexpr (PIPE) {
    ld.store(kmax - c_first * CHUNK, Ks[0], Vt[0], tid);
    __syncthreads();
  }
  if constexpr (PF2) ld.issue(p, btab[min(c_first + 2, c_stop)], g, tid);

  // the arithmetic of chunk c out of LDS buffer b (identical for every schedule)
  auto compute_chunk = [&](int c, int b) __attribute__((always_inline)) {
    const bool seg_start = (c % seg_chunks) == 0 || c == c_first;
    if (seg_start) m = -INFINITY;
    const u32x4_t* Kb = Ks[b];
    const bf16_t* Vb = Vt[b];

    // S^T = K . Q^T : 4 key blocks of 16, D/32 steps.  Each block's chain runs over the
    // steps in ascending order; the four chains are interleaved, and the K fragments
    // of step ks + 1 are read while step ks multiplies.
    f32x4_t sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    {
      bf16x8_t kf[D / 32][4];
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          kf[ks][kt] = __builtin_bit_cast(bf16x8_t, Kb[kswz<D>(kt * 16 + lc, ks * 4 + lg)]);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][kt], qf[ks], sacc[kt], 0, 0, 0);
      if constexpr (PIPE) {  // order: reads 0, reads 1, products 0, reads 2, products 1, ...
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          if (ks + 1 < D / 32) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
      }
    }
    // Causal mask.  It changes nothing for a chunk whose last key is at or before
    // the first (smallest) position of this wave's valid rows, so such chunks
    // skip it; rows past the tile's tokens are never stored.
    const bool need_mask = c * CHUNK + CHUNK - 1 > wave_qpos_min;  // wave-uniform
    float t[4][4];
    float mloc = -INFINITY;
    if constexpr (PIPE) {  // the mask as its own pass, skipped by whole chunks
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) t[kt][r] = sacc[kt][r] * p.scale_log2;
      if (need_mask) {
        const int kl = qpos - (c * CHUNK + 4 * lg);  // keys 16 kt + r <= kl are visible
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kt * 16 + r > kl) t[kt][r] = -INFINITY;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, t[kt][r]);
    } else {  // fused (fewer live registers)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sacc[kt][r] * p.scale_log2;
          if (need_mask) {
            const int key = c * CHUNK + kt * 16 + 4 * lg + r;
            t[kt][r] = key <= qpos ? v : -INFINITY;
          } else {
            t[kt][r] = v;
          }
          mloc = fmaxf(mloc, t[kt][r]);
        }
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
        pr[kt][r] = fexp2(t[kt][r] - mu);
        rs = rs + pr[kt][r];
      }
    rs = xrow_sum(rs);

    // O^T += V^T . P^T over two 32-key steps; from_zero: the first step accumulates
    // onto a literal zero
    auto pv = [&](auto from_zero) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        u32x4_t pw;
        pw[0] = pack_f2bf2(pr[2 * k2][0], pr[2 * k2][1]);
        pw[1] = pack_f2bf2(pr[2 * k2][2], pr[2 * k2][3]);
        pw[2] = pack_f2bf2(pr[2 * k2 + 1][0], pr[2 * k2 + 1][1]);
        pw[3] = pack_f2bf2(pr[2 * k2 + 1][2], pr[2 * k2 + 1][3]);
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
        const int ko = k2 * 32 + 4 * lg;
        u32x4_t vw[DPW];  // all fragments of the step are read, then multiplied
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          const bf16_t* vr = Vb + ((dt0 + j) * 16 + lc) * VT_STRIDE;
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr + ko);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + ko + 16);
          vw[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          const f32x4_t c0 = (decltype(from_zero)::value && k2 == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[j];
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vw[j]), pf, c0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, DPW, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, DPW, 0);
      }
    };
    // (m, l, acc) = (-inf, 0, 0) at a segment start: alpha = 2^(-inf) = 0, so
    // l * alpha + rs is rs and acc * alpha is +0, exactly what these shortcuts give
    if constexpr (PIPE) {
      if (seg_start) {
        l = rs;
        pv(std::true_type{});
      } else {
        const float alpha = fexp2(m - mu);
        l = mul_unless_one(l, alpha) + rs;
        scale_unless_one(acc, alpha);
        pv(std::false_type{});
      }
    } else {  // fewer registers: one copy of the products
      if (seg_start) {
        l = rs;
#pragma unroll
        for (int j = 0; j < DPW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      } else {
        const float alpha = fexp2(m - mu);
        l = mul_unless_one(l, alpha) + rs;
        scale_unless_one(acc, alpha);
      }
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
        for (int j = 0; j < DPW; ++j) {
          const bf16_t* vr = Vb + ((dt0 + j) * 16 + lc) * VT_STRIDE;
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vr + ko);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vr + ko + 16);
          const u32x4_t vw = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vw), pf, acc[j], 0, 0, 0);
        }
      }
    }
    m = mn;

    if constexpr (!SPLIT && !ONESEG) {
      if (c == c_stop || ((c + 1) % seg_chunks) == 0) {
        // merge the finished segment into the running state (ascending segment order)
        const float Mn = fmaxf(M, m);
        const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
        const float a = fexp2(M - Mu), bb = fexp2(m - Mu);
        L = mul_unless_one(L, a) + mul_unless_one(l, bb);
        scale_unless_one(ACC, a);
        scale_unless_one(acc, bb);
#pragma unroll
        for (int j = 0; j < DPW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) ACC[j][r] = ACC[j][r] + acc[j][r];
        M = Mn;
      }
    }

  };

  if constexpr (PF2) {
    // chunk c_first + i is held by ld (i even) or ld2 (i odd) until stored; at step i
    // the other set (chunk i + 1) is stored, then refilled with chunk i + 3
    auto step = [&](auto odd, int c) __attribute__((always_inline)) {
      constexpr int b = decltype(odd)::value ? 1 : 0;
      if (wave_active) compute_chunk(c, b);
      if constexpr (b == 0) ld2.store(kmax - (c + 1) * CHUNK, Ks[1], Vt[1], tid);
      else ld.store(kmax - (c + 1) * CHUNK, Ks[0], Vt[0], tid);
      __syncthreads();  // publishes buffer b^1, releases buffer b
      if constexpr (b == 0) ld2.issue(p, btab[min(c + 3, c_stop)], g, tid);
      else ld.issue(p, btab[min(c + 3, c_stop)], g, tid);
    };
    for (int c = c_first; c <= c_stop; c += 2) {
      step(std::false_type{}, c);
      if (c + 1 > c_stop) break;
      step(std::true_type{}, c + 1);
    }
  } else {
    for (int c = c_first; c <= c_stop; ++c) {
      const int b = (PIPE && !ONESEG) ? (c - c_first) & 1 : 0;
      const bool more = c < c_stop;
      if constexpr (PIPE) {
        if (more) ld.issue(p, btab[c + 1], g, tid);
      } else {
        if (c > c_first) __syncthreads();  // the previous chunk's LDS reads are done
        load_chunk_sync<D, FP8>(p, btab[c], g, kmax - c * CHUNK, Ks[0], Vt[0], tid);
        __syncthreads();
      }
      if (wave_active) compute_chunk(c, b);
      if constexpr (PIPE && ONESEG) {
        __syncthreads();  // every wave is done with the buffer
        if (more) ld.store(kmax - (c + 1) * CHUNK, Ks[0], Vt[0], tid);
        __syncthreads();  // publishes chunk c + 1
      } else if constexpr (PIPE) {
        // buffer b^1 was released by the previous iteration's barrier
        if (more) ld.store(kmax - (c + 1) * CHUNK, Ks[b ^ 1], Vt[b ^ 1], tid);
        __syncthreads();  // publishes buffer b^1, releases buffer b
      }
    }
  }

  if constexpr (SPLIT) {
    if (row_ok) {
      const size_t prow = ((size_t)blockIdx.z * p.n_tokens + tok_begin + tk) * p.nq + hq;
      float* pa = p.part_acc + prow * D;
#pragma unroll
      for (int j = 0; j < DPW; ++j)
        *reinterpret_cast<f32x4_t*>(pa + (dt0 + j) * 16 + 4 * lg) = acc[j];
      if (lg == 0) {
        p.part_ml[prow * 2] = m;
        p.part_ml[prow * 2 + 1] = l;
      }
    }
    return;
  }

  if (row_ok) {
    bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + (size_t)(tok_begin + tk) * qstride + hq * D;
    if constexpr (ONESEG) {
      // the merge of the only segment into (M, L, ACC) = (-inf, 0, +0): its scale factors
      // are 2^-inf = 0 and 2^0 = 1 exactly, leaving L = 0 + l and ACC = +0 + acc
      const float il = attn_inv_l(0.0f + l);
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        u32x2_t w;
        w[0] = pack_f2bf2((0.0f + acc[j][0]) * il, (0.0f + acc[j][1]) * il);
        w[1] = pack_f2bf2((0.0f + acc[j][2]) * il, (0.0f + acc[j][3]) * il);
        *reinterpret_cast<u32x2_t*>(orow + (dt0 + j) * 16 + 4 * lg) = w;
      }
    } else {
      const float il = attn_inv_l(L);
#pragma unroll
      for (int j = 0; j < DPW; ++j) {
        u32x2_t w;
        w[0] = pack_f2bf2(ACC[j][0] * il, ACC[j][1] * il);
        w[1] = pack_f2bf2(ACC[j][2] * il, ACC[j][3] * il);
        *reinterpret_cast<u32x2_t*>(orow + (dt0 + j) * 16 + 4 * lg) = w;
      }
    }
  }
}

// Split schedule, second pass: for each (token, head) row merge segments
// 0 .. pos / S in ascending order with exactly the expressions of the
// in-workgroup merge above (a later, fully masked segment of a deeper tile is
// an exact no-op there), then o = bf(ACC * rcp(L)).  One thread per output element.
template <int D>
__global__ __launch_bounds__(256) void attention_merge_kernel(AttnArgs p) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * (256 / D) + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (h >= p.nq) return;
  const int nseg = p.tok_pos[t] / p.seg_keys + 1;
  float M = -INFINITY, L = 0.0f, ACC = 0.0f;
  for (int z = 0; z < nseg; ++z) {
    const size_t prow = ((size_t)z * p.n_tokens + t) * p.nq + h;
    const float m = p.part_ml[prow * 2], l = p.part_ml[prow * 2 + 1];
    const float a_ = p.part_acc[prow * D + d];
    const float Mn = fmaxf(M, m);
    const float Mu = (Mn == -INFINITY) ? 0.0f : Mn;
    const float a = fexp2(M - Mu), b = fexp2(m - Mu);
    L = mul_unless_one(L, a) + mul_unless_one(l, b);
    ACC = mul_unless_one(ACC, a) + mul_unless_one(a_, b);
    M = Mn;
  }
  reinterpret_cast<bf16_t*>(p.o)[((size_t)t * p.nq + h) * D + d] = f2bf(ACC * attn_inv_l(L));
}

template <int D, bool FP8>
static void launch_d(const AttnArgs& a, hipStream_t s) {
  if (a.n_seg > 0) {
    hipLaunchKernelGGL((attention_kernel<D, FP8, true>), dim3(a.n_tiles, a.nkv, a.n_seg),
                       dim3(ATHREADS), 0, s, a);
    hipLaunchKernelGGL((attention_merge_kernel<D>), dim3(a.n_tokens, (a.nq * D + 255) / 256),
                       dim3(256), 0, s, a);
  } else if (a.pf2) {
    hipLaunchKernelGGL((attention_kernel<D, FP8, false, true>), dim3(a.n_tiles, a.nkv), dim3(ATHREADS),
                       0, s, a);
  } else if (a.dsplit) {
    hipLaunchKernelGGL((attention_kernel<D, FP8, false, false, true>), dim3(a.n_tiles, a.nkv),
                       dim3(ATHREADS), 0, s, a);
  } else if (a.one_seg) {
    hipLaunchKernelGGL((attention_kernel<D, FP8, false, false, false, true>), dim3(a.n_tiles, a.nkv),
                       dim3(ATHREADS), 0, s, a);
  } else {
    hipLaunchKernelGGL((attention_kernel<D, FP8, false>), dim3(a.n_tiles, a.nkv), dim3(ATHREADS),
                       0, s, a);
  }
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_tiles == 0) return hipSuccess;
  if (a.d == 128) {
    if (a.fp8) launch_d<128, true>(a, s);
    else launch_d<128, false>(a, s);
  } else if (a.d == 64) {
    if (a.fp8) launch_d<64, true>(a, s);
    else launch_d<64, false>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bci
