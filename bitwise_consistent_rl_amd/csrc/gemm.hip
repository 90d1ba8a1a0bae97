// Batch-invariant bf16 GEMM for gfx950, and the lm_head + log-softmax kernels.
//
// The pages make every dense GEMM batch-invariant, giving up the kernel and
// split switches that small batches usually get (page "Finish RL Training
// Faster" digest, section "让训练前向使用推理的数值"), because a request can
// otherwise land on a different kernel depending on what else is in the batch
// (same page, section "零差异需要一个精确的比较对象"; page "No More
// Train-Inference Mismatch", section "背景知识与关键观察").
//
// Invariance argument.  Output element (i, j) is accumulated in one fp32
// MFMA accumulator that starts at zero and receives
// v_mfma_f32_16x16x32_bf16(A[i, k:k+32], W[j, k:k+32]) for k = 0, 32, 64, ...
// in ascending order; nothing else is ever added to it.  The schedules below
// (256 x 256 x 64 tiles with 8 waves; the skinny one-wave-per-16-columns
// schedule for M <= 128, and up to 512 where it is faster; 16- and 64-row lm_head
// tiles for few scored rows) are chosen by the shape, but each runs exactly this chain
// for every element it owns, with
// no split-K, and an MFMA output element depends only on its own A row and W
// row, so the bits of row i are the same whatever M is, whichever schedule runs
// and wherever row i sits in a tile.
//
// Data path.  Global -> LDS directly (buffer_load_dwordx4 ... lds into two
// buffers of XOR-swizzled 16-byte chunks, conflict-free for the MFMA operand
// reads) -> MFMA.  While the waves multiply out of one LDS buffer, the next
// K-slab streams into the other, so one barrier per 64-wide K-slab suffices
// and a load has a whole slab of MFMA work to arrive.  The copies use the
// MUBUF form rather than global_load_lds: the compiler treats a pending FLAT
// copy into LDS as an outstanding LDS access of unknown order and then waits
// for every LDS read in flight (lgkmcnt(0)) before each use of a fragment,
// while with the MUBUF form it waits only for the fragment's own read.  8 waves (4 x 2) each own a 64 x 128 sub-tile, i.e.
// 4 x 8 MFMA blocks (128 fp32 accumulators per lane); two waves per SIMD, and
// a wave raises its priority while it issues MFMAs.
// Workgroups are remapped so each XCD (8 per chip, each with its own L2) gets
// a contiguous range of tiles, grouped 4 or 8 M-tiles at a time so that they
// share W tiles in L2.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// buffer_load_dwordx4 ... lds (the LLVM intrinsic llvm.amdgcn.raw.buffer.load.lds):
// each lane copies 16 bytes from the buffer at voffset + soffset into LDS at the
// wave-uniform base + 16 * lane.
__device__ void raw_buffer_load_lds(i32x4_t rsrc, __attribute__((address_space(3))) void* lds, int size,
                                    int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer descriptor (stride 0) of a global address with a 2 GiB range; callers
// rebase it at the first row a workgroup reads, so every offset stays far below it.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
  r.z = 0x7FFFFFFF;
  r.w = 0x00020000;
  return r;
}

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int KCH = BK / 8;  // 16-byte chunks per LDS row
constexpr int NWM = 4, NWN = 2;          // waves along M and N
constexpr int WTM = BM / NWM, WTN = BN / NWN;  // 64 x 128 per wave
constexpr int MI = WTM / 16, NI = WTN / 16;    // 4 x 8 MFMA blocks per wave
constexpr int THREADS = NWM * NWN * 64;
constexpr int STAGE = (BM + BN) * KCH;   // 16-byte chunks per LDS buffer
constexpr int LM_SMALL_M = 16;           // lm_head rows up to which 16-row tiles are used
constexpr int LM_MID_M = 128;            // ... and up to which 64-row tiles are used

enum { K_BF16 = 0, K_F32 = 1, K_SILU = 2, K_LMHEAD = 3, K_ATOMIC = 4, K_PART = 5, K_ROPE = 6, K_ADD = 7 };

struct GemmArgs {
  const bf16_t* A;
  const int32_t* a_rows;  // gather: A row of output row r is a_rows[r] / a_div
  int a_div;
  const bf16_t* W;
  void* C;
  int M, N, K;  // N: W rows (K_SILU: 2 * I; K_LMHEAD: vocab)
  int tiles_m, tiles_n;
  const int32_t* ids;
  float* part_m;
  float* part_s;
  float* zid;
  // grouped (per-expert) mode: m-tile i is gtiles[3i..3i+2] = (group, first row, rows),
  // valid for i < *n_gtiles; group g uses W + g * w_group_stride.
  const int32_t* gtiles;
  const int32_t* n_gtiles;
  size_t w_group_stride;
  // split-K: workgroup y covers K range [y * k_split, min(K, (y + 1) * k_split)).
  // K_ATOMIC (non-invariant mode only) atomically adds its fp32 partial to C; K_PART
  // stores it to C + y * M * N (fixed slices, summed later in slice order)
  int k_split;
  // K_ROPE: the QKV projection's epilogue rotates q and k at each token's position
  // and writes q to q_out [M, nq * 128] and k, v to the token's paged-cache slot
  bf16_t* q_out;
  const int32_t* tok_pos;
  const int32_t* tok_slot;
  const float* rcos;
  const float* rsin;
  KvLayer kv;
  int nq, nkv, fp8;
  // skinny NORM (M <= 4): A rows are RMSNorm(res rows) * gamma, computed in the kernel
  const bf16_t* res;
  const bf16_t* gamma;
  float eps;
};

// Row r of an LDS tile holds 8 chunks of 16 bytes; chunk c is stored at
// position c ^ ((r >> 1) & 7).  Rows alternate between the two 32-bank halves
// of the 64 banks and the XOR spreads 8 consecutive row pairs over all chunk
// positions, so 16 lanes reading 16 consecutive rows at one chunk hit 16
// distinct 4-bank groups.
__device__ __forceinline__ int swz(int row, int ch) { return row * KCH + (ch ^ ((row >> 1) & 7)); }

// LDS row of a wave's n-th 16-column MFMA block.  SiLU tiles hold BN/2 gate
// rows then the BN/2 matching up rows; a wave's first NI/2 blocks are gate
// columns and its last NI/2 the up columns of the same outputs.
template <int KIND>
__device__ __forceinline__ int b_lds_row(int wn, int ni) {
  if constexpr (KIND == K_SILU) {
    return (ni < NI / 2) ? wn * (WTN / 2) + ni * 16 : BN / 2 + wn * (WTN / 2) + (ni - NI / 2) * 16;
  } else {
    return wn * WTN + ni * 16;
  }
}

// TBM: rows per tile.  256 (4 waves along M) for every GEMM, or 16 / 64 (one wave
// along M) for the lm_head over a few rows (decode, small batches), which would
// otherwise stream up to 255 duplicated A rows per tile; the per-element chain and
// the epilogue's reduction order over the 256 columns are the same either way.
template <int KIND, bool GATHER, bool GROUPED, int TBM = BM>
__global__ __launch_bounds__((TBM >= 64 ? TBM / 64 : 1) * NWN * 64, 1) void gemm_kernel(GemmArgs p) {
  constexpr int KBM = TBM;
  constexpr int KNWM = TBM >= 64 ? TBM / 64 : 1;
  constexpr int KWTM = KBM / KNWM;
  constexpr int KMI = KWTM / 16;
  constexpr int KTHREADS = KNWM * NWN * 64;
  constexpr int KSTAGE = (KBM + BN) * KCH;
  __shared__ u32x4_t smem[2 * KSTAGE];  // two buffers (2 x 64 KiB at TBM = 256)

  // ---- tile id: XCD-contiguous ranges, then groups of GM M-tiles whose tiles run
  // column by column (GM tiles sharing a W tile in L2).  GM = 6 for the gate_up GEMM, 4 for
  // QKV, 8 for the others, measured in the recompute: gate_up 4 % faster with 4 than 8, then
  // 598 -> 592 us with 6 (2 and 3 slower; QKV and the others even with 6); the O / down
  // projections and the lm_head were slower with 4
  const int n_tiles = p.tiles_m * p.tiles_n;
  const int per_xcd = gridDim.x >> 3;  // grid is a multiple of 8
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= n_tiles) return;
  constexpr int GM = (KIND == K_SILU) ? 6 : (KIND == K_ROPE) ? 4 : 8;
  const int width = GM * p.tiles_n;
  const int first_m = (tile / width) * GM;
  const int gsz = min(p.tiles_m - first_m, GM);
  const int tm = first_m + (tile % width) % gsz;
  const int tn = (tile % width) / gsz;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int K = p.K;

  // rows [row_base, row_base + row_cnt) of C belong to this tile
  int row_base = tm * KBM, row_cnt = min(KBM, p.M - tm * KBM);
  const bf16_t* W = p.W;
  if constexpr (GROUPED) {
    if (tm >= *p.n_gtiles) return;
    const int grp = p.gtiles[3 * tm];
    row_base = p.gtiles[3 * tm + 1];
    row_cnt = p.gtiles[3 * tm + 2];
    W += (size_t)grp * p.w_group_stride;
  }

  // ---- loads: global -> LDS directly (buffer_load_dwordx4 ... lds, no VGPR staging).
  // One such load of a wave fills 64 consecutive 16-byte LDS chunks, lane l the
  // l-th, so the XOR swizzle is applied on the global side: the lane whose LDS
  // chunk position is P loads logical chunk (P % 8) ^ ((row >> 1) & 7) of row
  // P / 8 of the stacked [A tile; B tile].  Wave w issues loads i = 0..NL-1
  // covering positions (w * NL + i) * 64 + lane.  A load covers 8 whole LDS rows and
  // the A rows (the first KBM) end on a load boundary, so whether load i of a wave
  // reads A or W is the same for all its lanes.  Descriptors start at the tile's
  // first A row (the source base when rows are gathered) and first W row.
  constexpr int NL = KSTAGE / 64 / (KTHREADS / 64);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bf16_t* a_base = GATHER ? p.A : p.A + (size_t)row_base * K;
  int w_row0 = tn * BN;
  if constexpr (KIND == K_SILU) w_row0 = tn * (BN / 2);
  const i32x4_t rsA = buffer_rsrc(a_base);
  const i32x4_t rsW = buffer_rsrc(W + (size_t)w_row0 * K);
  int voff[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int P = (wv * NL + i) * 64 + lane;
    const int row = P / KCH;
    const int ch = (P % KCH) ^ ((row >> 1) & 7);
    if (row < KBM) {
      // rows past the tile's end duplicate its last row and are never stored
      int r = min(row, row_cnt - 1);
      if constexpr (GATHER) r = p.a_rows[row_base + r] / p.a_div;
      voff[i] = (int)(((size_t)r * K + ch * 8) * 2);
    } else {
      const int br = row - KBM;
      int n;
      if constexpr (KIND == K_SILU) {
        const int I = p.N >> 1;
        n = (br < BN / 2) ? br : I + (br - BN / 2);
      } else {
        n = min(br, p.N - 1 - w_row0);  // columns past N are masked in the epilogue
      }
      voff[i] = (int)(((size_t)n * K + ch * 8) * 2);
    }
  }
  auto issue = [&](int st, int k0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const bool is_a = (wv * NL + i) * 64 < KBM * KCH;
      raw_buffer_load_lds(is_a ? rsA : rsW,
                          (__attribute__((address_space(3))) void*)(smem + st * KSTAGE + (wv * NL + i) * 64), 16,
                          voff[i], k0 * 2, 0, 0);
    }
  };

  f32x4_t acc[KMI][NI];
#pragma unroll
  for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Operand order: the A fragment is the MFMA's first operand and the W fragment its
  // second for every kind, so a lane holds rows 4 (lane >> 4) + r and column lane & 15
  // of each 16x16 block.  The swapped order (W first, a lane holding 4 consecutive
  // columns of a row, for 8-byte epilogue accesses) gives every output element the same
  // chain and the same bits, but measured slower in the K loop: gate_up 609 -> 598 us
  // on this order, the recompute +1.1 % with the SiLU and residual-add epilogues moved
  // to it, and the QKV epilogue moved the other way 5 % slower.
  auto mfma = [&](const bf16x8_t& fa, const bf16x8_t& fb, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, c, 0, 0, 0);
  };
  auto lda = [&](int st, int ks, int mi) {
    return __builtin_bit_cast(
        bf16x8_t, smem[st * KSTAGE + swz(wm * KWTM + mi * 16 + (lane & 15), ks * 4 + (lane >> 4))]);
  };
  auto ldb = [&](int st, int ks, int ni) {
    return __builtin_bit_cast(
        bf16x8_t,
        smem[st * KSTAGE + KBM * KCH + swz(b_lds_row<KIND>(wn, ni) + (lane & 15), ks * 4 + (lane >> 4))]);
  };

  // Software pipeline over the two 32-wide K steps of each 64-wide slab.
  // Registers: fa0 / fa1 hold the A fragments of K step 0 / 1, fb the B
  // fragments of the step being multiplied; MFMAs run column block by column
  // block, and as soon as block ni is done its register takes block ni of the
  // next step.  step_a multiplies K step 0 of a slab while fetching step 1 of
  // the same slab; step_b multiplies step 1 while fetching step 0 of the next
  // slab, which the barrier between the two has published.  That barrier also
  // frees the slab's LDS buffer (its last fragments are in registers), so the
  // DMA of the slab after next is issued right after it.
  // The next step's A fragments are read after the MFMAs of the first column
  // blocks, FPG per block, never ahead of the step's first MFMAs: then at most 12
  // LDS reads are outstanding when an MFMA needs one of them, within what the LDS
  // counter can count, so the wait before it covers only reads issued a block or
  // more earlier instead of every read in flight.
  constexpr int FPG = (KMI + NI / 2 - 1) / (NI / 2);
  bf16x8_t fa0[KMI], fa1[KMI], fb[NI];
  auto step_a = [&](int st) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
      for (int mi = 0; mi < KMI; ++mi) acc[mi][ni] = mfma(fa0[mi], fb[ni], acc[mi][ni]);
      fb[ni] = ldb(st, 1, ni);
#pragma unroll
      for (int mi = 0; mi < KMI; ++mi)
        if (mi / FPG == ni) fa1[mi] = lda(st, 1, mi);
      __builtin_amdgcn_sched_group_barrier(0x008, KMI, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1 + FPG, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // copies(ni) runs before the MFMAs of column block ni (the slab copies' issue point)
  auto step_b = [&](int st, auto prefetch, auto copies) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      copies(ni);
#pragma unroll
      for (int mi = 0; mi < KMI; ++mi) acc[mi][ni] = mfma(fa1[mi], fb[ni], acc[mi][ni]);
      if constexpr (decltype(prefetch)::value) {
        fb[ni] = ldb(st ^ 1, 0, ni);
#pragma unroll
        for (int mi = 0; mi < KMI; ++mi)
          if (mi / FPG == ni) fa0[mi] = lda(st ^ 1, 0, mi);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KMI, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1 + FPG, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  int nk = K / BK;
  int kb = 0;
  if constexpr (KIND == K_ATOMIC || KIND == K_PART) {
    kb = blockIdx.y * p.k_split;
    nk = min(p.k_split, K - kb) / BK;
  }
  issue(0, kb);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < KMI; ++mi) fa0[mi] = lda(0, 0, mi);
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) fb[ni] = ldb(0, 0, ni);
  if (nk > 1) issue(1, kb + BK);
  step_a(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // The loop boundary sits right after a barrier, where no LDS read is in flight.  A wave
  // stalls while its copies are accepted, so the two waves of a SIMD issue theirs at
  // different points: the first half of the waves before the slab's first MFMAs, the
  // second half after the first half of the first K step's MFMA groups, while the first
  // half multiplies.  Measured against all waves issuing together: gate_up 647 -> 584 us,
  // QKV 228 -> 209, down 302 -> 281, lm_head (M = 8192) 4340 -> 4093; issuing later (the
  // second K step) or at four points was slower, copies spread over every MFMA group of
  // every wave slower in the recompute.
  const int copy_at = wv < (KTHREADS / 64) / 2 ? 0 : NI / 2;
  for (int kt = 0; kt + 1 < nk; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 2 < nk;
    step_b(st, std::true_type{}, [&](int ni) {
      if (more && ni == copy_at) issue(st, kb + (kt + 2) * BK);
    });
    step_a(st ^ 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads of slab kt+2 have landed
    __syncthreads();
  }
  step_b((nk - 1) & 1, std::false_type{}, [](int) {});

  // ---- epilogues.  Lane holds C[4*(lane>>4) + r][lane & 15] of each 16x16 block.
  const int lrow0 = wm * KWTM + 4 * (lane >> 4);  // row within the tile
  const int row0 = row_base + lrow0;
  if constexpr (KIND == K_ATOMIC) {
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + mi * 16 + r;
        if (lrow0 + mi * 16 + r < row_cnt) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int col = tn * BN + wn * WTN + ni * 16 + (lane & 15);
            if (col < p.N) atomicAdd(reinterpret_cast<float*>(p.C) + (size_t)row * p.N + col, acc[mi][ni][r]);
          }
        }
      }
  } else if constexpr (KIND == K_ADD) {
    // Residual add in place: a lane holds rows 4 (lane >> 4) + r, column lane & 15 of each
    // block; each element with the add+RMSNorm kernel's expression bf(bf(x) + r).  The
    // residual values of two row blocks are loaded together (rows past the tile read its
    // last row and are not written), then rewritten.
    static_assert(KMI % 2 == 0, "row blocks in pairs");
#pragma unroll
    for (int mp = 0; mp < KMI; mp += 2) {
      bf16_t old[2][4][NI];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = min(lrow0 + (mp + h) * 16 + r, row_cnt - 1);
          const bf16_t* rp = reinterpret_cast<const bf16_t*>(p.C) + (size_t)(row_base + lr) * p.N;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) old[h][r][ni] = rp[tn * BN + wn * WTN + ni * 16 + (lane & 15)];
        }
      asm volatile("" ::: "memory");   // the loads above stay ahead of the stores below
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = lrow0 + (mp + h) * 16 + r;
          if (lr < row_cnt) {
            bf16_t* rp = reinterpret_cast<bf16_t*>(p.C) + (size_t)(row_base + lr) * p.N;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              rp[tn * BN + wn * WTN + ni * 16 + (lane & 15)] =
                  f2bf(bf2f(f2bf(acc[mp + h][ni][r])) + bf2f(old[h][r][ni]));
          }
        }
    }
  } else if constexpr (KIND == K_BF16 || KIND == K_F32 || KIND == K_PART) {
    void* Cout = p.C;
    if constexpr (KIND == K_PART) Cout = reinterpret_cast<float*>(p.C) + (size_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + mi * 16 + r;
        if (lrow0 + mi * 16 + r < row_cnt) {
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int col = tn * BN + wn * WTN + ni * 16 + (lane & 15);
            if (col >= p.N) continue;
            if constexpr (KIND == K_BF16)
              reinterpret_cast<bf16_t*>(Cout)[(size_t)row * p.N + col] = f2bf(acc[mi][ni][r]);
            else
              reinterpret_cast<float*>(Cout)[(size_t)row * p.N + col] = acc[mi][ni][r];
          }
        }
      }
  } else if constexpr (KIND == K_SILU) {
    // silu(g) * u: the gate and up values of an output (row, column) sit in blocks ni and
    // ni + NI/2 of the same lane; 16 lanes store 16 consecutive columns of a row
    const int I = p.N >> 1;
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + mi * 16 + r;
        if (lrow0 + mi * 16 + r < row_cnt) {
          bf16_t* out = reinterpret_cast<bf16_t*>(p.C) + (size_t)row * I;
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) {
            const int col = tn * (BN / 2) + wn * (WTN / 2) + ni * 16 + (lane & 15);
            const float g = bf2f(f2bf(acc[mi][ni][r]));
            const float u = bf2f(f2bf(acc[mi][ni + NI / 2][r]));
            out[col] = f2bf(silu_f32(g) * u);
          }
        }
      }
  } else if constexpr (KIND == K_ROPE) {
    // Head dimension 128: wave wn of column tile tn holds head 2 tn + wn, and the
    // rotation pair (e, e + 64) of a row sits in blocks ni and ni + 4 of the same
    // lane.  Each value is first rounded to bf16 (what a qkv buffer would hold), then
    // rotated, rounded, scaled and encoded with the expressions of the standalone
    // RoPE/KV-write kernel, so both give the same bits.
    const int hd = tn * 2 + wn;
    const bool is_q = hd < p.nq, rot = hd < p.nq + p.nkv;
    const bool is_k = !is_q && rot;
    const int gk = is_q ? 0 : (is_k ? hd - p.nq : hd - p.nq - p.nkv);
    const int lc = lane & 15;
    // The loads are gathered ahead of the stores (which the compiler must otherwise
    // assume may alias them, serialising every row behind the previous one): the
    // positions and cache slots of the lane's rows first, then the rotation factors of
    // one block of 16 rows at a time (more at once would not fit the registers).
    int posr[KMI][4], slotr[KMI][4];
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = lrow0 + mi * 16 + r;
        const int t = row_base + (lr < row_cnt ? lr : 0);
        posr[mi][r] = rot ? p.tok_pos[t] : 0;
        slotr[mi][r] = is_q ? 0 : p.tok_slot[t];
      }
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi) {
      float rc[4][NI / 2], rs[4][NI / 2];
      if (rot) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) {
            const size_t k = (size_t)posr[mi][r] * 64 + ni * 16 + lc;
            rc[r][ni] = p.rcos[k];
            rs[r][ni] = p.rsin[k];
          }
      }
      asm volatile("" ::: "memory");   // the loads above stay ahead of the stores below
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = lrow0 + mi * 16 + r;
        const bool ok = lr < row_cnt;            // the same for the 16 lanes of a row
        const int t = row_base + (ok ? lr : 0);
        float y1[NI / 2], y2[NI / 2];
        if (rot) {
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) {
            const float c = rc[r][ni], sn = rs[r][ni];
            const float x1 = bf2f(f2bf(acc[mi][ni][r])), x2 = bf2f(f2bf(acc[mi][ni + NI / 2][r]));
            const float a1 = x1 * c, b1 = x2 * sn;
            const float a2 = x2 * c, b2 = x1 * sn;
            y1[ni] = bf2f(f2bf(a1 - b1));
            y2[ni] = bf2f(f2bf(a2 + b2));
          }
        } else {
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) {
            y1[ni] = bf2f(f2bf(acc[mi][ni][r]));
            y2[ni] = bf2f(f2bf(acc[mi][ni + NI / 2][r]));
          }
        }
        size_t crow = 0;  // cache row of (block, kv head, slot)
        if (!is_q) {
          const int slot = slotr[mi][r];
          crow = ((size_t)(slot >> 6) * p.nkv + gk) * 64 + (slot & 63);
        }
        if (is_q || !p.fp8) {
          bf16_t* dst = is_q ? p.q_out + (size_t)t * p.nq * 128 + hd * 128
                             : reinterpret_cast<bf16_t*>(is_k ? p.kv.k : p.kv.v) + crow * 128;
          if (ok) {
#pragma unroll
            for (int ni = 0; ni < NI / 2; ++ni) {
              dst[ni * 16 + lc] = f2bf(y1[ni]);
              dst[64 + ni * 16 + lc] = f2bf(y2[ni]);
            }
          }
        } else {
          // scale from the head's amax over its 128 rounded values (an exact max,
          // so the order does not matter): 8 per lane, then the row's 16 lanes
          float amax = 0.0f;
#pragma unroll
          for (int ni = 0; ni < NI / 2; ++ni) amax = fmaxf(amax, fmaxf(fabsf(y1[ni]), fabsf(y2[ni])));
          amax = fmaxf(amax, lane_xor<1>(amax));
          amax = fmaxf(amax, lane_xor<2>(amax));
          amax = fmaxf(amax, lane_xor<4>(amax));
          amax = fmaxf(amax, lane_xor<8>(amax));
          const float sc = kv_scale_from_amax(amax);
          uint8_t* dst = reinterpret_cast<uint8_t*>(is_k ? p.kv.k : p.kv.v) + crow * 128;
          if (ok) {
#pragma unroll
            for (int ni = 0; ni < NI / 2; ++ni) {
              dst[ni * 16 + lc] = (uint8_t)kv_encode(y1[ni], sc);
              dst[64 + ni * 16 + lc] = (uint8_t)kv_encode(y2[ni], sc);
            }
            if (lc == 0) (is_k ? p.kv.ks : p.kv.vs)[crow] = sc;
          }
        }
      }
    }
  } else {  // K_LMHEAD: per row, (max, sum exp) over this 256-column vocab chunk
    // Row lr's chunk max is max over the NWN waves of redm[w][lr]; its sum is
    // s_0 + s_1 (+ ...) over reds[w][lr] in wave order; within a wave the
    // columns reduce over the NI sub-blocks in order, then a fixed xor butterfly.
    const int V = p.N;
    float* redm = reinterpret_cast<float*>(smem);  // [NWN][KBM]; the loop ended on a barrier
    float* reds = redm + NWN * KBM;                  // [NWN][KBM]
    // the rows' token ids, loaded first so that their latency overlaps the two passes
    // (rows past the tile repeat its last row; they are never stored)
    int idr[KMI][4];
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) idr[mi][r] = p.ids[row_base + min(lrow0 + mi * 16 + r, row_cnt - 1)];
    if (tn * BN + BN > V) {
      // the vocabulary's last, partial chunk: columns past V become -inf, which adds
      // nothing to the max and exactly +0 (2^-inf) to the sum, so the passes below need
      // no per-logit bound checks
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if (tn * BN + wn * WTN + ni * 16 + (lane & 15) < V) continue;
#pragma unroll
        for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mi][ni][r] = -INFINITY;
      }
    }
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) mx = fmaxf(mx, acc[mi][ni][r]);
        mx = fmaxf(mx, lane_xor<1>(mx));
        mx = fmaxf(mx, lane_xor<2>(mx));
        mx = fmaxf(mx, lane_xor<4>(mx));
        mx = fmaxf(mx, lane_xor<8>(mx));
        if ((lane & 15) == 0) redm[wn * KBM + lrow0 + mi * 16 + r] = mx;
      }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = lrow0 + mi * 16 + r;
        float m = redm[lr];
#pragma unroll
        for (int w2 = 1; w2 < NWN; ++w2) m = fmaxf(m, redm[w2 * KBM + lr]);
        float s = 0.0f;
        // e^(z - m) as 2^((z - m) log2 e) on v_exp_f32: three instructions per logit
        // instead of the library expf's dozen, in every lm_head schedule alike
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) s = s + fexp2((acc[mi][ni][r] - m) * LOG2E);
        s = s + lane_xor<1>(s);
        s = s + lane_xor<2>(s);
        s = s + lane_xor<4>(s);
        s = s + lane_xor<8>(s);
        if ((lane & 15) == 0) reds[wn * KBM + lr] = s;
      }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < KMI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = lrow0 + mi * 16 + r;
        const int row = row_base + lr;
        if (lr < row_cnt) {
          if (wn == 0 && (lane & 15) == 0) {
            float m = redm[lr], s = reds[lr];
#pragma unroll
            for (int w2 = 1; w2 < NWN; ++w2) {
              m = fmaxf(m, redm[w2 * KBM + lr]);
              s = s + reds[w2 * KBM + lr];
            }
            p.part_m[(size_t)tn * p.M + row] = m;
            p.part_s[(size_t)tn * p.M + row] = s;
          }
          const int id = idr[mi][r];
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int col = tn * BN + wn * WTN + ni * 16 + (lane & 15);
            if (col == id) p.zid[row] = acc[mi][ni][r];
          }
        }
      }
  }
}


// ---- skinny schedule for M <= 128 (decode), and up to 512 rows where a latency model
// favours it.  The same per-element arithmetic as gemm_kernel -- one fp32 accumulator
// from zero, v_mfma_f32_16x16x32_bf16 over ascending 32-wide K steps, the same epilogue
// -- with a different assignment of output elements: a one-wave workgroup owns 16
// output columns (16 gate + 16 up for SiLU) and up to 2 (SiLU: 4) blocks of 16 rows,
// so N/16 waves per row group stream the weights instead of N/256 workgroups.  K is cut into stages of
// SK_KC (512 for a single row block and 256 for two when K allows); each stage's W rows and A
// rows are copied by buffer_load ... lds into a private LDS ring of D stages, so D
// stages of loads are in flight while the MFMAs consume the oldest.  A single
// wave needs no barrier, only vmcnt.  The stage width and the A rows a stage
// holds change which loads run, never the MFMA chain of an output element.
constexpr int SK_KC = 128;                  // K per stage (default)
constexpr int SK_NORM_MAX_K = 2048;         // NORM: K (the hidden size) up to one norm slice per thread


// s_waitcnt immediate for "vmcnt <= v" (gfx9 encoding; lgkmcnt/expcnt unconstrained)
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}


// GROUPED (the MoE expert GEMMs with few rows per expert): blockIdx.y is an entry of
// the device tile list (group, first row, rows <= 16), W is the group's slice, A rows
// are gathered through a_rows when GATHER.
// AR: A rows a stage holds.  16 * MT, or 4 when M <= 4 (decode): the MFMA's rows past
// AR read row AR - 1 (their outputs are never stored), so a stage copies 4 A rows
// instead of 16.  KC: K per stage (SK_KC, or 512 for one row block: each W row is then
// read in 1 KiB runs rather than 256-byte ones).
// NORM (M <= 4, K <= 2048, no gather): the A rows are not copied from memory but
// normalised by the wave itself from the residual rows p.res and the weight p.gamma,
// with the add+RMSNorm kernel's expressions and reduction tree (see norm_rows below),
// into an LDS region of their own; the weight stream starts before that work.
// CW: output columns (RoPE: rotation pairs) per wave, 16, or 8 for calls that would
// otherwise launch fewer waves than CUs: the wave streams 8 weight rows per stream, its
// MFMA lanes 8-15 read rows 0-7 again and their outputs are not stored, so twice as many
// CUs stream the weights.
template <int KIND, int MT, bool GATHER = false, bool GROUPED = false, int AR = 16 * MT, int KC = SK_KC,
          bool NORM = false, int CW = 16>
__global__ __launch_bounds__(64) void gemm_skinny_kernel(GemmArgs p) {
  static_assert(AR == 16 * MT || (MT == 1 && AR == 4), "A rows per stage");
  static_assert(CW == 16 || (CW == 8 && KIND != K_SILU && !GROUPED), "8 columns per wave: dense calls");
  static_assert(!NORM || (MT == 1 && AR == 4 && !GATHER && !GROUPED), "norm-fused A: M <= 4, plain rows");
  constexpr int ROWCH = KC / 8;                         // 16-byte chunks per row per stage
  // the copy swizzle (chunk ^ (row & 15)) must stay inside a row's stage: at fewer than
  // 16 chunks it would read past the stage, and past the matrix on its last row
  static_assert(ROWCH % 16 == 0, "a stage row holds a multiple of 16 chunks");
  // weight streams: (gate, up) rows for SiLU; for RoPE the rows e and e + 64 of a head
  constexpr int NB = (KIND == K_SILU || KIND == K_ROPE) ? 2 : 1;
  constexpr int WCH = NB * CW * ROWCH;                  // W chunks per stage
  constexpr int SCH = WCH + (NORM ? 0 : AR * ROWCH);    // chunks per stage
  constexpr int LPS = SCH / 64;                         // wave loads per stage
  static_assert(SCH % 64 == 0, "whole wave loads per stage");
  constexpr int NA_ROW = SK_NORM_MAX_K / 8;             // NORM: A chunks per row (rows 4 KiB apart)
  constexpr int D_LDS = (128 * 1024 / 16 - (NORM ? AR * NA_ROW : 0)) / SCH;
  constexpr int D_VM = 1 + 63 / LPS;
  constexpr int D0 = D_LDS < D_VM ? D_LDS : D_VM;
  constexpr int D = D0 > 16 ? 16 : D0;                  // ring depth (stages in flight)
  // chunk c of row r of a stage sits at r * ROWCH + (c ^ (r & 15)): 16 lanes reading
  // 16 rows at one chunk hit 16 distinct 4-bank groups
  auto swz = [](int row, int ch) { return row * ROWCH + (ch ^ (row & 15)); };
  static_assert(D >= 2, "ring too shallow");
  __shared__ u32x4_t ring[D * SCH];
  __shared__ u32x4_t a_nrm[NORM ? AR * NA_ROW : 1];
  const int lane = threadIdx.x;
  const int K = p.K;
  const int ncols = (KIND == K_SILU || KIND == K_ROPE) ? p.N / 2 : p.N;
  const int cb = blockIdx.x;
  const int col = cb * CW + (lane & 15);
  // K_ROPE (head_dim 128): wave cb holds rotation pairs e = CW (cb % (64 / CW)) + 0..CW-1 of
  // head cb / (64 / CW), i.e. QKV columns 128 h + e (stream 0) and 128 h + 64 + e (stream 1)
  const int rh = cb / (64 / CW), re0 = (cb % (64 / CW)) * CW;
  int row_base = 0, M = p.M;
  const bf16_t* W = p.W;
  if constexpr (GROUPED) {
    if ((int)blockIdx.y >= *p.n_gtiles) return;
    W += (size_t)p.gtiles[3 * blockIdx.y] * p.w_group_stride;
    row_base = p.gtiles[3 * blockIdx.y + 1];
    M = p.gtiles[3 * blockIdx.y + 2];
  } else {
    // blockIdx.y: which block of AR rows (the grid has ceil(M / AR) of them)
    row_base = blockIdx.y * AR;
    M = min(AR, p.M - row_base);
  }
  // load j of a stage fills ring chunks [j*64, j*64+64): lane's chunk P = j*64 + lane.
  // WCH is a multiple of 64, so a load reads W or A for all its lanes.  Descriptors
  // start at the wave's first W row and its first A row (the source base when rows
  // are gathered).
  const int w_row0 = (KIND == K_ROPE) ? rh * 128 : cb * CW;
  const i32x4_t rsW = buffer_rsrc(W + (size_t)w_row0 * K);
  const i32x4_t rsA = buffer_rsrc(GATHER ? p.A : p.A + (size_t)row_base * K);
  int voff[LPS];
#pragma unroll
  for (int j = 0; j < LPS; ++j) {
    const int P = j * 64 + lane;
    if (P < WCH) {
      const int r = P / ROWCH, ch = (P % ROWCH) ^ (r & 15);
      int wr;
      if constexpr (KIND == K_ROPE) {
        wr = re0 + (r & (CW - 1)) + (r >= CW ? 64 : 0);
      } else {
        wr = min(cb * CW + (r & (CW - 1)), ncols - 1) - w_row0;
        if (NB == 2 && r >= 16) wr += ncols;             // up rows follow the gate rows
      }
      voff[j] = (int)(((size_t)wr * K + ch * 8) * 2);
    } else {
      const int P2 = P - WCH;
      const int r = P2 / ROWCH, ch = (P2 % ROWCH) ^ (r & 15);
      int ar = min(r, M - 1);
      if constexpr (GATHER) ar = p.a_rows[row_base + ar] / p.a_div;
      voff[j] = (int)(((size_t)ar * K + ch * 8) * 2);
    }
  }
  auto issue = [&](int slot, int k0) {
#pragma unroll
    for (int j = 0; j < LPS; ++j)
      raw_buffer_load_lds(j * 64 < WCH ? rsW : rsA,
                          (__attribute__((address_space(3))) void*)(ring + slot * SCH + j * 64), 16, voff[j],
                          k0 * 2, 0, 0);
  };
  f32x4_t acc[NB][MT];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[b][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nst = K / KC;
  // NORM: the residual rows and the norm weight are loaded before the weight stream is
  // issued (loads complete in issue order, so waiting for them then waits for nothing
  // else) and normalised while the first stages stream in
  // (unconditional, at clamped addresses -- rows past M repeat row M - 1, columns past K
  // repeat the last 8 -- so that they issue back to back and are waited for once)
  uint4 xv[NORM ? 4 : 1][4], gv[4];
  if constexpr (NORM) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int c0 = min((w * 64 + lane) * 8, K - 8);
        xv[r][w] = *reinterpret_cast<const uint4*>(p.res + (size_t)min(r, M - 1) * K + c0);
      }
#pragma unroll
    for (int w = 0; w < 4; ++w) gv[w] = *reinterpret_cast<const uint4*>(p.gamma + min((w * 64 + lane) * 8, K - 8));
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int st = 0; st < D; ++st) {
    // NORM issues every stage unconditionally (a stage past the last one re-reads the
    // last into a slot never read): with a branch here the compiler's wait for the
    // residual rows would have to cover the path without copies and so wait for them
    if constexpr (NORM) issue(st, min(st, nst - 1) * KC);
    else if (st < nst) issue(st, st * KC);
  }
  if constexpr (NORM) {
    // The add+RMSNorm kernel runs 256 threads on a row, thread t over columns
    // [8t, 8t + 8) (one slice: K <= 2048): its sum of squares in column order, the
    // xor butterfly over each 64-thread wave, the four wave sums added in wave order,
    // inv = 1 / sqrt(sum / K + eps), h = bf((x * inv) * g).  Lane l plays threads
    // l, l + 64, l + 128 and l + 192, so every value and every addition is the same.
    // Row r's chunk c (8 columns) is stored at r * NA_ROW + (c ^ 4r): the MFMA reads
    // 4 consecutive chunks of 4 rows, which then fall in 16 distinct bank groups.
    // sums of squares of the M rows, then their butterflies step by step together
    // (the exchanges of the 4 per row overlap)
    float ssw[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float ss = 0.0f;
        if (r < M && (w * 64 + lane) * 8 < K) {
          const bf16_t* xp = reinterpret_cast<const bf16_t*>(&xv[r][w]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = bf2f(xp[i]);
            ss = ss + x * x;
          }
        }
        ssw[r][w] = ss;
      }
    auto bfly = [&](auto O) {
      constexpr int o = decltype(O)::value;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (r < M) {
#pragma unroll
          for (int w = 0; w < 4; ++w) ssw[r][w] = ssw[r][w] + lane_xor<o>(ssw[r][w]);
        }
    };
    bfly(std::integral_constant<int, 32>{});
    bfly(std::integral_constant<int, 16>{});
    bfly(std::integral_constant<int, 8>{});
    bfly(std::integral_constant<int, 4>{});
    bfly(std::integral_constant<int, 2>{});
    bfly(std::integral_constant<int, 1>{});
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r >= M) break;
      float tot = ssw[r][0];
#pragma unroll
      for (int w = 1; w < 4; ++w) tot = tot + ssw[r][w];
      const float inv = 1.0f / sqrtf(tot / (float)K + p.eps);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int t = w * 64 + lane;
        if (t * 8 < K) {
          const bf16_t* gp = reinterpret_cast<const bf16_t*>(&gv[w]);
          const bf16_t* xp = reinterpret_cast<const bf16_t*>(&xv[r][w]);
          u32x4_t hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float h0 = (bf2f(xp[2 * i]) * inv) * bf2f(gp[2 * i]);
            const float h1 = (bf2f(xp[2 * i + 1]) * inv) * bf2f(gp[2 * i + 1]);
            hv[i] = pack_bf2(f2bf(h0), f2bf(h1));
          }
          a_nrm[r * NA_ROW + (t ^ (4 * r))] = hv;
        }
      }
    }
  }
  for (int c = 0; c < nst; ++c) {
    if (c + D - 1 < nst) wait_vmcnt<(D - 1) * LPS>();   // stage c has landed
    else wait_vmcnt<0>();
    const u32x4_t* stg = ring + (c % D) * SCH;
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      const int ch = s * 4 + (lane >> 4);
      bf16x8_t bw[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) bw[b] = __builtin_bit_cast(bf16x8_t, stg[swz(b * CW + (lane & (CW - 1)), ch)]);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        bf16x8_t a;
        if constexpr (NORM) {
          const int ar = min(lane & 15, M - 1);
          a = __builtin_bit_cast(bf16x8_t, a_nrm[ar * NA_ROW + ((c * ROWCH + ch) ^ (4 * ar))]);
        } else {
          const int ar = AR == 16 * MT ? mi * 16 + (lane & 15) : min(lane & 15, AR - 1);
          a = __builtin_bit_cast(bf16x8_t, stg[WCH + swz(ar, ch)]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw[b], acc[b][mi], 0, 0, 0);
      }
    }
    if (c + D < nst) {
      __builtin_amdgcn_s_waitcnt(0x0070 | (0x3 << 14) | 0xF);   // lgkmcnt(0): this slot's reads are done
      issue(c % D, (c + D) * KC);
    }
  }
  if (cb * CW >= ncols || (lane & 15) >= CW) return;
  // lane holds C[16 mi + 4 (lane >> 4) + r][col]
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = mi * 16 + 4 * (lane >> 4) + r;
      if (lr >= M) continue;
      const int row = row_base + lr;
      if constexpr (KIND == K_SILU) {
        const float g = bf2f(f2bf(acc[0][mi][r]));
        const float u = bf2f(f2bf(acc[1][mi][r]));
        reinterpret_cast<bf16_t*>(p.C)[(size_t)row * ncols + col] = f2bf(silu_f32(g) * u);
      } else if constexpr (KIND == K_ROPE) {
        // bf16 cache only: the expressions of the standalone RoPE/KV-write kernel
        const int e = re0 + (lane & 15);
        const float x1 = bf2f(f2bf(acc[0][mi][r])), x2 = bf2f(f2bf(acc[1][mi][r]));
        float y1 = x1, y2 = x2;
        if (rh < p.nq + p.nkv) {
          const int pos = p.tok_pos[row];
          const float c = p.rcos[(size_t)pos * 64 + e], sn = p.rsin[(size_t)pos * 64 + e];
          const float a1 = x1 * c, b1 = x2 * sn;
          const float a2 = x2 * c, b2 = x1 * sn;
          y1 = bf2f(f2bf(a1 - b1));
          y2 = bf2f(f2bf(a2 + b2));
        }
        bf16_t* dst;
        if (rh < p.nq) {
          dst = p.q_out + (size_t)row * p.nq * 128 + rh * 128;
        } else {
          const bool is_k = rh < p.nq + p.nkv;
          const int gk = is_k ? rh - p.nq : rh - p.nq - p.nkv;
          const int slot = p.tok_slot[row];
          const size_t crow = ((size_t)(slot >> 6) * p.nkv + gk) * 64 + (slot & 63);
          dst = reinterpret_cast<bf16_t*>(is_k ? p.kv.k : p.kv.v) + crow * 128;
        }
        dst[e] = f2bf(y1);
        dst[64 + e] = f2bf(y2);
      } else if constexpr (KIND == K_BF16) {
        reinterpret_cast<bf16_t*>(p.C)[(size_t)row * p.N + col] = f2bf(acc[0][mi][r]);
      } else if constexpr (KIND == K_ADD) {
        // the residual add in place, with the tiled epilogue's expression bf(bf(x) + r);
        // each element is read and written by this lane only
        bf16_t* cp = reinterpret_cast<bf16_t*>(p.C) + (size_t)row * p.N + col;
        *cp = f2bf(bf2f(f2bf(acc[0][mi][r])) + bf2f(*cp));
      } else {
        reinterpret_cast<float*>(p.C)[(size_t)row * p.N + col] = acc[0][mi][r];
      }
    }
}

// A skinny wave multiplies its 16 weight rows with at most SK_ROW_BLOCKS blocks of 16 A
// rows; more rows go to more waves (grid.y), which stream the same weight rows again from
// L2.  Each wave's bandwidth is capped by the copies it can keep in flight, and with 64
// rows its A stream (256 KiB at K = 2048) was 4x its weight stream.  Measured on the
// decode step at B = 64, rows per wave 16 / 32 / 64: 3.08 / 2.57 / 2.79 ms; the rollout at
// a cap of 128 sequences 20.2 K -> 23.6 K tokens/s with 32.  Such 32-row waves take
// 256-wide K stages where K allows (each weight row read in 512-byte runs; same ring
// size): down at 64 rows 15.8 -> 14.6 us, the B = 64 decode step 2.437 -> 2.413 ms.
constexpr int SK_ROW_BLOCKS = 2;
// The SiLU form streams two weight rows per output column, so a second row group costs
// twice the re-read: 64 rows per wave there (B = 64 decode step 2.557 -> 2.470 ms
// against 32, the same as 128).
constexpr int SK_SILU_ROW_BLOCKS = 4;
constexpr int SKINNY_CUS = 256;  // compute units of the part

template <int KIND>
static hipError_t dispatch_skinny(const GemmArgs& a, hipStream_t s) {
  const int ncols = (KIND == K_SILU) ? a.N / 2 : a.N;
  const int grid = ncols / 16;
  const int mt = std::min((a.M + 15) / 16, KIND == K_SILU ? SK_SILU_ROW_BLOCKS : SK_ROW_BLOCKS);
  const bool wide = a.K % 512 == 0;
  const dim3 g1(grid), gm(grid, (a.M + 16 * mt - 1) / (16 * mt));
  // at most 4 rows, a single weight stream and fewer 16-column waves than CUs: 8 columns
  // per wave, so that every CU streams weights (same box, M = 1: O 5.4 -> 5.2 us, down 9.7 ->
  // 9.0, the B = 1 decode step 1.693 -> 1.652 ms).  With 16 or 32 A rows per wave the doubled
  // A stream cancels the gain (down at 24-32 rows 14.4 -> 14.7-14.9 us), so those keep 16.
  constexpr bool one_stream = KIND != K_SILU && KIND != K_ROPE;
  constexpr int CW8 = one_stream ? 8 : 16;
  const bool narrow = one_stream && grid < SKINNY_CUS && ncols % 8 == 0;
  const dim3 g1n(2 * grid);
  if (a.M <= 4 && wide && narrow)
    hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 1, false, false, 4, 512, false, CW8>), g1n, dim3(64), 0, s, a);
  else if (a.M <= 4 && wide) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 1, false, false, 4, 512>), g1, dim3(64), 0, s, a);
  else if (a.M <= 4) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 1, false, false, 4>), g1, dim3(64), 0, s, a);
  else if (mt == 1 && wide) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 1, false, false, 16, 512>), gm, dim3(64), 0, s, a);
  else if (mt == 1) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 1>), gm, dim3(64), 0, s, a);
  else if (mt == 2 && KIND != K_SILU && a.K % 256 == 0)
    hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 2, false, false, 32, 256>), gm, dim3(64), 0, s, a);
  else if (mt == 2) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 2>), gm, dim3(64), 0, s, a);
  else if (mt <= 4) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 4>), gm, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 8>), gm, dim3(64), 0, s, a);
  return hipGetLastError();
}

// Schedule choice for M in (SKINNY_MAX_M, SKINNY_DENSE_MAX_M]: a 256 x 256 tile takes
// ~42 us per 2048 of K, and a call with no more tiles than CUs takes one tile's time;
// the skinny schedule takes ~11 ns per (wave x 2048 of K x weight stream) plus ~5 us,
// with N/16 waves (N/32 for the two-stream SiLU and RoPE forms) per 32 rows.  Measured
// (us, tiled / skinny): M = 160: O 41 / 12, down 112 / 31, QKV 41 / 20, gate_up 42 / 39;
// M = 512: O 42 / 26, down 116 / 64, QKV 43 / 51, gate_up 46 / 111.  Either way every
// output element is the same chain.
bool gemm_prefers_skinny(int M, int N, int K, int epi, bool rope) {
  if (M <= SKINNY_MAX_M) return true;
  if (M > SKINNY_DENSE_MAX_M || K % SK_KC != 0 || N % 16 != 0) return false;
  const bool two = rope || epi == EPI_SILU;
  const double waves = (double)(two ? N / 32 : N / 16) * ((M + 31) / 32);
  const double skinny_us = 5.0 + 0.011 * waves * (K / 2048.0) * (two ? 2 : 1);
  const int tiles = ((M + BM - 1) / BM) * (two ? (N / 2) / (BN / 2) : (N + BN - 1) / BN);
  const double tiled_us = 42.0 * (K / 2048.0) * ((tiles + 255) / 256);
  return skinny_us < tiled_us;
}

template <int KIND>
static hipError_t dispatch(const GemmArgs& a, bool gather, hipStream_t s) {
  const int n_tiles = a.tiles_m * a.tiles_n;
  const int grid = (n_tiles + 7) / 8 * 8;
  if (gather)
    hipLaunchKernelGGL((gemm_kernel<KIND, true, false>), dim3(grid), dim3(THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<KIND, false, false>), dim3(grid), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const void* A, const int32_t* a_rows, const void* W, void* C, int M, int N,
                       int K, int epi, hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.a_rows = a_rows;
  a.W = (const bf16_t*)W;
  a.C = C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.a_div = 1;
  a.tiles_m = (M + BM - 1) / BM;
  a.tiles_n = (epi == EPI_SILU) ? (N / 2) / (BN / 2) : (N + BN - 1) / BN;
  if (epi == EPI_ADD) {
    if (a_rows) return hipErrorInvalidValue;
    // decode-sized and mid-sized calls: the skinny schedule with the same in-place add
    if (K % SK_KC == 0 && N % 16 == 0 && gemm_prefers_skinny(M, N, K, epi, false)) return dispatch_skinny<K_ADD>(a, s);
    return (N % BN) ? hipErrorInvalidValue : dispatch<K_ADD>(a, false, s);
  }
  // decode-sized M, and mid-sized M where it is faster: the skinny schedule (same
  // per-element arithmetic, more waves)
  if (!a_rows && K % SK_KC == 0 && N % 16 == 0 && gemm_prefers_skinny(M, N, K, epi, false)) {
    switch (epi) {
      case EPI_BF16: return dispatch_skinny<K_BF16>(a, s);
      case EPI_F32: return dispatch_skinny<K_F32>(a, s);
      case EPI_SILU: return dispatch_skinny<K_SILU>(a, s);
    }
  }
  switch (epi) {
    case EPI_BF16: return dispatch<K_BF16>(a, a_rows != nullptr, s);
    case EPI_F32: return dispatch<K_F32>(a, a_rows != nullptr, s);
    case EPI_SILU: return dispatch<K_SILU>(a, a_rows != nullptr, s);
  }
  return hipErrorInvalidValue;
}

// ---- non-invariant split-K for small M: zero an fp32 buffer, let
// n_split workgroups per tile add their K-range partials with atomics (the
// order of the additions, hence the bits, depends on timing), then convert
// with the requested epilogue.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] = 0.0f;
}

__global__ __launch_bounds__(256) void splitk_epilogue_kernel(const float* __restrict__ acc, void* __restrict__ C,
                                                              int M, int N, int epi) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (epi == EPI_SILU) {
    const int I = N >> 1;
    if (i >= (size_t)M * I) return;
    const size_t r = i / I, c = i % I;
    const float g = bf2f(f2bf(acc[r * N + c])), u = bf2f(f2bf(acc[r * N + I + c]));
    reinterpret_cast<bf16_t*>(C)[i] = f2bf(silu_f32(g) * u);
  } else {
    if (i >= (size_t)M * N) return;
    if (epi == EPI_F32) reinterpret_cast<float*>(C)[i] = acc[i];
    else reinterpret_cast<bf16_t*>(C)[i] = f2bf(acc[i]);
  }
}

hipError_t launch_gemm_splitk(const void* A, const void* W, void* C, int M, int N, int K, int epi,
                              float* ws, hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.a_div = 1;
  a.W = (const bf16_t*)W;
  a.C = ws;
  a.M = M;
  a.N = N;
  a.K = K;
  a.tiles_m = (M + BM - 1) / BM;
  a.tiles_n = (N + BN - 1) / BN;
  // enough workgroups to keep every CU streaming weights: ~2 per CU
  int n_split = 1;
  while (n_split * 2 * a.tiles_m * a.tiles_n <= 512 && K % (n_split * 2 * BK) == 0) n_split *= 2;
  a.k_split = K / n_split;
  const size_t n = (size_t)M * N;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 4096)), dim3(256), 0, s, ws, n);
  const int grid = (a.tiles_m * a.tiles_n + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<K_ATOMIC, false, false>), dim3(grid, n_split), dim3(THREADS), 0, s, a);
  const size_t outs = (epi == EPI_SILU) ? (size_t)M * (N / 2) : n;
  hipLaunchKernelGGL(splitk_epilogue_kernel, dim3((unsigned)((outs + 255) / 256)), dim3(256), 0, s, ws, C, M, N, epi);
  return hipGetLastError();
}

// Deterministic split-K: fixed contraction slices of k_split (the last may be
// shorter), each an fp32 partial of the tiled GEMM's per-element chain, then summed in
// ascending slice order and rounded once.  Element (i, j) depends only on row i of A,
// row j of W and k_split, so rows stay independent of M.
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(const float* __restrict__ ws, int S, size_t n,
                                                            void* __restrict__ C, int epi) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float acc = ws[i];
    for (int sl = 1; sl < S; ++sl) acc = acc + ws[(size_t)sl * n + i];
    if (epi == EPI_F32) reinterpret_cast<float*>(C)[i] = acc;
    else reinterpret_cast<bf16_t*>(C)[i] = f2bf(acc);
  }
}

hipError_t launch_gemm_ksplit(const void* A, const void* W, void* C, int M, int N, int K, int k_split, int epi,
                              float* ws, hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.a_div = 1;
  a.W = (const bf16_t*)W;
  a.C = ws;
  a.M = M;
  a.N = N;
  a.K = K;
  a.tiles_m = (M + BM - 1) / BM;
  a.tiles_n = (N + BN - 1) / BN;
  a.k_split = k_split;
  const int S = (K + k_split - 1) / k_split;
  const int grid = (a.tiles_m * a.tiles_n + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<K_PART, false, false>), dim3(grid, S), dim3(THREADS), 0, s, a);
  const size_t n = (size_t)M * N;
  hipLaunchKernelGGL(ksplit_reduce_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 8192)), dim3(256), 0, s,
                     ws, S, n, C, epi);
  return hipGetLastError();
}

template <int KIND, bool GATHER>
static void launch_skinny_grouped(const GemmArgs& a, dim3 grid, int mt, hipStream_t s) {
  if (mt == 1) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 1, GATHER, true>), grid, dim3(64), 0, s, a);
  else if (mt == 2) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 2, GATHER, true>), grid, dim3(64), 0, s, a);
  else if (mt <= 4) hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 4, GATHER, true>), grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((gemm_skinny_kernel<KIND, 8, GATHER, true>), grid, dim3(64), 0, s, a);
}

hipError_t launch_gemm_grouped(const void* A, const int32_t* a_rows, int a_div, const void* W,
                               size_t w_group_stride, void* C, const int32_t* gtiles,
                               const int32_t* n_gtiles, int max_mtiles, int max_rows, int N, int K,
                               int epi, hipStream_t s) {
  if (max_mtiles == 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.a_rows = a_rows;
  a.a_div = a_div;
  a.W = (const bf16_t*)W;
  a.C = C;
  a.M = 0;
  a.N = N;
  a.K = K;
  a.tiles_m = max_mtiles;
  a.tiles_n = (epi == EPI_SILU) ? (N / 2) / (BN / 2) : (N + BN - 1) / BN;
  a.gtiles = gtiles;
  a.n_gtiles = n_gtiles;
  a.w_group_stride = w_group_stride;
  const bool g = a_rows != nullptr;
  if (max_rows <= SKINNY_MAX_M && K % SK_KC == 0 && (epi == EPI_SILU || epi == EPI_BF16)) {
    // no group has more than SKINNY_MAX_M rows (few tokens): one wave per 16 columns
    // per group, covering the group's rows in ceil(max_rows / 16) row blocks
    const dim3 grid((epi == EPI_SILU ? N / 2 : N) / 16, max_mtiles);
    const int mt = (max_rows + 15) / 16;
    if (epi == EPI_SILU) {
      if (g) launch_skinny_grouped<K_SILU, true>(a, grid, mt, s);
      else launch_skinny_grouped<K_SILU, false>(a, grid, mt, s);
    } else {
      if (g) launch_skinny_grouped<K_BF16, true>(a, grid, mt, s);
      else launch_skinny_grouped<K_BF16, false>(a, grid, mt, s);
    }
    return hipGetLastError();
  }
  const int grid = (a.tiles_m * a.tiles_n + 7) / 8 * 8;
  if (epi == EPI_SILU) {
    if (g) hipLaunchKernelGGL((gemm_kernel<K_SILU, true, true>), dim3(grid), dim3(THREADS), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<K_SILU, false, true>), dim3(grid), dim3(THREADS), 0, s, a);
  } else if (epi == EPI_BF16) {
    if (g) hipLaunchKernelGGL((gemm_kernel<K_BF16, true, true>), dim3(grid), dim3(THREADS), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<K_BF16, false, true>), dim3(grid), dim3(THREADS), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_qkv_rope(const void* A, const void* W, int M, int N, int K, void* q_out,
                                const int32_t* tok_pos, const int32_t* tok_slot, const float* rope_cos,
                                const float* rope_sin, KvLayer kv, int nq, int nkv, bool fp8,
                                hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (N % BN != 0 || N != (nq + 2 * nkv) * 128 || K % BK != 0) return hipErrorInvalidValue;
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.a_div = 1;
  a.W = (const bf16_t*)W;
  a.M = M;
  a.N = N;
  a.K = K;
  a.tiles_m = (M + BM - 1) / BM;
  a.tiles_n = N / BN;
  a.q_out = (bf16_t*)q_out;
  a.tok_pos = tok_pos;
  a.tok_slot = tok_slot;
  a.rcos = rope_cos;
  a.rsin = rope_sin;
  a.kv = kv;
  a.nq = nq;
  a.nkv = nkv;
  a.fp8 = fp8 ? 1 : 0;
  if (M <= SKINNY_MAX_M || (!fp8 && gemm_prefers_skinny(M, N, K, EPI_BF16, true))) {
    // decode-sized calls (and mid-sized ones where it is faster), bf16 cache (an FP8
    // scale needs a head's 128 values, spread over 4 waves here): the skinny schedule,
    // one wave per 16 rotation pairs
    if (fp8 || K % SK_KC) return hipErrorInvalidValue;
    const int mt = std::min((M + 15) / 16, SK_ROW_BLOCKS);
    const dim3 grid(N / 32), gm(N / 32, (M + 16 * mt - 1) / (16 * mt));
    if (M <= 4 && K % 512 == 0)
      hipLaunchKernelGGL((gemm_skinny_kernel<K_ROPE, 1, false, false, 4, 512>), grid, dim3(64), 0, s, a);
    else if (mt == 1) hipLaunchKernelGGL((gemm_skinny_kernel<K_ROPE, 1>), gm, dim3(64), 0, s, a);
    else if (mt == 2) hipLaunchKernelGGL((gemm_skinny_kernel<K_ROPE, 2>), gm, dim3(64), 0, s, a);
    else if (mt <= 4) hipLaunchKernelGGL((gemm_skinny_kernel<K_ROPE, 4>), gm, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((gemm_skinny_kernel<K_ROPE, 8>), gm, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  const int grid = (a.tiles_m * a.tiles_n + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_kernel<K_ROPE, false, false>), dim3(grid), dim3(THREADS), 0, s, a);
  return hipGetLastError();
}

// Calls of at most 4 rows whose A is RMSNorm(res) * gamma (the norm before the QKV and
// gate_up projections): the skinny schedule normalises the rows itself, with the
// add+RMSNorm kernel's arithmetic, so the bits equal that kernel followed by the GEMM.
static bool norm_shape_ok(int M, int N, int K) {
  return M >= 1 && M <= 4 && K % 512 == 0 && K <= SK_NORM_MAX_K && N % 16 == 0;
}

hipError_t launch_gemm_norm(const void* res, const void* gamma, float eps, const void* W, void* C, int M, int N,
                            int K, int epi, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!norm_shape_ok(M, N, K) || (epi != EPI_BF16 && epi != EPI_SILU)) return hipErrorInvalidValue;
  GemmArgs a{};
  a.W = (const bf16_t*)W;
  a.C = C;
  a.M = M;
  a.N = N;
  a.K = K;
  a.a_div = 1;
  a.res = (const bf16_t*)res;
  a.gamma = (const bf16_t*)gamma;
  a.eps = eps;
  if (epi == EPI_SILU) {
    if ((N / 2) % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_skinny_kernel<K_SILU, 1, false, false, 4, 512, true>), dim3(N / 32), dim3(64), 0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<K_BF16, 1, false, false, 4, 512, true>), dim3(N / 16), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_qkv_rope_norm(const void* res, const void* gamma, float eps, const void* W, int M, int N,
                                     int K, void* q_out, const int32_t* tok_pos, const int32_t* tok_slot,
                                     const float* rope_cos, const float* rope_sin, KvLayer kv, int nq, int nkv,
                                     hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!norm_shape_ok(M, N, K) || N % BN != 0 || N != (nq + 2 * nkv) * 128) return hipErrorInvalidValue;
  GemmArgs a{};
  a.W = (const bf16_t*)W;
  a.M = M;
  a.N = N;
  a.K = K;
  a.a_div = 1;
  a.q_out = (bf16_t*)q_out;
  a.tok_pos = tok_pos;
  a.tok_slot = tok_slot;
  a.rcos = rope_cos;
  a.rsin = rope_sin;
  a.kv = kv;
  a.nq = nq;
  a.nkv = nkv;
  a.fp8 = 0;
  a.res = (const bf16_t*)res;
  a.gamma = (const bf16_t*)gamma;
  a.eps = eps;
  // 8 rotation pairs per wave: N / 16 waves (one per CU for the Qwen3 shape) instead of N / 32
  // (same box: B = 1 decode step 1.655 -> 1.628 ms).  The SiLU form, already at 384 waves, keeps
  // 16 columns: with 768 its ring and normalised rows (80 KiB) fit two waves per CU and the
  // step got slower; with a 2-stage ring (48 KiB, three per CU) it measured even.
  hipLaunchKernelGGL((gemm_skinny_kernel<K_ROPE, 1, false, false, 4, 512, true, 8>), dim3(N / 16), dim3(64), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_lmhead_partials(const void* A, const int32_t* a_rows, const void* E,
                                  const int32_t* ids, int M, int V, int K, float* part_m,
                                  float* part_s, float* zid, hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.a_rows = a_rows;
  a.a_div = 1;
  a.W = (const bf16_t*)E;
  a.M = M;
  a.N = V;
  a.K = K;
  a.tiles_n = (V + BN - 1) / BN;
  a.ids = ids;
  a.part_m = part_m;
  a.part_s = part_s;
  a.zid = zid;
  if (M <= LM_MID_M) {
    // few scored rows (decode, small batches): 16- or 64-row tiles with 2 waves, so the
    // weight stream is not accompanied by up to 255 duplicated A rows per tile
    const int tbm = M <= LM_SMALL_M ? LM_SMALL_M : LM_MID_M / 2;
    a.tiles_m = (M + tbm - 1) / tbm;
    const int grid = (a.tiles_m * a.tiles_n + 7) / 8 * 8;
    if (tbm == LM_SMALL_M) {
      if (a_rows)
        hipLaunchKernelGGL((gemm_kernel<K_LMHEAD, true, false, LM_SMALL_M>), dim3(grid), dim3(NWN * 64), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_kernel<K_LMHEAD, false, false, LM_SMALL_M>), dim3(grid), dim3(NWN * 64), 0, s, a);
    } else {
      if (a_rows)
        hipLaunchKernelGGL((gemm_kernel<K_LMHEAD, true, false, LM_MID_M / 2>), dim3(grid), dim3(NWN * 64), 0, s, a);
      else
        hipLaunchKernelGGL((gemm_kernel<K_LMHEAD, false, false, LM_MID_M / 2>), dim3(grid), dim3(NWN * 64), 0, s, a);
    }
    return hipGetLastError();
  }
  a.tiles_m = (M + BM - 1) / BM;
  return dispatch<K_LMHEAD>(a, a_rows != nullptr, s);
}

// Fixed merge order of the per-chunk (max, sum exp) pairs of one row: the
// chunks are split into 8 contiguous ranges; thread (row, q) merges range q in
// ascending chunk order; then range results 0..7 are merged in that order.
// The order depends only on the chunk count, never on the row count.  Lanes
// run over consecutive rows, so every load of the chunk-major partials is
// coalesced.  lp = (z[id] - max) - log(sum).
constexpr int COMB_ROWS = 64, COMB_SPLIT = 8;
constexpr int COMB_BATCH = 40;   // partials loaded together per thread (two batches per range at V = 151936)

// The rescale factors are 2^((m - m') log2 e) on v_exp_f32, the exponential of the
// chunks' own sums: the merge is one dependent chain per range, and the library expf's
// range reduction made it several times longer.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * fexp2((m - m2) * LOG2E) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s = s + s2 * fexp2((m2 - m) * LOG2E);
  }
}

__global__ __launch_bounds__(COMB_ROWS * COMB_SPLIT) void lmhead_combine_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const float* __restrict__ zid,
    const int32_t* __restrict__ ids, int M, int V, int nc, float* __restrict__ lp) {
  __shared__ float sm[COMB_SPLIT][COMB_ROWS], ss[COMB_SPLIT][COMB_ROWS];
  const int r = threadIdx.x, q = threadIdx.y;
  const int i = blockIdx.x * COMB_ROWS + r;
  const int per = (nc + COMB_SPLIT - 1) / COMB_SPLIT;
  float mx = -INFINITY, s = 0.0f;
  // the token id and its logit are loaded first, so their latency overlaps the merge
  const int ir = min(i, M - 1);
  const int id = ids[ir];
  const float z = zid[ir];
  if (i < M) {
    // the partials of COMB_BATCH chunks are loaded together (at clamped indices, so the
    // loads issue back to back and are waited for once), then merged in chunk order
    const int c0 = q * per, c1 = min(nc, (q + 1) * per);
    for (int c = c0; c < c1; c += COMB_BATCH) {
      float bm[COMB_BATCH], bs[COMB_BATCH];
#pragma unroll
      for (int u = 0; u < COMB_BATCH; ++u) {
        const size_t k = (size_t)min(c + u, c1 - 1) * M + i;
        bm[u] = pm[k];
        bs[u] = ps[k];
      }
#pragma unroll
      for (int u = 0; u < COMB_BATCH; ++u)
        if (c + u < c1) lse_merge(mx, s, bm[u], bs[u]);
    }
  }
  sm[q][r] = mx;
  ss[q][r] = s;
  __syncthreads();
  if (q == 0 && i < M) {
    for (int k = 1; k < COMB_SPLIT; ++k) lse_merge(mx, s, sm[k][r], ss[k][r]);
    lp[i] = (id < 0 || id >= V) ? __uint_as_float(0x7fc00000u) : (z - mx) - flog(s);
  }
}

hipError_t launch_lmhead_combine(const float* part_m, const float* part_s, const float* zid,
                                 const int32_t* ids, int M, int V, float* lp, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int nc = (V + BN - 1) / BN;
  hipLaunchKernelGGL(lmhead_combine_kernel, dim3((M + COMB_ROWS - 1) / COMB_ROWS),
                     dim3(COMB_ROWS, COMB_SPLIT), 0, s, part_m, part_s, zid, ids, M, V, nc, lp);
  return hipGetLastError();
}

}  // namespace bci
