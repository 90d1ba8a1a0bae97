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
// in ascending order; nothing else is ever added to it.  The tile shape
// (256 x 128 x 64, 4 waves) is the same for every M, there is no split-K, and
// an MFMA output element depends only on its own A row and W row, so the
// bits of row i are the same whatever M is and wherever row i sits in a tile.
//
// Data path.  Global -> registers (16-byte loads, prefetching the next
// K-slab) -> LDS (XOR-swizzled 16-byte chunks, conflict-free for the MFMA
// operand reads) -> MFMA.  Each wave owns a 128 x 64 sub-tile, i.e. 8 x 4
// MFMA blocks (128 fp32 accumulators per lane).  Workgroups are remapped so
// each XCD (8 per chip, each with its own L2) gets a contiguous range of
// tiles, grouped 8 M-tiles at a time so that they share W tiles in L2.
#include "common.h"
#include "kernels.h"

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int KCH = BK / 8;  // 16-byte chunks per LDS row
constexpr int THREADS = 256;

enum { K_BF16 = 0, K_F32 = 1, K_SILU = 2, K_LMHEAD = 3 };

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
};

// Row r of an LDS tile holds 8 chunks of 16 bytes; chunk c is stored at
// position c ^ ((r >> 1) & 7).  Rows alternate between the two 32-bank halves
// of the 64 banks and the XOR spreads 8 consecutive row pairs over all chunk
// positions, so 16 lanes reading 16 consecutive rows at one chunk hit 16
// distinct 4-bank groups.
__device__ __forceinline__ int swz(int row, int ch) { return row * KCH + (ch ^ ((row >> 1) & 7)); }

template <int KIND>
__device__ __forceinline__ int b_lds_row(int wn, int ni) {
  if constexpr (KIND == K_SILU) {
    // sub-tiles 0,1: gate columns; 2,3: the matching up columns
    return (ni < 2) ? wn * 32 + ni * 16 : 64 + wn * 32 + (ni - 2) * 16;
  } else {
    return wn * 64 + ni * 16;
  }
}

template <int KIND, bool GATHER, bool GROUPED>
__global__ __launch_bounds__(THREADS, 2) void gemm_kernel(GemmArgs p) {
  __shared__ u32x4_t smem[(BM + BN) * KCH];  // 48 KiB
  u32x4_t* As = smem;
  u32x4_t* Bs = smem + BM * KCH;

  // ---- tile id: XCD-contiguous ranges, then groups of 8 M-tiles
  const int n_tiles = p.tiles_m * p.tiles_n;
  const int per_xcd = gridDim.x >> 3;  // grid is a multiple of 8
  const int tile = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (tile >= n_tiles) return;
  constexpr int GM = 8;
  const int width = GM * p.tiles_n;
  const int first_m = (tile / width) * GM;
  const int gsz = min(p.tiles_m - first_m, GM);
  const int tm = first_m + (tile % width) % gsz;
  const int tn = (tile % width) / gsz;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = p.K;

  // rows [row_base, row_base + row_cnt) of C belong to this tile
  int row_base = tm * BM, row_cnt = min(BM, p.M - tm * BM);
  const bf16_t* W = p.W;
  if constexpr (GROUPED) {
    if (tm >= *p.n_gtiles) return;
    const int grp = p.gtiles[3 * tm];
    row_base = p.gtiles[3 * tm + 1];
    row_cnt = p.gtiles[3 * tm + 2];
    W += (size_t)grp * p.w_group_stride;
  }

  // ---- global load assignment: thread -> (row, 16-byte chunk)
  const int ld_ch = tid & 7, ld_row = tid >> 3;  // rows ld_row + 32 i
  const bf16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // rows past the tile's end duplicate its last row and are never stored
    int r = row_base + min(ld_row + 32 * i, row_cnt - 1);
    if constexpr (GATHER) r = p.a_rows[r] / p.a_div;
    a_src[i] = p.A + (size_t)r * K + ld_ch * 8;
  }
  const bf16_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ld_row + 32 * i;
    int n;
    if constexpr (KIND == K_SILU) {
      const int I = p.N >> 1;
      n = (r < 64) ? tn * 64 + r : I + tn * 64 + (r - 64);
    } else {
      n = min(tn * BN + r, p.N - 1);  // columns past N are masked in the epilogue
    }
    b_src[i] = W + (size_t)n * K + ld_ch * 8;
  }

  f32x4_t acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[8], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(b_src[i] + k0);
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) As[swz(ld_row + 32 * i, ld_ch)] = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) Bs[swz(ld_row + 32 * i, ld_ch)] = rb[i];
  };

  const int nk = K / BK;
  gload(0);
  sstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      bf16x8_t fa[8], fb[4];
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
        fa[mi] = __builtin_bit_cast(bf16x8_t, As[swz(wm * 128 + mi * 16 + (lane & 15), ch)]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        fb[ni] = __builtin_bit_cast(bf16x8_t, Bs[swz(b_lds_row<KIND>(wn, ni) + (lane & 15), ch)]);
#pragma unroll
      for (int mi = 0; mi < 8; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      sstore();
      __syncthreads();
    }
  }

  // ---- epilogues.  Lane holds C[4*(lane>>4) + r][lane & 15] of each 16x16 block.
  const int lrow0 = wm * 128 + 4 * (lane >> 4);  // row within the tile
  const int row0 = row_base + lrow0;
  if constexpr (KIND == K_BF16 || KIND == K_F32) {
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + mi * 16 + r;
        if (lrow0 + mi * 16 + r < row_cnt) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const int col = tn * BN + wn * 64 + ni * 16 + (lane & 15);
            if (col >= p.N) continue;
            if constexpr (KIND == K_BF16)
              reinterpret_cast<bf16_t*>(p.C)[(size_t)row * p.N + col] = f2bf(acc[mi][ni][r]);
            else
              reinterpret_cast<float*>(p.C)[(size_t)row * p.N + col] = acc[mi][ni][r];
          }
        }
      }
  } else if constexpr (KIND == K_SILU) {
    const int I = p.N >> 1;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + mi * 16 + r;
        if (lrow0 + mi * 16 + r < row_cnt) {
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const int col = tn * 64 + wn * 32 + ni * 16 + (lane & 15);
            const float g = bf2f(f2bf(acc[mi][ni][r]));
            const float u = bf2f(f2bf(acc[mi][ni + 2][r]));
            reinterpret_cast<bf16_t*>(p.C)[(size_t)row * I + col] = f2bf(silu_f32(g) * u);
          }
        }
      }
  } else {  // K_LMHEAD: per row, (max, sum exp) over this 128-column vocab chunk
    const int V = p.N;
    float* red = reinterpret_cast<float*>(smem);  // [2][BM]
    float mc[8][4];
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int col = tn * BN + wn * 64 + ni * 16 + (lane & 15);
          mx = fmaxf(mx, col < V ? acc[mi][ni][r] : -INFINITY);
        }
#pragma unroll
        for (int o = 1; o <= 8; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
        if ((lane & 15) == 0) red[wn * BM + wm * 128 + mi * 16 + 4 * (lane >> 4) + r] = mx;
      }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = wm * 128 + mi * 16 + 4 * (lane >> 4) + r;
        mc[mi][r] = fmaxf(red[lr], red[BM + lr]);
      }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = 0.0f;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int col = tn * BN + wn * 64 + ni * 16 + (lane & 15);
          const float e = col < V ? fexp(acc[mi][ni][r] - mc[mi][r]) : 0.0f;
          s = s + e;
        }
#pragma unroll
        for (int o = 1; o <= 8; o <<= 1) s = s + __shfl_xor(s, o, WAVE);
        if ((lane & 15) == 0) red[wn * BM + wm * 128 + mi * 16 + 4 * (lane >> 4) + r] = s;
      }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = wm * 128 + mi * 16 + 4 * (lane >> 4) + r;
        const int row = row_base + lr;
        if (lr < row_cnt) {
          if (wn == 0 && (lane & 15) == 0) {
            p.part_m[(size_t)tn * p.M + row] = mc[mi][r];
            p.part_s[(size_t)tn * p.M + row] = red[lr] + red[BM + lr];
          }
          const int id = p.ids[row];
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const int col = tn * BN + wn * 64 + ni * 16 + (lane & 15);
            if (col == id) p.zid[row] = acc[mi][ni][r];
          }
        }
      }
  }
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
  a.tiles_n = (epi == EPI_SILU) ? (N / 2) / 64 : (N + BN - 1) / BN;
  switch (epi) {
    case EPI_BF16: return dispatch<K_BF16>(a, a_rows != nullptr, s);
    case EPI_F32: return dispatch<K_F32>(a, a_rows != nullptr, s);
    case EPI_SILU: return dispatch<K_SILU>(a, a_rows != nullptr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_grouped(const void* A, const int32_t* a_rows, int a_div, const void* W,
                               size_t w_group_stride, void* C, const int32_t* gtiles,
                               const int32_t* n_gtiles, int max_mtiles, int N, int K, int epi,
                               hipStream_t s) {
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
  a.tiles_n = (epi == EPI_SILU) ? (N / 2) / 64 : (N + BN - 1) / BN;
  a.gtiles = gtiles;
  a.n_gtiles = n_gtiles;
  a.w_group_stride = w_group_stride;
  const int grid = (a.tiles_m * a.tiles_n + 7) / 8 * 8;
  const bool g = a_rows != nullptr;
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
  a.tiles_m = (M + BM - 1) / BM;
  a.tiles_n = (V + BN - 1) / BN;
  a.ids = ids;
  a.part_m = part_m;
  a.part_s = part_s;
  a.zid = zid;
  return dispatch<K_LMHEAD>(a, a_rows != nullptr, s);
}

// Fixed merge order of the per-chunk (max, sum exp) pairs of one row: the
// chunks are split into 8 contiguous ranges; thread (row, q) merges range q in
// ascending chunk order; then range results 0..7 are merged in that order.
// The order depends only on the chunk count, never on the row count.  Lanes
// run over consecutive rows, so every load of the chunk-major partials is
// coalesced.  lp = (z[id] - max) - log(sum).
constexpr int COMB_ROWS = 64, COMB_SPLIT = 8;

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * fexp(m - m2) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s = s + s2 * fexp(m2 - m);
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
  if (i < M) {
    const int c1 = min(nc, (q + 1) * per);
    for (int c = q * per; c < c1; ++c)
      lse_merge(mx, s, pm[(size_t)c * M + i], ps[(size_t)c * M + i]);
  }
  sm[q][r] = mx;
  ss[q][r] = s;
  __syncthreads();
  if (q == 0 && i < M) {
    for (int k = 1; k < COMB_SPLIT; ++k) lse_merge(mx, s, sm[k][r], ss[k][r]);
    const int id = ids[i];
    lp[i] = (id < 0 || id >= V) ? __uint_as_float(0x7fc00000u) : (zid[i] - mx) - flog(s);
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
