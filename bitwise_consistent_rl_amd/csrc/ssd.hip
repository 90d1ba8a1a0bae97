// Mamba-2-style selective state-space layer whose decode replays prefill's chunked
// arithmetic.
//
// Porting the method to Nemotron-3.5 meant recursive arithmetic in which decode
// replays the chunked computation order of prefill and training reuses the same
// operator (page "Finish RL Training Faster" digest, section
// "一致性有多个层面，修好一处还不能验收").  Here the recurrence
//     h_t = exp(A dt_t) h_{t-1} + dt_t B_t (outer) x_t,   y_t = C_t . h_t + D x_t
// is evaluated in chunks of 64 positions at fixed absolute positions (chunk c =
// positions 64c .. 64c+63).  The state is materialised only at chunk ends; inside a
// chunk every output comes from the chunk-start state and the chunk's inputs up to
// that position, by one routine, whether the position arrives in a prefill, a
// chunked prefill or a decode step.  Per head, with a_j = (A log2 e) dt_j and
// L_t the inclusive prefix of a over the chunk (one fixed shuffle scan):
//   y_t  = bf( (2^{L_t} (C_t . H) + sum_{j <= t} (C_t . B_j) 2^{L_t - L_j} dt_j x_j)
//              + D x_t )                         (H: state before the chunk)
//   H'   = 2^{L_63} H + S,  S = sum_j x_j (outer) bf(B_j 2^{L_63 - L_j} dt_j)
// with the dot products on v_mfma_f32_16x16x32_bf16 (ascending 32-wide steps),
// H rounded to bf16 for its product with C and the intra-chunk weights rounded to
// bf16 for their product with x (as P in attention).  Every MFMA output element
// depends only on its own row and column, so a decode step -- a tile holding the
// one new position -- gives the prefill's bits.
//
// Per call: state_walk (per sequence and head, the chunks that complete in the call
// in order: each chunk's state S on MFMA, the running state updated in registers, and
// each chunk's state-before handed to chunk_out in bf16, exactly the rounding chunk_out
// applies to the slot's fp32 state), chunk_out (every position of the call), and
// chunk_append (the positions of an unfinished last chunk into the slot's chunk
// buffer, which the next call reads back).
#include "common.h"
#include "kernels.h"

namespace bci {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int SQ = 64;            // chunk length
constexpr int SP = 64;            // head dimension
constexpr int XT_STRIDE = SQ + 8;  // bf16 per row of the transposed x tile

// inclusive prefix sum over the 64 lanes (lane j holds a_j): a fixed network, so
// the value at lane t depends only on a_0 .. a_t and always on the same tree
__device__ __forceinline__ float chunk_scan(float v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(v, o, WAVE);
    if (lane >= o) v = v + y;
  }
  return v;
}

// where position p of sequence s lives: the call's arrays (p >= pos0) or the
// slot's chunk buffer (an earlier position of the same chunk)
struct PosSrc {
  bool call;
  size_t row;  // token row of the call, or chunk-buffer row (slot * SQ + p % SQ)
};
__device__ __forceinline__ PosSrc pos_src(const SsdArgs& a, int s, int p) {
  const int* sq = a.seqs + 6 * s;
  const int cu = sq[0], pos0 = sq[1], slot = sq[3];
  if (p >= pos0) return PosSrc{true, (size_t)(cu + p - pos0)};
  return PosSrc{false, (size_t)slot * SQ + (p & (SQ - 1))};
}
__device__ __forceinline__ const bf16_t* x_row(const SsdArgs& a, PosSrc r, int h) {
  return (r.call ? a.x : a.xb) + (r.row * a.heads + h) * SP;
}
__device__ __forceinline__ const bf16_t* b_row(const SsdArgs& a, PosSrc r, int g) {
  return (r.call ? a.B : a.Bb) + (r.row * a.groups + g) * a.N;
}
__device__ __forceinline__ float dt_of(const SsdArgs& a, PosSrc r, int h) {
  return (r.call ? a.dt : a.dtb)[r.row * a.heads + h];
}

template <int N>
__device__ __forceinline__ int bswz(int row, int ch) {  // 16-byte chunks of an N-wide bf16 row
  return row * (N / 8) + (ch ^ (row & (N / 8 - 1)));
}

// ------------------------------------------------------------- state walk
// One workgroup (4 waves) per (sequence, head) walks the call's completed chunks in
// order, the state H held in registers in the MFMA accumulator layout (wave w, lane l:
// H[16w + 4(l/16) + r][16 nt + l%16]).  For each chunk: S = sum_j x_j (outer) bw_j on
// MFMA (x^T and the weighted B^T staged in LDS), hprev = bf(H) (the state before the
// chunk, for chunk_out), then H = 2^{L_63} H + S in fp32; no chunk state crosses HBM.
// The next chunk's dt, x and B rows are loaded into registers while the current chunk
// multiplies.  The final H goes back to the slot.
template <int N>
__global__ __launch_bounds__(256) void ssd_state_walk_kernel(SsdArgs a) {
  // staging units: two consecutive positions x 8 columns (lanes along the position
  // pairs, so the transposed 4-byte writes fall on consecutive banks)
  constexpr int NX = (SQ / 2) * (SP / 8) / 256;  // x units per thread per chunk
  constexpr int NB = (SQ / 2) * (N / 8) / 256;   // B units per thread per chunk
  __shared__ __attribute__((aligned(16))) bf16_t Xt[SP * XT_STRIDE];   // x^T [p][j]
  __shared__ __attribute__((aligned(16))) bf16_t Bt[N * XT_STRIDE];    // bw^T [n][j]
  __shared__ float wj[SQ];
  __shared__ float ek_s;
  const int s = blockIdx.x, h = blockIdx.y;
  const int* sq = a.seqs + 6 * s;
  const int slot = sq[3], k0 = sq[4], nd = sq[5];
  if (nd == 0) return;  // the whole workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int g = h / (a.heads / a.groups);
  const float A2 = a.A[h] * LOG2E;
  const size_t per = (size_t)SP * N;
  float* st = a.state + ((size_t)slot * a.heads + h) * per;
  const int c_first = a.inst[6 * a.done[k0] + 1];
  f32x4_t H[N / 16];
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      H[nt][r] = c_first == 0 ? 0.0f : st[(size_t)(16 * wave + 4 * lg + r) * N + 16 * nt + lc];

  // a chunk's inputs in registers: dt of position `lane` (wave 0), x and B pieces
  float rdt = 0.0f;
  u32x4_t rx[NX][2], rb[NB][2];
  auto load = [&](int c) {
    if (wave == 0) rdt = dt_of(a, pos_src(a, s, c * SQ + lane), h);
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int u = i * 256 + tid, j = 2 * (u % (SQ / 2)), pc = u / (SQ / 2);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        rx[i][q] = *reinterpret_cast<const u32x4_t*>(x_row(a, pos_src(a, s, c * SQ + j + q), h) + 8 * pc);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int u = i * 256 + tid, j = 2 * (u % (SQ / 2)), pc = u / (SQ / 2);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        rb[i][q] = *reinterpret_cast<const u32x4_t*>(b_row(a, pos_src(a, s, c * SQ + j + q), g) + 8 * pc);
    }
  };
  load(c_first);

  for (int k = k0; k < k0 + nd; ++k) {
    if (k > k0) __syncthreads();  // the previous chunk's LDS reads are done
    if (wave == 0) {
      const float L = chunk_scan(A2 * rdt, lane);
      const float Lend = __shfl(L, SQ - 1, WAVE);
      wj[lane] = fexp2(Lend - L) * rdt;
      if (lane == 0) ek_s = fexp2(Lend);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int u = i * 256 + tid, j = 2 * (u % (SQ / 2)), pc = u / (SQ / 2);
      const bf16_t* ea = reinterpret_cast<const bf16_t*>(&rx[i][0]);
      const bf16_t* eb = reinterpret_cast<const bf16_t*>(&rx[i][1]);
#pragma unroll
      for (int q = 0; q < 8; ++q) *reinterpret_cast<uint32_t*>(Xt + (8 * pc + q) * XT_STRIDE + j) = pack_bf2(ea[q], eb[q]);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int u = i * 256 + tid, j = 2 * (u % (SQ / 2)), pc = u / (SQ / 2);
      const bf16_t* ea = reinterpret_cast<const bf16_t*>(&rb[i][0]);
      const bf16_t* eb = reinterpret_cast<const bf16_t*>(&rb[i][1]);
      const float wa = wj[j], wb = wj[j + 1];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        *reinterpret_cast<uint32_t*>(Bt + (8 * pc + q) * XT_STRIDE + j) =
            pack_bf2(f2bf(bf2f(ea[q]) * wa), f2bf(bf2f(eb[q]) * wb));
    }
    __syncthreads();
    if (k + 1 < k0 + nd) load(a.inst[6 * a.done[k + 1] + 1]);  // in flight during the products
    const float ek = ek_s;
    bf16_t* hp = a.hprev + ((size_t)k * a.heads + h) * per;
    const bf16_t* xr = Xt + (16 * wave + lc) * XT_STRIDE;
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt) {
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const bf16_t* br = Bt + (16 * nt + lc) * XT_STRIDE;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8_t af = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xr + 32 * k2 + 8 * lg));
        const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(br + 32 * k2 + 8 * lg));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hp[(size_t)(16 * wave + 4 * lg + r) * N + 16 * nt + lc] = f2bf(H[nt][r]);
        H[nt][r] = ek * H[nt][r] + acc[r];
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) st[(size_t)(16 * wave + 4 * lg + r) * N + 16 * nt + lc] = H[nt][r];
}

// ------------------------------------------------------------- chunk outputs
// One workgroup (4 waves, 16 positions each) per (chunk of the call, head).
// Transposed products as in attention: S^T = B . C^T puts the intra weights in the
// layout of the B operand of Y^T = X^T . M^T, so they never leave registers.
template <int N>
__global__ __launch_bounds__(256) void ssd_chunk_out_kernel(SsdArgs a) {
  __shared__ __attribute__((aligned(16))) u32x4_t Bc[SQ * N / 8];   // B rows [j][n], swizzled
  __shared__ __attribute__((aligned(16))) u32x4_t Hb[SP * N / 8];   // bf(H) [p][n], swizzled
  __shared__ __attribute__((aligned(16))) bf16_t Xt[SP * XT_STRIDE];  // x^T [p][j]
  __shared__ float Ls[SQ], dts[SQ];
  const int ii = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int* in = a.inst + 6 * ii;
  const int s = in[0], c = in[1], r0 = in[2], r1 = in[3], k = in[4];
  const int g = h / (a.heads / a.groups);
  const int slot = a.seqs[6 * s + 3];
  const float A2 = a.A[h] * LOG2E;
  const int navail = r1 - c * SQ + 1;  // positions 0 .. navail-1 of the chunk exist

  if (wave == 0) {
    float dtj = 0.0f;
    if (lane < navail) dtj = dt_of(a, pos_src(a, s, c * SQ + lane), h);
    const float L = chunk_scan(A2 * dtj, lane);
    Ls[lane] = L;
    dts[lane] = dtj;
  }
  // B rows and x^T of the available positions (zeros past them)
  for (int u = tid; u < SQ * (N / 8); u += 256) {
    const int j = u / (N / 8), pc = u % (N / 8);
    u32x4_t v = u32x4_t{0, 0, 0, 0};
    if (j < navail) v = *reinterpret_cast<const u32x4_t*>(b_row(a, pos_src(a, s, c * SQ + j), g) + 8 * pc);
    Bc[bswz<N>(j, pc)] = v;
  }
  // x^T: a unit is two consecutive positions x 8 columns, written as 4-byte pairs by
  // lanes along the position pairs (consecutive banks)
  for (int u = tid; u < (SQ / 2) * (SP / 8); u += 256) {
    const int jp = u % (SQ / 2), pc = u / (SQ / 2), j = 2 * jp;
    u32x4_t va = u32x4_t{0, 0, 0, 0}, vb = va;
    if (j < navail) va = *reinterpret_cast<const u32x4_t*>(x_row(a, pos_src(a, s, c * SQ + j), h) + 8 * pc);
    if (j + 1 < navail) vb = *reinterpret_cast<const u32x4_t*>(x_row(a, pos_src(a, s, c * SQ + j + 1), h) + 8 * pc);
    const bf16_t* ea = reinterpret_cast<const bf16_t*>(&va);
    const bf16_t* eb = reinterpret_cast<const bf16_t*>(&vb);
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(Xt + (8 * pc + i) * XT_STRIDE + j) = pack_bf2(ea[i], eb[i]);
  }
  // the state before the chunk, rounded to bf16: zero for chunk 0, the state pass's
  // bf16 copy for a chunk completed in this call, the slot's state otherwise
  {
    const float* src = nullptr;
    const bf16_t* srcb = nullptr;
    if (c > 0) {
      if (k >= 0)
        srcb = a.hprev + (((size_t)k * a.heads + h) * SP) * N;
      else
        src = a.state + (((size_t)slot * a.heads + h) * SP) * N;
    }
    for (int u = tid; u < SP * (N / 8); u += 256) {
      const int p = u / (N / 8), pc = u % (N / 8);
      u32x4_t v = u32x4_t{0, 0, 0, 0};
      if (srcb) {
        v = *reinterpret_cast<const u32x4_t*>(srcb + (size_t)p * N + 8 * pc);
      } else if (src) {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src + (size_t)p * N + 8 * pc);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(src + (size_t)p * N + 8 * pc + 4);
        v = u32x4_t{pack_f2bf2(lo[0], lo[1]), pack_f2bf2(lo[2], lo[3]), pack_f2bf2(hi[0], hi[1]),
                    pack_f2bf2(hi[2], hi[3])};
      }
      Hb[bswz<N>(p, pc)] = v;
    }
  }
  __syncthreads();

  // this lane's output position (MFMA column): t = 16 wave + lc of the chunk
  const int tq = 16 * wave + lc;
  const int p_out = c * SQ + tq;
  const bool row_ok = p_out >= r0 && p_out <= r1;
  // a wave none of whose positions is an output of this call has nothing to do
  if (c * SQ + 16 * wave + 15 < r0 || c * SQ + 16 * wave > r1) return;

  bf16x8_t cf[N / 32];
  {
    const int* sq = a.seqs + 6 * s;
    const bf16_t* crow = a.C + ((size_t)(sq[0] + (row_ok ? p_out - sq[1] : 0)) * a.groups + g) * N;
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) {
      u32x4_t v = u32x4_t{0, 0, 0, 0};
      if (row_ok) v = *reinterpret_cast<const u32x4_t*>(crow + 32 * ks + 8 * lg);
      cf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  const float Lt = Ls[tq];

  // inter: Y^T[p][t] = sum_n bf(H)[p][n] C[t][n]
  f32x4_t yi[SP / 16];
#pragma unroll
  for (int dt = 0; dt < SP / 16; ++dt) {
    yi[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      yi[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, Hb[bswz<N>(16 * dt + lc, 4 * ks + lg)]), cf[ks], yi[dt], 0, 0, 0);
  }
  // intra: S^T[j][t] = B_j . C_t, weights m = S 2^{L_t - L_j} dt_j for j <= t
  float m[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, Bc[bswz<N>(16 * kt + lc, 4 * ks + lg)]), cf[ks], sacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * kt + 4 * lg + r;
      m[kt][r] = j <= tq ? (sacc[r] * fexp2(Lt - Ls[j])) * dts[j] : 0.0f;
    }
  }
  f32x4_t ya[SP / 16];
#pragma unroll
  for (int dt = 0; dt < SP / 16; ++dt) ya[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    u32x4_t pw;
    pw[0] = pack_f2bf2(m[2 * k2][0], m[2 * k2][1]);
    pw[1] = pack_f2bf2(m[2 * k2][2], m[2 * k2][3]);
    pw[2] = pack_f2bf2(m[2 * k2 + 1][0], m[2 * k2 + 1][1]);
    pw[3] = pack_f2bf2(m[2 * k2 + 1][2], m[2 * k2 + 1][3]);
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
    const int ko = k2 * 32 + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < SP / 16; ++dt) {
      const bf16_t* xr = Xt + (dt * 16 + lc) * XT_STRIDE;
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(xr + ko);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(xr + ko + 16);
      const u32x4_t xw = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      ya[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xw), pf, ya[dt], 0, 0, 0);
    }
  }
  if (!row_ok) return;
  const float et = fexp2(Lt);
  const float Dh = a.D[h];
  const int* sq = a.seqs + 6 * s;
  const size_t trow = (size_t)(sq[0] + p_out - sq[1]);
  const bf16_t* xo = a.x + (trow * a.heads + h) * SP;
  bf16_t* yo = a.y + (trow * a.heads + h) * SP;
#pragma unroll
  for (int dt = 0; dt < SP / 16; ++dt) {
    const int p0 = 16 * dt + 4 * lg;
    const u32x2_t xv = *reinterpret_cast<const u32x2_t*>(xo + p0);
    const bf16_t* xe = reinterpret_cast<const bf16_t*>(&xv);
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = (et * yi[dt][r] + ya[dt][r]) + Dh * bf2f(xe[r]);
    *reinterpret_cast<u32x2_t*>(yo + p0) = u32x2_t{pack_f2bf2(o[0], o[1]), pack_f2bf2(o[2], o[3])};
  }
}

// ------------------------------------------------------------- chunk append
// The call's positions in an unfinished last chunk -> the slot's chunk buffer.
__global__ __launch_bounds__(256) void ssd_chunk_append_kernel(SsdArgs a) {
  const int s = blockIdx.x, j = blockIdx.y;  // j: row of the chunk
  const int* sq = a.seqs + 6 * s;
  const int cu = sq[0], pos0 = sq[1], ql = sq[2], slot = sq[3];
  const int pend = pos0 + ql - 1;
  if ((pend & (SQ - 1)) == SQ - 1) return;       // the last chunk completed
  const int p = (pend & ~(SQ - 1)) + j;
  if (p < pos0 || p > pend) return;
  const size_t trow = (size_t)(cu + p - pos0), brow = (size_t)slot * SQ + j;
  const int xw = a.heads * SP / 8, bw = a.groups * a.N / 8;
  for (int u = threadIdx.x; u < xw; u += 256)
    reinterpret_cast<u32x4_t*>(a.xb + brow * a.heads * SP)[u] =
        reinterpret_cast<const u32x4_t*>(a.x + trow * a.heads * SP)[u];
  for (int u = threadIdx.x; u < bw; u += 256)
    reinterpret_cast<u32x4_t*>(a.Bb + brow * a.groups * a.N)[u] =
        reinterpret_cast<const u32x4_t*>(a.B + trow * a.groups * a.N)[u];
  for (int u = threadIdx.x; u < a.heads; u += 256) a.dtb[brow * a.heads + u] = a.dt[trow * a.heads + u];
}

template <int N>
static void launch_ssd_t(const SsdArgs& a, hipStream_t st) {
  if (a.n_done > 0)
    hipLaunchKernelGGL((ssd_state_walk_kernel<N>), dim3(a.n_seqs, a.heads), dim3(256), 0, st, a);
  hipLaunchKernelGGL((ssd_chunk_out_kernel<N>), dim3(a.n_inst, a.heads), dim3(256), 0, st, a);
  hipLaunchKernelGGL(ssd_chunk_append_kernel, dim3(a.n_seqs, SQ), dim3(256), 0, st, a);
}

hipError_t launch_ssd(const SsdArgs& a, hipStream_t st) {
  if (a.n_inst == 0) return hipSuccess;
  if (a.N == 128)
    launch_ssd_t<128>(a, st);
  else if (a.N == 64)
    launch_ssd_t<64>(a, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bci
