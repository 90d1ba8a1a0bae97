// Internal launch interface between the C-ABI layer (bci.cpp) and the kernel
// translation units.  Not installed; no C++ type crosses the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bci {

// ---- norm.hip
// r/h: [rows, cols]; when ids != nullptr the residual input is E[ids[row]]
// (embedding gather fused into the first norm; `a` must be null then).
hipError_t launch_add_rmsnorm(const void* a, const void* r_in, void* r_out, void* h,
                              const void* g, const int32_t* ids, const void* E, int rows,
                              int cols, float eps, hipStream_t s);
hipError_t launch_embed(const int32_t* ids, const void* E, void* out, int rows, int cols,
                        hipStream_t s);
hipError_t launch_gather_rows(const void* src, const int32_t* rows, void* dst, int n_rows,
                              int cols, hipStream_t s);

// ---- gemm.hip
// EPI_ADD (tiled schedule, or the skinny one for M <= 4): C is a bf16 residual [M, N]
// updated in place, C = bf(bf(A W^T) + C) -- the residual add of the add+RMSNorm that
// follows.
enum GemmEpi { EPI_BF16 = 0, EPI_F32 = 1, EPI_SILU = 2, EPI_ADD = 3 };
// C = A . W^T.  A [M, K] (rows gathered through a_rows when non-null), W [N, K].
hipError_t launch_gemm(const void* A, const int32_t* a_rows, const void* W, void* C, int M, int N,
                       int K, int epi, hipStream_t s);
// launch_gemm runs M <= SKINNY_MAX_M (when K % 128 == 0 and N % 16 == 0) on a
// skinny schedule with the same per-element arithmetic as the 256x256 tiles.
constexpr int SKINNY_MAX_M = 128;
// Between SKINNY_MAX_M and SKINNY_DENSE_MAX_M rows a dense GEMM (launch_gemm, the QKV +
// RoPE form with a bf16 cache) takes whichever schedule a latency model of the two
// predicts faster (gemm_prefers_skinny); the grouped expert GEMMs keep SKINNY_MAX_M.
constexpr int SKINNY_DENSE_MAX_M = 512;
// epi: EPI_BF16 / EPI_F32 / EPI_SILU / EPI_ADD; rope: the QKV + RoPE form (two weight
// streams per wave, like SiLU)
bool gemm_prefers_skinny(int M, int N, int K, int epi, bool rope);
// M <= 4, K % 512 == 0, K <= 2048: A = RMSNorm(res [M, K]) * gamma [K] computed inside
// the skinny GEMM with the add+RMSNorm kernel's arithmetic (its bits, without its
// launch); epi EPI_BF16 or EPI_SILU.  The QKV form has the RoPE / bf16 KV-write
// epilogue of launch_gemm_qkv_rope.
hipError_t launch_gemm_norm(const void* res, const void* gamma, float eps, const void* W, void* C, int M, int N,
                            int K, int epi, hipStream_t s);
// Non-invariant split-K for small M (BCI_MODE_FAST only): ws holds M*N fp32.
constexpr int FAST_SPLITK_MAX_M = 256;
hipError_t launch_gemm_splitk(const void* A, const void* W, void* C, int M, int N, int K, int epi,
                              float* ws, hipStream_t s);
// ---- probe.hip: back-to-back MFMAs on every SIMD (out: blocks * 512 floats)
hipError_t launch_mfma_rate(float* out, int blocks, int iters, int random, hipStream_t s);
constexpr int PROBE_BLOCK_THREADS = 512;
// ---- vendor_gemm.cpp (BCI_MODE_FAST only): C [M, N] bf16 = A [M, K] . W [N, K]^T
// through hipBLASLt, whose kernel choice depends on the shape (not batch-invariant).
struct VendorGemm;
bool vendor_gemm_create(VendorGemm** out, void* ws, size_t ws_bytes);
void vendor_gemm_destroy(VendorGemm* v);
bool vendor_gemm(VendorGemm* v, const void* A, const void* W, void* C, int M, int N, int K, hipStream_t s);
// Deterministic split-K (any mode): ws holds ceil(K / k_split) * M * N fp32 partials,
// summed in slice order.  k_split % GEMM_BK == 0; epi EPI_BF16 or EPI_F32.
hipError_t launch_gemm_ksplit(const void* A, const void* W, void* C, int M, int N, int K, int k_split, int epi,
                              float* ws, hipStream_t s);
// Grouped GEMM over a device tile list (see GemmArgs in gemm.hip): m-tile i covers
// rows gtiles[3i+1] .. +gtiles[3i+2] of C with weight W + gtiles[3i] * w_group_stride;
// A rows are a_rows[r] / a_div when a_rows is non-null, else r.
// max_rows: an upper bound on the rows of any group (<= 16 selects the skinny schedule)
hipError_t launch_gemm_grouped(const void* A, const int32_t* a_rows, int a_div, const void* W,
                               size_t w_group_stride, void* C, const int32_t* gtiles,
                               const int32_t* n_gtiles, int max_mtiles, int max_rows, int N, int K,
                               int epi, hipStream_t s);
// lm_head partials: for each row i < M and vocab chunk c (256 columns):
// part_m[c * M + i] = max_j z_ij, part_s[c * M + i] = sum_j exp(z_ij - max),
// and zid[i] = z[i, ids[i]].
hipError_t launch_lmhead_partials(const void* A, const int32_t* a_rows, const void* E,
                                  const int32_t* ids, int M, int V, int K, float* part_m,
                                  float* part_s, float* zid, hipStream_t s);
hipError_t launch_lmhead_combine(const float* part_m, const float* part_s, const float* zid,
                                 const int32_t* ids, int M, int V, float* lp, hipStream_t s);
constexpr int LM_CHUNK = 256;
constexpr int GEMM_BM = 256;
constexpr int GEMM_BN = 256;
constexpr int GEMM_BK = 64;

// ---- rope_kv.hip
struct KvLayer {
  void* k;         // [n_blocks, nkv, 64, d] bf16 or u8
  void* v;
  float* ks;       // [n_blocks, nkv, 64] (fp8 only)
  float* vs;
};
// QKV GEMM with RoPE and the KV write in its epilogue (tiled schedule, head_dim
// 128, N % 256 == 0): the same bits as launch_gemm(EPI_BF16) into a qkv buffer
// followed by launch_rope_kv_write, without the qkv buffer.
hipError_t launch_gemm_qkv_rope(const void* A, const void* W, int M, int N, int K, void* q_out,
                                const int32_t* tok_pos, const int32_t* tok_slot, const float* rope_cos,
                                const float* rope_sin, KvLayer kv, int nq, int nkv, bool fp8,
                                hipStream_t s);
hipError_t launch_gemm_qkv_rope_norm(const void* res, const void* gamma, float eps, const void* W, int M, int N,
                                     int K, void* q_out, const int32_t* tok_pos, const int32_t* tok_slot,
                                     const float* rope_cos, const float* rope_sin, KvLayer kv, int nq, int nkv,
                                     hipStream_t s);
hipError_t launch_rope_kv_write(const void* qkv, void* q_out, const int32_t* tok_pos,
                                const int32_t* tok_slot, const float* rope_cos,
                                const float* rope_sin, KvLayer kv, int T, int nq, int nkv, int d,
                                bool fp8, hipStream_t s);
hipError_t launch_kv_gather(KvLayer kv, const int32_t* block_row, int n_pos, int nkv, int d,
                            bool fp8, void* k_out, void* v_out, hipStream_t s);

// ---- attention.hip
struct AttnArgs {
  const void* q;               // [T, nq*d] bf16
  void* o;                     // [T, nq*d] bf16
  KvLayer kv;
  // [n_tiles, ATTN_TILE_WORDS]: seq, tok_begin, n_tok, pos_begin, then the physical
  // blocks of the sequence's chunks 0 and 1 (chunk 1's = chunk 0's when it has one), which
  // the unsplit schedules load without waiting for the block table
  const int32_t* tiles;
  const int32_t* block_table;  // [n_seqs, max_blocks]
  const int32_t* tok_pos;      // [T] absolute position of each token (split merge)
  int n_tiles, max_blocks, nq, nkv, d, seg_keys;
  bool fp8;
  float scale_log2;            // (1/sqrt(d)) * log2(e), fp32
  // split schedule: one workgroup per (tile, kv head, segment) writes the
  // segment's (m, l, acc) to part_* and a merge kernel combines segments in
  // ascending order; n_seg = segments of the deepest tile (0: no split).
  int n_seg, n_tokens;
  float* part_acc;             // [n_seg][T][nq][d]
  float* part_ml;              // [n_seg][T][nq][2]
  // unsplit schedule with two chunks in flight (tiles of at most 16 rows: decode)
  bool pf2;
  // tiles of at most 16 rows: the four waves split the PV work (implied by pf2)
  bool dsplit;
  // every position of the call lies in the first segment (prefill schedule only)
  bool one_seg;
};
constexpr int ATTN_ROWS = 64;  // query rows (token x head-in-group) per tile
constexpr int ATTN_TILE_WORDS = 8;  // ints per attention tile record (32 bytes)
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// ---- sparse.hip (sparse attention over a Top-K selected key set)
// index keys [T, DI] bf16 -> paged FP8 index cache (codes [n_blocks*64, DI], scales
// [n_blocks*64]) at each token's cache slot
hipError_t launch_index_key_write(const void* kidx, const int32_t* tok_slot, void* codes,
                                  float* scales, int T, int DI, hipStream_t s);
struct IdxArgs {
  const uint16_t* q;           // [T, heads, dim] bf16 index queries
  const float* w;              // [T, heads] head weights
  const uint8_t* codes;        // [n_blocks * 64, dim] e4m3 index keys
  const float* scales;         // [n_blocks * 64]
  const int32_t* block_table;  // [n_seqs, max_blocks]
  const int32_t* tok_pos;      // [T]
  const int32_t* tok_seq;      // [T]
  const int32_t* tiles;        // [n_tiles, 4] (seq, tok_begin, n_tok, pos_begin), <= 4 tokens
  float* scores;               // [T, stride]
  size_t stride;
  int T, heads, dim, max_blocks, n_tiles, max_pos;
};
constexpr int IDX_TILE_TOKENS = 4;
hipError_t launch_index_scores(const IdxArgs& a, bool staged, hipStream_t s);
hipError_t launch_sparse_topk(const float* scores, size_t stride, const int32_t* tok_pos, int T,
                              int K, int32_t* sel, hipStream_t s);
struct SparseAttnArgs {
  const void* q;               // [T, nq*d] bf16
  void* o;                     // [T, nq*d] bf16
  KvLayer kv;                  // FP8 cache layer
  const int32_t* sel;          // [T, K] selected positions
  const int32_t* block_table;
  const int32_t* tok_pos;
  const int32_t* tok_seq;
  int T, K, max_blocks, nq, nkv, d;
  float scale_log2;
};
constexpr int SPARSE_MAX_K = 2048;
hipError_t launch_sparse_attention(const SparseAttnArgs& a, hipStream_t s);

// ---- ssd.hip (state-space layer, chunked; decode replays prefill's chunks)
struct SsdArgs {
  const uint16_t *x, *B, *C;   // call inputs: x [T, heads, 64], B/C [T, groups, N] bf16
  const float *dt, *A, *D;     // dt [T, heads]; A, D [heads]
  uint16_t* y;                 // [T, heads, 64] bf16
  uint16_t *xb, *Bb;           // chunk buffers [slots][64][heads][64], [slots][64][groups][N]
  float* dtb;                  // [slots][64][heads]
  float* state;                // [slots][heads][64][N] fp32
  uint16_t* hprev;             // [max_done][heads][64][N] bf16 (state before each chunk)
  const int32_t* seqs;         // [n_seqs][6]: cu, pos0, q_len, slot, first done index, n done
  const int32_t* inst;         // [n_inst][6]: seq, chunk, first pos, last pos, done index or -1, 0
  const int32_t* done;         // [n_done]: instance of each completed chunk
  int heads, groups, N, n_seqs, n_inst, n_done;
};
hipError_t launch_ssd(const SsdArgs& a, hipStream_t s);

// ---- backward.hip
hipError_t launch_transpose_bf16(const void* src, void* dst, int R, int C, int ldd, hipStream_t s);
constexpr int BW_DG_ROWS = 64;  // rows per partial sum of the gain gradient
hipError_t launch_rmsnorm_backward(const void* r, const void* g, const void* dh, const void* dr_in,
                                   void* dr, float* rstd, float* dg, float* part, int rows, int cols,
                                   float eps, hipStream_t s);
hipError_t launch_silu_mul_backward(const void* gu, const void* dact, void* dgu, int rows, int inter,
                                    hipStream_t s);
hipError_t launch_logprob_dz(const float* z, const int32_t* ids, const float* gout, void* dz, int M, int V,
                             hipStream_t s);
hipError_t launch_rope_backward(const void* dq, const void* dk, const void* dv, void* dqkv,
                                const int32_t* tok_pos, const float* rcos, const float* rsin, int T, int nq,
                                int nkv, int d, hipStream_t s);

// ---- attn_backward.hip (one sequence at positions 0..L-1)
struct AttnBwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;  // q, o, dout [L, nq, d]; k, v [L, nkv, d] bf16
  uint16_t *dq, *dk, *dv;                // bf16, same shapes
  float *lse, *dsum;                     // workspace [L, nq]: log2-sum-exp2, sum dO o
  float* part;                           // null, or fp32 [AB_MAX_PARTS][L][nkv][d] x 2 (dK, dV)
  int L, nq, nkv, d;
  float scale, scale_log2;               // 1/sqrt(d), log2(e)/sqrt(d)
};
// the dK/dV pass splits each key tile's rows into at most AB_MAX_PARTS fixed parts of
// >= AB_PART_MIN_ROWS rows (when a part buffer is given), summed in part order
constexpr int AB_MAX_PARTS = 4;
constexpr int AB_PART_MIN_ROWS = 2048;
hipError_t launch_attention_backward(const AttnBwdArgs& a, hipStream_t s);

// ---- moe.hip
constexpr int MOE_MAX_K = 8;
hipError_t launch_moe_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                           hipStream_t s);
hipError_t launch_moe_sort(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                           int32_t* perm, int32_t* inv, int32_t* tiles, int32_t* n_tiles,
                           hipStream_t s);
hipError_t launch_moe_combine(const void* y, const void* ys, const int32_t* ids, const float* w,
                              const int32_t* inv, int T, int k, int E, int H, void* out,
                              hipStream_t s);

}  // namespace bci
