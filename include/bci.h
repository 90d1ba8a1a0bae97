/*
 * bci.h -- C ABI of the batch-invariant logprob-recompute forward for MI355X (gfx950).
 *
 * What the library computes.  In on-policy RL the rollout engine samples tokens
 * and the trainer recomputes the log-probability of every sampled token under
 * the same weights; the two must agree bit for bit (page "Finish RL Training
 * Faster" digest, section "零差异需要一个精确的比较对象"; news page "A vLLM bitre
 * azonosította az RL-tréning és az inferencia eredményeit", section "A tréning
 * közvetlenül a vLLM inferenciás kerneljeit használja").  The trainer's forward
 * calls the same inference kernels (digest, section "让训练前向使用推理的数值";
 * page "No More Train-Inference Mismatch", section "方法细节").  Every entry point
 * below produces, for each row, a result that does not depend on the other rows
 * of the call, on how the sequence was split into prefill chunks and decode
 * steps, or on which entry point ran it.
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers unless the name says "host".
 *     bf16 tensors are 16-bit bit patterns (void*); fp32 tensors are float*.
 *     Matrices are row-major and dense (leading dimension = number of columns).
 *   - The caller owns every tensor (weights, KV cache, inputs, outputs).  The
 *     library owns only its context and the one workspace that bci_create
 *     allocates; it never allocates again, so workspace addresses are stable.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; outputs are valid after the stream synchronises.
 *     Use one stream per context at a time.
 *   - Every argument is validated on the host before any launch; on error
 *     nothing is enqueued and bci_last_error() explains.  A failed launch
 *     returns BCI_E_HIP with the HIP error text.
 *   - No entry point throws or aborts across the ABI.
 *
 * Numeric contract (identical in every entry point and every phase)
 *   - GEMMs: bf16 operands; each output element is ONE fp32 accumulator that
 *     starts at zero and receives v_mfma_f32_16x16x32_bf16 of its own A row and
 *     W row over ascending 32-wide K steps, and nothing else.  Several schedules
 *     assign elements to workgroups -- 256 x 256 tiles, a skinny one-wave-per-16-
 *     columns-and-32-rows schedule for M <= 128 (and up to 512 where a latency
 *     model of the call's M, N and K favours it), 16- and 64-row lm_head tiles for
 *     few scored rows -- and which one runs depends on the shape, but every one performs this
 *     same per-element chain (no split-K, no atomics), so the bits of a row never
 *     depend on M or on the row's place in a tile (page "Finish RL Training
 *     Faster" digest, section "让训练前向使用推理的数值": batch-invariant dense GEMM
 *     that gives up small-batch kernel switches).
 *   - Norm and softmax reductions: fixed shuffle/LDS trees that depend only on
 *     the column position, never on the row count.
 *   - Attention: keys walked in 64-key chunks at absolute positions (chunk c =
 *     keys 64c..64c+63), grouped into segments of `attn_segment_keys` keys that
 *     are computed from scratch and merged in ascending order, for prefill,
 *     chunked prefill and decode alike.
 *   - FP8 KV (e4m3fn, per-token-per-head fp32 scale): every phase quantises
 *     through one rule and reads keys/values back as bf(fp32(code) * scale).
 *   - lm_head: fp32 logits never materialised; per 256-column vocab chunk a
 *     (max, sum-exp) pair; the pairs are merged in one fixed order that depends
 *     only on the vocabulary size (8 contiguous chunk ranges, each ascending,
 *     then the 8 range results in order).
 */
#ifndef BCI_H
#define BCI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bci_ctx bci_ctx;

typedef enum {
  BCI_OK = 0,
  BCI_E_INVALID = -1,      /* bad argument (shape, range, null pointer)           */
  BCI_E_UNSUPPORTED = -2,  /* valid request this build does not implement          */
  BCI_E_HIP = -3,          /* a HIP call or kernel launch failed                   */
  BCI_E_WORKSPACE = -4,    /* request exceeds the limits given at bci_create       */
  BCI_E_STATE = -5         /* weights / cache / batch not bound yet                */
} bci_status;

/* BCI_MODE_FAST is the non-invariant reference schedule, kept only to quote
 * the cost of invariance.  It takes the choices a throughput engine takes where
 * they are faster: the O and down projections of calls above 256 tokens run on
 * the vendor GEMM (hipBLASLt, whose kernel choice depends on the shape), with the
 * residual adds in the norms after them; GEMMs with
 * 128 < M <= 256 and K >= 4096 split K across workgroups and add fp32 partials
 * with atomics (order, hence bits, depend on timing); and attention sizes its KV
 * segments from each call's shape, splitting calls with fewer workgroups than CUs
 * (prefill and decode meet different reduction trees).  Its results are NOT
 * batch-invariant. */
typedef enum { BCI_MODE_INVARIANT = 0, BCI_MODE_FAST = 1 } bci_mode;
typedef enum { BCI_KV_BF16 = 0, BCI_KV_FP8_E4M3 = 1 } bci_kv_dtype;
typedef enum { BCI_EPI_BF16 = 0, BCI_EPI_F32 = 1, BCI_EPI_SILU_MUL = 2 } bci_epilogue;

/* Model shape and numeric contract; copied by bci_create.
 *   head_dim must be 64 or 128; hidden, n_q_heads*head_dim and intermediate
 *   multiples of 128; n_q_heads a multiple of n_kv_heads.
 *   kv_block_tokens must be 64 (= the attention chunk).  attn_segment_keys is a
 *   positive multiple of 64 (default 2048 when 0).
 *   max_* bound every later call and size the workspace. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
  float rms_eps, rope_theta;
  int32_t kv_dtype;            /* bci_kv_dtype */
  int32_t kv_block_tokens;     /* 64 */
  int32_t attn_segment_keys;   /* S, multiple of 64; 0 -> 2048 */
  int32_t max_tokens_per_call; /* T_max: new tokens in one forward call           */
  int32_t max_seqs_per_call;
  int32_t max_scored_per_call;
  int32_t max_position;        /* context capacity per sequence (RoPE table size)  */
  int32_t mode;                /* bci_mode; fixed for the life of the context      */
  /* MoE layer (0 experts = dense only).  n_experts <= 64, 1 <= top_k <= min(8,
   * n_experts), expert_intermediate % 128 == 0, n_shared_experts 0 or 1.  The
   * MoE entry points use `hidden` as the model width and size their workspace
   * for max_tokens_per_call * top_k routed rows. */
  int32_t n_experts, top_k, expert_intermediate, n_shared_experts;
  /* Attention schedule (never changes a bit, only where the work runs):
   * 0 = auto (split a call's KV segments across workgroups when it has few
   * query tiles and at most max_seqs_per_call tokens), 1 = never split,
   * 2 = split whenever the workspace allows. */
  int32_t attn_split_mode;
} bci_model_config;

/* One varlen forward call; HOST arrays.  Sequences are packed back to back:
 * sequence i owns tokens [cu_q[i], cu_q[i+1]) at absolute positions
 * pos0[i] .. pos0[i] + q_len - 1 (q_len >= 1).  Its keys/values for positions
 * < pos0[i] must already be in the bound KV cache; this call writes the new
 * ones.  block_table[i * max_blocks_per_seq + j] is the cache block holding
 * positions 64j .. 64j+63 of sequence i.  score_rows[r] is a token index whose
 * NEXT token score_ids[r] is scored (the logprob of a valid response token). */
typedef struct {
  int32_t n_seqs, n_tokens, n_scored, max_blocks_per_seq;
  const int32_t* tokens;       /* [n_tokens], each in [0, vocab)                  */
  const int32_t* cu_q;         /* [n_seqs + 1], cu_q[0] = 0, cu_q[n_seqs] = n_tokens */
  const int32_t* pos0;         /* [n_seqs]                                         */
  const int32_t* block_table;  /* [n_seqs * max_blocks_per_seq]                    */
  const int32_t* score_rows;   /* [n_scored], each in [0, n_tokens)                */
  const int32_t* score_ids;    /* [n_scored], each in [0, vocab)                   */
} bci_batch;

/* ---- context ------------------------------------------------------------ */

/* Creates a context on HIP device `device` and allocates its workspace (sized
 * from the max_* fields) and the fp32 RoPE table [max_position, head_dim/2].
 * On failure *out is NULL and the status says why (no context to query). */
bci_status bci_create(const bci_model_config* cfg, int32_t device, bci_ctx** out);
/* Frees the workspace.  Safe on NULL.  The caller must have synchronised. */
void bci_destroy(bci_ctx* ctx);
/* Text of the last error on this context ("" if none).  Valid until the next call. */
const char* bci_last_error(const bci_ctx* ctx);
/* Bytes of device workspace the context holds. */
uint64_t bci_workspace_bytes(const bci_ctx* ctx);

/* Binds the weights (pointers are kept; the caller keeps the memory alive and
 * rebinds after reallocating).  Order (n_ptrs = 2 + 6 * n_layers):
 *   [0] embed [vocab, hidden] (tied lm_head), then per layer l:
 *   attn_norm [hidden], wqkv [(nq + 2 nkv) * d, hidden] (q heads, k heads, v heads),
 *   wo [hidden, nq * d], mlp_norm [hidden], wgu [2 * intermediate, hidden] (gate rows
 *   then up rows), wd [hidden, intermediate]; last: final_norm [hidden].
 * weight_version identifies the weights (same version => comparable logprobs). */
bci_status bci_bind_weights(bci_ctx* ctx, const void* const* ptrs, int32_t n_ptrs,
                            uint64_t weight_version);
uint64_t bci_weight_version(const bci_ctx* ctx);

/* Binds a paged KV cache.  Layout, per tensor:
 *   k, v   : [n_layers, n_blocks, n_kv_heads, 64, head_dim]  bf16, or uint8 e4m3fn codes
 *   k_scale, v_scale (FP8 only, else NULL): [n_layers, n_blocks, n_kv_heads, 64] fp32
 * Every buffer must be 16-byte aligned (BCI_E_INVALID otherwise).
 * The rollout call and the training recompute bind different buffers (the
 * private cache copy of the digest's FP8 paragraph), written through the same
 * quantiser. */
bci_status bci_bind_kv_cache(bci_ctx* ctx, void* k, void* v, float* k_scale, float* v_scale,
                             int32_t n_blocks);

/* Validates a host batch and uploads its metadata (token ids, positions, cache
 * slots, attention tile list, scored rows) into the workspace on `stream`.  It
 * stays the context's current batch for bci_forward_logprobs and the bci_op_*
 * calls that take no explicit shape. */
bci_status bci_set_batch(bci_ctx* ctx, const bci_batch* batch, void* stream);

/* The whole forward of the current batch (page "Finish RL Training Faster" digest,
 * section "零差异需要一个精确的比较对象": the quantity compared between rollout and
 * training is the logprob of every valid response token under one weight version
 * and one token prefix; the same section requires one computation path whatever
 * the batch and the phase): embedding, n_layers x [add+RMSNorm,
 * QKV GEMM, RoPE + KV write, attention, O GEMM, add+RMSNorm, gate_up GEMM with
 * SiLU*up, down GEMM], final add+RMSNorm, lm_head + fp32 log-softmax + gather.
 * Writes d_logprobs[n_scored] (fp32).  This is the "rollout" entry point.  Batches
 * of more than 128 tokens (256 in BCI_MODE_FAST) run RoPE + KV write inside the QKV
 * GEMM's epilogue (head_dim 128) and (not in BCI_MODE_FAST) the residual adds inside
 * the O and down GEMMs' epilogues (hidden % 256 == 0).  Batches of at most 4 tokens with hidden % 512
 * == 0 and hidden <= 2048 add the O and down projections into the residual in those
 * GEMMs' epilogues and normalise the QKV and gate_up GEMMs' A rows inside those GEMMs
 * (with RoPE + a bf16 KV write in the QKV epilogue when head_dim is 128), so only
 * the first and the final add+RMSNorm run as kernels of their own.  Every logprob
 * and cache byte equals what the same sequence of bci_op_* calls produces. */
bci_status bci_forward_logprobs(bci_ctx* ctx, float* d_logprobs, void* stream);

/* bci_forward_logprobs replayed from a HIP graph.  On the first call for a batch
 * shape (n_tokens, n_seqs, n_scored, attention tiles, block-table width) the forward
 * is captured on a private stream into a graph kept by the context (up to 16 shapes,
 * least recently used dropped); later calls with the same shape launch that graph on
 * `stream` and copy the logprobs to d_logprobs.  The graph reads the batch metadata
 * that bci_set_batch uploads to the workspace's fixed addresses, so a decode loop
 * calls bci_set_batch then this function each step; positions, tokens and block ids
 * may change between replays.  Bits equal bci_forward_logprobs (the captured forward
 * launches every KV segment the context can hold; the ones past a row's position are
 * no-ops).  Weights updated in place (same buffers, e.g. after an optimiser step) are
 * read by the next replay; a rebind that moves any weight or cache buffer drops the
 * graphs and the next call captures again (the stable workspace and in-place weight
 * update of the digest's section "让训练前向使用推理的数值", which also requires a
 * stable batch shape for capture).  The block-table width is part of the shape, so a
 * decode loop keeps it fixed (pads the table).  Invariant mode and dense models only
 * (BCI_E_UNSUPPORTED otherwise); errors as bci_forward_logprobs, plus BCI_E_HIP when
 * capture or instantiation fails (nothing is launched then). */
bci_status bci_forward_logprobs_graph(bci_ctx* ctx, float* d_logprobs, void* stream);
/* Number of graphs the context holds; bci_graph_reset drops them all. */
int32_t bci_graph_count(const bci_ctx* ctx);
bci_status bci_graph_reset(bci_ctx* ctx);

/* ---- per-operator entry points ("the training forward calls the inference
 *      kernels"); each is bitwise identical to its use inside the forward ---- */

/* r[i] = E[tokens[i]] for the current batch (exact row copy): the first step of the
 * forward that recomputes the token probabilities of a prefix (page "Finish RL
 * Training Faster" digest, opening paragraph and section "零差异需要一个精确的比较对象").
 * E [vocab, hidden] bf16, r [n_tokens, hidden] bf16; BCI_E_STATE without a batch. */
bci_status bci_op_embed(bci_ctx* ctx, const void* E, void* r, void* stream);

/* Fused residual add + RMSNorm over `rows` rows of `cols` bf16 values
 * (page "No More Train-Inference Mismatch", section "方法细节"):
 *   if a != NULL: r <- bf(fp32(a) + fp32(r))   (r is updated in place)
 *   h <- bf(r * rsqrt(mean(r^2) + eps) * g), the mean over the rounded r.
 * a, r, h: [rows, cols] bf16; g: [cols] bf16.  cols % 8 == 0, cols <= 8192. */
bci_status bci_op_add_rmsnorm(bci_ctx* ctx, const void* a, void* r, void* h, const void* g,
                              int32_t rows, int32_t cols, float eps, void* stream);

/* C = A . W^T with A [M, K] bf16 and W [N, K] bf16 (nn.Linear layout), fp32
 * accumulation in ascending K order, the same for every M (page "Finish RL
 * Training Faster" digest, section "让训练前向使用推理的数值": batch-invariant
 * dense GEMM).  Epilogues:
 *   BCI_EPI_BF16:     C [M, N] bf16 = bf(acc)
 *   BCI_EPI_F32:      C [M, N] fp32 = acc
 *   BCI_EPI_SILU_MUL: W holds gate rows then up rows (N = 2 I); C [M, I] bf16 =
 *                     bf(silu(bf(acc_gate)) * bf(acc_up))   (fused SiLU MLP)
 * K % 64 == 0; N >= 1 (BCI_EPI_SILU_MUL: I % 128 == 0); M >= 0; A and W 16-byte aligned;
 * (I + 256) * K * 2 and min(M, 512) * K * 2 below 2^31 (the copies' descriptor range);
 * otherwise BCI_E_INVALID and nothing is launched. */
bci_status bci_op_gemm_bf16(bci_ctx* ctx, const void* A, const void* W, void* C, int32_t M,
                            int32_t N, int32_t K, int32_t epilogue, void* stream);

/* C = A . W^T as bci_op_gemm_bf16, with the contraction cut into fixed slices of
 * k_split (the last may be shorter) for products with few output tiles and a long
 * contraction (the logits' gradient times the embedding in the lm_head backward):
 * slice s's fp32 partial (the same ascending 32-wide MFMA chain from zero over the
 * slice) goes to workspace + s * M * N, then C = bf16 or fp32 of the partials summed in
 * ascending slice order.  Deterministic, and row i depends only on row i of A, W and
 * k_split (never on M) -- the fixed reduction order of page "Finish RL Training Faster"
 * digest, section "让训练前向使用推理的数值".  A [M, K], W [N, K] bf16, 16-byte aligned;
 * K and k_split multiples of 64; epilogue BCI_EPI_BF16 or BCI_EPI_F32; workspace fp32
 * [ceil(K / k_split) * M * N], owned by the caller. */
bci_status bci_op_gemm_bf16_ksplit(bci_ctx* ctx, const void* A, const void* W, void* C, int32_t M, int32_t N,
                                   int32_t K, int32_t k_split, int32_t epilogue, float* workspace,
                                   void* stream);

/* For the current batch and layer: rotates q and k of qkv [n_tokens, (nq + 2 nkv) d]
 * (half-split RoPE at each token's absolute position, fp32 table, bf16 result),
 * writes q' to q_out [n_tokens, nq * d] and k', v into the bound cache (bf16, or
 * e4m3 with the per-token-per-head scale rule a = max|x|, s = a / 448, code =
 * e4m3_rne(clamp(x / s, +-448)); page "Finish RL Training Faster" digest, section
 * "让训练前向使用推理的数值", FP8 KV paragraph).  qkv and q_out must be 16-byte
 * aligned (BCI_E_INVALID otherwise). */
bci_status bci_op_rope_kv_write(bci_ctx* ctx, const void* qkv, void* q_out, int32_t layer,
                                void* stream);

/* FP8 KV gather / dequantise (page "Finish RL Training Faster" digest, section
 * "让训练前向使用推理的数值", the FP8 KV paragraph and the figure caption before it:
 * the cache stays FP8, and prefill, decode and the training recompute all gather
 * and dequantise it to BF16 before one attention operator, the recompute from a
 * private cache copy written through the same FP8 round trip).  Gathers sequence
 * `seq` of the current batch, positions 0 .. n_pos - 1, of one layer out of the
 * paged cache: k_out, v_out [n_pos, n_kv_heads, head_dim] bf16 = bf(fp32(code) *
 * scale) (a plain copy for a bf16 cache), caller owned.  This is the conversion
 * the attention kernel applies on load, through the same device function, so the
 * materialised and the fused paths give the same bits.  n_pos <= pos0 + q_len of
 * the sequence (BCI_E_INVALID otherwise); BCI_E_STATE without a batch. */
bci_status bci_op_kv_gather_dequant(bci_ctx* ctx, int32_t seq, int32_t n_pos, int32_t layer,
                                    void* k_out, void* v_out, void* stream);

/* Causal GQA attention of the current batch for one layer: q [n_tokens, nq * d]
 * bf16 (rotated) against the bound cache, o [n_tokens, nq * d] bf16.  Query head
 * h reads kv head h / (nq / nkv).  One kernel for prefill, chunked prefill and
 * decode; keys in 64-key chunks at absolute positions, ascending; segments of S
 * keys merged ascending (digest, sections "零差异需要一个精确的比较对象" and
 * "让训练前向使用推理的数值"). */
bci_status bci_op_attention(bci_ctx* ctx, const void* q, int32_t layer, void* o, void* stream);

/* ---- sparse attention over a Top-K selected key set --------------------------
 * The DeepSeek-V4-Flash recipe runs sparse attention whose Top-K breaks ties by a
 * fixed rule and lists the selected set in fixed position order, and feeds every
 * phase the FP8 cache gathered and dequantised to BF16 before one sparse attention
 * operator (page "Finish RL Training Faster" digest, section "让训练前向使用推理的数值"
 * and its figure caption).  The pages give no scoring function; these calls use the
 * indexer of DeepSeek's sparse attention:
 *   score(t, s) = sum_h w[t,h] * relu(q_idx[t,h,:] . k_idx[s,:]),  0 <= s <= pos(t),
 * with the index keys in an FP8 index cache (one e4m3 row and one fp32 scale per
 * token, the KV cache's quantisation rule) read back as bf(fp32(code) * scale).
 * The index cache is paged like the KV cache and uses the same block ids:
 *   icodes [n_index_blocks, 64, index_dim] uint8, iscale [n_index_blocks, 64] fp32,
 * caller owned, 16-byte aligned, n_index_blocks >= the bound KV cache's n_blocks;
 * one such pair per layer.  index_dim is 64 or 128; index_heads 16, 32 or 64.
 * Every token's scores, selection and output are bitwise independent of the batch,
 * of prefill / chunked prefill / decode and of the score schedule. */

/* Quantises kidx [n_tokens, index_dim] bf16 (one index key per token of the current
 * batch) into the index cache at each token's position. */
bci_status bci_op_index_key_write(bci_ctx* ctx, const void* kidx, int32_t index_dim, void* icodes,
                                  float* iscale, int32_t n_index_blocks, void* stream);

/* scores[t * score_stride + s] = score(t, s) (fp32) for s = 0 .. pos(t); later
 * entries of the row are not written.  qidx [n_tokens, index_heads, index_dim] bf16
 * (16-byte aligned), w [n_tokens, index_heads] fp32, scores 16-byte aligned,
 * score_stride a multiple of 4 and > every position of the batch.  Per (t, s): fp32
 * MFMA dot products in ascending 32-wide steps of index_dim, then one fixed
 * relu-weighted chain over the heads.  schedule: 0 chooses from the batch shape,
 * 1 forces keys read per token, 2 forces keys staged for four tokens of a sequence
 * (testing; the bits are the same). */
bci_status bci_op_index_scores(bci_ctx* ctx, const void* qidx, const float* w, int32_t index_heads,
                               int32_t index_dim, const void* icodes, const float* iscale,
                               int32_t n_index_blocks, float* scores, int64_t score_stride,
                               int32_t schedule, void* stream);

/* Top-K selection per token of the current batch: the topk positions s <= pos(t)
 * with the largest scores, ranked by (score descending, position ascending) -- an
 * equal score goes to the earlier position; NaN ranks above every number and
 * -0 equals +0 -- written to sel[t * topk ..] in ascending position order.  When
 * pos(t) + 1 <= topk every position 0 .. pos(t) is selected and the row is padded
 * with -1.  scores as written by bci_op_index_scores (same stride rules);
 * sel [n_tokens, topk] int32. */
bci_status bci_op_sparse_topk(bci_ctx* ctx, const float* scores, int64_t score_stride, int32_t topk,
                              int32_t* sel, void* stream);

/* Attention of q [n_tokens, nq * d] bf16 (rotated) over the keys listed in
 * sel [n_tokens, topk] (positions; an entry outside [0, pos(t)], e.g. the -1
 * padding, is skipped) of layer `layer` of the bound FP8 cache; o as q.  K and V
 * rows are gathered by position and dequantised with the cache's one rule.  Per
 * (token, kv head): the list is cut into segments of 256 entries, each walked in
 * 64-entry chunks in list order with the online softmax of bci_op_attention, and
 * the segments are merged in ascending order; with every position selected the
 * bits equal bci_op_attention on a context with attn_segment_keys = 256.  topk a
 * multiple of 64 in [64, 2048]; FP8 cache and a GQA group <= 16 only
 * (BCI_E_UNSUPPORTED otherwise). */
bci_status bci_op_sparse_attention(bci_ctx* ctx, const void* q, int32_t layer, const int32_t* sel,
                                   int32_t topk, void* o, void* stream);

/* Scored-row select: out[r] = src[score_rows[r]] for the current batch, [n_scored,
 * cols] bf16 (an exact copy).  Only valid response tokens are compared (page
 * "Finish RL Training Faster" digest, section "零差异需要一个精确的比较对象"), so
 * the lm_head runs on these rows only.  cols % 8 == 0; BCI_E_STATE without a batch. */
bci_status bci_op_gather_scored(bci_ctx* ctx, const void* src, int32_t cols, void* out,
                                void* stream);

/* lm_head + fp32 log-softmax + gather of the sampled token (digest, section
 * "零差异需要一个精确的比较对象": the compared quantity):
 *   z = hf . E^T in fp32 (never stored), lp[i] = z[i, ids[i]] - logsumexp(z[i, :]).
 * hf [M, H] bf16, E [V, H] bf16, ids [M] int32 (device; an id outside [0, V)
 * yields NaN), lp [M] fp32.  H % 64 == 0; hf and E 16-byte aligned; M <=
 * max_scored_per_call (the partials live in the workspace). */
bci_status bci_op_lmhead_logprob(bci_ctx* ctx, const void* hf, const void* E, const int32_t* ids,
                                 int32_t M, int32_t H, int32_t V, float* lp, void* stream);

/* bci_op_lmhead_logprob for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It needs
 * no context and allocates nothing (no hipMalloc, hipFree or allocating library
 * call): the per-(row, vocab chunk) partials live in a fixed device array of the
 * library, 2 * BCI_LMHEAD_NOALLOC_MAX_PAIRS + BCI_LMHEAD_NOALLOC_MAX_ROWS fp32
 * (2.4 MiB), that each GPU the library runs on holds until the process ends; its
 * address is looked up on the first call made with that device current.  Same
 * arguments and the same kernels, hence the same bits, as bci_op_lmhead_logprob:
 * hf [M, H] bf16, E [V, H] bf16, ids [M] int32 (an id outside [0, V) yields NaN),
 * lp [M] fp32, all device pointers; H % 64 == 0.  Limits: M <=
 * BCI_LMHEAD_NOALLOC_MAX_ROWS and M * ceil(V / 256) <= BCI_LMHEAD_NOALLOC_MAX_PAIRS
 * (M <= 512 at V = 151936), else BCI_E_WORKSPACE with nothing enqueued; bad
 * pointers or shapes give BCI_E_INVALID, a failed launch BCI_E_HIP (there is no
 * context, so no error text).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams, two host threads) race and must be ordered
 * by the caller; nothing in the array needs clearing between calls. */
#define BCI_LMHEAD_NOALLOC_MAX_ROWS 1024
#define BCI_LMHEAD_NOALLOC_MAX_PAIRS 304128
bci_status bci_lmhead_logprob_noalloc(const void* hf, const void* E, const int32_t* ids, int32_t M,
                                      int32_t H, int32_t V, float* lp, void* stream);

/* ---- MoE (configured through n_experts / top_k / expert_intermediate) ------ */

/* Router top-K with a fixed tie rule (digest, section "零差异需要一个精确的比较对象":
 * tie handling in discrete Top-K; section "让训练前向使用推理的数值": MoE).
 * logits [T, n_experts] fp32 (device).  Experts are ranked by (logit descending,
 * expert index ascending); slots 0..top_k-1 take them in that order.
 * ids [T, top_k] int32, w [T, top_k] fp32 = softmax over the selected logits
 * (the denominator summed in slot order).  NaN logits rank above every number. */
bci_status bci_op_moe_topk(bci_ctx* ctx, const float* logits, int32_t T, int32_t* ids, float* w,
                           void* stream);

/* One MoE layer: out[t] = bf( sum over slots s = 0..top_k-1, in slot order, of
 * fp32 w[t,s] * y_{ids[t,s]}(h[t]) accumulated with one fp32 FMA chain, then +
 * y_shared(h[t]) ), where y_e(x) = bf( bf(silu(bf(x Wg_e^T)) * bf(x Wu_e^T)) Wd_e^T )
 * (digest, section "让训练前向使用推理的数值": row-wise expert compute and an FP32
 * combine in fixed slot order).  Pairs (t, s) are grouped by expert with a
 * stable sort in (t, s) order and run through one grouped GEMM per projection.
 *   h [T, hidden] bf16; ids, w as produced by bci_op_moe_topk (device; an id
 *   outside [0, n_experts) makes that token's row NaN);
 *   wgu [n_experts, 2 I, hidden] (gate rows then up rows), wd [n_experts, hidden, I];
 *   swgu [2 I, hidden], swd [hidden, I] the ungated shared expert (NULL when
 *   n_shared_experts == 0); out [T, hidden] bf16, 16-byte aligned.
 *   T <= max_tokens_per_call. */
bci_status bci_op_moe_forward(bci_ctx* ctx, const void* h, const int32_t* ids, const float* w,
                              int32_t T, const void* wgu, const void* wd, const void* swgu,
                              const void* swd, void* out, void* stream);

/* ---- backward pieces ---------------------------------------------------------
 * The trainer keeps the inference forward and adds its own backward, whose gradients
 * are checked against an independent reference (page "Finish RL Training Faster"
 * digest, section "让训练前向使用推理的数值").  The backward's GEMMs are
 * bci_op_gemm_bf16 on transposed operands (dX = dY . W as dY . (W^T)^T; dW = dY^T . X
 * as (dY^T) . (X^T)^T with the token dimension padded to 64 by zeros), so every element
 * is one ascending fp32 MFMA chain; the calls below are the pieces around them.  The
 * forward's roundings are taken as the identity (straight-through) and the backward
 * is evaluated at the forward's stored bf16 values.  Activation gradients are bf16,
 * weight and gain gradients fp32. */

/* dst[c * ld_dst + r] = src[r * C + c] for r < R, c < C; 0 for R <= r < ld_dst (bf16).
 * C and ld_dst multiples of 8, ld_dst >= R, both pointers 16-byte aligned. */
bci_status bci_op_transpose_bf16(bci_ctx* ctx, const void* src, void* dst, int32_t R, int32_t C,
                                 int32_t ld_dst, void* stream);

/* Backward of h = bf(r * s * g), s = 1 / sqrt(mean(r^2) + eps) (the forward's
 * expression), per row of r [rows, cols] (the forward's rounded residual):
 *   dr = bf((g dh) s - r (s^3 sum_k g_k dh_k r_k / cols) + dr_in)   (dr_in may be NULL:
 *        the gradient reaching r through the residual stream; dr is then also the
 *        gradient of both inputs of the forward's add),
 *   rstd[row] = s (fp32), dg[k] = sum over rows in ascending order (partial sums over
 *   blocks of 64 rows, then the blocks in order) of dh r s (fp32).
 * g [cols] bf16; dh, dr_in, dr [rows, cols] bf16.  cols % 8 == 0, cols <= 8192,
 * rows <= max_tokens_per_call. */
bci_status bci_op_add_rmsnorm_backward(bci_ctx* ctx, const void* r, const void* g, const void* dh,
                                       const void* dr_in, void* dr, float* rstd, float* dg,
                                       int32_t rows, int32_t cols, float eps, void* stream);

/* Backward of act = bf(silu(gate) * up): gu [rows, 2 I] (gate columns then up columns,
 * the gate_up GEMM's bf16 output), dact [rows, I] bf16 -> dgu [rows, 2 I] bf16 =
 * [bf(dact up silu'(gate)), bf(dact silu(gate))], silu'(x) = sig(x)(1 + x(1 - sig(x))). */
bci_status bci_op_silu_mul_backward(bci_ctx* ctx, const void* gu, const void* dact, void* dgu,
                                    int32_t rows, int32_t inter, void* stream);

/* The logprob's gradient with respect to the logits: z [M, V] fp32 (the lm_head GEMM
 * with the fp32 epilogue), ids [M] int32, gout [M] fp32 (dL/dlp) -> dz [M, V] bf16 =
 * bf(gout_i ((j == ids_i) - exp(z_ij - m_i) / S_i)), (m_i, S_i) the row's max and sum of
 * exp(z - m), folded per thread and merged by a fixed tree (an id outside [0, V) gives
 * a NaN row).  V % 4 == 0 uses 16-byte loads; z and dz then 16- and 8-byte aligned.  dhf = dz . E and
 * dE = dz^T . hf follow as GEMMs. */
bci_status bci_op_logprob_backward_dz(bci_ctx* ctx, const float* z, const int32_t* ids,
                                      const float* gout, int32_t M, int32_t V, void* dz,
                                      void* stream);

/* Backward of bci_op_rope_kv_write's rotation for the current batch: dq [n_tokens, nq d],
 * dk and dv [n_tokens, nkv d] bf16 (gradients with respect to the rotated q, the keys
 * written to the cache and the values) -> dqkv [n_tokens, (nq + 2 nkv) d] bf16, laid out
 * as the forward's qkv input.  Per rotation pair (e, d/2 + e) of a q or k head, at the
 * token's position and with the forward's fp32 table (c, s):
 *   dx1 = bf(dr1 c + dr2 s),  dx2 = bf(dr2 c - dr1 s)   (the rotation's transpose),
 * and dv is copied.  The forward's bf16 roundings (and, for an FP8 cache, the key's
 * quantiser) are taken as the identity, the straight-through of page "Finish RL
 * Training Faster" digest, section "让训练前向使用推理的数值".  All tensors 16-byte
 * aligned (BCI_E_INVALID otherwise); BCI_E_STATE without a batch. */
bci_status bci_op_rope_backward(bci_ctx* ctx, const void* dq, const void* dk, const void* dv, void* dqkv,
                                void* stream);

/* Backward of the causal GQA attention of one sequence at positions 0..L-1 (the
 * context's heads and head_dim): q, o, dout [L, nq, d], k, v [L, nkv, d] bf16 -- k and v
 * the keys and values the forward attended to (for an FP8 cache the dequantised ones:
 * the quantiser's gradient is taken as the identity, so dk and dv are also the
 * gradients of the keys and values before quantisation, the straight-through of the
 * digest's section "让训练前向使用推理的数值").  With P the weights and D = sum dO o:
 *   dq = dS k / sqrt(d),  dk = dS^T q / sqrt(d),  dv = P^T dO,  dS = P (dO v^T - D),
 * summed over the query heads of each kv head; dq, dk, dv bf16, same shapes.  Each
 * element accumulates in one fixed order (dq over 64-key chunks ascending, dk and dv
 * over 64-row chunks ascending; no atomics), so the result is deterministic.  The row
 * statistics (log-sum-exp, D) are recomputed into the context's workspace.  workspace:
 * NULL, or fp32 [2 * 4 * L * nkv * d] owned by the caller, 16-byte aligned: with it and
 * at least 4096 (token, query head) rows per kv head, the dK/dV pass cuts the rows into
 * at most 4 fixed parts (by row index), sums each part in fp32 and adds the parts in
 * ascending order -- deterministic, balanced across the causal key tiles; different bits
 * from the unsplit order.  L <= max_tokens_per_call; all tensors 16-byte aligned. */
bci_status bci_op_attention_backward(bci_ctx* ctx, const void* q, const void* k, const void* v,
                                     const void* o, const void* dout, int32_t L, void* dq, void* dk,
                                     void* dv, float* workspace, void* stream);

/* ---- state-space layer (Mamba-2-style), chunked ---------------------------------
 * Porting the method to Nemotron-3.5 meant recursive arithmetic in which decode
 * replays prefill's chunked computation order and training reuses the same operator
 * (page "Finish RL Training Faster" digest, sections "一致性有多个层面，修好一处还不能验收"
 * and "两组结果，要连同分母一起读").  The pages give no formula; the layer computed is
 * the Mamba-2 selective state-space recurrence, per head h (B, C shared by the heads of
 * a group g = h / (n_heads / n_groups)), from a zero state at position 0:
 *   h_t = exp(A[h] dt[t,h]) h_{t-1} + dt[t,h] B[t,g] (outer) x[t,h]
 *   y[t,h] = bf( C[t,g] . h_t + D[h] x[t,h] )
 * evaluated in chunks of 64 positions at fixed absolute positions.  The state is kept
 * only at chunk ends; every position's output is computed from the state before its
 * chunk and the chunk's inputs up to it by one routine, so a token's output bits do
 * not depend on the batch, on how its sequence was split into calls (prefill, chunked
 * prefill, decode) or on the call.  The context is separate from bci_ctx: a layer of
 * this kind holds no KV cache.
 *
 * Per-slot memory is the caller's (one slot per sequence in flight):
 *   state     [n_slots, n_heads, 64 (head dim), d_state] fp32 -- the state at the last
 *             chunk end of the slot's sequence (never read for chunk 0, so a new
 *             sequence needs no clearing);
 *   chunk_buf [x: n_slots, 64, n_heads, 64 bf16][B: n_slots, 64, n_groups, d_state bf16]
 *             [dt: n_slots, 64, n_heads fp32] -- the inputs of the slot's unfinished
 *             chunk.  bci_ssd_slot_bytes(which = 0 / 1) gives one slot's size of each.
 * A slot's pos0 in a call must equal the number of positions its sequence has already
 * run through this layer (0 for a new sequence); calls that overlap on a slot race. */
typedef struct bci_ssd bci_ssd;
typedef struct {
  int32_t n_heads;     /* multiple of n_groups */
  int32_t head_dim;    /* 64 */
  int32_t d_state;     /* 64 or 128 */
  int32_t n_groups;
  int32_t max_tokens_per_call;
  int32_t max_seqs_per_call;
} bci_ssd_config;

/* Validates the configuration and allocates the workspace (chunk states of up to
 * max_tokens_per_call / 64 + max_seqs_per_call chunks, and the call tables). */
bci_status bci_ssd_create(const bci_ssd_config* cfg, int32_t device, bci_ssd** out);
void bci_ssd_destroy(bci_ssd* ctx);
const char* bci_ssd_last_error(const bci_ssd* ctx);
/* Bytes of one slot: which = 0 the state, 1 the chunk buffer (0 for other values). */
uint64_t bci_ssd_slot_bytes(const bci_ssd* ctx, int32_t which);

/* The next call's layout (host arrays): sequence i owns tokens [cu_q[i], cu_q[i+1])
 * (at least one) at positions pos0[i] .. and uses slot[i] (distinct within a call).
 * Uploads the chunk tables on `stream`; errors leave nothing enqueued. */
bci_status bci_ssd_set_batch(bci_ssd* ctx, int32_t n_seqs, const int32_t* cu_q, const int32_t* pos0,
                             const int32_t* slot, void* stream);

/* One layer over the current batch.  x [T, n_heads, 64] bf16, dt [T, n_heads] fp32 (the
 * step after its softplus), A [n_heads] fp32 (< 0), B and C [T, n_groups, d_state] bf16,
 * D [n_heads] fp32 (device pointers; x, dt, B, C, state, chunk_buf and y 16-byte
 * aligned); y [T, n_heads, 64] bf16.  Updates the slots' state and chunk buffer.  Per
 * head, with a_j = fp32(A log2 e) dt_j and L_t their inclusive prefix over the chunk:
 *   y_t = bf((2^L_t (C_t . bf(H)) + sum_{j<=t} bf((C_t . B_j) 2^(L_t - L_j) dt_j) x_j) + D x_t),
 *   H <- 2^L_63 H + sum_j x_j (outer) bf(B_j 2^(L_63 - L_j) dt_j)  at each chunk end,
 * dot products on fp32-accumulating MFMA in ascending 32-wide steps. */
bci_status bci_ssd_forward(bci_ssd* ctx, const void* x, const float* dt, const float* A, const void* B,
                           const void* C, const float* D, float* state, void* chunk_buf, int32_t n_slots,
                           void* y, void* stream);

/* ---- instrumentation ----------------------------------------------------- */

/* While enabled, bci_forward_logprobs records a HIP event pair on its stream
 * around every launch of the gate_up GEMM (the SiLU*up-epilogue kernel, the
 * largest single kernel of the forward) together with the launch's row count M.
 * bci_profile_begin creates the events for `capacity` launches up front (0 means
 * 8192), so no event is created inside a timed region; launches beyond the
 * capacity are not timed and are counted in *dropped.  bci_profile_end
 * synchronises the events and returns the summed kernel time in ms, the number
 * of launches timed and the sum of their M (so that the caller counts the FLOPs
 * of exactly the timed launches: 2 * rows * 2 * intermediate * hidden). */
bci_status bci_profile_begin(bci_ctx* ctx, int32_t capacity);
bci_status bci_profile_end(bci_ctx* ctx, double* total_ms, int32_t* launches, int64_t* rows,
                           int32_t* dropped);

/* The sustained dense bf16 MFMA rate of HIP device `device`, measured: every SIMD issues
 * v_mfma_f32_16x16x32_bf16 back to back for ~50 ms (16 independent chains per wave, two
 * waves per SIMD, operands in registers: pseudo-random bf16 values when random_operands
 * is non-zero, zeros otherwise) after a warm-up.  *tflops receives the rate in TFLOP/s:
 * a denominator beside the datasheet peak that includes the power-limited clock.
 * Allocates and frees a small buffer; synchronises the device's null stream. */
bci_status bci_measure_mfma_rate(int32_t device, int32_t random_operands, double* tflops);

#ifdef __cplusplus
}
#endif
#endif /* BCI_H */
