// C-ABI layer of libbci: context, validation, batch metadata upload, the
// forward orchestration and the per-operator entry points.
//
// Everything here runs on the host.  Every argument is checked before any
// launch, so a bad request enqueues nothing; device work is only ever
// launched through the kernels of the *.hip translation units.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/bci.h"
#include "kernels.h"

using namespace bci;

namespace {

constexpr int KV_BLOCK = 64;
constexpr int DEFAULT_PROFILE = 8192;
constexpr size_t VENDOR_WS_BYTES = (size_t)64 << 20;  // the vendor GEMM's workspace (fast mode)
// Fast mode on the tiled range: the O and down projections on the vendor GEMM with the
// residual adds in the norms; the QKV projection keeps the fused GEMM + RoPE + KV write
// (measured on the recompute, same box, fast-mode tokens/s: vendor QKV and O/down 224.1 /
// 223.7 K, vendor O/down only 224.8 / 224.5 K, vendor QKV only 223.2 / 223.0 K, neither
// 224.0 / 225.1 K: within noise of each other and of the invariant mode's 225 K)
constexpr bool FAST_VENDOR_QKV = false;
constexpr bool FAST_VENDOR_OD = true;

struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
};

}  // namespace

struct bci_ctx {
  bci_model_config cfg{};
  int device = 0;
  std::string err;
  // derived shape
  int qkv_w = 0, qd = 0, group = 0, max_blocks = 0, max_tiles = 0, n_chunks = 0, tpt = 0;
  // workspace (one allocation, carved)
  void* ws = nullptr;
  size_t ws_bytes = 0;
  uint16_t *bufR = nullptr, *bufH = nullptr, *bufQKV = nullptr, *bufQ = nullptr,
           *bufO = nullptr, *bufX = nullptr, *bufACT = nullptr;
  float *part_m = nullptr, *part_s = nullptr, *zid = nullptr;
  // MoE workspace (n_experts > 0)
  int32_t *moe_perm = nullptr, *moe_inv = nullptr, *moe_counts = nullptr, *moe_offsets = nullptr,
          *moe_tiles = nullptr, *moe_ntiles = nullptr;
  uint16_t *moe_act = nullptr, *moe_y = nullptr, *moe_act_s = nullptr, *moe_y_s = nullptr;
  int moe_max_mtiles = 0;
  float *rope_cos = nullptr, *rope_sin = nullptr;
  // split-attention partials: [max_seg][split_tokens][nq][d] and [..][2]
  float *attn_part_acc = nullptr, *attn_part_ml = nullptr;
  int max_seg = 1, split_tokens = 0;
  // backward: partial sums of the RMSNorm gain gradient [max_tokens / 64][8192] fp32,
  // and the attention backward's per-row statistics [max_tokens][nq] fp32 (x2)
  float* bw_part = nullptr;
  float *ab_lse = nullptr, *ab_dsum = nullptr;
  // non-invariant mode: split-K accumulation buffer [FAST_SPLITK_MAX_M, max_n] fp32, and
  // the vendor GEMM for large-M projections (null if the library offers no algorithm)
  float* splitk_ws = nullptr;
  int splitk_max_n = 0;
  void* vendor_ws = nullptr;
  VendorGemm* vg = nullptr;
  int32_t* meta = nullptr;  // device metadata region
  size_t meta_words = 0;
  // metadata offsets (int32 words)
  size_t o_tok = 0, o_pos = 0, o_slot = 0, o_tiles = 0, o_btab = 0, o_srow = 0, o_sid = 0;
  size_t o_tseq = 0, o_itiles = 0;  // token -> sequence; 4-token index-score tiles
  int max_itiles = 0;
  // pinned staging for uploads (2 slots, each guarded by an event)
  int32_t* stage[2] = {nullptr, nullptr};
  hipEvent_t stage_ev[2] = {nullptr, nullptr};
  bool stage_used[2] = {false, false};
  int stage_next = 0;
  // bindings
  std::vector<const void*> w;
  uint64_t weight_version = 0;
  bool weights_bound = false;
  void *kc = nullptr, *vc = nullptr;
  float *kscale = nullptr, *vscale = nullptr;
  int n_blocks = 0;
  bool cache_bound = false;
  // current batch (host copy of what was uploaded)
  bool batch_valid = false;
  int n_seqs = 0, n_tokens = 0, n_scored = 0, n_tiles = 0, batch_seg = 1;
  int n_itiles = 0, batch_max_pos = 0;
  std::vector<int32_t> h_cu, h_pos0, h_btab;  // h_btab with stride max_blocks
  // profiling of the gate_up GEMM launches (HIP events on the launch stream): one event
  // pair and the row count M per timed launch; launches past the capacity are counted
  // in prof_dropped and not timed
  bool prof_on = false;
  int prof_n = 0, prof_dropped = 0, prof_cap = 0;
  std::vector<hipEvent_t> prof_ev;
  std::vector<int32_t> prof_rows;
  // captured forwards, keyed by batch shape; bind_epoch changes whenever a rebind
  // moves a weight or cache buffer, which invalidates every captured graph
  struct Graph {
    int n_tokens, n_seqs, n_scored, n_tiles, max_blocks;
    uint64_t epoch;
    hipGraph_t graph;
    hipGraphExec_t exec;
    uint64_t last_use;
  };
  std::vector<Graph> graphs;
  uint64_t bind_epoch = 1, graph_clock = 0;
  bool graph_mode = false;  // set while capturing: attention schedule independent of positions
  hipStream_t cap_stream = nullptr;
  float* graph_lp = nullptr;  // logprob output of captured forwards [max_scored]
};

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static bci_status fail(bci_ctx* c, bci_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return st;
}

static bci_status hipfail(bci_ctx* c, hipError_t e, const char* what) {
  return fail(c, BCI_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(c, expr)                                         \
  do {                                                           \
    hipError_t e_ = (expr);                                      \
    if (e_ != hipSuccess) return hipfail((c), e_, #expr);        \
  } while (0)

static inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static KvLayer kv_layer(const bci_ctx* c, int layer) {
  const auto& g = c->cfg;
  const size_t rows = (size_t)c->n_blocks * g.n_kv_heads * KV_BLOCK;  // cache rows per layer
  const size_t esz = (g.kv_dtype == BCI_KV_FP8_E4M3) ? 1 : 2;
  KvLayer kv;
  kv.k = (char*)c->kc + (size_t)layer * rows * g.head_dim * esz;
  kv.v = (char*)c->vc + (size_t)layer * rows * g.head_dim * esz;
  kv.ks = c->kscale ? c->kscale + (size_t)layer * rows : nullptr;
  kv.vs = c->vscale ? c->vscale + (size_t)layer * rows : nullptr;
  return kv;
}

extern "C" {

bci_status bci_create(const bci_model_config* cfg_in, int32_t device, bci_ctx** out) {
  if (!out) return BCI_E_INVALID;
  *out = nullptr;
  if (!cfg_in) return BCI_E_INVALID;
  bci_model_config g = *cfg_in;
  if (g.attn_segment_keys == 0) g.attn_segment_keys = 2048;
  if (g.n_layers < 1 || g.hidden < 128 || g.hidden % 128 || g.hidden > 8192 || g.n_q_heads < 1 ||
      g.n_kv_heads < 1 || g.n_q_heads % g.n_kv_heads || (g.head_dim != 64 && g.head_dim != 128) ||
      (g.n_q_heads * g.head_dim) % 128 || g.intermediate < 64 || g.intermediate % 128 ||
      g.vocab < 1 || !(g.rms_eps >= 0.0f) || !(g.rope_theta > 0.0f))
    return BCI_E_INVALID;
  if (64 % (g.n_q_heads / g.n_kv_heads)) return BCI_E_INVALID;  // GQA group must divide 64
  if (g.kv_dtype != BCI_KV_BF16 && g.kv_dtype != BCI_KV_FP8_E4M3) return BCI_E_INVALID;
  if (g.kv_block_tokens != KV_BLOCK) return BCI_E_INVALID;
  if (g.attn_segment_keys < KV_BLOCK || g.attn_segment_keys % KV_BLOCK) return BCI_E_INVALID;
  if (g.max_tokens_per_call < 1 || g.max_seqs_per_call < 1 || g.max_scored_per_call < 0 ||
      g.max_position < 1)
    return BCI_E_INVALID;
  if (g.n_experts < 0 || g.n_experts > 64) return BCI_E_INVALID;
  if (g.n_experts > 0 &&
      (g.top_k < 1 || g.top_k > MOE_MAX_K || g.top_k > g.n_experts || g.expert_intermediate < 128 ||
       g.expert_intermediate % 128 || g.n_shared_experts < 0 || g.n_shared_experts > 1))
    return BCI_E_INVALID;
  if (g.attn_split_mode < 0 || g.attn_split_mode > 2) return BCI_E_INVALID;
  if (g.mode != BCI_MODE_INVARIANT && g.mode != BCI_MODE_FAST) return BCI_E_INVALID;
  if (hipSetDevice(device) != hipSuccess) return BCI_E_HIP;

  bci_ctx* c = new bci_ctx();
  c->cfg = g;
  c->device = device;
  c->qkv_w = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim;
  c->qd = g.n_q_heads * g.head_dim;
  c->group = g.n_q_heads / g.n_kv_heads;
  c->tpt = ATTN_ROWS / c->group;
  c->max_blocks = (g.max_position + KV_BLOCK - 1) / KV_BLOCK;
  c->max_tiles = g.max_tokens_per_call / c->tpt + g.max_seqs_per_call;
  c->n_chunks = (g.vocab + LM_CHUNK - 1) / LM_CHUNK;
  c->w.assign(2 + 6 * g.n_layers, nullptr);

  const size_t T = g.max_tokens_per_call, H = g.hidden, R = std::max(1, g.max_scored_per_call);
  // metadata words
  c->o_tok = 0;
  c->o_pos = c->o_tok + T;
  c->o_slot = c->o_pos + T;
  c->o_tiles = c->o_slot + T;
  c->o_btab = c->o_tiles + ATTN_TILE_WORDS * (size_t)c->max_tiles;
  c->o_srow = c->o_btab + (size_t)g.max_seqs_per_call * c->max_blocks;
  c->o_sid = c->o_srow + R;
  c->max_itiles = (int)(T / IDX_TILE_TOKENS) + g.max_seqs_per_call;
  c->o_tseq = c->o_sid + R;
  c->o_itiles = c->o_tseq + T;
  c->meta_words = c->o_itiles + 4 * (size_t)c->max_itiles;

  struct Part {
    void** dst;
    size_t bytes;
  };
  std::vector<Part> parts = {
      {(void**)&c->bufR, T * H * 2},
      {(void**)&c->bufH, T * H * 2},
      {(void**)&c->bufQKV, T * c->qkv_w * 2},
      {(void**)&c->bufQ, T * c->qd * 2},
      {(void**)&c->bufO, T * c->qd * 2},
      {(void**)&c->bufX, T * H * 2},
      {(void**)&c->bufACT, T * (size_t)g.intermediate * 2},
      {(void**)&c->part_m, (size_t)c->n_chunks * R * 4},
      {(void**)&c->part_s, (size_t)c->n_chunks * R * 4},
      {(void**)&c->zid, R * 4},
      {(void**)&c->graph_lp, R * 4},
      {(void**)&c->rope_cos, (size_t)g.max_position * (g.head_dim / 2) * 4},
      {(void**)&c->rope_sin, (size_t)g.max_position * (g.head_dim / 2) * 4},
      {(void**)&c->meta, c->meta_words * 4},
      {(void**)&c->bw_part, (T + BW_DG_ROWS - 1) / BW_DG_ROWS * (size_t)8192 * 4},
      {(void**)&c->ab_lse, T * (size_t)g.n_q_heads * 4},
      {(void**)&c->ab_dsum, T * (size_t)g.n_q_heads * 4},
  };
  c->max_seg = (g.max_position + g.attn_segment_keys - 1) / g.attn_segment_keys;
  if (g.mode == BCI_MODE_FAST) {
    // the non-invariant schedule sizes segments per call: up to 64 of them
    c->max_seg = std::min(64, (g.max_position + KV_BLOCK - 1) / KV_BLOCK);
    c->splitk_max_n = std::max({c->qkv_w, 2 * g.intermediate, g.hidden});
    parts.push_back({(void**)&c->splitk_ws, (size_t)FAST_SPLITK_MAX_M * c->splitk_max_n * 4});
    parts.push_back({(void**)&c->vendor_ws, VENDOR_WS_BYTES});
  }
  if (c->max_seg > 1 && g.attn_split_mode != 1) {
    c->split_tokens = g.max_seqs_per_call;
    const size_t rows = (size_t)c->max_seg * c->split_tokens * g.n_q_heads;
    parts.push_back({(void**)&c->attn_part_acc, rows * g.head_dim * 4});
    parts.push_back({(void**)&c->attn_part_ml, rows * 2 * 4});
  }
  if (g.n_experts > 0) {
    const size_t P = T * (size_t)g.top_k, I = g.expert_intermediate;
    c->moe_max_mtiles = (int)((P + GEMM_BM - 1) / GEMM_BM) + g.n_experts;
    std::vector<Part> moe = {
        {(void**)&c->moe_perm, P * 4},
        {(void**)&c->moe_inv, P * 4},
        {(void**)&c->moe_counts, (size_t)g.n_experts * 4},
        {(void**)&c->moe_offsets, (size_t)(g.n_experts + 1) * 4},
        {(void**)&c->moe_tiles, (size_t)c->moe_max_mtiles * 3 * 4},
        {(void**)&c->moe_ntiles, 4},
        {(void**)&c->moe_act, P * I * 2},
        {(void**)&c->moe_y, P * H * 2},
        {(void**)&c->moe_act_s, T * I * 2},
        {(void**)&c->moe_y_s, T * H * 2},
    };
    parts.insert(parts.end(), moe.begin(), moe.end());
  }
  size_t total = 0;
  for (auto& p : parts) total += align_up(p.bytes, 256);
  if (hipMalloc(&c->ws, total) != hipSuccess) {
    delete c;
    return BCI_E_WORKSPACE;
  }
  c->ws_bytes = total;
  size_t off = 0;
  for (auto& p : parts) {
    *p.dst = (char*)c->ws + off;
    off += align_up(p.bytes, 256);
  }
  if (g.mode == BCI_MODE_FAST && !vendor_gemm_create(&c->vg, c->vendor_ws, VENDOR_WS_BYTES)) c->vg = nullptr;
  for (int i = 0; i < 2; ++i) {
    if (hipHostMalloc((void**)&c->stage[i], c->meta_words * 4, hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming) != hipSuccess) {
      bci_destroy(c);
      return BCI_E_WORKSPACE;
    }
  }
  // RoPE table: cos/sin(t * theta^(-2i/d)) in double, rounded to fp32.
  {
    const int half = g.head_dim / 2;
    std::vector<float> cs((size_t)g.max_position * half), sn((size_t)g.max_position * half);
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)g.rope_theta, -2.0 * i / g.head_dim);
      for (int t = 0; t < g.max_position; ++t) {
        const double a = (double)t * inv;
        cs[(size_t)t * half + i] = (float)std::cos(a);
        sn[(size_t)t * half + i] = (float)std::sin(a);
      }
    }
    if (hipMemcpy(c->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(c->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
      bci_destroy(c);
      return BCI_E_HIP;
    }
  }
  *out = c;
  return BCI_OK;
}

static void drop_graphs(bci_ctx* c) {
  for (auto& g : c->graphs) {
    (void)hipGraphExecDestroy(g.exec);
    (void)hipGraphDestroy(g.graph);
  }
  c->graphs.clear();
}

// Teardown is best effort: there is no caller to report a failure to, so the
// status of each release call is deliberately dropped.
void bci_destroy(bci_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  drop_graphs(c);
  vendor_gemm_destroy(c->vg);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  for (auto& e : c->prof_ev)
    if (e) (void)hipEventDestroy(e);
  for (int i = 0; i < 2; ++i) {
    if (c->stage_ev[i]) {
      (void)hipEventSynchronize(c->stage_ev[i]);  // the staging slot may still be read
      (void)hipEventDestroy(c->stage_ev[i]);
    }
    if (c->stage[i]) (void)hipHostFree(c->stage[i]);
  }
  if (c->ws) (void)hipFree(c->ws);
  delete c;
}

const char* bci_last_error(const bci_ctx* c) { return c ? c->err.c_str() : "null context"; }

uint64_t bci_workspace_bytes(const bci_ctx* c) { return c ? c->ws_bytes : 0; }

bci_status bci_bind_weights(bci_ctx* c, const void* const* ptrs, int32_t n, uint64_t version) {
  if (!c) return BCI_E_INVALID;
  if (!ptrs || n != (int32_t)c->w.size())
    return fail(c, BCI_E_INVALID, "bind_weights: expected %d pointers, got %d", (int)c->w.size(), n);
  for (int i = 0; i < n; ++i)
    if (!ptrs[i]) return fail(c, BCI_E_INVALID, "bind_weights: pointer %d is null", i);
  bool moved = !c->weights_bound;
  for (int i = 0; i < n; ++i) moved = moved || c->w[i] != ptrs[i];
  if (moved) ++c->bind_epoch;  // captured graphs hold the old addresses
  for (int i = 0; i < n; ++i) c->w[i] = ptrs[i];
  c->weight_version = version;
  c->weights_bound = true;
  return BCI_OK;
}

uint64_t bci_weight_version(const bci_ctx* c) { return c ? c->weight_version : 0; }

bci_status bci_bind_kv_cache(bci_ctx* c, void* k, void* v, float* ks, float* vs, int32_t n_blocks) {
  if (!c) return BCI_E_INVALID;
  const bool fp8 = c->cfg.kv_dtype == BCI_KV_FP8_E4M3;
  if (!k || !v || n_blocks < 1) return fail(c, BCI_E_INVALID, "bind_kv_cache: null buffer or n_blocks < 1");
  if (fp8 && (!ks || !vs)) return fail(c, BCI_E_INVALID, "bind_kv_cache: FP8 cache needs scales");
  if (!fp8 && (ks || vs)) return fail(c, BCI_E_INVALID, "bind_kv_cache: bf16 cache takes no scales");
  if (!aligned16(k) || !aligned16(v) || (fp8 && (!aligned16(ks) || !aligned16(vs))))
    return fail(c, BCI_E_INVALID, "bind_kv_cache: buffers must be 16-byte aligned");
  if (!c->cache_bound || c->kc != k || c->vc != v || c->kscale != ks || c->vscale != vs ||
      c->n_blocks != n_blocks)
    ++c->bind_epoch;
  c->kc = k;
  c->vc = v;
  c->kscale = ks;
  c->vscale = vs;
  c->n_blocks = n_blocks;
  c->cache_bound = true;
  c->batch_valid = false;  // block ids were validated against the old cache
  return BCI_OK;
}

bci_status bci_set_batch(bci_ctx* c, const bci_batch* b, void* stream) {
  if (!c) return BCI_E_INVALID;
  c->batch_valid = false;
  const auto& g = c->cfg;
  if (!b) return fail(c, BCI_E_INVALID, "set_batch: null batch");
  if (!c->cache_bound) return fail(c, BCI_E_STATE, "set_batch: bind a KV cache first");
  if (b->n_seqs < 1 || b->n_seqs > g.max_seqs_per_call)
    return fail(c, BCI_E_WORKSPACE, "set_batch: n_seqs %d outside [1, %d]", b->n_seqs, g.max_seqs_per_call);
  if (b->n_tokens < 1 || b->n_tokens > g.max_tokens_per_call)
    return fail(c, BCI_E_WORKSPACE, "set_batch: n_tokens %d outside [1, %d]", b->n_tokens, g.max_tokens_per_call);
  if (b->n_scored < 0 || b->n_scored > g.max_scored_per_call)
    return fail(c, BCI_E_WORKSPACE, "set_batch: n_scored %d outside [0, %d]", b->n_scored, g.max_scored_per_call);
  if (b->max_blocks_per_seq < 1) return fail(c, BCI_E_INVALID, "set_batch: max_blocks_per_seq < 1");
  if (!b->tokens || !b->cu_q || !b->pos0 || !b->block_table || (b->n_scored && (!b->score_rows || !b->score_ids)))
    return fail(c, BCI_E_INVALID, "set_batch: null array");
  if (b->cu_q[0] != 0 || b->cu_q[b->n_seqs] != b->n_tokens)
    return fail(c, BCI_E_INVALID, "set_batch: cu_q must start at 0 and end at n_tokens");
  for (int i = 0; i < b->n_seqs; ++i) {
    const int ql = b->cu_q[i + 1] - b->cu_q[i];
    if (ql < 1) return fail(c, BCI_E_INVALID, "set_batch: sequence %d has q_len %d", i, ql);
    const int p0 = b->pos0[i];
    if (p0 < 0 || (int64_t)p0 + ql > g.max_position)
      return fail(c, BCI_E_INVALID, "set_batch: sequence %d positions [%d, %d) exceed max_position %d", i, p0,
                  p0 + ql, g.max_position);
    const int need = (p0 + ql + KV_BLOCK - 1) / KV_BLOCK;
    if (need > b->max_blocks_per_seq)
      return fail(c, BCI_E_INVALID, "set_batch: sequence %d needs %d blocks, table has %d", i, need,
                  b->max_blocks_per_seq);
    for (int j = 0; j < need; ++j) {
      const int blk = b->block_table[(size_t)i * b->max_blocks_per_seq + j];
      if (blk < 0 || blk >= c->n_blocks)
        return fail(c, BCI_E_INVALID, "set_batch: sequence %d block %d id %d outside [0, %d)", i, j, blk,
                    c->n_blocks);
    }
  }
  for (int t = 0; t < b->n_tokens; ++t)
    if (b->tokens[t] < 0 || b->tokens[t] >= g.vocab)
      return fail(c, BCI_E_INVALID, "set_batch: token %d id %d outside [0, %d)", t, b->tokens[t], g.vocab);
  for (int r = 0; r < b->n_scored; ++r) {
    if (b->score_rows[r] < 0 || b->score_rows[r] >= b->n_tokens)
      return fail(c, BCI_E_INVALID, "set_batch: score row %d = %d outside [0, %d)", r, b->score_rows[r],
                  b->n_tokens);
    if (b->score_ids[r] < 0 || b->score_ids[r] >= g.vocab)
      return fail(c, BCI_E_INVALID, "set_batch: score id %d = %d outside [0, %d)", r, b->score_ids[r], g.vocab);
  }
  // count tiles and the deepest segment
  int n_tiles = 0, bseg = 1;
  for (int i = 0; i < b->n_seqs; ++i) {
    n_tiles += (b->cu_q[i + 1] - b->cu_q[i] + c->tpt - 1) / c->tpt;
    bseg = std::max(bseg, (b->pos0[i] + b->cu_q[i + 1] - b->cu_q[i] - 1) / g.attn_segment_keys + 1);
  }
  if (n_tiles > c->max_tiles) return fail(c, BCI_E_WORKSPACE, "set_batch: %d attention tiles > %d", n_tiles, c->max_tiles);

  // wait until the staging slot's previous upload has been consumed
  const int sl = c->stage_next;
  c->stage_next ^= 1;
  if (c->stage_used[sl]) HIP_TRY(c, hipEventSynchronize(c->stage_ev[sl]));
  int32_t* h = c->stage[sl];
  std::memcpy(h + c->o_tok, b->tokens, sizeof(int32_t) * b->n_tokens);
  c->h_cu.assign(b->cu_q, b->cu_q + b->n_seqs + 1);
  c->h_pos0.assign(b->pos0, b->pos0 + b->n_seqs);
  c->h_btab.assign((size_t)b->n_seqs * c->max_blocks, 0);
  for (int i = 0; i < b->n_seqs; ++i) {
    const int need = (b->pos0[i] + b->cu_q[i + 1] - b->cu_q[i] + KV_BLOCK - 1) / KV_BLOCK;
    for (int j = 0; j < need; ++j)
      c->h_btab[(size_t)i * c->max_blocks + j] = b->block_table[(size_t)i * b->max_blocks_per_seq + j];
  }
  std::memcpy(h + c->o_btab, c->h_btab.data(), c->h_btab.size() * sizeof(int32_t));
  int tix = 0, iix = 0, max_pos = 0;
  for (int i = 0; i < b->n_seqs; ++i) {
    const int q0 = b->cu_q[i], ql = b->cu_q[i + 1] - q0, p0 = b->pos0[i];
    max_pos = std::max(max_pos, p0 + ql - 1);
    for (int t0 = 0; t0 < ql; t0 += IDX_TILE_TOKENS) {
      int32_t* tl = h + c->o_itiles + 4 * (size_t)iix++;
      tl[0] = i;
      tl[1] = q0 + t0;
      tl[2] = std::min(IDX_TILE_TOKENS, ql - t0);
      tl[3] = p0 + t0;
    }
    for (int t = 0; t < ql; ++t) {
      const int p = p0 + t;
      h[c->o_tseq + q0 + t] = i;
      h[c->o_pos + q0 + t] = p;
      h[c->o_slot + q0 + t] = c->h_btab[(size_t)i * c->max_blocks + p / KV_BLOCK] * KV_BLOCK + p % KV_BLOCK;
    }
    const int32_t* brow = c->h_btab.data() + (size_t)i * c->max_blocks;
    const int need = (p0 + ql + KV_BLOCK - 1) / KV_BLOCK;
    for (int t0 = 0; t0 < ql; t0 += c->tpt) {
      int32_t* tl = h + c->o_tiles + ATTN_TILE_WORDS * (size_t)tix++;
      tl[0] = i;
      tl[1] = q0 + t0;
      tl[2] = std::min(c->tpt, ql - t0);
      tl[3] = p0 + t0;
      tl[4] = brow[0];
      tl[5] = brow[need > 1 ? 1 : 0];
      tl[6] = tl[7] = 0;
    }
  }
  if (b->n_scored) {
    std::memcpy(h + c->o_srow, b->score_rows, sizeof(int32_t) * b->n_scored);
    std::memcpy(h + c->o_sid, b->score_ids, sizeof(int32_t) * b->n_scored);
  }
  HIP_TRY(c, hipSetDevice(c->device));
  HIP_TRY(c, hipMemcpyAsync(c->meta, h, c->meta_words * 4, hipMemcpyHostToDevice, S(stream)));
  HIP_TRY(c, hipEventRecord(c->stage_ev[sl], S(stream)));
  c->stage_used[sl] = true;
  c->n_seqs = b->n_seqs;
  c->n_tokens = b->n_tokens;
  c->n_scored = b->n_scored;
  c->n_tiles = n_tiles;
  c->batch_seg = bseg;
  c->n_itiles = iix;
  c->batch_max_pos = max_pos;
  c->batch_valid = true;
  return BCI_OK;
}

// ---------------------------------------------------------------- ops

static bci_status need_batch(bci_ctx* c, const char* who) {
  if (!c->batch_valid) return fail(c, BCI_E_STATE, "%s: no current batch (call bci_set_batch)", who);
  return BCI_OK;
}

static bci_status op_rope(bci_ctx* c, const void* qkv, void* q_out, int layer, hipStream_t s) {
  const auto& g = c->cfg;
  HIP_TRY(c, launch_rope_kv_write(qkv, q_out, c->meta + c->o_pos, c->meta + c->o_slot, c->rope_cos,
                                  c->rope_sin, kv_layer(c, layer), c->n_tokens, g.n_q_heads,
                                  g.n_kv_heads, g.head_dim, g.kv_dtype == BCI_KV_FP8_E4M3, s));
  return BCI_OK;
}

static bci_status op_attn(bci_ctx* c, const void* q, void* o, int layer, hipStream_t s) {
  const auto& g = c->cfg;
  AttnArgs a{};
  a.q = q;
  a.o = o;
  a.kv = kv_layer(c, layer);
  a.tiles = c->meta + c->o_tiles;
  a.block_table = c->meta + c->o_btab;
  a.n_tiles = c->n_tiles;
  a.max_blocks = c->max_blocks;
  a.nq = g.n_q_heads;
  a.nkv = g.n_kv_heads;
  a.d = g.head_dim;
  a.seg_keys = g.attn_segment_keys;
  a.fp8 = g.kv_dtype == BCI_KV_FP8_E4M3;
  a.scale_log2 = (float)(1.0 / std::sqrt((double)g.head_dim) * 1.4426950408889634);
  a.tok_pos = c->meta + c->o_pos;
  a.n_tokens = c->n_tokens;
  // schedule: split the KV segments across workgroups when the call has few
  // query tiles (decode, short chunks); bits are the same either way
  const bool few_tiles = c->n_tiles * g.n_kv_heads < 1024;
  if (g.mode == BCI_MODE_FAST) {
    // non-invariant: segment size chosen from this call's shape (prefill: one
    // segment; calls with fewer workgroups than CUs, i.e. small decode batches:
    // enough segments for ~1024 workgroups), so the same query meets different
    // reduction trees in different calls.  (Splitting calls of 256-1023 workgroups
    // measured slower: B = 64 decode 2.78 -> 2.99 ms.)
    const bool fast_split = c->n_tiles * g.n_kv_heads < 256;
    int max_pos = 0;
    for (int i = 0; i < c->n_seqs; ++i)
      max_pos = std::max(max_pos, c->h_pos0[i] + c->h_cu[i + 1] - c->h_cu[i] - 1);
    const int chunks = max_pos / KV_BLOCK + 1;
    int n_split = fast_split ? std::min({c->max_seg, chunks, (1024 + c->n_tiles * g.n_kv_heads - 1) /
                                                              (c->n_tiles * g.n_kv_heads)})
                             : 1;
    if (c->n_tokens > c->split_tokens || !c->attn_part_acc) n_split = 1;
    const int cps = (chunks + n_split - 1) / n_split;
    a.seg_keys = cps * KV_BLOCK;
    a.n_seg = n_split > 1 ? (max_pos / a.seg_keys + 1) : 0;
  } else {
    // a captured forward must not depend on positions: it launches every segment the
    // context can have; segments past a tile's last position return at once and the
    // merge stops at each row's own last segment, so the bits are the same
    const int nseg = c->graph_mode ? c->max_seg : c->batch_seg;
    const bool can_split = c->attn_part_acc && nseg > 1 && c->n_tokens <= c->split_tokens;
    const bool want_split = g.attn_split_mode == 2 || (g.attn_split_mode == 0 && few_tiles);
    a.n_seg = (can_split && want_split) ? nseg : 0;
  }
  a.part_acc = c->attn_part_acc;
  a.part_ml = c->attn_part_ml;
  // every tile at most 16 rows (one wave's worth) and fewer workgroups than CUs (small
  // decode batches, where each chunk's loads would otherwise wait a memory latency):
  // the unsplit schedule with two chunks in flight.  Measured, same box: B = 1 decode
  // step 1.752 -> 1.727 ms; at B = 64 (512 workgroups) its two extra clamped chunk
  // loads per tile cost more than they hide (2.77 -> 2.83 ms), so it stays off there
  int max_q = 0;
  for (int i = 0; i < c->n_seqs; ++i) max_q = std::max(max_q, c->h_cu[i + 1] - c->h_cu[i]);
  a.dsplit = max_q * (g.n_q_heads / g.n_kv_heads) <= 16;
  a.pf2 = a.dsplit && c->n_tiles * g.n_kv_heads < 256;
  // a captured forward is replayed with other positions, so it keeps the general kernel
  a.one_seg = !c->graph_mode && a.n_seg == 0 && c->batch_max_pos < a.seg_keys;
  HIP_TRY(c, launch_attention(a, s));
  return BCI_OK;
}

static bci_status gemm_checked(bci_ctx* c, const void* A, const int32_t* rows, const void* W, void* C,
                               int M, int N, int K, int epi, hipStream_t s) {
  // non-invariant mode: split-K with atomics where it beats the invariant schedules --
  // between the skinny range and 256 rows, for long contractions (K >= 4096: the down
  // projection, 114 -> 50-71 us at 160-256 rows); with K = 2048 the zero-fill and
  // epilogue launches cost more than the split gains (e.g. QKV 42 -> 78-125 us), and on the
  // skinny schedule too (decode step B = 1 1.76 -> 2.05 ms), so those keep the same kernels
  if (c->cfg.mode == BCI_MODE_FAST && !rows && M > SKINNY_MAX_M && M <= FAST_SPLITK_MAX_M &&
      N <= c->splitk_max_n && K >= 4096 && !gemm_prefers_skinny(M, N, K, epi, false)) {
    HIP_TRY(c, launch_gemm_splitk(A, W, C, M, N, K, epi, c->splitk_ws, s));
    return BCI_OK;
  }
  HIP_TRY(c, launch_gemm(A, rows, W, C, M, N, K, epi, s));
  return BCI_OK;
}

bci_status bci_op_embed(bci_ctx* c, const void* E, void* r, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_embed")) return st;
  if (!E || !r) return fail(c, BCI_E_INVALID, "op_embed: null pointer");
  HIP_TRY(c, launch_embed(c->meta + c->o_tok, E, r, c->n_tokens, c->cfg.hidden, S(stream)));
  return BCI_OK;
}

bci_status bci_op_add_rmsnorm(bci_ctx* c, const void* a, void* r, void* h, const void* g, int32_t rows,
                              int32_t cols, float eps, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!r || !h || !g || rows < 0) return fail(c, BCI_E_INVALID, "op_add_rmsnorm: null pointer or rows < 0");
  if (cols < 8 || cols % 8 || cols > 8192) return fail(c, BCI_E_INVALID, "op_add_rmsnorm: cols %d", cols);
  HIP_TRY(c, launch_add_rmsnorm(a, r, r, h, g, nullptr, nullptr, rows, cols, eps, S(stream)));
  return BCI_OK;
}

bci_status bci_op_gemm_bf16(bci_ctx* c, const void* A, const void* W, void* C, int32_t M, int32_t N,
                            int32_t K, int32_t epi, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!A || !W || !C || M < 0 || N < 1 || K < 1) return fail(c, BCI_E_INVALID, "op_gemm: bad pointer or shape");
  if (K % GEMM_BK) return fail(c, BCI_E_INVALID, "op_gemm: K %d not a multiple of %d", K, GEMM_BK);
  if (epi == BCI_EPI_SILU_MUL) {
    if (N % 256) return fail(c, BCI_E_INVALID, "op_gemm: SILU_MUL needs N = 2*I with I %% 128 == 0 (N=%d)", N);
  } else if (epi == BCI_EPI_BF16 || epi == BCI_EPI_F32) {
    // any N: columns past the last full 128-column tile are masked
  } else {
    return fail(c, BCI_E_INVALID, "op_gemm: unknown epilogue %d", epi);
  }
  // the operand copies are 16-byte loads at row offsets of K * 2 bytes
  if (!aligned16(A) || !aligned16(W)) return fail(c, BCI_E_INVALID, "op_gemm: A and W must be 16-byte aligned");
  // buffer descriptors cover 2 GiB from a tile's first row: the SiLU form reads its up
  // rows N / 2 rows past its gate rows, and the skinny schedule reads all M rows of A
  const size_t row_bytes = (size_t)K * 2;
  if ((epi == BCI_EPI_SILU_MUL && (size_t)(N / 2 + 256) * row_bytes > (size_t)INT32_MAX) ||
      (size_t)(M < 512 ? M : 512) * row_bytes > (size_t)INT32_MAX || 256 * row_bytes > (size_t)INT32_MAX)
    return fail(c, BCI_E_INVALID, "op_gemm: operand rows beyond the 2 GiB a copy descriptor covers (N %d, K %d)",
                N, K);
  return gemm_checked(c, A, nullptr, W, C, M, N, K, epi, S(stream));
}

bci_status bci_op_gemm_bf16_ksplit(bci_ctx* c, const void* A, const void* W, void* C, int32_t M, int32_t N,
                                   int32_t K, int32_t k_split, int32_t epi, float* workspace, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!A || !W || !C || !workspace || M < 0 || N < 1 || K < 1)
    return fail(c, BCI_E_INVALID, "op_gemm_ksplit: bad pointer or shape");
  if (K % GEMM_BK || k_split < GEMM_BK || k_split % GEMM_BK)
    return fail(c, BCI_E_INVALID, "op_gemm_ksplit: K %d and k_split %d must be multiples of %d", K, k_split,
                GEMM_BK);
  if (epi != BCI_EPI_BF16 && epi != BCI_EPI_F32)
    return fail(c, BCI_E_INVALID, "op_gemm_ksplit: epilogue %d (BF16 or F32 only)", epi);
  if (!aligned16(A) || !aligned16(W)) return fail(c, BCI_E_INVALID, "op_gemm_ksplit: A and W must be 16-byte aligned");
  HIP_TRY(c, launch_gemm_ksplit(A, W, C, M, N, K, k_split, epi, workspace, S(stream)));
  return BCI_OK;
}

bci_status bci_op_rope_kv_write(bci_ctx* c, const void* qkv, void* q_out, int32_t layer, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_rope_kv_write")) return st;
  if (!qkv || !q_out || layer < 0 || layer >= c->cfg.n_layers)
    return fail(c, BCI_E_INVALID, "op_rope_kv_write: null pointer or layer %d", layer);
  if (!aligned16(qkv) || !aligned16(q_out))
    return fail(c, BCI_E_INVALID, "op_rope_kv_write: qkv and q_out must be 16-byte aligned");
  return op_rope(c, qkv, q_out, layer, S(stream));
}

bci_status bci_op_kv_gather_dequant(bci_ctx* c, int32_t seq, int32_t n_pos, int32_t layer, void* k_out,
                                    void* v_out, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_kv_gather_dequant")) return st;
  if (seq < 0 || seq >= c->n_seqs || layer < 0 || layer >= c->cfg.n_layers || !k_out || !v_out)
    return fail(c, BCI_E_INVALID, "op_kv_gather_dequant: bad seq/layer/pointer");
  const int hi = c->h_pos0[seq] + c->h_cu[seq + 1] - c->h_cu[seq];  // positions known to the batch
  if (n_pos < 0 || n_pos > hi)
    return fail(c, BCI_E_INVALID, "op_kv_gather_dequant: n_pos %d outside [0, %d]", n_pos, hi);
  const auto& g = c->cfg;
  HIP_TRY(c, launch_kv_gather(kv_layer(c, layer), c->meta + c->o_btab + (size_t)seq * c->max_blocks, n_pos,
                              g.n_kv_heads, g.head_dim, g.kv_dtype == BCI_KV_FP8_E4M3, k_out, v_out,
                              S(stream)));
  return BCI_OK;
}

bci_status bci_op_attention(bci_ctx* c, const void* q, int32_t layer, void* o, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_attention")) return st;
  if (!q || !o || layer < 0 || layer >= c->cfg.n_layers)
    return fail(c, BCI_E_INVALID, "op_attention: null pointer or layer %d", layer);
  return op_attn(c, q, o, layer, S(stream));
}

// ------------------------------------------------------- backward pieces

bci_status bci_op_transpose_bf16(bci_ctx* c, const void* src, void* dst, int32_t R, int32_t C, int32_t ld_dst,
                                 void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!src || !dst || R < 0 || C < 0 || C % 8 || ld_dst < R || ld_dst % 8 || !aligned16(src) || !aligned16(dst))
    return fail(c, BCI_E_INVALID, "op_transpose_bf16: bad pointer or shape (C and ld_dst multiples of 8, "
                                  "ld_dst >= R, 16-byte aligned)");
  HIP_TRY(c, launch_transpose_bf16(src, dst, R, C, ld_dst, S(stream)));
  return BCI_OK;
}

bci_status bci_op_add_rmsnorm_backward(bci_ctx* c, const void* r, const void* g, const void* dh,
                                       const void* dr_in, void* dr, float* rstd, float* dg, int32_t rows,
                                       int32_t cols, float eps, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!r || !g || !dh || !dr || !rstd || !dg || rows < 0 || cols < 8 || cols > 8192 || cols % 8)
    return fail(c, BCI_E_INVALID, "op_add_rmsnorm_backward: bad pointer or shape");
  if (rows > c->cfg.max_tokens_per_call)
    return fail(c, BCI_E_WORKSPACE, "op_add_rmsnorm_backward: rows %d > max_tokens_per_call %d", rows,
                c->cfg.max_tokens_per_call);
  HIP_TRY(c, launch_rmsnorm_backward(r, g, dh, dr_in, dr, rstd, dg, c->bw_part, rows, cols, eps, S(stream)));
  return BCI_OK;
}

bci_status bci_op_silu_mul_backward(bci_ctx* c, const void* gu, const void* dact, void* dgu, int32_t rows,
                                    int32_t inter, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!gu || !dact || !dgu || rows < 0 || inter < 1)
    return fail(c, BCI_E_INVALID, "op_silu_mul_backward: bad pointer or shape");
  HIP_TRY(c, launch_silu_mul_backward(gu, dact, dgu, rows, inter, S(stream)));
  return BCI_OK;
}

bci_status bci_op_rope_backward(bci_ctx* c, const void* dq, const void* dk, const void* dv, void* dqkv,
                                void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_rope_backward")) return st;
  if (!dq || !dk || !dv || !dqkv) return fail(c, BCI_E_INVALID, "op_rope_backward: null pointer");
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dqkv))
    return fail(c, BCI_E_INVALID, "op_rope_backward: all tensors must be 16-byte aligned");
  const auto& g = c->cfg;
  HIP_TRY(c, launch_rope_backward(dq, dk, dv, dqkv, c->meta + c->o_pos, c->rope_cos, c->rope_sin, c->n_tokens,
                                  g.n_q_heads, g.n_kv_heads, g.head_dim, S(stream)));
  return BCI_OK;
}

bci_status bci_op_logprob_backward_dz(bci_ctx* c, const float* z, const int32_t* ids, const float* gout,
                                      int32_t M, int32_t V, void* dz, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!z || !ids || !gout || !dz || M < 0 || V < 1)
    return fail(c, BCI_E_INVALID, "op_logprob_backward_dz: bad pointer or shape");
  HIP_TRY(c, launch_logprob_dz(z, ids, gout, dz, M, V, S(stream)));
  return BCI_OK;
}

bci_status bci_op_attention_backward(bci_ctx* c, const void* q, const void* k, const void* v,
                                     const void* o, const void* dout, int32_t L, void* dq, void* dk,
                                     void* dv, float* workspace, void* stream) {
  if (!c) return BCI_E_INVALID;
  const auto& g = c->cfg;
  if (!q || !k || !v || !o || !dout || !dq || !dk || !dv || L < 0)
    return fail(c, BCI_E_INVALID, "op_attention_backward: bad pointer or length");
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(p)) return fail(c, BCI_E_INVALID, "op_attention_backward: tensors must be 16-byte aligned");
  if (L > g.max_tokens_per_call)
    return fail(c, BCI_E_WORKSPACE, "op_attention_backward: L %d > max_tokens_per_call %d", L,
                g.max_tokens_per_call);
  AttnBwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.lse = c->ab_lse;
  a.dsum = c->ab_dsum;
  if (workspace && !aligned16(workspace))
    return fail(c, BCI_E_INVALID, "op_attention_backward: workspace must be 16-byte aligned");
  a.part = workspace;
  a.L = L;
  a.nq = g.n_q_heads;
  a.nkv = g.n_kv_heads;
  a.d = g.head_dim;
  a.scale = (float)(1.0 / std::sqrt((double)g.head_dim));
  a.scale_log2 = (float)(1.0 / std::sqrt((double)g.head_dim) * 1.4426950408889634);
  HIP_TRY(c, launch_attention_backward(a, S(stream)));
  return BCI_OK;
}

// ------------------------------------------------------- sparse attention

static bci_status check_index_cache(bci_ctx* c, const char* who, int dim, const void* codes,
                                    const float* scales, int32_t n_index_blocks) {
  if (dim != 64 && dim != 128) return fail(c, BCI_E_INVALID, "%s: index_dim %d is not 64 or 128", who, dim);
  if (!codes || !scales) return fail(c, BCI_E_INVALID, "%s: null index cache", who);
  if (!aligned16(codes) || !aligned16(scales))
    return fail(c, BCI_E_INVALID, "%s: index cache buffers must be 16-byte aligned", who);
  if (n_index_blocks < c->n_blocks)
    return fail(c, BCI_E_INVALID, "%s: index cache has %d blocks, the bound KV cache %d", who,
                n_index_blocks, c->n_blocks);
  return BCI_OK;
}

bci_status bci_op_index_key_write(bci_ctx* c, const void* kidx, int32_t index_dim, void* icodes,
                                  float* iscale, int32_t n_index_blocks, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_index_key_write")) return st;
  if (bci_status st = check_index_cache(c, "op_index_key_write", index_dim, icodes, iscale, n_index_blocks))
    return st;
  if (!kidx || !aligned16(kidx)) return fail(c, BCI_E_INVALID, "op_index_key_write: kidx null or unaligned");
  HIP_TRY(c, launch_index_key_write(kidx, c->meta + c->o_slot, icodes, iscale, c->n_tokens, index_dim,
                                    S(stream)));
  return BCI_OK;
}

bci_status bci_op_index_scores(bci_ctx* c, const void* qidx, const float* w, int32_t index_heads,
                               int32_t index_dim, const void* icodes, const float* iscale,
                               int32_t n_index_blocks, float* scores, int64_t score_stride,
                               int32_t schedule, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_index_scores")) return st;
  if (bci_status st = check_index_cache(c, "op_index_scores", index_dim, icodes, iscale, n_index_blocks))
    return st;
  if (index_heads != 16 && index_heads != 32 && index_heads != 64)
    return fail(c, BCI_E_INVALID, "op_index_scores: index_heads %d is not 16, 32 or 64", index_heads);
  if (!qidx || !w || !scores || !aligned16(qidx) || !aligned16(scores))
    return fail(c, BCI_E_INVALID, "op_index_scores: null or unaligned qidx/w/scores");
  if (score_stride < (int64_t)c->batch_max_pos + 1 || score_stride % 4)
    return fail(c, BCI_E_INVALID, "op_index_scores: score_stride %lld must be a multiple of 4 and >= %d",
                (long long)score_stride, c->batch_max_pos + 1);
  if (schedule < 0 || schedule > 2) return fail(c, BCI_E_INVALID, "op_index_scores: schedule %d", schedule);
  IdxArgs a{};
  a.q = static_cast<const uint16_t*>(qidx);
  a.w = w;
  a.codes = static_cast<const uint8_t*>(icodes);
  a.scales = iscale;
  a.block_table = c->meta + c->o_btab;
  a.tok_pos = c->meta + c->o_pos;
  a.tok_seq = c->meta + c->o_tseq;
  a.tiles = c->meta + c->o_itiles;
  a.scores = scores;
  a.stride = (size_t)score_stride;
  a.T = c->n_tokens;
  a.heads = index_heads;
  a.dim = index_dim;
  a.max_blocks = c->max_blocks;
  a.n_tiles = c->n_itiles;
  a.max_pos = c->batch_max_pos;
  // the two schedules compute the same chain per (token, key); staging pays off when
  // several query tokens of a sequence share each key block
  const bool staged = schedule == 2 || (schedule == 0 && c->n_tokens >= 2 * c->n_seqs);
  HIP_TRY(c, launch_index_scores(a, staged, S(stream)));
  return BCI_OK;
}

bci_status bci_op_sparse_topk(bci_ctx* c, const float* scores, int64_t score_stride, int32_t topk,
                              int32_t* sel, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_sparse_topk")) return st;
  if (!scores || !sel || !aligned16(scores))
    return fail(c, BCI_E_INVALID, "op_sparse_topk: null or unaligned scores/sel");
  if (topk < 1) return fail(c, BCI_E_INVALID, "op_sparse_topk: topk %d < 1", topk);
  if (score_stride < (int64_t)c->batch_max_pos + 1 || score_stride % 4)
    return fail(c, BCI_E_INVALID, "op_sparse_topk: score_stride %lld must be a multiple of 4 and >= %d",
                (long long)score_stride, c->batch_max_pos + 1);
  HIP_TRY(c, launch_sparse_topk(scores, (size_t)score_stride, c->meta + c->o_pos, c->n_tokens, topk, sel,
                                S(stream)));
  return BCI_OK;
}

bci_status bci_op_sparse_attention(bci_ctx* c, const void* q, int32_t layer, const int32_t* sel,
                                   int32_t topk, void* o, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_sparse_attention")) return st;
  const auto& g = c->cfg;
  if (!q || !o || !sel || layer < 0 || layer >= g.n_layers)
    return fail(c, BCI_E_INVALID, "op_sparse_attention: null pointer or layer %d", layer);
  if (!aligned16(q) || !aligned16(o))
    return fail(c, BCI_E_INVALID, "op_sparse_attention: q and o must be 16-byte aligned");
  if (g.kv_dtype != BCI_KV_FP8_E4M3)
    return fail(c, BCI_E_UNSUPPORTED, "op_sparse_attention: needs an FP8 KV cache");
  if (c->group > 16)
    return fail(c, BCI_E_UNSUPPORTED, "op_sparse_attention: GQA group %d > 16", c->group);
  if (topk < 64 || topk > SPARSE_MAX_K || topk % 64)
    return fail(c, BCI_E_INVALID, "op_sparse_attention: topk %d must be a multiple of 64 in [64, %d]", topk,
                SPARSE_MAX_K);
  SparseAttnArgs a{};
  a.q = q;
  a.o = o;
  a.kv = kv_layer(c, layer);
  a.sel = sel;
  a.block_table = c->meta + c->o_btab;
  a.tok_pos = c->meta + c->o_pos;
  a.tok_seq = c->meta + c->o_tseq;
  a.T = c->n_tokens;
  a.K = topk;
  a.max_blocks = c->max_blocks;
  a.nq = g.n_q_heads;
  a.nkv = g.n_kv_heads;
  a.d = g.head_dim;
  a.scale_log2 = (float)(1.0 / std::sqrt((double)g.head_dim) * 1.4426950408889634);
  HIP_TRY(c, launch_sparse_attention(a, S(stream)));
  return BCI_OK;
}

bci_status bci_op_gather_scored(bci_ctx* c, const void* src, int32_t cols, void* out, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (bci_status st = need_batch(c, "op_gather_scored")) return st;
  if (!src || !out || cols < 8 || cols % 8) return fail(c, BCI_E_INVALID, "op_gather_scored: bad args");
  HIP_TRY(c, launch_gather_rows(src, c->meta + c->o_srow, out, c->n_scored, cols, S(stream)));
  return BCI_OK;
}

bci_status bci_op_lmhead_logprob(bci_ctx* c, const void* hf, const void* E, const int32_t* ids, int32_t M,
                                 int32_t H, int32_t V, float* lp, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!hf || !E || !ids || !lp || M < 0 || V < 1 || H < 64 || H % GEMM_BK)
    return fail(c, BCI_E_INVALID, "op_lmhead_logprob: bad pointer or shape");
  if (!aligned16(hf) || !aligned16(E))
    return fail(c, BCI_E_INVALID, "op_lmhead_logprob: hf and E must be 16-byte aligned");
  if (M > c->cfg.max_scored_per_call)
    return fail(c, BCI_E_WORKSPACE, "op_lmhead_logprob: M %d > max_scored_per_call %d", M,
                c->cfg.max_scored_per_call);
  if ((V + LM_CHUNK - 1) / LM_CHUNK > c->n_chunks)
    return fail(c, BCI_E_WORKSPACE, "op_lmhead_logprob: vocab %d larger than the context's %d", V, c->cfg.vocab);
  HIP_TRY(c, launch_lmhead_partials(hf, nullptr, E, ids, M, V, H, c->part_m, c->part_s, c->zid, S(stream)));
  HIP_TRY(c, launch_lmhead_combine(c->part_m, c->part_s, c->zid, ids, M, V, lp, S(stream)));
  return BCI_OK;
}

// ------------------------------------------------------------ MoE

bci_status bci_op_moe_topk(bci_ctx* c, const float* logits, int32_t T, int32_t* ids, float* w,
                           void* stream) {
  if (!c) return BCI_E_INVALID;
  const auto& g = c->cfg;
  if (g.n_experts == 0) return fail(c, BCI_E_STATE, "op_moe_topk: the context has no MoE layer");
  if (!logits || !ids || !w || T < 0) return fail(c, BCI_E_INVALID, "op_moe_topk: bad pointer or T");
  if (T > g.max_tokens_per_call)
    return fail(c, BCI_E_WORKSPACE, "op_moe_topk: T %d > max_tokens_per_call %d", T, g.max_tokens_per_call);
  HIP_TRY(c, launch_moe_topk(logits, T, g.n_experts, g.top_k, ids, w, S(stream)));
  return BCI_OK;
}

bci_status bci_op_moe_forward(bci_ctx* c, const void* h, const int32_t* ids, const float* w, int32_t T,
                              const void* wgu, const void* wd, const void* swgu, const void* swd, void* out,
                              void* stream) {
  if (!c) return BCI_E_INVALID;
  const auto& g = c->cfg;
  if (g.n_experts == 0) return fail(c, BCI_E_STATE, "op_moe_forward: the context has no MoE layer");
  if (!h || !ids || !w || !wgu || !wd || !out || T < 0)
    return fail(c, BCI_E_INVALID, "op_moe_forward: null pointer or T < 0");
  if ((g.n_shared_experts > 0) != (swgu && swd))
    return fail(c, BCI_E_INVALID, "op_moe_forward: shared-expert weights must match n_shared_experts");
  if (T > g.max_tokens_per_call)
    return fail(c, BCI_E_WORKSPACE, "op_moe_forward: T %d > max_tokens_per_call %d", T, g.max_tokens_per_call);
  if (!aligned16(out)) return fail(c, BCI_E_INVALID, "op_moe_forward: out must be 16-byte aligned");
  if (T == 0) return BCI_OK;
  const hipStream_t s = S(stream);
  const int H = g.hidden, I = g.expert_intermediate, E = g.n_experts, k = g.top_k, P = T * k;
  const int max_mt = (P + GEMM_BM - 1) / GEMM_BM + E;
  HIP_TRY(c, launch_moe_sort(ids, P, E, c->moe_counts, c->moe_offsets, c->moe_perm, c->moe_inv, c->moe_tiles,
                             c->moe_ntiles, s));
  // a token picks an expert at most once, so no expert gets more than T rows
  HIP_TRY(c, launch_gemm_grouped(h, c->moe_perm, k, wgu, (size_t)2 * I * H, c->moe_act, c->moe_tiles,
                                 c->moe_ntiles, max_mt, T, 2 * I, H, EPI_SILU, s));
  HIP_TRY(c, launch_gemm_grouped(c->moe_act, nullptr, 1, wd, (size_t)H * I, c->moe_y, c->moe_tiles,
                                 c->moe_ntiles, max_mt, T, H, I, EPI_BF16, s));
  if (swgu) {
    HIP_TRY(c, launch_gemm(h, nullptr, swgu, c->moe_act_s, T, 2 * I, H, EPI_SILU, s));
    HIP_TRY(c, launch_gemm(c->moe_act_s, nullptr, swd, c->moe_y_s, T, H, I, EPI_BF16, s));
  }
  HIP_TRY(c, launch_moe_combine(c->moe_y, swgu ? c->moe_y_s : nullptr, ids, w, c->moe_inv, T, k, E, H, out, s));
  return BCI_OK;
}

// ------------------------------------------------------------ forward

static bci_status forward_impl(bci_ctx* c, float* lp, hipStream_t s);

bci_status bci_forward_logprobs(bci_ctx* c, float* lp, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!c->weights_bound) return fail(c, BCI_E_STATE, "forward: bind weights first");
  if (bci_status st = need_batch(c, "forward")) return st;
  if (c->n_scored && !lp) return fail(c, BCI_E_INVALID, "forward: null logprob output");
  HIP_TRY(c, hipSetDevice(c->device));
  return forward_impl(c, lp, S(stream));
}

static bci_status forward_impl(bci_ctx* c, float* lp, hipStream_t s) {
  const auto& g = c->cfg;
  const int T = c->n_tokens, H = g.hidden;
  const void* E = c->w[0];
  // layer 0 norm: residual = E[token] (exact copy), no add
  HIP_TRY(c, launch_add_rmsnorm(nullptr, nullptr, c->bufR, c->bufH, c->w[1], c->meta + c->o_tok, E, T, H,
                                g.rms_eps, s));
  // Calls on the tiled GEMM schedule (more rows than the skinny one takes, and in the
  // non-invariant mode more than its split-K range) fuse RoPE and the KV write into the
  // QKV epilogue and the residual add into the O and down epilogues (the norm after
  // them then only normalises); the bits are those of the unfused op sequence.
  const bool tiled = T > SKINNY_MAX_M && (g.mode != BCI_MODE_FAST || T > FAST_SPLITK_MAX_M);
  // the non-invariant mode runs the tiled-range projections (QKV, O, down) on the vendor
  // GEMM, with RoPE and the residual adds in their own kernels
  const bool vendor = g.mode == BCI_MODE_FAST && tiled && c->vg != nullptr;
  // calls of at most 4 tokens (latency-bound decode) fuse RoPE into the skinny QKV
  // schedule too, for bf16 caches; above that its two weight streams per wave (half the
  // waves of the plain skinny GEMM) cost about what the launch saves (up to 128 tokens,
  // same box: B = 64 decode step 2.559 vs 2.560 ms, rollout caps 8 / 32 / 128 -0.3 /
  // -1.0 / +1.6 %)
  const bool fuse_rope = g.head_dim == 128 && c->qkv_w % GEMM_BN == 0 && !(vendor && FAST_VENDOR_QKV) &&
                         (tiled || (T <= 4 && g.kv_dtype != BCI_KV_FP8_E4M3 && H % 512 == 0));
  // calls of at most 4 tokens (decode) fold the norms into the GEMMs after them: the O
  // and down projections add into the residual in their epilogue and the QKV and gate_up
  // projections normalise their A rows themselves (launch_gemm_norm), so of the add+RMSNorm
  // launches only the embedding's and the final one remain; the bits are unchanged
  const bool fuse_norm = !tiled && T <= 4 && H % 512 == 0 && H <= 2048;
  const bool vendor_od = vendor && FAST_VENDOR_OD;
  const bool fuse_add = (tiled && H % GEMM_BN == 0 && !vendor_od) || fuse_norm;
  auto vgemm = [&](const void* A, const void* W, void* C, int N, int K) -> bci_status {
    if (!vendor_gemm(c->vg, A, W, C, T, N, K, s))
      return gemm_checked(c, A, nullptr, W, C, T, N, K, EPI_BF16, s);
    return BCI_OK;
  };
  // the O or down projection, into bufX or (fused) added into the residual bufR
  auto project = [&](const void* A, const void* W, int K) -> bci_status {
    if (fuse_add) {
      HIP_TRY(c, launch_gemm(A, nullptr, W, c->bufR, T, H, K, EPI_ADD, s));
      return BCI_OK;
    }
    if (vendor_od) return vgemm(A, W, c->bufX, H, K);
    return gemm_checked(c, A, nullptr, W, c->bufX, T, H, K, EPI_BF16, s);
  };
  const void* addend = fuse_add ? nullptr : c->bufX;  // what the norms still add
  for (int l = 0; l < g.n_layers; ++l) {
    const void* const* lw = &c->w[1 + 6 * l];  // attn_norm, wqkv, wo, mlp_norm, wgu, wd
    // the layer's A rows: bufH, or normalised inside the QKV GEMM from the residual
    const bool qkv_norm = fuse_norm && l > 0;
    if (l > 0 && !qkv_norm)
      HIP_TRY(c, launch_add_rmsnorm(addend, c->bufR, c->bufR, c->bufH, lw[0], nullptr, nullptr, T, H,
                                    g.rms_eps, s));
    if (fuse_rope && qkv_norm) {
      HIP_TRY(c, launch_gemm_qkv_rope_norm(c->bufR, lw[0], g.rms_eps, lw[1], T, c->qkv_w, H, c->bufQ,
                                           c->meta + c->o_pos, c->meta + c->o_slot, c->rope_cos, c->rope_sin,
                                           kv_layer(c, l), g.n_q_heads, g.n_kv_heads, s));
    } else if (qkv_norm) {
      HIP_TRY(c, launch_gemm_norm(c->bufR, lw[0], g.rms_eps, lw[1], c->bufQKV, T, c->qkv_w, H, EPI_BF16, s));
      if (bci_status st = op_rope(c, c->bufQKV, c->bufQ, l, s)) return st;
    } else if (fuse_rope) {
      // tiled QKV GEMM with RoPE and the KV write in its epilogue: the same bits as the
      // GEMM into bufQKV followed by op_rope (the op-by-op path), without bufQKV
      HIP_TRY(c, launch_gemm_qkv_rope(c->bufH, lw[1], T, c->qkv_w, H, c->bufQ, c->meta + c->o_pos,
                                      c->meta + c->o_slot, c->rope_cos, c->rope_sin, kv_layer(c, l),
                                      g.n_q_heads, g.n_kv_heads, g.kv_dtype == BCI_KV_FP8_E4M3, s));
    } else {
      if (vendor && FAST_VENDOR_QKV) {
        if (bci_status st = vgemm(c->bufH, lw[1], c->bufQKV, c->qkv_w, H)) return st;
      } else if (bci_status st = gemm_checked(c, c->bufH, nullptr, lw[1], c->bufQKV, T, c->qkv_w, H, EPI_BF16, s)) {
        return st;
      }
      if (bci_status st = op_rope(c, c->bufQKV, c->bufQ, l, s)) return st;
    }
    if (bci_status st = op_attn(c, c->bufQ, c->bufO, l, s)) return st;
    if (bci_status st = project(c->bufO, lw[2], c->qd)) return st;
    if (!fuse_norm)
      HIP_TRY(c, launch_add_rmsnorm(addend, c->bufR, c->bufR, c->bufH, lw[3], nullptr, nullptr, T, H,
                                    g.rms_eps, s));
    const bool prof = c->prof_on && !c->graph_mode && c->prof_n < c->prof_cap;
    if (c->prof_on && !c->graph_mode && !prof) ++c->prof_dropped;
    if (prof) HIP_TRY(c, hipEventRecord(c->prof_ev[2 * c->prof_n], s));
    if (fuse_norm) {
      HIP_TRY(c, launch_gemm_norm(c->bufR, lw[3], g.rms_eps, lw[4], c->bufACT, T, 2 * g.intermediate, H, EPI_SILU,
                                  s));
    } else if (bci_status st = gemm_checked(c, c->bufH, nullptr, lw[4], c->bufACT, T, 2 * g.intermediate, H,
                                            EPI_SILU, s)) {
      return st;
    }
    if (prof) {
      HIP_TRY(c, hipEventRecord(c->prof_ev[2 * c->prof_n + 1], s));
      c->prof_rows[c->prof_n++] = T;
    }
    if (bci_status st = project(c->bufACT, lw[5], g.intermediate)) return st;
  }
  HIP_TRY(c, launch_add_rmsnorm(addend, c->bufR, c->bufR, c->bufH, c->w[1 + 6 * g.n_layers], nullptr, nullptr,
                                T, H, g.rms_eps, s));
  if (c->n_scored) {
    HIP_TRY(c, launch_lmhead_partials(c->bufH, c->meta + c->o_srow, E, c->meta + c->o_sid, c->n_scored, g.vocab,
                                      H, c->part_m, c->part_s, c->zid, s));
    HIP_TRY(c, launch_lmhead_combine(c->part_m, c->part_s, c->zid, c->meta + c->o_sid, c->n_scored, g.vocab, lp,
                                     s));
  }
  return BCI_OK;
}

// ------------------------------------------------------------ captured forward

bci_status bci_forward_logprobs_graph(bci_ctx* c, float* lp, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!c->weights_bound) return fail(c, BCI_E_STATE, "forward_graph: bind weights first");
  if (bci_status st = need_batch(c, "forward_graph")) return st;
  if (c->n_scored && !lp) return fail(c, BCI_E_INVALID, "forward_graph: null logprob output");
  if (c->cfg.mode != BCI_MODE_INVARIANT)
    return fail(c, BCI_E_UNSUPPORTED, "forward_graph: only the invariant mode is captured");
  if (c->cfg.n_experts > 0)
    return fail(c, BCI_E_UNSUPPORTED, "forward_graph: the MoE layer is not captured");
  HIP_TRY(c, hipSetDevice(c->device));
  const hipStream_t s = S(stream);
  bci_ctx::Graph* hit = nullptr;
  for (auto& g : c->graphs)
    if (g.n_tokens == c->n_tokens && g.n_seqs == c->n_seqs && g.n_scored == c->n_scored &&
        g.n_tiles == c->n_tiles && g.max_blocks == c->max_blocks && g.epoch == c->bind_epoch)
      hit = &g;
  if (!hit) {
    // drop graphs of an older binding, then the least recently used beyond 16
    for (size_t i = 0; i < c->graphs.size();) {
      if (c->graphs[i].epoch != c->bind_epoch) {
        (void)hipGraphExecDestroy(c->graphs[i].exec);
        (void)hipGraphDestroy(c->graphs[i].graph);
        c->graphs.erase(c->graphs.begin() + i);
      } else {
        ++i;
      }
    }
    if (c->graphs.size() >= 16) {
      size_t lru = 0;
      for (size_t i = 1; i < c->graphs.size(); ++i)
        if (c->graphs[i].last_use < c->graphs[lru].last_use) lru = i;
      (void)hipGraphExecDestroy(c->graphs[lru].exec);
      (void)hipGraphDestroy(c->graphs[lru].graph);
      c->graphs.erase(c->graphs.begin() + lru);
    }
    if (!c->cap_stream) HIP_TRY(c, hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
    // the capture only records launches; the batch metadata it reads is uploaded by
    // bci_set_batch before every launch of the graph
    HIP_TRY(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
    c->graph_mode = true;
    const bci_status st = forward_impl(c, c->graph_lp, c->cap_stream);
    c->graph_mode = false;
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(c->cap_stream, &graph);
    if (st != BCI_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return hipfail(c, e, "hipStreamEndCapture");
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (ei != hipSuccess) {
      (void)hipGraphDestroy(graph);
      return hipfail(c, ei, "hipGraphInstantiate");
    }
    c->graphs.push_back({c->n_tokens, c->n_seqs, c->n_scored, c->n_tiles, c->max_blocks, c->bind_epoch,
                         graph, exec, 0});
    hit = &c->graphs.back();
  }
  hit->last_use = ++c->graph_clock;
  HIP_TRY(c, hipGraphLaunch(hit->exec, s));
  if (c->n_scored)
    HIP_TRY(c, hipMemcpyAsync(lp, c->graph_lp, (size_t)c->n_scored * 4, hipMemcpyDeviceToDevice, s));
  return BCI_OK;
}

int32_t bci_graph_count(const bci_ctx* c) { return c ? (int32_t)c->graphs.size() : 0; }

bci_status bci_graph_reset(bci_ctx* c) {
  if (!c) return BCI_E_INVALID;
  HIP_TRY(c, hipSetDevice(c->device));
  drop_graphs(c);
  return BCI_OK;
}

// ------------------------------------------------------------ profiling

bci_status bci_profile_begin(bci_ctx* c, int32_t capacity) {
  if (!c) return BCI_E_INVALID;
  if (capacity < 0) return fail(c, BCI_E_INVALID, "profile_begin: capacity %d < 0", capacity);
  if (capacity == 0) capacity = DEFAULT_PROFILE;
  HIP_TRY(c, hipSetDevice(c->device));
  // events are created here, outside any timed region; the ring only grows
  if (c->prof_ev.size() < 2 * (size_t)capacity) c->prof_ev.resize(2 * (size_t)capacity, nullptr);
  for (size_t i = 0; i < 2 * (size_t)capacity; ++i)
    if (!c->prof_ev[i]) HIP_TRY(c, hipEventCreate(&c->prof_ev[i]));
  c->prof_cap = capacity;
  c->prof_rows.assign(capacity, 0);
  c->prof_on = true;
  c->prof_n = 0;
  c->prof_dropped = 0;
  return BCI_OK;
}

bci_status bci_profile_end(bci_ctx* c, double* total_ms, int32_t* launches, int64_t* rows, int32_t* dropped) {
  if (!c || !total_ms || !launches || !rows || !dropped) return BCI_E_INVALID;
  c->prof_on = false;
  double tot = 0.0;
  int64_t m = 0;
  for (int i = 0; i < c->prof_n; ++i) {
    HIP_TRY(c, hipEventSynchronize(c->prof_ev[2 * i + 1]));
    float ms = 0.0f;
    HIP_TRY(c, hipEventElapsedTime(&ms, c->prof_ev[2 * i], c->prof_ev[2 * i + 1]));
    tot += ms;
    m += c->prof_rows[i];
  }
  *total_ms = tot;
  *launches = c->prof_n;
  *rows = m;
  *dropped = c->prof_dropped;
  return BCI_OK;
}

bci_status bci_measure_mfma_rate(int32_t device, int32_t random_operands, double* tflops) {
  if (!tflops) return BCI_E_INVALID;
  *tflops = 0.0;
  if (hipSetDevice(device) != hipSuccess) return BCI_E_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return BCI_E_HIP;
  const int blocks = 2 * prop.multiProcessorCount, iters = 100000;
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  bci_status st = BCI_E_HIP;
  if (hipMalloc(&out, (size_t)blocks * PROBE_BLOCK_THREADS * sizeof(float)) == hipSuccess &&
      hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
    // warm up (clocks settle), then time one launch of ~50 ms
    bool ok = launch_mfma_rate(out, blocks, iters / 2, random_operands, nullptr) == hipSuccess &&
              launch_mfma_rate(out, blocks, iters / 2, random_operands, nullptr) == hipSuccess &&
              hipEventRecord(e0, nullptr) == hipSuccess &&
              launch_mfma_rate(out, blocks, iters, random_operands, nullptr) == hipSuccess &&
              hipEventRecord(e1, nullptr) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.0f;
    if (ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms > 0.0f) {
      const double flops = (double)blocks * (PROBE_BLOCK_THREADS / 64) * iters * 16 * 16384.0;
      *tflops = flops / (ms * 1e-3) / 1e12;
      st = BCI_OK;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  return st;
}

}  // extern "C"
