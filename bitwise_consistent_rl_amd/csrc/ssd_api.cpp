// C ABI of the chunked state-space layer (include/bci.h, "state-space layer").
// Host side only: validation, the per-call chunk tables, the launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/bci.h"
#include "kernels.h"

using namespace bci;

namespace {
constexpr int SSD_CHUNK = 64;
constexpr int SSD_HEAD_DIM = 64;
}  // namespace

struct bci_ssd {
  bci_ssd_config cfg{};
  int device = 0;
  std::string err;
  int max_inst = 0, max_done = 0;
  void* ws = nullptr;
  uint16_t* hprev = nullptr;
  int32_t* meta = nullptr;
  size_t meta_words = 0, o_seq = 0, o_inst = 0, o_done = 0;
  int32_t* stage = nullptr;
  hipEvent_t stage_ev = nullptr;
  bool stage_used = false;
  bool batch_valid = false;
  int n_seqs = 0, n_tokens = 0, n_inst = 0, n_done = 0;
  std::vector<int32_t> h_slot;
};

static bci_status sfail(bci_ssd* c, bci_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return st;
}

#define SSD_TRY(c, expr)                                                                   \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return sfail((c), BCI_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static size_t slot_state_bytes(const bci_ssd_config& g) {
  return (size_t)g.n_heads * SSD_HEAD_DIM * g.d_state * 4;
}
static size_t slot_chunk_bytes(const bci_ssd_config& g) {
  return (size_t)SSD_CHUNK * ((size_t)g.n_heads * SSD_HEAD_DIM * 2 + (size_t)g.n_groups * g.d_state * 2 +
                              (size_t)g.n_heads * 4);
}

extern "C" {

bci_status bci_ssd_create(const bci_ssd_config* cfg, int32_t device, bci_ssd** out) {
  if (!out) return BCI_E_INVALID;
  *out = nullptr;
  if (!cfg) return BCI_E_INVALID;
  const bci_ssd_config g = *cfg;
  if (g.head_dim != SSD_HEAD_DIM || (g.d_state != 64 && g.d_state != 128) || g.n_groups < 1 ||
      g.n_heads < 1 || g.n_heads % g.n_groups || g.max_tokens_per_call < 1 || g.max_seqs_per_call < 1)
    return BCI_E_INVALID;
  if (hipSetDevice(device) != hipSuccess) return BCI_E_HIP;
  bci_ssd* c = new bci_ssd();
  c->cfg = g;
  c->device = device;
  c->max_inst = g.max_tokens_per_call / SSD_CHUNK + 2 * g.max_seqs_per_call;
  c->max_done = g.max_tokens_per_call / SSD_CHUNK + g.max_seqs_per_call;
  c->o_seq = 0;
  c->o_inst = c->o_seq + 6 * (size_t)g.max_seqs_per_call;
  c->o_done = c->o_inst + 6 * (size_t)c->max_inst;
  c->meta_words = c->o_done + (size_t)c->max_done;
  const size_t hp = ((size_t)c->max_done * slot_state_bytes(g) / 2 + 255) / 256 * 256;  // bf16 states
  const size_t mw = (c->meta_words * 4 + 255) / 256 * 256;
  if (hipMalloc(&c->ws, hp + mw) != hipSuccess) {
    delete c;
    return BCI_E_WORKSPACE;
  }
  c->hprev = static_cast<uint16_t*>(c->ws);
  c->meta = reinterpret_cast<int32_t*>(static_cast<char*>(c->ws) + hp);
  if (hipHostMalloc((void**)&c->stage, c->meta_words * 4, hipHostMallocDefault) != hipSuccess ||
      hipEventCreateWithFlags(&c->stage_ev, hipEventDisableTiming) != hipSuccess) {
    bci_ssd_destroy(c);
    return BCI_E_WORKSPACE;
  }
  *out = c;
  return BCI_OK;
}

void bci_ssd_destroy(bci_ssd* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  if (c->stage_ev) (void)hipEventDestroy(c->stage_ev);
  if (c->stage) (void)hipHostFree(c->stage);
  if (c->ws) (void)hipFree(c->ws);
  delete c;
}

const char* bci_ssd_last_error(const bci_ssd* c) { return c ? c->err.c_str() : "null context"; }

uint64_t bci_ssd_slot_bytes(const bci_ssd* c, int32_t which) {
  if (!c) return 0;
  return which == 0 ? slot_state_bytes(c->cfg) : which == 1 ? slot_chunk_bytes(c->cfg) : 0;
}

bci_status bci_ssd_set_batch(bci_ssd* c, int32_t n_seqs, const int32_t* cu_q, const int32_t* pos0,
                             const int32_t* slot, void* stream) {
  if (!c) return BCI_E_INVALID;
  c->batch_valid = false;
  const auto& g = c->cfg;
  if (n_seqs < 1 || n_seqs > g.max_seqs_per_call)
    return sfail(c, BCI_E_WORKSPACE, "ssd_set_batch: n_seqs %d outside [1, %d]", n_seqs, g.max_seqs_per_call);
  if (!cu_q || !pos0 || !slot) return sfail(c, BCI_E_INVALID, "ssd_set_batch: null array");
  if (cu_q[0] != 0) return sfail(c, BCI_E_INVALID, "ssd_set_batch: cu_q must start at 0");
  for (int i = 0; i < n_seqs; ++i) {
    if (cu_q[i + 1] - cu_q[i] < 1) return sfail(c, BCI_E_INVALID, "ssd_set_batch: sequence %d is empty", i);
    if (pos0[i] < 0) return sfail(c, BCI_E_INVALID, "ssd_set_batch: pos0[%d] < 0", i);
    if (slot[i] < 0) return sfail(c, BCI_E_INVALID, "ssd_set_batch: slot[%d] < 0", i);
    for (int j = 0; j < i; ++j)
      if (slot[j] == slot[i]) return sfail(c, BCI_E_INVALID, "ssd_set_batch: slot %d used twice", slot[i]);
  }
  const int T = cu_q[n_seqs];
  if (T > g.max_tokens_per_call)
    return sfail(c, BCI_E_WORKSPACE, "ssd_set_batch: %d tokens > %d", T, g.max_tokens_per_call);
  if (c->stage_used) SSD_TRY(c, hipEventSynchronize(c->stage_ev));
  int32_t* h = c->stage;
  std::vector<int32_t> done;
  int n_inst = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int ql = cu_q[i + 1] - cu_q[i], p0 = pos0[i], pend = p0 + ql - 1;
    int32_t* sq = h + c->o_seq + 6 * i;
    sq[0] = cu_q[i];
    sq[1] = p0;
    sq[2] = ql;
    sq[3] = slot[i];
    sq[4] = (int32_t)done.size();
    sq[5] = 0;
    for (int ch = p0 / SSD_CHUNK; ch <= pend / SSD_CHUNK; ++ch) {
      if (n_inst >= c->max_inst) return sfail(c, BCI_E_WORKSPACE, "ssd_set_batch: too many chunks");
      int32_t* in = h + c->o_inst + 6 * n_inst;
      in[0] = i;
      in[1] = ch;
      in[2] = std::max(p0, ch * SSD_CHUNK);
      in[3] = std::min(pend, ch * SSD_CHUNK + SSD_CHUNK - 1);
      in[4] = -1;
      in[5] = 0;
      if (ch * SSD_CHUNK + SSD_CHUNK - 1 <= pend) {  // the chunk completes in this call
        if ((int)done.size() >= c->max_done) return sfail(c, BCI_E_WORKSPACE, "ssd_set_batch: too many chunks");
        in[4] = (int32_t)done.size();
        done.push_back(n_inst);
        ++sq[5];
      }
      ++n_inst;
    }
  }
  std::memcpy(h + c->o_done, done.data(), done.size() * 4);
  SSD_TRY(c, hipSetDevice(c->device));
  SSD_TRY(c, hipMemcpyAsync(c->meta, h, c->meta_words * 4, hipMemcpyHostToDevice,
                            reinterpret_cast<hipStream_t>(stream)));
  SSD_TRY(c, hipEventRecord(c->stage_ev, reinterpret_cast<hipStream_t>(stream)));
  c->stage_used = true;
  c->h_slot.assign(slot, slot + n_seqs);
  c->n_seqs = n_seqs;
  c->n_tokens = T;
  c->n_inst = n_inst;
  c->n_done = (int)done.size();
  c->batch_valid = true;
  return BCI_OK;
}

bci_status bci_ssd_forward(bci_ssd* c, const void* x, const float* dt, const float* A, const void* B,
                           const void* C, const float* D, float* state, void* chunk_buf, int32_t n_slots,
                           void* y, void* stream) {
  if (!c) return BCI_E_INVALID;
  if (!c->batch_valid) return sfail(c, BCI_E_STATE, "ssd_forward: no current batch (call bci_ssd_set_batch)");
  if (!x || !dt || !A || !B || !C || !D || !state || !chunk_buf || !y)
    return sfail(c, BCI_E_INVALID, "ssd_forward: null pointer");
  for (const void* p : {(const void*)x, (const void*)dt, (const void*)B, (const void*)C, (const void*)state,
                        (const void*)chunk_buf, (const void*)y})
    if (!al16(p)) return sfail(c, BCI_E_INVALID, "ssd_forward: tensors must be 16-byte aligned");
  for (int i = 0; i < c->n_seqs; ++i)
    if (c->h_slot[i] >= n_slots)
      return sfail(c, BCI_E_INVALID, "ssd_forward: slot %d outside [0, %d)", c->h_slot[i], n_slots);
  const auto& g = c->cfg;
  SsdArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.B = static_cast<const uint16_t*>(B);
  a.C = static_cast<const uint16_t*>(C);
  a.dt = dt;
  a.A = A;
  a.D = D;
  a.y = static_cast<uint16_t*>(y);
  char* cb = static_cast<char*>(chunk_buf);
  a.xb = reinterpret_cast<uint16_t*>(cb);
  a.Bb = reinterpret_cast<uint16_t*>(cb + (size_t)n_slots * SSD_CHUNK * g.n_heads * SSD_HEAD_DIM * 2);
  a.dtb = reinterpret_cast<float*>(cb + (size_t)n_slots * SSD_CHUNK *
                                            ((size_t)g.n_heads * SSD_HEAD_DIM * 2 + (size_t)g.n_groups * g.d_state * 2));
  a.state = state;
  a.hprev = c->hprev;
  a.seqs = c->meta + c->o_seq;
  a.inst = c->meta + c->o_inst;
  a.done = c->meta + c->o_done;
  a.heads = g.n_heads;
  a.groups = g.n_groups;
  a.N = g.d_state;
  a.n_seqs = c->n_seqs;
  a.n_inst = c->n_inst;
  a.n_done = c->n_done;
  SSD_TRY(c, hipSetDevice(c->device));
  SSD_TRY(c, launch_ssd(a, reinterpret_cast<hipStream_t>(stream)));
  return BCI_OK;
}

}  // extern "C"
