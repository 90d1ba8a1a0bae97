// bci_lmhead_logprob_noalloc: the lm_head + fp32 log-softmax + gather of
// bci_op_lmhead_logprob for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// It runs the same two kernels as bci_op_lmhead_logprob (per-256-column-chunk
// (max, sum exp) partials and z[id], then the fixed-order combine), so the bits
// are the same; only the partials live elsewhere: in `scratch`, a file-scope
// device array the loader places on every GPU the library runs on, held until
// the process ends.  Host code never passes `scratch` itself (its name is a
// host-side stand-in); the device address comes from hipGetSymbolAddress, looked
// up once per device on the first call made with that device current.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/bci.h"
#include "kernels.h"

using namespace bci;

namespace {

// (row, chunk) pairs of partials the array holds, and the row limit (zid).
constexpr int64_t NOALLOC_PAIRS = BCI_LMHEAD_NOALLOC_MAX_PAIRS;
constexpr int NOALLOC_ROWS = BCI_LMHEAD_NOALLOC_MAX_ROWS;
constexpr int MAX_DEVICES = 64;

// [part_m: NOALLOC_PAIRS][part_s: NOALLOC_PAIRS][zid: NOALLOC_ROWS] fp32
static __device__ __align__(256) float scratch[2 * NOALLOC_PAIRS + NOALLOC_ROWS];

std::mutex g_lookup;
std::atomic<float*> g_ptr[MAX_DEVICES];

// Device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  float* p = g_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_lookup);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!q) return hipErrorInvalidSymbol;
      p = static_cast<float*>(q);
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" bci_status bci_lmhead_logprob_noalloc(const void* hf, const void* E, const int32_t* ids, int32_t M,
                                                 int32_t H, int32_t V, float* lp, void* stream) {
  if (!hf || !E || !ids || !lp || M < 0 || V < 1 || H < 64 || H % GEMM_BK) return BCI_E_INVALID;
  const int64_t chunks = (V + LM_CHUNK - 1) / LM_CHUNK;
  if (M > NOALLOC_ROWS || (int64_t)M * chunks > NOALLOC_PAIRS) return BCI_E_WORKSPACE;
  if (M == 0) return BCI_OK;
  float* base = nullptr;
  if (scratch_ptr(&base) != hipSuccess) return BCI_E_HIP;
  // partials packed for this call's M: chunk c of row i at c * M + i, as in the
  // context workspace; every (chunk, row) and every valid row's z[id] is written
  // before it is read, so nothing needs clearing between calls
  float* part_m = base;
  float* part_s = base + NOALLOC_PAIRS;
  float* zid = base + 2 * NOALLOC_PAIRS;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (launch_lmhead_partials(hf, nullptr, E, ids, M, V, H, part_m, part_s, zid, s) != hipSuccess) return BCI_E_HIP;
  if (launch_lmhead_combine(part_m, part_s, zid, ids, M, V, lp, s) != hipSuccess) return BCI_E_HIP;
  return BCI_OK;
}
