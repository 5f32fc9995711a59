// nq_quantize_kv_noalloc: quantize for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace -- the RoPE table, the frequencies, the
// counters and queues of the fp64 pass -- is `scratch`, a file-scope device
// array of kScratchBytes that each GPU holds until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/nq.h"
#include "nq_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's copy of `scratch` (host code never
// passes the array's name to a kernel: that is a host-side stand-in).  Looked
// up once per device, with that device current.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return NQ_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NQ_OK;
}

}  // namespace

extern "C" int nq_quantize_kv_noalloc(const nq_config* cfg, const void* k, const void* v,
                                      int64_t S, int32_t H, int64_t T,
                                      const int32_t* positions, const nq_packed* pk,
                                      const nq_packed* pv, void* stream) {
  // a config or shape that nq_workspace_bytes rejects gets its precise status
  // from the checks of the shared body; one that needs more than the scratch
  // array holds is rejected here, before anything is enqueued
  const size_t need = nq_workspace_bytes(cfg, S, H, T);
  if (need == 0)
    return nq::quantize_impl(cfg, k, v, S, H, T, positions, pk, pv, nullptr, 0, stream);
  if (need > kScratchBytes) return NQ_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_for_current_device(&ws);
  if (st != NQ_OK) return st;
  return nq::quantize_impl(cfg, k, v, S, H, T, positions, pk, pv, ws, kScratchBytes, stream);
}
