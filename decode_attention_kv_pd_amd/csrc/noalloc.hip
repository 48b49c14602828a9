// pd_attention_run_noalloc: pd_attention_run (optionally preceded by
// pd_kv_append) for callers that cannot allocate device memory.  The plan's
// tables and the split-KV partial results live in `scratch`, a static device
// array of kNoallocScratchBytes that every GPU the library runs on holds
// until the process ends; the call itself allocates nothing (no hipMalloc,
// no hipHostMalloc, no pinned staging block).
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// first call on a device looks up that device's address of the array with
// hipGetSymbolAddress (with the device current) and keeps it per device;
// only that address is handed to copies and kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_internal.hpp"
#include "pd_attn.h"

namespace {

constexpr size_t kNoallocScratchBytes = (size_t)PD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kNoallocScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (looked up once per device).
pd_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pdh::hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return pdh::set_error(PD_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return pdh::hip_error(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PD_OK;
}

}  // namespace

extern "C" {

pd_status pd_attention_run_noalloc(pd_plan_t plan, const void* q, void* kv_pool, const void* k_new,
                                   const void* v_new, float* out, float* lse, void* stream) {
  try {
    if (!plan) return pdh::set_error(PD_ERR_INVALID_ARG, "NULL plan");
    const pdh::PlanImage im = pdh::plan_image(plan);
    if (im.mla) return pdh::set_error(PD_ERR_INVALID_ARG, "an MLA plan: not supported by the no-allocation call");
    if ((k_new == nullptr) != (v_new == nullptr))
      return pdh::set_error(PD_ERR_INVALID_ARG, "k_new and v_new must both be given or both be NULL");
    if (im.ws_bytes > kNoallocScratchBytes)
      return pdh::set_error(PD_ERR_WORKSPACE, "the plan needs more device scratch than the no-allocation call's "
                                              "static buffer (PD_NOALLOC_SCRATCH_BYTES)");
    if (im.total_rows == 0) return PD_OK;
    if (!q || !kv_pool || !out) return pdh::set_error(PD_ERR_INVALID_ARG, "NULL q, pool or out");
    void* ws = nullptr;
    pd_status s = device_scratch(&ws);
    if (s != PD_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    // the tables come from the plan's host memory (pageable: the copy has read
    // them when it returns); the partial results need no clearing, every slot
    // is written before the merge reads it
    hipError_t e = hipMemcpyAsync(ws, im.tables, im.table_bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return pdh::hip_error(e, "table upload to the static scratch");
    if (k_new && (s = pdh::enqueue_append(plan, ws, kv_pool, k_new, v_new, stream)) != PD_OK) return s;
    return pdh::enqueue_attention(plan, ws, q, kv_pool, out, lse, stream);
  } catch (...) {
    return pdh::set_error(PD_ERR_HIP, "unexpected error in pd_attention_run_noalloc");
  }
}

}  // extern "C"
