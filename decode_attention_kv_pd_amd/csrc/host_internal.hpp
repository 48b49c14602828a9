// Host-side helpers shared by the C entry points of api.cpp and noalloc.hip.
// Not part of the public ABI (include/pd_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pd_attn.h"

namespace pdh {

// Records msg as the calling thread's last error (pd_last_error) and returns s.
pd_status set_error(pd_status s, const char* msg);
// PD_ERR_HIP with the runtime's message for e.
pd_status hip_error(hipError_t e, const char* what);

// The device tables of a plan as built on the host: table_bytes bytes at
// `tables` go to the start of a workspace of ws_bytes (the rest holds the
// split-KV partial results, written before they are read).
struct PlanImage {
  const void* tables;
  size_t table_bytes;
  size_t ws_bytes;
  bool mla;
  int32_t total_rows;
};
PlanImage plan_image(pd_plan_t plan);

// Launches of pd_kv_append and pd_attention_run over a workspace the plan's
// tables are (or will be, earlier on the same stream) uploaded to.  The
// arguments are checked by the caller.
pd_status enqueue_append(pd_plan_t plan, void* d_ws, void* kv_pool, const void* k_new, const void* v_new,
                         void* stream);
pd_status enqueue_attention(pd_plan_t plan, void* d_ws, const void* q, const void* kv_pool, float* out, float* lse,
                            void* stream);

}  // namespace pdh
