/* One step of the path driven from C through the C ABI alone (HIP runtime for
 * device memory; no PyTorch): plan, upload, append, attention, pack, unpack.
 *   c_step IN OUT
 * IN holds the batch as the GPU test writes it (int32 header and tables, then
 * float32 pool, q, k_new, v_new, then the pack / unpack page lists); OUT
 * receives out, lse, the pool after the step and the packed buffer. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <hip/hip_runtime_api.h>

#include "pd_attn.h"

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      exit(2);                                                             \
    }                                                                      \
  } while (0)
#define PD_OK_(x)                                                          \
  do {                                                                     \
    pd_status s_ = (x);                                                    \
    if (s_ != PD_OK) {                                                     \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, pd_status_string(s_), pd_last_error()); \
      exit(3);                                                             \
    }                                                                      \
  } while (0)

static void* read_n(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input\n");
    exit(4);
  }
  return p;
}

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: c_step IN OUT\n");
    return 1;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 1;
  int32_t* hdr = (int32_t*)read_n(f, 10 * sizeof(int32_t));
  float scale;
  if (fread(&scale, sizeof scale, 1, f) != 1) return 4;
  pd_attn_desc d;
  d.num_qo_heads = hdr[0]; d.num_kv_heads = hdr[1]; d.head_dim = hdr[2]; d.page_size = hdr[3];
  d.dtype = hdr[4]; d.causal = hdr[5]; d.sm_scale = scale;
  const int32_t B = hdr[6], num_pool_pages = hdr[7], n_pages = hdr[8], rows = hdr[9];
  if (d.dtype != PD_F32) return 5;
  int32_t* qo = (int32_t*)read_n(f, sizeof(int32_t) * B);
  int32_t* kv = (int32_t*)read_n(f, sizeof(int32_t) * B);
  int32_t* indptr = (int32_t*)read_n(f, sizeof(int32_t) * (B + 1));
  int32_t* indices = (int32_t*)read_n(f, sizeof(int32_t) * n_pages);
  const size_t page_elems = 2 * (size_t)d.num_kv_heads * d.page_size * d.head_dim;
  const size_t pool_bytes = sizeof(float) * page_elems * num_pool_pages;
  const size_t q_bytes = sizeof(float) * (size_t)rows * d.num_qo_heads * d.head_dim;
  const size_t kv_bytes = sizeof(float) * (size_t)rows * d.num_kv_heads * d.head_dim;
  void* pool_h = read_n(f, pool_bytes);
  void* q_h = read_n(f, q_bytes);
  void* k_h = read_n(f, kv_bytes);
  void* v_h = read_n(f, kv_bytes);
  int32_t n_pack;
  if (fread(&n_pack, sizeof n_pack, 1, f) != 1) return 4;
  int32_t* pack_ids = (int32_t*)read_n(f, sizeof(int32_t) * n_pack);
  int32_t* unpack_ids = (int32_t*)read_n(f, sizeof(int32_t) * n_pack);
  fclose(f);

  void* pool = to_device(pool_h, pool_bytes);
  void* q = to_device(q_h, q_bytes);
  void* k_new = to_device(k_h, kv_bytes);
  void* v_new = to_device(v_h, kv_bytes);
  const size_t out_bytes = q_bytes, lse_bytes = sizeof(float) * (size_t)rows * d.num_qo_heads;
  float *out = NULL, *lse = NULL;
  HIP_OK(hipMalloc((void**)&out, out_bytes ? out_bytes : 16));
  HIP_OK(hipMalloc((void**)&lse, lse_bytes ? lse_bytes : 16));

  pd_plan_t plan = NULL;
  PD_OK_(pd_plan(&d, B, qo, kv, indptr, indices, num_pool_pages, NULL, &plan));
  const size_t ws_bytes = pd_plan_workspace_bytes(plan);
  void* ws = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 16));
  PD_OK_(pd_plan_upload(plan, ws, ws_bytes, NULL));
  PD_OK_(pd_kv_append(plan, ws, pool, k_new, v_new, NULL));
  PD_OK_(pd_attention_run(plan, ws, q, pool, out, lse, NULL));
  const size_t buf_bytes = pd_kv_pack_bytes(&d, n_pack);
  void *buf = NULL, *scratch = NULL;
  HIP_OK(hipMalloc(&buf, buf_bytes));
  HIP_OK(hipMalloc(&scratch, 4 * (size_t)n_pack));
  PD_OK_(pd_kv_pack(&d, pool, num_pool_pages, pack_ids, n_pack, buf, buf_bytes, scratch, 4 * (size_t)n_pack, NULL));
  PD_OK_(pd_kv_unpack(&d, pool, num_pool_pages, unpack_ids, n_pack, buf, buf_bytes, scratch, 4 * (size_t)n_pack,
                      NULL));
  HIP_OK(hipDeviceSynchronize());
  pd_plan_free(plan);

  void* out_h = malloc(out_bytes + lse_bytes + pool_bytes + buf_bytes);
  char* o = (char*)out_h;
  HIP_OK(hipMemcpy(o, out, out_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(o + out_bytes, lse, lse_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(o + out_bytes + lse_bytes, pool, pool_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(o + out_bytes + lse_bytes + pool_bytes, buf, buf_bytes, hipMemcpyDeviceToHost));
  FILE* g = fopen(argv[2], "wb");
  if (!g || fwrite(out_h, 1, out_bytes + lse_bytes + pool_bytes + buf_bytes, g) !=
                out_bytes + lse_bytes + pool_bytes + buf_bytes)
    return 6;
  fclose(g);
  printf("c_step: %d rows, %d pages packed and unpacked\n", rows, n_pack);
  return 0;
}
