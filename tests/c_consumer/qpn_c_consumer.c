/*
 * A plain C99 consumer of include/qpn.h: it must compile as C (no C++ in the
 * header), link against libqpn.so with every declared entry point resolved,
 * and see the same struct layouts as the Python binding. It makes host-only
 * calls (sizes, plans, argument checks that fail before any HIP call), so it
 * runs without a GPU. Prints "key value" lines for the test to compare.
 */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "qpn.h"

typedef void (*entry_fn)(void);

#define FAIL(msg)                          \
  do {                                     \
    fprintf(stderr, "FAILED: %s\n", msg);  \
    return 1;                              \
  } while (0)

int main(void) {
  /* Every entry point the header declares, taken by address: an unresolved
   * one fails the link. */
  const entry_fn entries[] = {
      (entry_fn)qpn_status_string,      (entry_fn)qpn_packed_bytes,
      (entry_fn)qpn_pack_nvfp4,         (entry_fn)qpn_pack_fp8,
      (entry_fn)qpn_unpack_nvfp4,       (entry_fn)qpn_unpack_fp8,
      (entry_fn)qpn_absmax_f32,         (entry_fn)qpn_nvfp4_tensor_scale,
      (entry_fn)qpn_quantize_nvfp4,     (entry_fn)qpn_quantize_fp8,
      (entry_fn)qpn_fp8_absmax,         (entry_fn)qpn_requantize_fp8_nvfp4,
      (entry_fn)qpn_workspace_bytes,    (entry_fn)qpn_gemm,
      (entry_fn)qpn_gemm_tuned,         (entry_fn)qpn_workspace_bytes_tuned,
      (entry_fn)qpn_gemm_plan,          (entry_fn)qpn_gemm_swiglu,
      (entry_fn)qpn_gemm_f32,           (entry_fn)qpn_gemm_argmax,
      (entry_fn)qpn_read_ceiling,       (entry_fn)qpn_read_ceiling_grid,
      (entry_fn)qpn_gemm_noalloc,       (entry_fn)qpn_mlp,
      (entry_fn)qpn_mlp_workspace_bytes,
  };
  size_t i;
  for (i = 0; i < sizeof entries / sizeof entries[0]; ++i)
    if (!entries[i]) FAIL("null entry point");
  printf("entries %d\n", (int)(sizeof entries / sizeof entries[0]));

  printf("sizeof_weight %d\n", (int)sizeof(qpn_weight));
  printf("offset_weight_n %d\n", (int)offsetof(qpn_weight, n));
  printf("offset_weight_packed %d\n", (int)offsetof(qpn_weight, packed));
  printf("offset_weight_tensor_scale %d\n", (int)offsetof(qpn_weight, tensor_scale));
  printf("offset_weight_row_scales %d\n", (int)offsetof(qpn_weight, row_scales));
  printf("sizeof_launch %d\n", (int)sizeof(qpn_launch));
  printf("offset_launch_whole_groups %d\n", (int)offsetof(qpn_launch, whole_groups));
  printf("offset_launch_block_columns %d\n", (int)offsetof(qpn_launch, block_columns));
  printf("sizeof_mlp_launch %d\n", (int)sizeof(qpn_mlp_launch));
  printf("offset_mlp_launch_stream_after %d\n", (int)offsetof(qpn_mlp_launch, stream_after));
  printf("max_m %d\n", QPN_MAX_M);

  if (strcmp(qpn_status_string(QPN_OK), "ok") != 0) FAIL("status string");
  if (qpn_packed_bytes(QPN_FMT_NVFP4, 512, 1024) != (size_t)32 * 4 * 2304) FAIL("packed bytes");
  if (qpn_nvfp4_tensor_scale(2688.0f) != 1.0f) FAIL("tensor scale");

  {
    /* The gate_up matrix of the 27B decoder at M = 1: a tuned plan. No
     * pointer is dereferenced by a plan query. */
    qpn_weight w;
    qpn_launch resolved;
    memset(&w, 0, sizeof w);
    w.format = QPN_FMT_NVFP4;
    w.n = 34816;
    w.k = 5120;
    w.tensor_scale = 1.0f;
    if (qpn_gemm_plan(&w, 1, NULL, &resolved) != QPN_OK) FAIL("plan");
    printf("plan_gate_up_m1 %d %d %d %d %d %d %d\n", resolved.split_k, resolved.waves_per_group,
           resolved.depth, resolved.k_slices, resolved.epilogue, resolved.x_stage, resolved.whole_groups);
    printf("workspace_gate_up_m8 %lu\n", (unsigned long)qpn_workspace_bytes(&w, 8));
    /* argument checks that fail on the host, before any HIP call */
    if (qpn_gemm(NULL, &w, NULL, 1, NULL, 0, NULL) != QPN_ERR_INVALID_ARG) FAIL("null pointers");
    if (qpn_gemm(NULL, &w, NULL, QPN_MAX_M + 1, NULL, 0, NULL) != QPN_ERR_INVALID_ARG) FAIL("m too large");
    w.reserved = 1;
    if (qpn_gemm_plan(&w, 1, NULL, &resolved) != QPN_ERR_INVALID_ARG) FAIL("reserved field");
  }
  printf("ok 1\n");
  return 0;
}
