/*
 * A plain C user of liblcv_bsa through include/lcv_bsa.h (no Python, no C++): it shows that
 * the boundary is usable from C and lets the tests check it from outside the Python binding.
 *
 *   lcv_client query N LOCAL STRIDE COND
 *       host only: the ABI version and the layout's closed-form sizes, one "key value" line
 *       each.
 *   lcv_client forward T H W HEADS LOCAL STRIDE COND IN OUT
 *       reads Q, K, V (bf16 bits, [1, HEADS, N, 64] each, N = T*H*W, in that order) from
 *       the file IN, runs lcv_bsa_build_layout and lcv_bsa_forward with the 3D-RoPE applied
 *       to Q and K (theta 1e4), and writes out (bf16 bits) and then lse (fp32) to OUT.
 *   lcv_client cross_bwd_noquery HEADS KV_LEN
 *       the cross-attention backward with no query (n_q = 0): every query-side pointer and
 *       the workspace are NULL (its size is 0), dK and dV are filled with NaN bits first;
 *       prints "zeros" if both come back as exact zeros.
 *
 * Every call's status is checked; on failure the library's message is printed and the
 * program exits with status 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lcv_bsa.h"

static void check_lcv(lcv_status st, const char* what) {
  if (st != LCV_OK) {
    fprintf(stderr, "%s failed (%d): %s\n", what, (int)st, lcv_last_error());
    exit(1);
  }
}

static void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s failed: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

static int query(int argc, char** argv) {
  if (argc != 6) return 2;
  lcv_bsa_layout_params p;
  p.n_tokens = atoi(argv[2]);
  p.block = LCV_BLOCK;
  p.local_blocks = atoi(argv[3]);
  p.global_stride = atoi(argv[4]);
  p.cond_len = atoi(argv[5]);
  lcv_bsa_layout_info info;
  check_lcv(lcv_bsa_layout_query(&p, &info), "lcv_bsa_layout_query");
  printf("abi_version %d\n", (int)lcv_abi_version());
  printf("n_blocks %d\n", (int)info.n_blocks);
  printf("max_row_len %d\n", (int)info.max_row_len);
  printf("nnz %lld\n", (long long)info.nnz);
  printf("attended_pairs %lld\n", (long long)info.attended_pairs);
  return 0;
}

static int forward(int argc, char** argv) {
  if (argc != 11) return 2;
  lcv_rope3d_grid grid;
  grid.T = atoi(argv[2]);
  grid.H = atoi(argv[3]);
  grid.W = atoi(argv[4]);
  grid.theta = 10000.0f;
  const int heads = atoi(argv[5]);
  lcv_bsa_layout_params p;
  p.n_tokens = grid.T * grid.H * grid.W;
  p.block = LCV_BLOCK;
  p.local_blocks = atoi(argv[6]);
  p.global_stride = atoi(argv[7]);
  p.cond_len = atoi(argv[8]);
  const size_t elems = (size_t)heads * (size_t)p.n_tokens * LCV_HEAD_DIM;
  const size_t bytes = elems * sizeof(uint16_t);
  const size_t rows = (size_t)heads * (size_t)p.n_tokens;

  uint16_t* host = (uint16_t*)malloc(4 * bytes);
  float* lse_host = (float*)malloc(rows * sizeof(float));
  if (host == NULL || lse_host == NULL) {
    fprintf(stderr, "host allocation failed\n");
    return 1;
  }
  FILE* f = fopen(argv[9], "rb");
  if (f == NULL || fread(host, 1, 3 * bytes, f) != 3 * bytes) {
    fprintf(stderr, "cannot read %zu bytes from %s\n", 3 * bytes, argv[9]);
    return 1;
  }
  fclose(f);

  void *q, *k, *v, *out;
  float* lse;
  check_hip(hipMalloc(&q, bytes), "hipMalloc q");
  check_hip(hipMalloc(&k, bytes), "hipMalloc k");
  check_hip(hipMalloc(&v, bytes), "hipMalloc v");
  check_hip(hipMalloc(&out, bytes), "hipMalloc out");
  check_hip(hipMalloc((void**)&lse, rows * sizeof(float)), "hipMalloc lse");
  check_hip(hipMemcpy(q, host, bytes, hipMemcpyHostToDevice), "copy q");
  check_hip(hipMemcpy(k, host + elems, bytes, hipMemcpyHostToDevice), "copy k");
  check_hip(hipMemcpy(v, host + 2 * elems, bytes, hipMemcpyHostToDevice), "copy v");

  lcv_bsa_layout* layout = NULL;
  check_lcv(lcv_bsa_build_layout(&p, 0, &layout), "lcv_bsa_build_layout");
  check_lcv(lcv_bsa_forward(q, k, v, 1, heads, layout, p.cond_len, LCV_ROPE_Q | LCV_ROPE_K, &grid, out, lse, 0),
            "lcv_bsa_forward");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");
  check_hip(hipMemcpy(host + 3 * elems, out, bytes, hipMemcpyDeviceToHost), "copy out");
  check_hip(hipMemcpy(lse_host, lse, rows * sizeof(float), hipMemcpyDeviceToHost), "copy lse");
  lcv_bsa_layout_destroy(layout);
  hipFree(q);
  hipFree(k);
  hipFree(v);
  hipFree(out);
  hipFree(lse);

  f = fopen(argv[10], "wb");
  if (f == NULL || fwrite(host + 3 * elems, 1, bytes, f) != bytes ||
      fwrite(lse_host, sizeof(float), rows, f) != rows) {
    fprintf(stderr, "cannot write %s\n", argv[10]);
    return 1;
  }
  fclose(f);
  free(host);
  free(lse_host);
  printf("forward ok\n");
  return 0;
}

static int cross_bwd_noquery(int argc, char** argv) {
  if (argc != 4) return 2;
  const int heads = atoi(argv[2]);
  const int kv_len = atoi(argv[3]);
  const size_t elems = (size_t)heads * (size_t)kv_len * LCV_HEAD_DIM;
  const size_t bytes = elems * sizeof(uint16_t);
  const int64_t ws = lcv_cross_attention_backward_workspace(1, heads, 0, kv_len);
  if (ws != 0) {
    fprintf(stderr, "workspace for n_q = 0 is %lld, expected 0\n", (long long)ws);
    return 1;
  }
  uint16_t* host = (uint16_t*)malloc(bytes);
  if (host == NULL) {
    fprintf(stderr, "host allocation failed\n");
    return 1;
  }
  for (size_t i = 0; i < elems; ++i) host[i] = (uint16_t)(0x3c00u + (i % 97u));   /* finite keys and values */
  void *k, *v, *dk, *dv;
  check_hip(hipMalloc(&k, bytes), "hipMalloc k");
  check_hip(hipMalloc(&v, bytes), "hipMalloc v");
  check_hip(hipMalloc(&dk, bytes), "hipMalloc dk");
  check_hip(hipMalloc(&dv, bytes), "hipMalloc dv");
  check_hip(hipMemcpy(k, host, bytes, hipMemcpyHostToDevice), "copy k");
  check_hip(hipMemcpy(v, host, bytes, hipMemcpyHostToDevice), "copy v");
  check_hip(hipMemset(dk, 0xff, bytes), "poison dk");
  check_hip(hipMemset(dv, 0xff, bytes), "poison dv");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");
  check_lcv(lcv_cross_attention_backward(NULL, k, v, NULL, NULL, NULL, 1, heads, 0, kv_len, NULL, NULL, dk, dv, NULL,
                                         0, 0),
            "lcv_cross_attention_backward");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");
  int zeros = 1;
  void* grads[2] = {dk, dv};
  for (int t = 0; t < 2; ++t) {
    check_hip(hipMemcpy(host, grads[t], bytes, hipMemcpyDeviceToHost), "copy gradient");
    for (size_t i = 0; i < elems; ++i)
      if (host[i] != 0) zeros = 0;
  }
  hipFree(k);
  hipFree(v);
  hipFree(dk);
  hipFree(dv);
  free(host);
  printf("%s\n", zeros ? "zeros" : "nonzero");
  return 0;
}

int main(int argc, char** argv) {
  int rc = 2;
  if (argc > 1 && strcmp(argv[1], "query") == 0) rc = query(argc, argv);
  if (argc > 1 && strcmp(argv[1], "forward") == 0) rc = forward(argc, argv);
  if (argc > 1 && strcmp(argv[1], "cross_bwd_noquery") == 0) rc = cross_bwd_noquery(argc, argv);
  if (rc == 2)
    fprintf(stderr, "usage: lcv_client query N LOCAL STRIDE COND\n"
                    "       lcv_client forward T H W HEADS LOCAL STRIDE COND IN OUT\n"
                    "       lcv_client cross_bwd_noquery HEADS KV_LEN\n");
  return rc;
}
