/*
 * Exercises the host side of the C ABI (include/epoch.h) without touching a GPU: descriptor
 * validation and workspace sizes of the benchmark shapes and of invalid descriptors, every
 * argument error that is returned before anything is enqueued, and the status strings.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer on the host code of libepoch
 * (tests/test_sanitizers.py).  Exit status 0 when every call returned what its declaration says.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/epoch.h"

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); exit(1); } } while (0)

static epoch_desc base_desc(int H, int E, int K, int I, int shared, int batch, int block) {
  epoch_desc d;
  memset(&d, 0, sizeof d);
  d.n_layers = 2; d.hidden = H; d.n_experts = E; d.top_k = K; d.inter = I;
  d.n_shared = shared; d.shared_inter = shared ? I : 0; d.batch = batch; d.block = block;
  d.gate = EPOCH_GATE_SIGMOID; d.norm_topk = 1; d.act_dtype = EPOCH_DTYPE_BF16;
  d.staleness_R = 4; d.atlas_m = K; d.atlas_B = (E + 1) / 2; d.atlas_c = K;
  d.alpha_num = 9; d.alpha_den = 10; d.q_num = 95; d.q_den = 100; d.beta_num = 1; d.beta_den = 1;
  d.routing = EPOCH_ROUTING_EXACT;
  return d;
}

int main(void) {
  size_t n = 0;
  const int shapes[][7] = {{64, 8, 2, 64, 0, 1, 16}, {2048, 64, 8, 1024, 0, 8, 32},
                           {2048, 256, 8, 512, 1, 32, 32}, {4096, 256, 8, 1536, 1, 64, 32},
                           {2048, 256, 8, 512, 1, 128, 64}, {64, 1024, 16, 64, 0, 3, 7}};
  size_t prev = 0;
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    const int* s = shapes[i];
    epoch_desc d = base_desc(s[0], s[1], s[2], s[3], s[4], s[5], s[6]);
    CHECK(epoch_plan_workspace_bytes(&d, &n) == EPOCH_OK && n > 0 && n % 256 == 0);
    d.routing = EPOCH_ROUTING_RESTRICTED;
    d.atlas_period = 3;
    CHECK(epoch_plan_workspace_bytes(&d, &n) == EPOCH_OK);
    prev = n;
  }
  (void)prev;
  /* invalid descriptors */
  epoch_desc d = base_desc(2048, 64, 8, 1024, 0, 8, 32);
  epoch_desc b;
  b = d; b.hidden = 100; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  b = d; b.top_k = 0; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  b = d; b.n_experts = 5000; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  b = d; b.act_dtype = 9; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_DTYPE);
  b = d; b.gate = 9; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_DTYPE);
  b = d; b.flags = 1; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  b = d; b.atlas_period = 2; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  b = d; b.n_group = 3; b.topk_group = 1; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  b = d; b.batch = 1 << 20; CHECK(epoch_plan_workspace_bytes(&b, &n) == EPOCH_E_SHAPE);
  CHECK(epoch_plan_workspace_bytes(NULL, &n) == EPOCH_E_NULL);
  CHECK(epoch_plan_workspace_bytes(&d, NULL) == EPOCH_E_NULL);
  /* plan build: argument errors are returned before any launch */
  epoch_layer_weights w[2];
  memset(w, 0, sizeof w);
  epoch_plan* plan = (epoch_plan*)0x1;
  CHECK(epoch_block_plan_build(&d, w, (void*)256, (size_t)1 << 30, NULL, &plan) == EPOCH_E_NULL);
  CHECK(plan == NULL);
  CHECK(epoch_block_plan_build(&d, w, (void*)100, (size_t)1 << 30, NULL, &plan) == EPOCH_E_WORKSPACE);
  for (int l = 0; l < 2; ++l) {
    w[l].router_w = (const float*)(uintptr_t)4096; w[l].w1 = (const void*)(uintptr_t)8192;
    w[l].w3 = (const void*)(uintptr_t)8200; w[l].w2 = (const void*)(uintptr_t)12288;
  }
  CHECK(epoch_block_plan_build(&d, w, (void*)256, (size_t)1 << 30, NULL, &plan) == EPOCH_E_ALIGN);
  w[0].w3 = (const void*)(uintptr_t)8208; w[1].w3 = (const void*)(uintptr_t)8208;
  CHECK(epoch_block_plan_build(&d, w, (void*)256, 16, NULL, &plan) == EPOCH_E_WORKSPACE);
  CHECK(epoch_block_plan_build(NULL, w, (void*)256, 16, NULL, &plan) == EPOCH_E_NULL);
  /* calls on a NULL plan */
  CHECK(epoch_moe_fresh_forward(NULL, 0, (void*)256, (const uint8_t*)256, NULL, (void*)256, NULL, NULL) == EPOCH_E_NULL);
  CHECK(epoch_cache_update(NULL, 0, NULL) == EPOCH_E_NULL);
  epoch_inspect ins;
  CHECK(epoch_plan_inspect(NULL, 0, &ins) == EPOCH_E_NULL);
  CHECK(epoch_plan_set_timing(NULL, -1) == EPOCH_E_NULL);
  CHECK(epoch_plan_timing(NULL, NULL, NULL, 0) == EPOCH_E_NULL);
  CHECK(epoch_block_plan_destroy(NULL) == EPOCH_OK);
  /* live decoding */
  epoch_decode_desc dd = {8, 32, 2048, 32768, EPOCH_DTYPE_BF16, 0, 0.95};
  CHECK(epoch_decode_workspace_bytes(&dd, &n) == EPOCH_OK && n % 256 == 0);
  epoch_decode_desc db = dd; db.vocab = 100;
  CHECK(epoch_decode_workspace_bytes(&db, &n) == EPOCH_E_SHAPE);
  db = dd; db.tau = 1.5; CHECK(epoch_decode_workspace_bytes(&db, &n) == EPOCH_E_SHAPE);
  db = dd; db.act_dtype = EPOCH_DTYPE_F32; CHECK(epoch_decode_workspace_bytes(&db, &n) == EPOCH_E_DTYPE);
  CHECK(epoch_live_decode(&dd, NULL, (void*)256, (uint8_t*)256, (uint8_t*)256, (int32_t*)256, NULL,
                          (void*)256, n, NULL) == EPOCH_E_NULL);
  CHECK(epoch_live_decode(&dd, (void*)8, (void*)256, (uint8_t*)256, (uint8_t*)256, (int32_t*)256, NULL,
                          (void*)256, n, NULL) == EPOCH_E_ALIGN);
  CHECK(epoch_live_decode(&dd, (void*)256, (void*)256, (uint8_t*)256, (uint8_t*)256, (int32_t*)256, NULL,
                          (void*)256, 16, NULL) == EPOCH_E_WORKSPACE);
  epoch_decode_desc big = {256, 32, 2048, 131072, EPOCH_DTYPE_BF16, 0, 0.95};
  CHECK(epoch_live_decode_static(&big, (void*)256, (void*)256, (uint8_t*)256, (uint8_t*)256,
                                 (int32_t*)256, NULL, NULL) == EPOCH_E_SCRATCH);
  for (int code = 1; code >= -10; --code) CHECK(epoch_status_string(code) != NULL);
  printf("abi sanitizer check ok\n");
  return 0;
}
