/*
 * Drives every function of the CPU oracle (oracle/oracle.c) over small seeded blocks, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
 * Shapes include the edges: one position, K = E, K_ext capped at E, a fresh set that empties.
 * Exit status 0 when every call returned sane values; the sanitizers abort on any error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t rng_state = 88172645463325252ull;
static double urand(void) {  /* xorshift64 */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0;
}
static float nrand(void) { return (float)(sqrt(-2.0 * log(urand() + 1e-300)) * cos(6.283185307 * urand())); }
static uint16_t bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static void* xmalloc(size_t n) {
  void* p = calloc(n ? n : 1, 1);
  if (!p) exit(3);
  return p;
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); exit(1); } } while (0)

static void run_block(int batch, int block, int H, int E, int K, int m, int I, int Is, int R,
                      int iters, int bf, int sigmoid, int norm, int restricted, int n_group,
                      int topk_group) {
  const int M = batch * block, Kext = K + m < E ? K + m : E;
  const size_t es = bf ? 2 : 4;
  char* x = xmalloc((size_t)M * H * es);
  float* Wg = xmalloc(sizeof(float) * E * H);
  float* bias = xmalloc(sizeof(float) * E);
  char* W1 = xmalloc((size_t)E * I * H * es);
  char* W3 = xmalloc((size_t)E * I * H * es);
  char* W2 = xmalloc((size_t)E * H * I * es);
  char *SW1 = NULL, *SW3 = NULL, *SW2 = NULL;
  for (int i = 0; i < E * H; ++i) Wg[i] = 0.1f * nrand();
  for (int e = 0; e < E; ++e) bias[e] = 0.2f * nrand();
  for (size_t i = 0; i < (size_t)E * I * H; ++i) {
    float a = 0.05f * nrand(), b = 0.05f * nrand(), c = 0.05f * nrand();
    if (bf) {
      ((uint16_t*)W1)[i] = bf16(a); ((uint16_t*)W3)[i] = bf16(b); ((uint16_t*)W2)[i] = bf16(c);
    } else {
      ((float*)W1)[i] = a; ((float*)W3)[i] = b; ((float*)W2)[i] = c;
    }
  }
  if (Is) {
    SW1 = xmalloc((size_t)Is * H * es); SW3 = xmalloc((size_t)Is * H * es); SW2 = xmalloc((size_t)H * Is * es);
    for (size_t i = 0; i < (size_t)Is * H; ++i) {
      float a = 0.05f * nrand(), b = 0.05f * nrand(), c = 0.05f * nrand();
      if (bf) { ((uint16_t*)SW1)[i] = bf16(a); ((uint16_t*)SW3)[i] = bf16(b); ((uint16_t*)SW2)[i] = bf16(c); }
      else { ((float*)SW1)[i] = a; ((float*)SW3)[i] = b; ((float*)SW2)[i] = c; }
    }
  }
  float* G = xmalloc(sizeof(float) * M * E);
  int32_t* ids = xmalloc(sizeof(int32_t) * M * Kext);
  double* s = xmalloc(sizeof(double) * M * Kext);
  double* w = xmalloc(sizeof(double) * M * K);
  int64_t* q = xmalloc(sizeof(int64_t) * M * Kext);
  uint8_t* allowed = xmalloc((size_t)M * E);
  uint8_t* inS = xmalloc(E);
  uint8_t* inA = xmalloc(E);
  int32_t* slot_of = xmalloc(sizeof(int32_t) * E);
  int32_t* S_list = xmalloc(sizeof(int32_t) * E);
  int32_t* slotA = xmalloc(sizeof(int32_t) * E);
  int32_t* SA = xmalloc(sizeof(int32_t) * E);
  int64_t stats[5];
  uint8_t* valid = xmalloc(M);
  int32_t* last_fresh = xmalloc(sizeof(int32_t) * M);
  uint8_t* prev_D = xmalloc(M);
  uint8_t* D = xmalloc(M);
  uint8_t* fresh = xmalloc(M);
  int32_t* wl_pos = xmalloc(sizeof(int32_t) * M * K);
  int32_t* wl_k = xmalloc(sizeof(int32_t) * M * K);
  double* wl_w = xmalloc(sizeof(double) * M * K);
  int32_t* offs = xmalloc(sizeof(int32_t) * (E + 1));
  int32_t* inv = xmalloc(sizeof(int32_t) * M * K);
  int32_t* rows = xmalloc(sizeof(int32_t) * M);
  int32_t* rids = xmalloc(sizeof(int32_t) * M * K);
  double* rw = xmalloc(sizeof(double) * M * K);
  double* cache = xmalloc(sizeof(double) * M * H);
  double* Rout = xmalloc(sizeof(double) * M * H);
  double* Yout = xmalloc(sizeof(double) * M * H);
  for (int t = 0; t < M; ++t) { last_fresh[t] = -(1 << 30); rows[t] = t; }
  int support_valid = 0;
  for (int it = 0; it < iters; ++it) {
    for (size_t i = 0; i < (size_t)M * H; ++i) {
      float v = nrand();
      if (bf) ((uint16_t*)x)[i] = bf16(v); else ((float*)x)[i] = v;
    }
    for (int t = 0; t < M; ++t) D[t] = (uint8_t)(it > 0 && urand() < (double)it / iters);
    orc_router_logits(M, H, E, bf, x, Wg, bias, G);
    const uint8_t* al = NULL;
    if (n_group > 1) {
      orc_group_allowed(M, E, n_group, topk_group, G, NULL, allowed);
      al = allowed;
    }
    orc_route(M, E, K, Kext, sigmoid, norm, G, al, ids, s, w, q);
    orc_score_given(M, E, K, Kext, sigmoid, norm, G, ids, s, w, q);
    const int path = orc_support_status(M, K, Kext, ids, inS, support_valid);
    CHECK(path >= 0 && path <= 2);
    if (path) {
      int nS = orc_support_build(M, E, K, Kext, ids, q, (E + 1) / 2, K, 9, 10, 95, 100, 1, 1, inS,
                                 slot_of, S_list, stats);
      CHECK(nS >= K && nS <= E);
      support_valid = 1;
    }
    if (restricted) {
      int nA = orc_atlas_build(M, E, K, Kext, ids, q, (E + 1) / 2, K, 9, 10, 95, 100, 1, 1, inA,
                               slotA, SA, stats);
      CHECK(nA >= 0 && nA <= E);
      for (int t = 0; t < M; ++t) memcpy(allowed + (size_t)t * E, inS, E);
      CHECK(orc_route_restricted(M, E, K, sigmoid, norm, G, allowed, rids, rw) >= 0);
      CHECK(orc_under_covered(M, K, Kext, ids, q, inA, 9, 10) <= M);
    }
    int an = orc_fresh_set(M, R, it, valid, last_fresh, prev_D, D, NULL, fresh);
    CHECK(an == 0 || an == 1);
    int nS = 0;
    for (int e = 0; e < E; ++e) nS += inS[e];
    int P = orc_worklist(M, K, Kext, ids, w, fresh, slot_of, nS, wl_pos, wl_k, wl_w, offs, inv);
    CHECK(P >= 0 && P <= M * K);
    orc_moe_rows(M, H, I, Is, E, K, Kext, bf, x, ids, w, fresh, W1, W3, W2, SW1, SW3, SW2, M, rows,
                 cache, Rout, Yout);
    orc_commit(M, it, fresh, D, valid, last_fresh, prev_D);
  }
  orc_dense_moe(M, H, I, Is, E, K, sigmoid, norm, bf, x, Wg, bias, W1, W3, W2, SW1, SW3, SW2, Rout,
                Yout);
  for (size_t i = 0; i < (size_t)M * H; ++i) CHECK(isfinite(Yout[i]));
  free(x); free(Wg); free(bias); free(W1); free(W3); free(W2); free(SW1); free(SW3); free(SW2);
  free(G); free(ids); free(s); free(w); free(q); free(allowed); free(inS); free(inA);
  free(slot_of); free(S_list); free(slotA); free(SA); free(valid); free(last_fresh); free(prev_D); free(D); free(fresh);
  free(wl_pos); free(wl_k); free(wl_w); free(offs); free(inv); free(rows); free(rids); free(rw);
  free(cache); free(Rout); free(Yout);
}

static void run_decode(int batch, int block, int H, int V) {
  const int M = batch * block;
  uint16_t* h = xmalloc(sizeof(uint16_t) * M * H);
  uint16_t* Wv = xmalloc(sizeof(uint16_t) * V * H);
  for (int i = 0; i < M * H; ++i) h[i] = bf16(nrand());
  for (int i = 0; i < V * H; ++i) Wv[i] = bf16(0.05f * nrand());
  uint8_t* D = xmalloc(M);
  uint8_t* Dn = xmalloc(M);
  int32_t* token = xmalloc(sizeof(int32_t) * M);
  int32_t* top = xmalloc(sizeof(int32_t) * M);
  double* conf = xmalloc(sizeof(double) * M);
  double* gap = xmalloc(sizeof(double) * M);
  for (int t = 0; t < M; ++t) { D[t] = (uint8_t)(urand() < 0.3); token[t] = -1; }
  int commits = orc_live_decode(M, H, V, block, 1, h, Wv, D, 0.95, Dn, token, conf, gap, top);
  CHECK(commits >= 0 && commits <= M);
  free(h); free(Wv); free(D); free(Dn); free(token); free(top); free(conf); free(gap);
}

int main(void) {
  /* batch, block, H, E, K, m, I, Is, R, iters, bf16, sigmoid, norm, restricted, groups, kept */
  run_block(2, 8, 64, 16, 4, 4, 24, 20, 3, 6, 1, 1, 1, 0, 0, 0);
  run_block(1, 16, 64, 8, 2, 2, 32, 0, 2, 4, 0, 0, 0, 0, 0, 0);   /* fp32, softmax */
  run_block(1, 1, 32, 4, 4, 4, 16, 0, 1, 3, 1, 0, 0, 0, 0, 0);    /* one position, K = E */
  run_block(3, 5, 32, 12, 3, 3, 16, 16, 2, 5, 1, 1, 1, 1, 0, 0);  /* restricted routing */
  run_block(2, 6, 32, 16, 2, 2, 16, 0, 4, 4, 1, 1, 1, 0, 4, 2);   /* group-limited top-k */
  run_decode(3, 8, 32, 200);
  run_decode(1, 1, 16, 128);
  printf("oracle sanitizer check ok\n");
  return 0;
}
