/*
 * oracle.h -- plain CPU oracle of the liveness-sparse routed-expert MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the product path (the HIP
 * library and its binding) never calls it and shares no code with it.
 *
 * Sources: "Epoch: Compiling Diffusion Blocks for Sparse MoE Serving" (paper
 * card abstract) and the pinghaoyang.com.cn teardown of it ("Epoch 完全拆解"),
 * cited per function in oracle.c by section and equation.
 *
 * Conventions: position t = b * block + p, row-major arrays, bf16 tensors are
 * uint16 bit patterns (act_bf16 = 1) else fp32.  All sums are in double.  The
 * router logits are rounded once to fp32 because the top-k decision is taken on
 * fp32 logits; nothing else is rounded.
 */
#ifndef EPOCH_ORACLE_H
#define EPOCH_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int orc_num_threads(void);
void orc_set_num_threads(int n);

void orc_router_logits(int M, int H, int E, int act_bf16, const void* x, const float* Wg,
                       const float* bias, float* G);

/* allowed: [M x E] selectable experts per row, or NULL for all */
void orc_route(int M, int E, int K, int Kext, int gate_sigmoid, int norm_topk, const float* G,
               const uint8_t* allowed, int32_t* ids, double* s, double* w, int64_t* q);
void orc_score_given(int M, int E, int K, int Kext, int gate_sigmoid, int norm_topk,
                     const float* G, const int32_t* ids, double* s, double* w, int64_t* q);

void orc_group_allowed(int M, int E, int n_group, int topk_group, const float* G,
                       const uint8_t* base, uint8_t* allowed);

int orc_support_status(int M, int K, int Kext, const int32_t* ids, const uint8_t* inS,
                       int support_valid);

int orc_support_build(int M, int E, int K, int Kext, const int32_t* ids, const int64_t* q, int B,
                      int c, int alpha_num, int alpha_den, int q_num, int q_den, int beta_num,
                      int beta_den, uint8_t* inS, int32_t* slot_of, int32_t* S_list,
                      int64_t* stats);

int orc_atlas_build(int M, int E, int K, int Kext, const int32_t* ids, const int64_t* q, int B,
                    int c, int alpha_num, int alpha_den, int q_num, int q_den, int beta_num,
                    int beta_den, uint8_t* inA, int32_t* slot_of, int32_t* S_list,
                    int64_t* stats);

/* allowed: [M x E]; returns the number of rows with fewer than K selectable experts (then
   nothing is written) */
int orc_route_restricted(int M, int E, int K, int gate_sigmoid, int norm_topk, const float* G,
                         const uint8_t* allowed, int32_t* rids, double* rw);

int64_t orc_under_covered(int M, int K, int Kext, const int32_t* ids, const int64_t* q,
                          const uint8_t* inS, int alpha_num, int alpha_den);

int orc_fresh_set(int M, int R, int iter, const uint8_t* valid, const int32_t* last_fresh,
                  const uint8_t* prev_D, const uint8_t* D, const uint8_t* force, uint8_t* fresh);

/* Returns the number of pairs, or -1 when a fresh position selects an expert without a slot. */
int orc_worklist(int M, int K, int Kext, const int32_t* ids, const double* w,
                 const uint8_t* fresh, const int32_t* slot_of, int nS, int32_t* wl_pos,
                 int32_t* wl_k, double* wl_w, int32_t* offs, int32_t* inv);

void orc_expert(int H, int I, int act_bf16, const void* x_row, const void* W1e, const void* W3e,
                const void* W2e, double* y);

void orc_moe_rows(int M, int H, int I, int Is, int E, int K, int Kext, int act_bf16,
                  const void* x, const int32_t* ids, const double* w, const uint8_t* fresh,
                  const void* W1, const void* W3, const void* W2, const void* SW1,
                  const void* SW3, const void* SW2, int n_rows, const int32_t* rows,
                  double* cache, double* R_out, double* Y_out);

void orc_commit(int M, int iter, const uint8_t* fresh, const uint8_t* D, uint8_t* valid,
                int32_t* last_fresh, uint8_t* prev_D);

void orc_dense_moe(int M, int H, int I, int Is, int E, int K, int gate_sigmoid, int norm_topk,
                   int act_bf16, const void* x, const float* Wg, const float* bias,
                   const void* W1, const void* W3, const void* W2, const void* SW1,
                   const void* SW3, const void* SW2, double* R_out, double* Y_out);

int orc_live_decode(int M, int H, int V, int block, int act_bf16, const void* h, const void* Wv,
                    const uint8_t* D, double tau, uint8_t* D_next, int32_t* token, double* conf,
                    double* gap, int32_t* top);

#ifdef __cplusplus
}
#endif
#endif
