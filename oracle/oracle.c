/*
 * oracle.c -- plain, slow CPU oracle of the liveness-sparse routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.
 *
 * Every function below follows one passage of the pages:
 *   [P1]  "Epoch: Compiling Diffusion Blocks for Sparse MoE Serving", abstract.
 *   [T]   pinghaoyang.com.cn teardown "Epoch 完全拆解", cited by its section:
 *         "MoE bottleneck" (the MoE-layer equation), "Expert Atlas" (G, K_ext,
 *         r_t, C_t, U_l, p_e, G_e, H_e, score equations and the three steps),
 *         "Liveness-Shard Parallelism" (Z_i, N_i, F_i equations, the hot-iteration
 *         state machine and the Compact / SparseMoE / merge equations),
 *         "refresh period" (the age bound), "FreshLane" (pack, counts, light
 *         expert kernel, scatter/merge) and "cold / hot-update / hot-skip".
 *
 * Arithmetic: double everywhere.  Router logits are rounded to fp32 once, because
 * the top-k decision is taken on fp32 logits.  Atlas weights are integers
 * q = floor(s * 2^16 + 1/2) so that the support arithmetic is exact.
 *
 * Planted mistakes: building with -DORC_MUTATE=<n> changes one step on purpose;
 * the test-suite uses this to show that its pins catch each kind of mistake.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORC_MUTATE
#define ORC_MUTATE 0
#endif

#define ATLAS_Q 65536LL

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* threads of the oracle's parallel loops from here on (n >= 1); the baseline timing uses it
   to time one host core beside all of them */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* element h of a row of bf16 bit patterns (act_bf16) or fp32 values, as double */
static double ld(const void* base, int act_bf16, size_t idx) {
  if (act_bf16) {
    uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

static size_t act_size(int act_bf16) { return act_bf16 ? 2u : 4u; }

static const void* offset(const void* base, int act_bf16, size_t elems) {
  return (const char*)base + elems * act_size(act_bf16);
}

/*
 * Router logits G in R^{N x E} ([T] Expert Atlas, the G equation; [P1] "recomputing
 * gate logits every iteration"): G[t,e] = sum_h x[t,h] W_g[e,h] + b_e, a plain linear
 * gate with bias, summed in double and rounded once to fp32.
 */
void orc_router_logits(int M, int H, int E, int act_bf16, const void* x, const float* Wg,
                       const float* bias, float* G) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < M; ++t) {
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += ld(x, act_bf16, (size_t)t * H + h) * (double)Wg[(size_t)e * H + h];
#if ORC_MUTATE != 1
      if (bias) acc += (double)bias[e];
#endif
      G[(size_t)t * E + e] = (float)acc;
    }
  }
}

/* key order of the top-k: larger logit first, equal logits -> lower expert id first */
static int before(float ga, int ea, float gb, int eb) {
#if ORC_MUTATE == 4
  return ga > gb || (ga == gb && ea > eb);
#else
  return ga > gb || (ga == gb && ea < eb);
#endif
}

/* Scores of one position's ranked candidates ids[0..Kext): s = sigma(G) (softmax over all E
   experts, or sigmoid), the Atlas integer weight q = floor(s * 2^16 + 1/2), and the routing
   weights of the first K (s, or s / sum_{j<K} s when norm_topk). */
static void score_row(int E, int K, int Kext, int gate_sigmoid, int norm_topk, const float* g,
                      const int32_t* ids, double* s, double* w, int64_t* q) {
  double zmax = -INFINITY, z = 0.0;
  if (!gate_sigmoid) {
    for (int e = 0; e < E; ++e) zmax = fmax(zmax, (double)g[e]);
    for (int e = 0; e < E; ++e) z += exp((double)g[e] - zmax);
  }
  for (int j = 0; j < Kext; ++j) {
    double ge = (double)g[ids[j]];
    double sj = gate_sigmoid ? 1.0 / (1.0 + exp(-ge)) : exp(ge - zmax) / z;
    s[j] = sj;
    q[j] = (int64_t)floor(sj * (double)ATLAS_Q + 0.5);
  }
  double denom = 0.0;
  for (int k = 0; k < K; ++k) denom += s[k];
  for (int k = 0; k < K; ++k) w[k] = norm_topk ? s[k] / denom : s[k];
}

/*
 * Top-k selection and routing weights ([T] MoE bottleneck, y_t = sum over TopK(g(x_t))
 * of w_{t,e} E_e(x_t); [T] Expert Atlas: top-k taken over sigma(G), extended to
 * K_ext = K + m candidates I_{t,j} with weights W_{t,j} for the planner).
 * ids: the first K_ext experts in key order; the first K are the routing selection.
 * s:   gate score sigma(G) of each candidate (softmax over all E, or sigmoid).
 * w:   routing weight of the first K (= s, or s / sum_{j<K} s when norm_topk).
 * q:   the Atlas integer weight floor(s * 2^16 + 1/2) of each candidate.
 */
void orc_route(int M, int E, int K, int Kext, int gate_sigmoid, int norm_topk, const float* G,
               const uint8_t* allowed, int32_t* ids, double* s, double* w, int64_t* q) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < M; ++t) {
    const float* g = G + (size_t)t * E;
    const uint8_t* al = allowed ? allowed + (size_t)t * E : NULL;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    for (int j = 0; j < Kext; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if ((!al || al[e]) && !taken[e] && (best < 0 || before(g[e], e, g[best], best))) best = e;
      taken[best] = 1;
      ids[(size_t)t * Kext + j] = best;
    }
    free(taken);
    score_row(E, K, Kext, gate_sigmoid, norm_topk, g, ids + (size_t)t * Kext,
              s + (size_t)t * Kext, w + (size_t)t * K, q + (size_t)t * Kext);
  }
}

/*
 * The scores, weights and planner weights of a given selection (the scoring half of orc_route,
 * for selections fixed elsewhere): ids [M x Kext] holds each position's candidates in rank
 * order.  The harness uses it for positions whose order is a tie of their logits (two logits
 * closer than the near-tie gap), where either order is correct.
 */
void orc_score_given(int M, int E, int K, int Kext, int gate_sigmoid, int norm_topk,
                     const float* G, const int32_t* ids, double* s, double* w, int64_t* q) {
  for (int t = 0; t < M; ++t)
    score_row(E, K, Kext, gate_sigmoid, norm_topk, G + (size_t)t * E, ids + (size_t)t * Kext,
              s + (size_t)t * Kext, w + (size_t)t * K, q + (size_t)t * Kext);
}

/*
 * Which lifecycle path a forward takes for the support ([T] cold / hot-update /
 * hot-skip): 1 = cold (no support built in this block yet), 2 = hot-update (some
 * position's current top-K expert lies outside the support), 0 = hot-skip.
 */
int orc_support_status(int M, int K, int Kext, const int32_t* ids, const uint8_t* inS,
                       int support_valid) {
  if (!support_valid) return 1;
#if ORC_MUTATE == 11
  const int n_checked = Kext;
#else
  const int n_checked = K;
#endif
  for (int t = 0; t < M; ++t)
    for (int k = 0; k < n_checked; ++k)
      if (!inS[ids[(size_t)t * Kext + k]]) return 2;
  return 0;
}

/* R_t = sum_{j<K} W_{t,j}  and  C_t(S) = sum_{j<K_ext, I_{t,j} in S} W_{t,j}  ([T] Expert Atlas) */
static void coverage(int M, int K, int Kext, const int32_t* ids, const int64_t* q,
                     const uint8_t* inS, int64_t* R, int64_t* C) {
  for (int t = 0; t < M; ++t) {
    int64_t r = 0, c = 0;
    for (int j = 0; j < K; ++j) r += q[(size_t)t * Kext + j];
    for (int j = 0; j < Kext; ++j)
      if (inS[ids[(size_t)t * Kext + j]]) c += q[(size_t)t * Kext + j];
    R[t] = r;
    C[t] = c;
  }
}

/* |U| with U = { t : C_t(S) < alpha R_t }  ([T] Expert Atlas, the U_l equation) */
int64_t orc_under_covered(int M, int K, int Kext, const int32_t* ids, const int64_t* q,
                          const uint8_t* inS, int alpha_num, int alpha_den) {
  int64_t* R = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
  int64_t* C = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
  coverage(M, K, Kext, ids, q, inS, R, C);
  int64_t n = 0;
  for (int t = 0; t < M; ++t)
#if ORC_MUTATE == 12
    if ((int64_t)alpha_den * C[t] <= (int64_t)alpha_num * R[t]) ++n;
#else
    if ((int64_t)alpha_den * C[t] < (int64_t)alpha_num * R[t]) ++n;
#endif
  free(R);
  free(C);
  return n;
}

/*
 * Expert Atlas support construction ([T] Expert Atlas, steps one and two, and the
 * coverage goal |U_l| <= (1 - q) N).  Integer form: W = q_{t,j} (units of 2^-16),
 * alpha, q and beta as rationals, so every comparison is exact.
 *   (i)   p_e = sum_{t,j: I_{t,j}=e} W_{t,j}; start from the top-B experts by p_e
 *         (p desc, id asc), taking only experts with p_e > 0.
 *   (ii)  while |U| > (1 - q) M: for every e outside S,
 *           G_e = sum_{t in U, j: I_{t,j}=e} min(W_{t,j}, r_t - C_t)
 *           H_e = #{t in U : C_t + W_{t,j} >= r_t}
 *           score_e = H_e + beta G_e
 *         (scaled by alpha_den * Q * beta_den to stay integral), add up to c experts
 *         with positive score (score desc, id asc); stop when none is positive.
 *   (iii) closure: every expert some position selects in its top-K joins S, since
 *         routing here is over all experts and every selected expert needs a slot.
 *   (iv)  slots: S sorted by expert id; slot_of[e] = rank in S or -1.
 * stats: [0] final |U| (before closure), [1] repair rounds, [2] coverage unmet,
 *        [3] initial size, [4] size before closure.  Returns |S|.
 */
static int support_build(int M, int E, int K, int Kext, const int32_t* ids, const int64_t* q,
                         int B, int c, int alpha_num, int alpha_den, int q_num, int q_den,
                         int beta_num, int beta_den, int closure, uint8_t* inS, int32_t* slot_of,
                         int32_t* S_list, int64_t* stats) {
  const int64_t an = alpha_num, ad = alpha_den, qn = q_num, qd = q_den;
  const int64_t bn = beta_num, bd = beta_den;
  int64_t* p = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* Ge = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* He = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* score = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  uint8_t* pick = (uint8_t*)calloc((size_t)E, 1);
  int64_t* R = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
  int64_t* C = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));

  /* (i) popularity and the initial top-B set */
  for (int t = 0; t < M; ++t)
    for (int j = 0; j < Kext; ++j) p[ids[(size_t)t * Kext + j]] += q[(size_t)t * Kext + j];
  memset(inS, 0, (size_t)E);
  int npos = 0;
  for (int e = 0; e < E; ++e) npos += p[e] > 0;
  int n_init = B < npos ? B : npos;
  for (int r = 0; r < n_init; ++r) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!inS[e] && p[e] > 0 && (best < 0 || p[e] > p[best])) best = e; /* ties: lower id */
    inS[best] = 1;
  }

  /* (ii) greedy repair of under-covered positions */
  coverage(M, K, Kext, ids, q, inS, R, C);
  int64_t nU = 0;
  for (int t = 0; t < M; ++t) nU += (ad * C[t] < an * R[t]);
  int64_t rounds = 0, unmet = 0;
  while (qd * nU > (qd - qn) * (int64_t)M) {
    memset(Ge, 0, sizeof(int64_t) * (size_t)E);
    memset(He, 0, sizeof(int64_t) * (size_t)E);
    for (int t = 0; t < M; ++t) {
      if (!(ad * C[t] < an * R[t])) continue;
      int64_t gap = an * R[t] - ad * C[t]; /* (r_t - C_t) scaled by alpha_den */
      for (int j = 0; j < Kext; ++j) {
        int e = ids[(size_t)t * Kext + j];
        if (inS[e]) continue;
        int64_t v = ad * q[(size_t)t * Kext + j];
        Ge[e] += v < gap ? v : gap;
#if ORC_MUTATE == 7
        if (ad * (C[t] + q[(size_t)t * Kext + j]) > an * R[t]) He[e] += 1;
#else
        if (ad * (C[t] + q[(size_t)t * Kext + j]) >= an * R[t]) He[e] += 1;
#endif
      }
    }
    for (int e = 0; e < E; ++e) score[e] = bd * He[e] * ad * ATLAS_Q + bn * Ge[e];
    memset(pick, 0, (size_t)E);
    int added = 0;
    for (int r = 0; r < c; ++r) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!inS[e] && !pick[e] && score[e] > 0 && (best < 0 || score[e] > score[best])) best = e;
      if (best < 0) break;
      pick[best] = 1;
      ++added;
    }
    if (!added) {
      unmet = 1;
      break;
    }
    for (int e = 0; e < E; ++e)
      if (pick[e]) inS[e] = 1;
    ++rounds;
    coverage(M, K, Kext, ids, q, inS, R, C);
    nU = 0;
    for (int t = 0; t < M; ++t) nU += (ad * C[t] < an * R[t]);
  }
  int size_before = 0;
  for (int e = 0; e < E; ++e) size_before += inS[e];

  /* (iii) closure over the current top-K selections */
  if (closure)
    for (int t = 0; t < M; ++t)
      for (int k = 0; k < K; ++k) inS[ids[(size_t)t * Kext + k]] = 1;

  /* (iv) slots in expert-id order */
  int n = 0;
  for (int e = 0; e < E; ++e) {
    if (inS[e]) {
      slot_of[e] = n;
      S_list[n] = e;
      ++n;
    } else {
      slot_of[e] = -1;
    }
  }
  if (stats) {
    stats[0] = nU;
    stats[1] = rounds;
    stats[2] = unmet;
    stats[3] = n_init;
    stats[4] = size_before;
  }
  free(p);
  free(Ge);
  free(He);
  free(score);
  free(pick);
  free(R);
  free(C);
  return n;
}

/* The support with the closure (iii): routing over all experts (the exact mode). */
int orc_support_build(int M, int E, int K, int Kext, const int32_t* ids, const int64_t* q, int B,
                      int c, int alpha_num, int alpha_den, int q_num, int q_den, int beta_num,
                      int beta_den, uint8_t* inS, int32_t* slot_of, int32_t* S_list,
                      int64_t* stats) {
  return support_build(M, E, K, Kext, ids, q, B, c, alpha_num, alpha_den, q_num, q_den, beta_num,
                       beta_den, 1, inS, slot_of, S_list, stats);
}

/*
 * The Atlas support alone, steps (i), (ii) and (iv) without the closure: the set of
 * selectable experts of support-restricted routing ([T] Expert Atlas, third step: the hot
 * path keeps the support mask and selects each position's experts inside it).
 */
int orc_atlas_build(int M, int E, int K, int Kext, const int32_t* ids, const int64_t* q, int B,
                    int c, int alpha_num, int alpha_den, int q_num, int q_den, int beta_num,
                    int beta_den, uint8_t* inA, int32_t* slot_of, int32_t* S_list,
                    int64_t* stats) {
  return support_build(M, E, K, Kext, ids, q, B, c, alpha_num, alpha_den, q_num, q_den, beta_num,
                       beta_den, 0, inA, slot_of, S_list, stats);
}

/*
 * Support-restricted top-K ([T] Expert Atlas, third step): the same selection rule as
 * orc_route (key: logit desc, expert id asc) over the experts e with inA[e] = 1 only; the
 * gate score of a selected expert keeps its definition over all E experts (softmax over
 * all E, or sigmoid); the weights are the selected scores, normalised over the K selected
 * when norm_topk.  Needs at least K experts in the support.  rids, rw: [M x K].
 */
int orc_route_restricted(int M, int E, int K, int gate_sigmoid, int norm_topk, const float* G,
                         const uint8_t* allowed, int32_t* rids, double* rw) {
  int n_short = 0;
  for (int t = 0; t < M; ++t) {
    int n = 0;
    for (int e = 0; e < E; ++e) n += allowed[(size_t)t * E + e] != 0;
    n_short += n < K;
  }
  if (n_short) return n_short;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < M; ++t) {
    const float* g = G + (size_t)t * E;
    const uint8_t* inA = allowed + (size_t)t * E;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    double zmax = -INFINITY, z = 0.0;
    if (!gate_sigmoid) {
      for (int e = 0; e < E; ++e) zmax = fmax(zmax, (double)g[e]);
      for (int e = 0; e < E; ++e) z += exp((double)g[e] - zmax);
    }
    double sk[64];
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int e = 0; e < E; ++e)
#if ORC_MUTATE == 8
        if (!taken[e] && (best < 0 || before(g[e], e, g[best], best))) best = e;
#else
        if (inA[e] && !taken[e] && (best < 0 || before(g[e], e, g[best], best))) best = e;
#endif
      taken[best] = 1;
      rids[(size_t)t * K + k] = best;
      const double ge = (double)g[best];
      sk[k] = gate_sigmoid ? 1.0 / (1.0 + exp(-ge)) : exp(ge - zmax) / z;
    }
    free(taken);
    double denom = 0.0;
    for (int k = 0; k < K; ++k) denom += sk[k];
    for (int k = 0; k < K; ++k) rw[(size_t)t * K + k] = norm_topk ? sk[k] / denom : sk[k];
  }
  return 0;
}

/*
 * Group-limited selectable set ([T] Expert Atlas, step three: routing there applies the
 * model's own grouped expert selection, restricted to the experts of the support).
 * Experts form n_group contiguous groups of E / n_group ids.  Among the experts that base
 * allows (base = NULL: all; else a [E] support mask), a group is ranked by its best expert
 * under the selection key (logit desc, id asc), groups without an allowed expert last; the
 * first topk_group groups are kept.  allowed[t][e] = base[e] and e's group kept for row t.
 */
void orc_group_allowed(int M, int E, int n_group, int topk_group, const float* G,
                       const uint8_t* base, uint8_t* allowed) {
  const int gs = E / n_group;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < M; ++t) {
    const float* g = G + (size_t)t * E;
    int* best = (int*)malloc(sizeof(int) * (size_t)n_group);
    unsigned char* kept = (unsigned char*)calloc((size_t)n_group, 1);
    for (int gr = 0; gr < n_group; ++gr) {
      best[gr] = -1;
      for (int e = gr * gs; e < (gr + 1) * gs; ++e)
        if ((!base || base[e]) && (best[gr] < 0 || before(g[e], e, g[best[gr]], best[gr])))
          best[gr] = e;
    }
    for (int r = 0; r < topk_group; ++r) {
      int pick = -1;
      for (int gr = 0; gr < n_group; ++gr) {
        if (kept[gr] || best[gr] < 0) continue;
#if ORC_MUTATE == 9
        /* planted: a group ranked by its first allowed expert instead of its best */
        int fg = -1, fp = -1;
        for (int e = gr * gs; e < (gr + 1) * gs && fg < 0; ++e)
          if (!base || base[e]) fg = e;
        if (pick >= 0)
          for (int e = pick * gs; e < (pick + 1) * gs && fp < 0; ++e)
            if (!base || base[e]) fp = e;
        if (pick < 0 || before(g[fg], fg, g[fp], fp)) pick = gr;
#else
        if (pick < 0 || before(g[best[gr]], best[gr], g[best[pick]], best[pick])) pick = gr;
#endif
      }
      if (pick < 0) break;
      kept[pick] = 1;
    }
    for (int e = 0; e < E; ++e)
      allowed[(size_t)t * E + e] = (uint8_t)((!base || base[e]) && kept[e / gs]);
    free(best);
    free(kept);
  }
}

/*
 * Fresh set F_i ([T] Liveness-Shard Parallelism: Z_i = D_i ∩ D_{i-1}, N_i = D_i \ D_{i-1},
 * F_i = all on cache miss or refresh due, else not Z_i; newly decoded positions run
 * fresh once; [T] refresh period: 0 <= age <= M_C - 1, so a cached row is reused only
 * while iter - last_fresh <= R - 1; [T] cold/hot paths: a liveness-transition anomaly
 * falls back to a full fresh pass).  Per position t:
 *   fresh = anomaly or force_t or not valid_t or not (D_i[t] and D_{i-1}[t])
 *           or iter - last_fresh_t >= R
 * where anomaly = some position decoded in the previous forward is live again.
 * Returns the anomaly flag.
 */
int orc_fresh_set(int M, int R, int iter, const uint8_t* valid, const int32_t* last_fresh,
                  const uint8_t* prev_D, const uint8_t* D, const uint8_t* force, uint8_t* fresh) {
  int anomaly = 0;
  for (int t = 0; t < M; ++t)
    if (prev_D[t] && !D[t]) anomaly = 1;
  for (int t = 0; t < M; ++t) {
    int stable = D[t] && prev_D[t];
    int miss = !valid[t];
#if ORC_MUTATE == 5
    int due = 0;
#else
    int due = (int64_t)iter - (int64_t)last_fresh[t] >= (int64_t)R;
#endif
    int forced = force ? force[t] != 0 : 0;
    fresh[t] = (uint8_t)(anomaly || forced || miss || !stable || due);
  }
  return anomaly;
}

/*
 * Fresh token-expert worklist ([P1] "fresh token--expert worklist"; [T] FreshLane
 * pack and count steps; [T] LSP: B_i = Compact(H, F_i)).  Pairs (t, k) for fresh t and
 * k < K, ordered by (expert id, position); per-slot exclusive offsets; inv[t*K + k] is
 * the pair index or -1 when t is not fresh.  Returns the pair count P.
 */
int orc_worklist(int M, int K, int Kext, const int32_t* ids, const double* w,
                 const uint8_t* fresh, const int32_t* slot_of, int nS, int32_t* wl_pos,
                 int32_t* wl_k, double* wl_w, int32_t* offs, int32_t* inv) {
  /* every routed expert of a fresh position needs a slot (the support covers every
     selected expert); -1 reports a selection outside the slot set */
  for (int t = 0; t < M; ++t)
    if (fresh[t])
      for (int k = 0; k < K; ++k) {
        const int e = ids[(size_t)t * Kext + k];
        if (slot_of[e] < 0 || slot_of[e] >= nS) return -1;
      }
  int32_t* cursor = (int32_t*)calloc((size_t)(nS > 0 ? nS : 1), sizeof(int32_t));
  for (int s = 0; s <= nS; ++s) offs[s] = 0;
  for (int t = 0; t < M; ++t)
    if (fresh[t])
      for (int k = 0; k < K; ++k) offs[slot_of[ids[(size_t)t * Kext + k]] + 1] += 1;
  for (int s = 0; s < nS; ++s) offs[s + 1] += offs[s];
  for (int s = 0; s < nS; ++s) cursor[s] = offs[s];
#if ORC_MUTATE == 6
  /* planted: position-major order instead of expert-major */
  int p = 0;
  for (int t = 0; t < M; ++t)
    for (int k = 0; k < K; ++k) {
      inv[(size_t)t * K + k] = -1;
      if (!fresh[t]) continue;
      wl_pos[p] = t;
      wl_k[p] = k;
      wl_w[p] = w[(size_t)t * K + k];
      inv[(size_t)t * K + k] = p++;
    }
#else
  for (int t = 0; t < M; ++t) {
    for (int k = 0; k < K; ++k) {
      inv[(size_t)t * K + k] = -1;
      if (!fresh[t]) continue;
      int s = slot_of[ids[(size_t)t * Kext + k]];
      int p = cursor[s]++;
      wl_pos[p] = t;
      wl_k[p] = k;
      wl_w[p] = w[(size_t)t * K + k];
      inv[(size_t)t * K + k] = p;
    }
  }
#endif
  free(cursor);
  return offs[nS];
}

/*
 * One SwiGLU expert E_e(x) ([T] MoE bottleneck, E_e in the MoE equation; the expert
 * MLP of the fused-MoE kernel): g = W1 x, u = W3 x, h = silu(g) * u, y = W2 h, with
 * silu(z) = z / (1 + e^{-z}).  W1, W3 are [I x H] and W2 is [H x I], row-major.
 */
void orc_expert(int H, int I, int act_bf16, const void* x_row, const void* W1e, const void* W3e,
                const void* W2e, double* y) {
  double* hbuf = (double*)malloc(sizeof(double) * (size_t)(I > 0 ? I : 1));
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      double xv = ld(x_row, act_bf16, (size_t)h);
      g += xv * ld(W1e, act_bf16, (size_t)i * H + h);
      u += xv * ld(W3e, act_bf16, (size_t)i * H + h);
    }
#if ORC_MUTATE == 3
    hbuf[i] = g / (1.0 + exp(g)) * u;
#else
    hbuf[i] = g / (1.0 + exp(-g)) * u;
#endif
  }
  for (int j = 0; j < H; ++j) {
    double acc = 0.0;
    for (int i = 0; i < I; ++i)
#if ORC_MUTATE == 2
      acc += ld(W2e, act_bf16, (size_t)(i % H) * I + (size_t)(j % I)) * hbuf[i];
#else
      acc += ld(W2e, act_bf16, (size_t)j * I + i) * hbuf[i];
#endif
    y[j] = acc;
  }
  free(hbuf);
}

/*
 * Routed output, stale merge and dense restore for a list of rows ([T] LSP:
 * Y_F = SparseMoE(B_i, S_l), Y[F] = Y_F, Y[not F] = C_l[not F]; the cache stores the
 * routed-expert output, not the layer output; LSP leaves the shared expert alone, so
 * it runs for every position).  For each listed row t:
 *   fresh t:  R_t = sum_{k<K} w_{t,k} E_{I_{t,k}}(x_t), summed in k order; cache[t] = R_t
 *   stable t: R_t = cache[t]
 *   Y_t = R_t + S(x_t) (shared expert with weight 1, if present), else Y_t = R_t.
 * R_out / Y_out are [n_rows x H] in list order.
 */
void orc_moe_rows(int M, int H, int I, int Is, int E, int K, int Kext, int act_bf16,
                  const void* x, const int32_t* ids, const double* w, const uint8_t* fresh,
                  const void* W1, const void* W3, const void* W2, const void* SW1,
                  const void* SW3, const void* SW2, int n_rows, const int32_t* rows,
                  double* cache, double* R_out, double* Y_out) {
  (void)M;
  (void)E;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < n_rows; ++r) {
    int t = rows[r];
    const void* xt = offset(x, act_bf16, (size_t)t * H);
    double* Rt = R_out + (size_t)r * H;
    double* yt = (double*)malloc(sizeof(double) * (size_t)H);
    if (fresh[t]) {
      for (int j = 0; j < H; ++j) Rt[j] = 0.0;
      for (int k = 0; k < K; ++k) {
        int e = ids[(size_t)t * Kext + k];
        size_t ew = (size_t)e * I * H;
        orc_expert(H, I, act_bf16, xt, offset(W1, act_bf16, ew), offset(W3, act_bf16, ew),
                   offset(W2, act_bf16, ew), yt);
        double wk = w[(size_t)t * K + k];
        for (int j = 0; j < H; ++j) Rt[j] += wk * yt[j];
      }
      for (int j = 0; j < H; ++j) cache[(size_t)t * H + j] = Rt[j];
    } else {
      for (int j = 0; j < H; ++j) Rt[j] = cache[(size_t)t * H + j];
    }
    double* Yt = Y_out + (size_t)r * H;
    if (SW1) {
      orc_expert(H, Is, act_bf16, xt, SW1, SW3, SW2, yt);
      for (int j = 0; j < H; ++j) Yt[j] = Rt[j] + yt[j];
    } else {
      for (int j = 0; j < H; ++j) Yt[j] = Rt[j];
    }
    free(yt);
  }
}

/*
 * Cache commit after a forward ([T] LSP state machine: newly decoded -> fresh once ->
 * cache update; [T] refresh period: age restarts at a fresh write): fresh rows become
 * valid with last_fresh = iter; the decoded set seen by this forward becomes D_{i-1}.
 */
void orc_commit(int M, int iter, const uint8_t* fresh, const uint8_t* D, uint8_t* valid,
                int32_t* last_fresh, uint8_t* prev_D) {
  for (int t = 0; t < M; ++t) {
    if (fresh[t]) {
      valid[t] = 1;
      last_fresh[t] = iter;
    }
    prev_D[t] = D[t];
  }
}

/*
 * Brute-force dense MoE layer ([T] MoE bottleneck equation, evaluated literally):
 * every expert is evaluated on every position, and the routed output keeps the
 * top-K of them: R_t = sum_e 1[e in TopK_t] w_{t,e} E_e(x_t); Y_t = R_t + S(x_t).
 * The gate is computed from scratch here (fp32 logits, key (G desc, id asc)).
 */
void orc_dense_moe(int M, int H, int I, int Is, int E, int K, int gate_sigmoid, int norm_topk,
                   int act_bf16, const void* x, const float* Wg, const float* bias,
                   const void* W1, const void* W3, const void* W2, const void* SW1,
                   const void* SW3, const void* SW2, double* R_out, double* Y_out) {
#pragma omp parallel for schedule(dynamic)
  for (int t = 0; t < M; ++t) {
    const void* xt = offset(x, act_bf16, (size_t)t * H);
    float* g = (float*)malloc(sizeof(float) * (size_t)E);
    double* all = (double*)malloc(sizeof(double) * (size_t)E * H);
    double* sc = (double*)malloc(sizeof(double) * (size_t)E);
    uint8_t* top = (uint8_t*)calloc((size_t)E, 1);
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += ld(xt, act_bf16, (size_t)h) * (double)Wg[(size_t)e * H + h];
      if (bias) acc += (double)bias[e];
      g[e] = (float)acc;
      size_t ew = (size_t)e * I * H;
      orc_expert(H, I, act_bf16, xt, offset(W1, act_bf16, ew), offset(W3, act_bf16, ew),
                 offset(W2, act_bf16, ew), all + (size_t)e * H);
    }
    /* membership in the top-K: e is in it iff fewer than K experts precede it */
    for (int e = 0; e < E; ++e) {
      int ahead = 0;
      for (int f = 0; f < E; ++f)
        if (g[f] > g[e] || (g[f] == g[e] && f < e)) ++ahead;
      top[e] = ahead < K;
    }
    double zmax = -INFINITY, z = 0.0;
    for (int e = 0; e < E; ++e) zmax = fmax(zmax, (double)g[e]);
    for (int e = 0; e < E; ++e) z += exp((double)g[e] - zmax);
    double tot = 0.0;
    for (int e = 0; e < E; ++e) {
      sc[e] = gate_sigmoid ? 1.0 / (1.0 + exp(-(double)g[e])) : exp((double)g[e] - zmax) / z;
      if (top[e]) tot += sc[e];
    }
    double* Rt = R_out + (size_t)t * H;
    for (int j = 0; j < H; ++j) Rt[j] = 0.0;
    for (int e = 0; e < E; ++e) {
      if (!top[e]) continue;
      double we = norm_topk ? sc[e] / tot : sc[e];
      for (int j = 0; j < H; ++j) Rt[j] += we * all[(size_t)e * H + j];
    }
    double* Yt = Y_out + (size_t)t * H;
    if (SW1) {
      double* ys = (double*)malloc(sizeof(double) * (size_t)H);
      orc_expert(H, Is, act_bf16, xt, SW1, SW3, SW2, ys);
      for (int j = 0; j < H; ++j) Yt[j] = Rt[j] + ys[j];
      free(ys);
    } else {
      for (int j = 0; j < H; ++j) Yt[j] = Rt[j];
    }
    free(g);
    free(all);
    free(sc);
    free(top);
  }
}

/*
 * Live-only output decoding ([T] evaluation setup: greedy threshold decoding with commit
 * threshold tau = 0.95, only live positions decoded; [T] LSP section: live logits z_{i,t} and
 * their commit / no-commit decision).  For every live position t (D[t] = 0) of the block
 * batch (t = b * block + p):
 *   z_v = sum_h h[t,h] W[v,h]  (double)          top token v* = argmax z (lower id on ties)
 *   conf_t = max_v softmax(z)_v = 1 / sum_v exp(z_v - z_{v*})
 *   gap_t = z_{v*} - (second largest z)           (for reporting near ties)
 * Commit: every live t with conf_t >= tau; a sequence b none of whose live positions reaches
 * tau commits its single most confident live position (lower position on ties), so every
 * refinement step decodes at least one position of a sequence that still has live ones.
 * D_next = D with the commits set; token[t] = v* for committed t (others left unchanged).
 * conf / gap are written for live positions (0 elsewhere).  Returns the number of commits.
 */
int orc_live_decode(int M, int H, int V, int block, int act_bf16, const void* h, const void* Wv,
                    const uint8_t* D, double tau, uint8_t* D_next, int32_t* token, double* conf,
                    double* gap, int32_t* top) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < M; ++t) {
    conf[t] = 0.0;
    gap[t] = 0.0;
    top[t] = -1;
    if (D[t]) continue;
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    int best = 0;
    for (int v = 0; v < V; ++v) {
      double acc = 0.0;
      for (int k = 0; k < H; ++k)
        acc += ld(h, act_bf16, (size_t)t * H + k) * ld(Wv, act_bf16, (size_t)v * H + k);
      z[v] = acc;
#if ORC_MUTATE == 10
      if (acc >= z[best]) best = v; /* planted: ties toward the higher token id */
#else
      if (acc > z[best]) best = v;
#endif
    }
    double second = -INFINITY, Z = 0.0;
    for (int v = 0; v < V; ++v) {
      if (v != best && z[v] > second) second = z[v];
      Z += exp(z[v] - z[best]);
    }
    top[t] = best;
    conf[t] = 1.0 / Z;
    gap[t] = V > 1 ? z[best] - second : INFINITY;
    free(z);
  }
  int commits = 0;
  for (int t = 0; t < M; ++t) D_next[t] = D[t];
  const int nb = M / block;
  for (int b = 0; b < nb; ++b) {
    int any = 0, arg = -1;
    for (int p = 0; p < block; ++p) {
      const int t = b * block + p;
      if (D[t]) continue;
      if (conf[t] >= tau) {
        D_next[t] = 1;
        token[t] = top[t];
        ++commits;
        any = 1;
      }
      if (arg < 0 || conf[t] > conf[arg]) arg = t;
    }
    if (!any && arg >= 0) {
      D_next[arg] = 1;
      token[arg] = top[arg];
      ++commits;
    }
  }
  return commits;
}
