/*
 * epoch.h -- C ABI of the liveness-sparse routed-expert MoE layer forward on MI355X (gfx950).
 *
 * The operation is the MoE layer of a block-diffusion language model during one
 * refinement iteration, as described by "Epoch: Compiling Diffusion Blocks for
 * Sparse MoE Serving" (abstract) and the pinghaoyang.com.cn teardown of it
 * ("Epoch 完全拆解"):
 *   - route: gate logits recomputed over every block position every iteration
 *     (abstract; teardown, Expert Atlas section, the G equation and step three);
 *   - support: a coverage-driven active expert set per layer, built on the block
 *     clock (teardown, Expert Atlas, steps one and two; "cold / hot-update /
 *     hot-skip" section);
 *   - fresh set: live, newly decoded and refresh-due positions (teardown,
 *     Liveness-Shard Parallelism, the Z_i / N_i / F_i equations; refresh-period
 *     section, the age bound);
 *   - worklist, expert compute, combine and dense restore (teardown, LSP
 *     equations B_i = Compact(H, F_i), Y[F] = Y_F, Y[not F] = C_l[not F];
 *     FreshLane steps pack, light expert kernel, combine, scatter/merge).
 * Routing is over all experts by default (the support is then a compact layout and
 * a rebuild trigger); with EPOCH_ROUTING_RESTRICTED each position's top-K is taken
 * inside the layer's support, as in the teardown's Expert Atlas step three.  One GPU
 * holds every expert, so no collective is involved.
 *
 * Conventions for every call:
 *   - Positions: M = batch * block, position t = b * block + p.  Tensors are dense,
 *     row-major and contiguous.  "act" is the activation / expert-weight dtype of
 *     the descriptor: bf16 (raw 16-bit bfloat16) or fp32.
 *   - Device pointers must be 16-byte aligned.  The caller owns every device
 *     buffer (weights, inputs, outputs, workspace); the library never allocates
 *     device memory (its one device array, the scratch of epoch_live_decode_static,
 *     is part of the loaded code object).  The only allocations are host-side: the
 *     plan object, three
 *     events per plan for shapes with a shared expert or compute-bound routed tiles
 *     (created by epoch_block_plan_build, released by epoch_block_plan_destroy), and
 *     one side stream per device for the whole process (default priority, created at
 *     the first plan build on that device that needs it, never destroyed).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     only enqueue work on it: no host synchronisation, no host<->device copies.
 *     A forward with a shared expert forks that expert onto the device's side
 *     stream (an event recorded on `stream`) and joins it back before the combine,
 *     so all of its work is still ordered after earlier work on `stream` and before
 *     later work on it (graph capture of `stream` captures both branches).  Plans of
 *     one device share the side stream, so their side work runs in submission order.
 *   - Return value: EPOCH_OK (0) or a negative EPOCH_E_* code; nothing is enqueued
 *     when a call fails its argument checks.  A kernel fault surfaces at the
 *     caller's next synchronisation of the stream.
 *   - A plan is not thread-safe; use one stream at a time per plan.
 */
#ifndef EPOCH_H
#define EPOCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  EPOCH_OK = 0,
  EPOCH_E_NULL = -1,      /* a required pointer is NULL */
  EPOCH_E_SHAPE = -2,     /* descriptor values out of the supported range */
  EPOCH_E_DTYPE = -3,     /* unknown dtype or gate */
  EPOCH_E_WORKSPACE = -4, /* workspace too small or misaligned */
  EPOCH_E_LAYER = -5,     /* layer index out of range */
  EPOCH_E_STATE = -6,     /* commit without a preceding forward of that layer */
  EPOCH_E_HIP = -7,       /* a kernel launch failed */
  EPOCH_E_ALIGN = -8,     /* a tensor pointer is not 16-byte aligned */
  EPOCH_E_SCRATCH = -9    /* the call needs more scratch than the library's static array holds */
};

enum { EPOCH_GATE_SOFTMAX = 0, EPOCH_GATE_SIGMOID = 1 };
enum { EPOCH_DTYPE_F32 = 0, EPOCH_DTYPE_BF16 = 1 };
/* Routing modes (epoch_desc.routing):
 *   EXACT: every position's top-K over all E experts.  The support is the Atlas set plus
 *     every routed expert (closure); it is rebuilt at the block's first forward (cold) and
 *     whenever a routed expert falls outside it (hot-update).
 *   RESTRICTED: the support is the Atlas set alone (no closure), and a forward that keeps it
 *     (hot-skip) routes each position to the top-K experts inside it (teardown, Expert
 *     Atlas, step three: ids, order and weights still change every iteration; scores keep
 *     their definition over all E).  Every forward still ranks the K_ext candidates over
 *     all experts; the support is rebuilt from them at the first forward (cold), after
 *     atlas_period iterations (if > 0), or when they show it misses the coverage goal
 *     |U| <= (1 - q) M or holds fewer than K experts (hot-update; the block-plan
 *     lifecycle and its fallback to the full path).  A forward that rebuilds routes over
 *     all experts, giving the routed experts outside the support slots for that forward. */
enum { EPOCH_ROUTING_EXACT = 0, EPOCH_ROUTING_RESTRICTED = 1 };

/* Per-layer counters, int64, readable through epoch_plan_inspect().counters. */
enum {
  EPOCH_CNT_COLD = 0,          /* forwards that built the support for the first time in the block */
  EPOCH_CNT_HOT_UPDATE = 1,    /* forwards that rebuilt it because a top-K expert left it */
  EPOCH_CNT_HOT_SKIP = 2,      /* forwards that reused it */
  EPOCH_CNT_ANOMALY = 3,       /* forwards that fell back to all-fresh (decoded -> live) */
  EPOCH_CNT_FRESH_ROWS = 4,    /* sum over forwards of |F| */
  EPOCH_CNT_PAIRS = 5,         /* sum over forwards of fresh token-expert pairs */
  EPOCH_CNT_UNMET = 6,         /* support builds that stopped before the coverage goal */
  EPOCH_CNT_FORCED_ROWS = 7,   /* sum of rows fresh because of force_fresh */
  EPOCH_CNT_DUE_ROWS = 8,      /* sum of rows fresh because their cached output reached age R */
  EPOCH_CNT_SUPPORT_SIZE = 9,  /* |S| after the latest build */
  EPOCH_CNT_U_FINAL = 10,      /* under-covered positions after the latest build's repair */
  EPOCH_CNT_REPAIR_ROUNDS = 11,/* sum of greedy repair rounds */
  EPOCH_CNT_TOUCHED = 12,      /* sum over forwards of experts with at least one fresh pair */
  EPOCH_CNT_FORWARDS = 13,
  EPOCH_CNT_RESERVED14 = 14,   /* unused: the commit count is epoch_inspect.iteration */
  EPOCH_CNT_RESTRICTED = 15,   /* forwards routed inside the support (restricted mode) */
  EPOCH_CNT_COVERAGE_FALLBACK = 16, /* restricted-mode rebuilds forced by the coverage check */
  EPOCH_CNT_PERIOD_UPDATE = 17,/* restricted-mode rebuilds forced by atlas_period */
  EPOCH_CNT_BIG_EXPERTS = 18,  /* sum over forwards of experts run on 256-row compute-bound tiles */
  EPOCH_CNT_BIG_PAIRS = 19,    /* sum over forwards of those experts' fresh pairs */
  EPOCH_NUM_COUNTERS = 20
};

typedef struct epoch_desc {
  /* shape */
  int32_t n_layers;     /* >= 1 */
  int32_t hidden;       /* H: multiple of 64, <= 16384 */
  int32_t n_experts;    /* E: 1..1024 */
  int32_t top_k;        /* K: 1..min(E, 16) */
  int32_t inter;        /* I: expert SwiGLU width; multiple of 64 for bf16 */
  int32_t n_shared;     /* 0 or 1 always-on shared expert */
  int32_t shared_inter; /* I_s of the shared expert (multiple of 64 for bf16), ignored if n_shared = 0 */
  int32_t batch;        /* sequences in the block batch */
  int32_t block;        /* positions per diffusion block */
  /* gate */
  int32_t gate;         /* EPOCH_GATE_SOFTMAX (softmax over all E) or EPOCH_GATE_SIGMOID */
  int32_t norm_topk;    /* 1: w_k = s_k / sum_{j<K} s_j; 0: w_k = s_k */
  int32_t act_dtype;    /* EPOCH_DTYPE_BF16 or EPOCH_DTYPE_F32 */
  /* bounded staleness: a cached routed output is reused while iter - last_fresh <= R - 1 */
  int32_t staleness_R;  /* >= 1; 1 = exact (every position fresh every iteration) */
  /* Expert Atlas planner (teardown, Expert Atlas): K_ext = min(K + m, E) candidates per
     position, initial top-B by popularity, at most c experts added per repair round,
     coverage floor alpha, goal fraction q, score weight beta, as rationals */
  int32_t atlas_m, atlas_B, atlas_c;
  int32_t alpha_num, alpha_den, q_num, q_den, beta_num, beta_den;
  int32_t flags;        /* reserved, must be 0 */
  int32_t routing;      /* EPOCH_ROUTING_EXACT or EPOCH_ROUTING_RESTRICTED */
  int32_t atlas_period; /* restricted mode: rebuild the support after this many iterations
                           (0 = only on the coverage check); must be 0 in exact mode */
  /* group-limited top-k (teardown, Expert Atlas step three, which names the model's own
     grouped selection rule without defining it): the experts form n_group contiguous
     groups of E / n_group ids; each position ranks the groups by their best expert
     (selection key: logit desc, id asc; in restricted mode among the support's experts)
     and selects its K_ext candidates and K routed experts among the experts of its
     topk_group best groups.  n_group <= 1: off.
     Otherwise 2 <= n_group <= 64, E % n_group == 0, 1 <= topk_group <= n_group and
     topk_group * E / n_group >= K_ext.  A restricted forward in which some position's
     groups hold fewer than K support experts routes over all experts (full path). */
  int32_t n_group;
  int32_t topk_group;
} epoch_desc;

/* Device pointers of one layer's weights; all row-major, contiguous, caller-owned and
   kept alive until the plan is destroyed. */
typedef struct epoch_layer_weights {
  const float* router_w; /* [E x H] fp32 gate weight */
  const float* router_b; /* [E] fp32 gate bias, added to the logits; NULL = none */
  const void* w1;        /* [E x I x H] act, gate projection */
  const void* w3;        /* [E x I x H] act, up projection */
  const void* w2;        /* [E x H x I] act, down projection */
  const void* sw1;       /* shared expert [I_s x H] act, or NULL when n_shared = 0 */
  const void* sw3;       /* [I_s x H] act */
  const void* sw2;       /* [H x I_s] act */
} epoch_layer_weights;

/* Device pointers into the workspace (read-only views for checks and statistics). */
typedef struct epoch_inspect {
  /* stage outputs of the most recent forward (of layer last_forward_layer) */
  const float* logits;        /* [M x E]  G = x W_g^T + b, fp32 */
  const int32_t* ids;         /* [M x K_ext] candidates, key (G desc, id asc); first K are routed */
  const float* scores;        /* [M x K_ext] gate score s (softmax prob. or sigmoid) */
  const int32_t* atlas_q;     /* [M x K_ext] planner weight floor(s * 2^16 + 1/2) */
  const float* weights;       /* [M x K] routing weights w */
  const uint8_t* fresh;       /* [M] 1 if position t ran fresh */
  const int32_t* fresh_list;  /* [n_fresh] fresh positions, ascending */
  const int32_t* n_fresh;     /* [1] */
  const int32_t* n_pairs;     /* [1] P = n_fresh * K */
  const int32_t* wl_pos;      /* [P] pair -> position, ordered by (expert, position) */
  const int32_t* wl_k;        /* [P] pair -> rank k in the position's top-K */
  const float* wl_w;          /* [P] pair -> routing weight */
  const int32_t* offs;        /* [|S| + 1] exclusive pair offsets per support slot */
  const int32_t* inv;         /* [M x K] (t, k) -> pair index, -1 if t is not fresh */
  const int32_t* routed_ids;  /* [M x K] experts the worklist used (= ids[:, :K] unless the
                                 forward routed inside the support) */
  const float* routed_w;      /* [M x K] their routing weights */
  /* per-layer state of the requested layer */
  const uint8_t* in_support;  /* [E] */
  const int32_t* slot_of;     /* [E] slot = rank of e in the sorted support, -1 outside */
  const int32_t* support;     /* [E] sorted support ids (first support_size valid) */
  const int32_t* support_size;/* [1] */
  const uint8_t* atlas;       /* [E] restricted mode: the Atlas support (no closure) */
  const void* cache;          /* [M x H] act: cached routed output C_l */
  const uint8_t* valid;       /* [M] cache row written in this block */
  const int32_t* last_fresh;  /* [M] iteration of the last fresh write */
  const uint8_t* prev_decoded;/* [M] D_{i-1} */
  const int64_t* counters;    /* [EPOCH_NUM_COUNTERS] */
  int32_t k_ext;
  int32_t iteration;          /* host-side iteration counter of the layer (commits so far) */
  int32_t last_forward_layer; /* -1 before the first forward */
} epoch_inspect;

typedef struct epoch_plan epoch_plan;

/* Bytes of device workspace a plan for `d` needs (caches, masks, support, worklist,
   expert intermediates, scratch).  Returns EPOCH_E_* for an invalid descriptor. */
int32_t epoch_plan_workspace_bytes(const epoch_desc* d, size_t* out_bytes);

/*
 * Block-plan build, the cold path (teardown, Two Clocks: the block plan holds ids,
 * versions and maps, never live values or weights; "cold / hot-update / hot-skip":
 * the cold path clears the per-block caches and prepares the per-layer metadata;
 * a plan is never reused across blocks).  Enqueues one init kernel that clears every
 * layer's cache validity, decoded set, last-fresh ages, support and counters.  The
 * support itself is built by the first forward of each layer, from that iteration's
 * logits.  `weights` is an array of n_layers structs (copied; the tensors are not).
 * `workspace` (device, >= epoch_plan_workspace_bytes, 256-byte aligned) is owned by
 * the caller and must outlive the plan.  On success *out_plan receives a new plan.
 */
int32_t epoch_block_plan_build(const epoch_desc* d, const epoch_layer_weights* weights,
                               void* workspace, size_t workspace_bytes, void* stream,
                               epoch_plan** out_plan);

/*
 * One layer, one refinement iteration (teardown, LSP state machine and equations;
 * FreshLane pack / light expert kernel / combine / scatter-merge):
 *   x         [M x H] act (device): the layer input of every position;
 *   decoded   [M] uint8 (device): D_i, 1 = committed token, 0 = still [Mask];
 *   force_fresh [M] uint8 (device) or NULL: rows forced through the fresh path;
 *   y         [M x H] act (device): the dense layer output, routed (+ shared) expert;
 *   y_routed  [M x H] act (device) or NULL: the routed part alone (fresh or cached).
 * Enqueues: gate + top-k over all positions; support check and (cold / hot-update)
 * rebuild; fresh set; expert-grouped worklist; grouped SwiGLU experts on the fresh
 * pairs; shared expert on all positions; weighted combine, stale-cache merge and
 * dense restore.  Writes the cache rows of fresh positions only and reads those of
 * stable positions, so repeating the call for the same iteration gives the same y.
 * A position decoded in the previous forward that is live again makes the whole
 * layer-iteration fresh (counted as an anomaly), as the pages prescribe.
 */
int32_t epoch_moe_fresh_forward(epoch_plan* plan, int32_t layer, const void* x,
                                const uint8_t* decoded, const uint8_t* force_fresh, void* y,
                                void* y_routed, void* stream);

/*
 * Cache commit of the layer's latest forward (teardown, LSP state machine: a fresh
 * output updates the cache; refresh-period section: the age restarts at a fresh
 * write): fresh rows become valid with last_fresh = iteration, D_i becomes D_{i-1},
 * and the layer's iteration counter advances.  EPOCH_E_STATE if the layer has no
 * forward since its last commit.  The forward already wrote this state into a second
 * copy of the per-position state (so that repeating a forward stays idempotent); the
 * commit makes that copy current on the host and enqueues nothing on `stream`.  It is
 * ordered after the forward by the stream the next forward runs on.
 */
int32_t epoch_cache_update(epoch_plan* plan, int32_t layer, void* stream);

/* Fills *out with device pointers to the plan's stage outputs and the layer's state.
   Enqueues nothing; read the buffers after synchronising the stream. */
int32_t epoch_plan_inspect(const epoch_plan* plan, int32_t layer, epoch_inspect* out);

/* Block end (teardown, Two Clocks: the block plan lives for one diffusion block and is
 * never carried into the next; a new block starts with a new build).  Frees the host-side
 * plan object and its events; the workspace stays the caller's.  Waits first for the
 * plan's latest work on the device's side stream.  NULL is a no-op. */
int32_t epoch_block_plan_destroy(epoch_plan* plan);

/* Static text for a status code. */
const char* epoch_status_string(int32_t status);

/*
 * Kernel timing for measurement.  `groups` is a bitmask of kernel groups (bit g = group g;
 * -1 = all): 0 router + top-k + fresh test, 1 plan (support check / build, worklist scans),
 * 2 worklist placement, 3 routed gate/up (weight-stream tiles), 4 routed down (weight-stream
 * tiles), 5 shared expert, 6 combine, 7 routed gate/up on 256-row compute-bound tiles, 8 routed
 * down on those tiles (7 and 8 only for shapes with big tiles).  While set, the kernels of every
 * selected group of each forward carry a pair of HIP events on the stream the group runs on
 * (the forward's stream, or the device's side stream for 5, 7 and 8), stamped by the dispatches
 * themselves: the start of the group's first kernel and the end of its last (events come from
 * a process-wide pool, so a measured region reuses events created earlier; a timed dispatch
 * still waits a few microseconds longer for its neighbours, so a measurement that must not
 * disturb the work can set the mask on some forwards only).  epoch_plan_timing synchronises the
 * recorded events, adds their durations (ms) and counts per group into the plan's sums,
 * writes the sums for up to n groups and returns the events to the pool.  Setting the mask
 * clears the sums.  0 = off (the default).
 */
enum { EPOCH_TIMING_GROUPS = 9 };
int32_t epoch_plan_set_timing(epoch_plan* plan, int32_t groups);
int32_t epoch_plan_timing(epoch_plan* plan, float* ms, int64_t* launches, int32_t n);

/* ------------------------------------------------------------------ live-only output decoding */

/* One refinement step's output decoding of the block batch. */
typedef struct epoch_decode_desc {
  int32_t batch;     /* sequences */
  int32_t block;     /* positions per sequence, <= 1024 */
  int32_t hidden;    /* H: multiple of 64 */
  int32_t vocab;     /* V: multiple of 128 */
  int32_t act_dtype; /* EPOCH_DTYPE_BF16 (the only dtype of this call) */
  int32_t flags;     /* reserved, must be 0 */
  double tau;        /* commit threshold on the top softmax probability, in (0, 1] */
} epoch_decode_desc;

/* Bytes of device workspace epoch_live_decode needs for `d` (live list, per-position
   live index, per-row partial reductions of max(min(M, 128) x V/128, M x ceil(V/256)) entries,
   per-position confidence and top token). */
int32_t epoch_decode_workspace_bytes(const epoch_decode_desc* d, size_t* out_bytes);

/*
 * Live-only output decoding (teardown, evaluation setup: greedy threshold decoding with
 * commit threshold tau; LSP section: only live positions reach the output decoding, and each
 * commit / no-commit decision is taken on the live logits z_{i,t}).  For every live position
 * t (decoded[t] = 0) of the block batch:
 *   z_v = sum_h h[t,h] w_vocab[v,h]  (bf16 products, fp32 accumulation on MFMA)
 *   top token = argmax_v z_v (lower id on ties);  conf_t = 1 / sum_v exp(z_v - max z)
 * Every live position with conf_t >= tau commits; a sequence none of whose live positions
 * reaches tau commits its most confident one (lower position on ties).
 *   h            [M x H] bf16 (device): the final hidden states of every position;
 *   w_vocab      [V x H] bf16 (device): the LM head;
 *   decoded      [M] u8 (device): D_i;
 *   decoded_next [M] u8 (device, written): D_{i+1} = D_i plus the commits;
 *   tokens       [M] i32 (device): written at the committed positions only;
 *   conf         [M] f32 (device, written, nullable): conf_t of live positions, 0 elsewhere;
 *   workspace    (device, 256-byte aligned, >= epoch_decode_workspace_bytes), caller-owned.
 * Decoded positions are never decoded again: their logits are not computed.  Errors as for
 * every call (EPOCH_E_DTYPE for a dtype other than bf16).
 */
int32_t epoch_live_decode(const epoch_decode_desc* d, const void* h, const void* w_vocab,
                          const uint8_t* decoded, uint8_t* decoded_next, int32_t* tokens,
                          float* conf, void* workspace, size_t workspace_bytes, void* stream);

/*
 * epoch_live_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same kernels and outputs as epoch_live_decode, with its scratch (live list,
 * per-row partial reductions, per-position confidences) in a device array of
 * EPOCH_DECODE_STATIC_SCRATCH_BYTES that the library holds on each device it runs on until
 * the process ends; the device address of that array is looked up once per device, at the
 * first call on it (with that device current).  The call allocates nothing and calls no
 * allocating routine.  A shape whose epoch_decode_workspace_bytes exceeds
 * EPOCH_DECODE_STATIC_SCRATCH_BYTES returns EPOCH_E_SCRATCH and enqueues nothing (for example
 * 2048 positions at a 131072-token vocabulary fit, 8192 do not).  Every call on a device uses
 * the same array: calls whose work overlaps on one device (unordered streams, several host
 * threads) race and give undefined results; order them on one stream.  The array keeps the
 * latest call's contents; every buffer in it is written before it is read, so nothing needs
 * clearing between calls.  Arguments and errors otherwise as for epoch_live_decode.
 */
enum { EPOCH_DECODE_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024 };
int32_t epoch_live_decode_static(const epoch_decode_desc* d, const void* h, const void* w_vocab,
                                 const uint8_t* decoded, uint8_t* decoded_next, int32_t* tokens,
                                 float* conf, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EPOCH_H */
