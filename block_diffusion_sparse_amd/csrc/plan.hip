// Block-clock and bookkeeping kernels: plan init, the per-iteration plan step (Expert Atlas
// support check / build and the worklist scans), stable worklist placement and the cache
// commit (gfx950).
#include "device_common.h"
#include "epoch_internal.h"

namespace epoch {

constexpr int32_t kNeverFresh = -(1 << 30);

// ---------------------------------------------------------------------------- plan init
// Cold path of the block plan (teardown, "cold / hot-update / hot-skip": clear the per-block
// caches, initialise the live set, prepare the per-layer metadata).  Cache rows are not
// touched: valid = 0 keeps them unread until a fresh write.
__global__ void k_init_layer(int M, int E, LayerState L) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < M) {
    L.valid[i] = 0;
    L.last_fresh[i] = kNeverFresh;
    L.prev_D[i] = 0;
    L.fresh[i] = 0;
  }
  if (i < E) {
    L.inS[i] = 0;
    L.slot_of[i] = -1;
    L.S_list[i] = 0;
    L.inA[i] = 0;
  }
  if (i < 4) L.A_state[i] = 0;
  if (i < EPOCH_NUM_COUNTERS) L.counters[i] = 0;
  if (i == 0) {
    *L.S_size = 0;
    *L.S_valid = 0;
  }
}

hipError_t launch_init_layer(const Shape& s, const LayerState& L, hipStream_t st) {
  const int n = max(max(s.M, s.E), (int)EPOCH_NUM_COUNTERS);
  launch(k_init_layer, dim3((n + 255) / 256), dim3(256), 0, st, s.M, s.E, L);
  return hipGetLastError();
}

// The per-forward accumulators start at zero once per plan; afterwards each forward leaves them
// at zero for the next: the plan step clears the per-chunk counts and the router flags after
// reading them.
__global__ void k_zero_i32(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_init_scratch(const Shape& s, const Scratch& W, hipStream_t st) {
  // cnt_f, cnt_a and chunk_fresh are carved back to back
  const int n = (int)(W.chunk_fresh + s.n_chunks - W.cnt_f);
  launch(k_zero_i32, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024), dim3(256), 0, st, W.cnt_f, n);
  launch(k_zero_i32, dim3(1), dim3(64), 0, st, W.flags, (int)FLAG_WORDS);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- plan step
constexpr int kPlanThreads = 1024;

constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS traffic): shifts
// by 1, 2, 4, 8 inside each row of 16 lanes, then each row's total carried into the rows
// after it (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).  Lanes whose
// source falls outside the row, or whose row the mask leaves out, add 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Inclusive scan over the workgroup, one value per thread (thread order); also returns the
// total.  wsum is kPlanWaves ints of LDS owned by the caller; two barriers, and a third on
// return so that wsum may be reused at once.
__device__ __forceinline__ int block_incl_scan(int v, int32_t* wsum, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kPlanWaves ? wsum[lane] : 0;
    w = wave_incl_scan(w);
    if (lane < kPlanWaves) wsum[lane] = w;
  }
  __syncthreads();
  const int r = inc + (wave ? wsum[wave - 1] : 0);
  *total = wsum[kPlanWaves - 1];
  __syncthreads();
  return r;
}

// Counter increments are device-scope atomics that return nothing, so the issuing wave never
// waits for them (a read-modify-write would hold every barrier after it for a memory round trip).
__device__ __forceinline__ void counter_add(const LayerState& L, int idx, long long v) {
  if (v) atomicAdd((unsigned long long*)&L.counters[idx], (unsigned long long)v);
}

// Inclusive scans of N values per thread over the workgroup at once (two barriers); msum is
// N x kPlanWaves ints of LDS owned by the caller, free again after the caller's next barrier.
template <int N>
__device__ __forceinline__ void block_multi_scan(int (&v)[N], int32_t (*msum)[kPlanWaves],
                                                 int (&total)[N]) {
  static_assert(N <= kPlanWaves, "one wave scans each column of wave sums");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int n = 0; n < N; ++n) v[n] = wave_incl_scan(v[n]);
  if (lane == 63)
#pragma unroll
    for (int n = 0; n < N; ++n) msum[n][wave] = v[n];
  __syncthreads();
  if (wave < N) {
    int w = lane < kPlanWaves ? msum[wave][lane] : 0;
    w = wave_incl_scan(w);
    if (lane < kPlanWaves) msum[wave][lane] = w;
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < N; ++n) {
    v[n] += wave ? msum[n][wave - 1] : 0;
    total[n] = msum[n][kPlanWaves - 1];
  }
}

// The uniform state the plan step starts from, read in one batch after the per-thread
// prefetches so that a single wait covers all of them.
struct PlanState {
  int anomaly, miss, under, short_rows;  // router flags of this forward
  int s_valid, s_size;                   // the slot lists
  int a_valid, a_built, a_size;          // the Atlas set (restricted routing)
};

__device__ __forceinline__ PlanState load_plan_state(const LayerState& L, const Scratch& W) {
  PlanState ps;
  ps.anomaly = W.flags[FLAG_ANOMALY];
  ps.miss = W.flags[FLAG_MISS];
  ps.under = W.flags[FLAG_UNDER];
  ps.short_rows = W.flags[FLAG_SHORT];
  ps.s_valid = *L.S_valid;
  ps.s_size = *L.S_size;
  ps.a_valid = L.A_state[0];
  ps.a_built = L.A_state[1];
  ps.a_size = L.A_state[2];
  return ps;
}

struct SupportLds {
  unsigned long long p[kMaxExperts];
  unsigned long long G[kMaxExperts];
  int32_t H[kMaxExperts];
  int32_t scan[kMaxExperts];
  int32_t wsum[kPlanWaves];
  int32_t slist[kMaxExperts];  // the slot list as last written (bit 1 of support_phase)
  uint8_t inS[kMaxExperts];
  uint8_t pick[kMaxExperts];
  int nU, added, size;
};

// Entries [j0, min(j0 + kRowGroup, n)) of one position's candidates (ids, and the planner
// weights when WITH_Q), rows of `stride` entries: all loads of a group issue together (uniform
// guards; 16-byte loads when the stride allows), one memory round trip per group instead of one
// per candidate.
constexpr int kRowGroup = 8;
struct RowGroup {
  int32_t id[kRowGroup];
  int32_t q[kRowGroup];
};

template <bool WITH_Q>
__device__ __forceinline__ void load_row_group(const int32_t* __restrict__ ids,
                                               const int32_t* __restrict__ q, int t, int stride,
                                               int j0, int n, RowGroup& g) {
  const int32_t* it = ids + (size_t)t * stride + j0;
  const int32_t* qt = q + (size_t)t * stride + j0;
  if ((stride & 3) == 0 && (n & 3) == 0) {
#pragma unroll
    for (int v = 0; v < kRowGroup / 4; ++v) {
      if (j0 + 4 * v < n) {
        const int4 a = *reinterpret_cast<const int4*>(it + 4 * v);
        g.id[4 * v] = a.x, g.id[4 * v + 1] = a.y, g.id[4 * v + 2] = a.z, g.id[4 * v + 3] = a.w;
        if (WITH_Q) {
          const int4 b = *reinterpret_cast<const int4*>(qt + 4 * v);
          g.q[4 * v] = b.x, g.q[4 * v + 1] = b.y, g.q[4 * v + 2] = b.z, g.q[4 * v + 3] = b.w;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kRowGroup; ++j) {
      if (j0 + j < n) {
        g.id[j] = it[j];
        if (WITH_Q) g.q[j] = qt[j];
      }
    }
  }
}

__device__ __forceinline__ void coverage_pass(const int32_t* __restrict__ ids,
                                              const int32_t* __restrict__ q, const uint8_t* inS,
                                              int M, int K, int Kext, int an, int ad,
                                              int32_t* __restrict__ Crow,
                                              int32_t* __restrict__ Rrow, int* nU) {
  int local = 0;
  for (int t = threadIdx.x; t < M; t += kPlanThreads) {
    int64_t r = 0, c = 0;
    for (int j0 = 0; j0 < Kext; j0 += kRowGroup) {
      RowGroup g;
      load_row_group<true>(ids, q, t, Kext, j0, Kext, g);
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j) {
        if (j0 + j < Kext) {
          if (j0 + j < K) r += g.q[j];
          if (inS[g.id[j]]) c += g.q[j];
        }
      }
    }
    Rrow[t] = (int32_t)r;
    Crow[t] = (int32_t)c;
    local += ((int64_t)ad * c < (int64_t)an * r);
  }
  if (local) atomicAdd(nU, local);
}

// Expert Atlas (teardown, Expert Atlas section, steps one and two, coverage goal
// |U| <= (1 - q) N; "cold / hot-update / hot-skip" for when it runs).  Planner weights are the
// integers q_{t,j} (units of 2^-16), alpha / q / beta are rationals, so every sum is an exact
// integer and the result does not depend on the order of the atomics.  Runs when the layer has
// no support yet (cold) or when the router found a routed expert outside it (hot-update);
// otherwise counts a hot-skip.  Whole-workgroup function: every thread must call it.
//
// Support-restricted routing (restricted shapes) keeps the Atlas set itself (no closure) in
// L.inA and decides here which routing the forward uses: a forward without a support (cold),
// past the update period, or whose candidates leave more than (1 - q) M positions
// under-covered by the support (or with fewer than K experts in it) rebuilds the support
// and routes over all experts, its routed experts getting slots for this forward only;
// otherwise (hot-skip) the slots are the support and the forward routes inside it.
// Returns bit 0 = the forward routes inside the support, bit 1 = the slot lists were rewritten.
__device__ int support_phase(const Shape& s, int iter, const LayerState& L, const Scratch& W,
                             const PlanState& ps, SupportLds& sh) {
  const int tid = threadIdx.x;
  const int M = s.M, E = s.E, K = s.K, Kext = s.Kext;
  const long long an = s.an, ad = s.ad, qn = s.qn, qd = s.qd, bn = s.bn, bd = s.bd;
  const int32_t* ids = W.ids;
  const int32_t* q = W.q;
  const bool valid = ps.s_valid != 0;
  int path;        // 0 hot-skip, 1 cold, 2 hot-update
  int reason = 0;  // restricted hot-update: 1 coverage check, 2 update period
  if (!s.restricted) {
    path = !valid ? 1 : (ps.miss != 0 ? 2 : 0);
    if (path == 0) {
      if (tid == 0) counter_add(L, EPOCH_CNT_HOT_SKIP, 1);
      return 0;  // slots unchanged
    }
  } else {
    const int a_valid = ps.a_valid, built = ps.a_built, a_size = ps.a_size;
    const long long nU = ps.under;
    if (!a_valid) {
      path = 1;
    } else if (s.atlas_period > 0 && iter - built >= s.atlas_period) {
      path = 2;
      reason = 2;
    } else if (a_size < K || ps.short_rows != 0 || qd * nU > (qd - qn) * (long long)M) {
      path = 2;
      reason = 1;
    } else {
      path = 0;
    }
  }
  int rounds = 0, unmet = 0, nU_final = 0, a_size_new = 0;
  if (path == 0) {
    // restricted hot-skip: the slots are the support
    for (int e = tid; e < E; e += kPlanThreads) sh.inS[e] = L.inA[e];
    __syncthreads();
  } else {
  const long long Q = 65536;
  // (i) popularity p_e = sum_{t,j: I_{t,j} = e} W_{t,j}
  for (int e = tid; e < E; e += kPlanThreads) sh.p[e] = 0;
  if (tid == 0) sh.nU = 0;
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) sh.H[e] = 0;
  for (int t = tid; t < M; t += kPlanThreads)
    for (int j0 = 0; j0 < Kext; j0 += kRowGroup) {
      RowGroup g;
      load_row_group<true>(ids, q, t, Kext, j0, Kext, g);
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j)
        if (j0 + j < Kext) atomicAdd(&sh.p[g.id[j]], (unsigned long long)(long long)g.q[j]);
    }
  __syncthreads();
  // initial support: experts with p_e > 0 whose rank by (p desc, id asc) is below B; the
  // E x E comparisons go to every thread (adjacent threads on adjacent experts, each group of
  // Epad threads a range of the others), the partial ranks summed in sh.H
  {
    int Epad = 1;
    while (Epad < E) Epad <<= 1;
    const int groups = kPlanThreads / Epad, e = tid & (Epad - 1), grp = tid / Epad;
    const int seg = (E + groups - 1) / groups, f0 = min(E, grp * seg), f1 = min(E, f0 + seg);
    if (e < E) {
      const unsigned long long pe = sh.p[e];
      int rank = 0;
#pragma unroll 8
      for (int f = f0; f < f1; ++f) rank += (sh.p[f] > pe) || (sh.p[f] == pe && f < e);
      if (rank) atomicAdd(&sh.H[e], rank);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) sh.inS[e] = (sh.p[e] > 0 && sh.H[e] < s.B) ? 1 : 0;
  __syncthreads();
  coverage_pass(ids, q, sh.inS, M, K, Kext, s.an, s.ad, W.Crow, W.Rrow, &sh.nU);
  __syncthreads();
  // (ii) greedy repair while |U| > (1 - q) M
  while (qd * sh.nU > (qd - qn) * M) {
    for (int e = tid; e < E; e += kPlanThreads) {
      sh.G[e] = 0;
      sh.H[e] = 0;
      sh.pick[e] = 0;
    }
    if (tid == 0) sh.added = 0;
    __syncthreads();
    for (int t = tid; t < M; t += kPlanThreads) {
      const long long R = W.Rrow[t], C = W.Crow[t];
      if (!(ad * C < an * R)) continue;
      const long long gap = an * R - ad * C;
      for (int j0 = 0; j0 < Kext; j0 += kRowGroup) {
        RowGroup g;
        load_row_group<true>(ids, q, t, Kext, j0, Kext, g);
#pragma unroll
        for (int j = 0; j < kRowGroup; ++j) {
          if (j0 + j >= Kext) continue;
          const int e = g.id[j];
          if (sh.inS[e]) continue;
          const long long v = ad * g.q[j];
          atomicAdd(&sh.G[e], (unsigned long long)(v < gap ? v : gap));
          if (ad * (C + g.q[j]) >= an * R) atomicAdd(&sh.H[e], 1);
        }
      }
    }
    __syncthreads();
    // score_e = H_e + beta G_e, scaled by alpha_den * Q * beta_den; add the best c positive
    for (int e = tid; e < E; e += kPlanThreads) {
      if (sh.inS[e]) continue;
      const long long se = bd * sh.H[e] * ad * Q + bn * (long long)sh.G[e];
      if (se <= 0) continue;
      int rank = 0;
      for (int f = 0; f < E; ++f) {
        if (sh.inS[f]) continue;
        const long long sf = bd * sh.H[f] * ad * Q + bn * (long long)sh.G[f];
        rank += (sf > se) || (sf == se && f < e);
      }
      if (rank < s.c) {
        sh.pick[e] = 1;
        atomicAdd(&sh.added, 1);
      }
    }
    __syncthreads();
    if (sh.added == 0) {
      unmet = 1;
      break;
    }
    for (int e = tid; e < E; e += kPlanThreads)
      if (sh.pick[e]) sh.inS[e] = 1;
    ++rounds;
    if (tid == 0) sh.nU = 0;
    __syncthreads();
    coverage_pass(ids, q, sh.inS, M, K, Kext, s.an, s.ad, W.Crow, W.Rrow, &sh.nU);
    __syncthreads();
  }
  nU_final = sh.nU;
  if (s.restricted) {
    // the Atlas support itself: kept for the next forwards, before the closure below
    const int incl_a = block_incl_scan(tid < E ? sh.inS[tid] : 0, sh.wsum, &a_size_new);
    (void)incl_a;
    if (tid < E) L.inA[tid] = sh.inS[tid];
    if (tid == 0) {
      L.A_state[0] = 1;
      L.A_state[1] = iter;
      L.A_state[2] = a_size_new;
    }
  }
  // (iii) closure: every routed expert of the current iteration gets a slot
  for (int t = tid; t < M; t += kPlanThreads)
    for (int j0 = 0; j0 < K; j0 += kRowGroup) {
      RowGroup g;
      load_row_group<false>(ids, q, t, Kext, j0, K, g);
#pragma unroll
      for (int j = 0; j < kRowGroup; ++j)
        if (j0 + j < K) sh.inS[g.id[j]] = 1;
    }
  __syncthreads();
  }
  // (iv) slots in expert-id order (E <= kMaxExperts == kPlanThreads: one expert per thread)
  int size;
  const int incl = block_incl_scan(tid < E ? sh.inS[tid] : 0, sh.wsum, &size);
  if (tid < E) {
    L.inS[tid] = sh.inS[tid];
    if (sh.inS[tid]) {
      L.slot_of[tid] = incl - 1;
      L.S_list[incl - 1] = tid;
      sh.slist[incl - 1] = tid;
    } else {
      L.slot_of[tid] = -1;
    }
  }
  if (tid == 0) {
    *L.S_size = size;
    *L.S_valid = 1;
    sh.size = size;
    if (path == 0) {
      counter_add(L, EPOCH_CNT_HOT_SKIP, 1);
      counter_add(L, EPOCH_CNT_RESTRICTED, 1);
    } else {
      counter_add(L, path == 1 ? EPOCH_CNT_COLD : EPOCH_CNT_HOT_UPDATE, 1);
      if (reason == 1) counter_add(L, EPOCH_CNT_COVERAGE_FALLBACK, 1);
      if (reason == 2) counter_add(L, EPOCH_CNT_PERIOD_UPDATE, 1);
      counter_add(L, EPOCH_CNT_UNMET, unmet);
      L.counters[EPOCH_CNT_SUPPORT_SIZE] = s.restricted ? a_size_new : size;
      L.counters[EPOCH_CNT_U_FINAL] = nU_final;
      counter_add(L, EPOCH_CNT_REPAIR_ROUNDS, rounds);
    }
  }
  __syncthreads();
  return (path == 0 ? 1 : 0) | 2;  // bit 0: route inside the support; bit 1: slots rewritten
}

// One position's routing as the placement reads it: the pre-anomaly flags and the K routed
// ids and weights, the all-expert top-K (first K candidates) or, when the forward routes inside
// the support, the in-support top-K.  Rows past M read position 0; every guard is uniform over
// the wave, so the loads issue back to back (16-byte loads when K and the row stride allow).
constexpr int kMaxTopK = 16;
struct RowRouting {
  int id[kMaxTopK];
  float w[kMaxTopK];
  uint8_t fp;
  bool inside;  // which routing the ids are
};

__device__ __forceinline__ void load_row_routing(int t, int M, int K, int Kext, bool inside,
                                                 const Scratch& W, RowRouting& r) {
  const size_t tt = t < M ? (size_t)t : 0;
  const int stride = inside ? K : Kext;
  const int32_t* it = (inside ? W.rids : W.ids) + tt * stride;
  const float* wt = (inside ? W.rw : W.w) + tt * K;
  if ((K & 3) == 0 && (stride & 3) == 0) {
#pragma unroll
    for (int j = 0; j < kMaxTopK / 4; ++j) {
      if (4 * j < K) {
        const int4 a = *reinterpret_cast<const int4*>(it + 4 * j);
        const float4 b = *reinterpret_cast<const float4*>(wt + 4 * j);
        r.id[4 * j] = a.x, r.id[4 * j + 1] = a.y, r.id[4 * j + 2] = a.z, r.id[4 * j + 3] = a.w;
        r.w[4 * j] = b.x, r.w[4 * j + 1] = b.y, r.w[4 * j + 2] = b.z, r.w[4 * j + 3] = b.w;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
      if (k < K) {
        r.id[k] = it[k];
        r.w[k] = wt[k];
      }
    }
  }
  r.fp = W.fpre[tt];
  r.inside = inside;
}

// Stable placement of one chunk by one wave (teardown, FreshLane pack: fresh rows with their
// owner positions and routing metadata in a contiguous buffer, here grouped by expert for the
// expert kernel).  Final fresh flag = pre-anomaly test or anomaly.  Pair (t, k) of expert e
// lands at eoffs[e] + chunk_base[chunk][e] + rank, where rank counts the chunk's earlier fresh
// positions routed to e (a 64-bit mask per expert, in LDS, cleared by the wave beforehand).
// foff = fresh positions in chunks before this one.  r holds this lane's row (loaded by the
// caller, possibly long before).  Wave-level function: all 64 lanes call it; mask holds E
// entries owned by this wave.  Issues no global load; the per-position rows (inv and the
// routing used) go out as 16-byte stores when K allows.
__device__ __forceinline__ void place_chunk(int chunk, int M, int E, int K, bool anomaly,
                                            const LayerState& L, const Scratch& W,
                                            unsigned long long* mask, const int32_t* eoffs,
                                            const int32_t* cbase, int foff, const RowRouting& r) {
  const int lane = threadIdx.x & 63;
  const int t = chunk * kChunk + lane;
  const bool in = t < M;
  for (int e = lane; e < E; e += 64) mask[e] = 0ull;
  const uint8_t fp = in ? r.fp : 0;
  const bool fresh = in && (anomaly || (fp & 1));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (fresh)
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
      if (k < K) atomicOr(&mask[r.id[k]], 1ull << lane);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int pk[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    pk[k] = -1;
    if (k < K && fresh) {
      const int e = r.id[k];
      const int p = eoffs[e] + cbase[e] + __popcll(mask[e] & below);
      W.wl_pos[p] = t;
      W.wl_k[p] = k;
      W.wl_w[p] = r.w[k];
      pk[k] = p;
    }
  }
  if (in) {
    // the slot of every pair (-1: not fresh) and the routing the worklist used
    int32_t* iv = W.inv + (size_t)t * K;
    int32_t* ri = W.routed_ids + (size_t)t * K;
    float* rw = W.routed_w + (size_t)t * K;
    if ((K & 3) == 0) {
#pragma unroll
      for (int j = 0; j < kMaxTopK / 4; ++j) {
        if (4 * j < K) {
          const int k = 4 * j;
          *reinterpret_cast<int4*>(iv + k) = make_int4(pk[k], pk[k + 1], pk[k + 2], pk[k + 3]);
          *reinterpret_cast<int4*>(ri + k) =
              make_int4(r.id[k], r.id[k + 1], r.id[k + 2], r.id[k + 3]);
          *reinterpret_cast<float4*>(rw + k) =
              make_float4(r.w[k], r.w[k + 1], r.w[k + 2], r.w[k + 3]);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kMaxTopK; ++k) {
        if (k < K) {
          iv[k] = pk[k];
          ri[k] = r.id[k];
          rw[k] = r.w[k];
        }
      }
    }
    L.fresh[t] = fresh ? 1 : 0;
  }
  const uint64_t fb = ballot64(fresh);
  if (fresh) W.fresh_list[foff + __popcll(fb & below)] = t;
  const int n_forced = __popcll(ballot64((fp & 2) != 0));
  const int n_due = __popcll(ballot64((fp & 4) != 0));
  if (lane == 0) {
    counter_add(L, EPOCH_CNT_FORCED_ROWS, n_forced);
    counter_add(L, EPOCH_CNT_DUE_ROWS, n_due);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Shapes whose placement runs inside the plan workgroup (one wave per chunk, kPlanWaves
// chunks at a time): the per-wave masks fit in LDS and there are few chunks to walk.
constexpr int kFusedPlaceMaxExperts = 256;
constexpr int kFusedPlaceMaxChunks = kPlanWaves;

// The plan step of one forward, one workgroup: the support check / build above, then the
// worklist bookkeeping over the router's per-chunk counts (the fresh-pair counts, or the counts
// of every position when a liveness anomaly makes the whole layer-iteration fresh):
//   chunk_base[c][e] = pairs of expert e in chunks before c   (stable order inside an expert)
//   eoffs[e]         = pairs of experts before e               (expert-major worklist)
//   offs[s]          = eoffs of the s-th support expert; tile tables (kTileRows pairs per
//                      tile, or kBigTile for experts with at least kBigRows pairs)
//   chunk_foff[c]    = fresh positions in chunks before c      (the fresh list)
// and, when FUSED_PLACE, the placement of every chunk.
template <bool FUSED_PLACE>
__global__ __launch_bounds__(kPlanThreads) void k_plan(Shape s, int iter, LayerState L,
                                                       Scratch W) {
  __shared__ SupportLds sh;
  __shared__ int32_t part[kPlanThreads];
  __shared__ int32_t tot[kMaxExperts];
  __shared__ unsigned long long pmask[FUSED_PLACE ? kPlanWaves : 1]
                                     [FUSED_PLACE ? kFusedPlaceMaxExperts : 1];
  // chunk bases and fresh-list offsets of the fused placement, kept in LDS: [chunk][expert]
  __shared__ int32_t cbl[FUSED_PLACE ? kFusedPlaceMaxChunks * kFusedPlaceMaxExperts : 1];
  __shared__ int32_t foffl[FUSED_PLACE ? kFusedPlaceMaxChunks : 1];
  __shared__ int32_t msum[9][kPlanWaves];
  const int tid = threadIdx.x;
  const int E = s.E, nch = s.n_chunks;
  // per-expert totals and chunk bases: Gp groups of Epad threads, adjacent threads on adjacent
  // experts (coalesced rows of the [chunk][expert] tables), each group a contiguous chunk range
  int Epad = 1;
  while (Epad < E) Epad <<= 1;
  const int Gp = kPlanThreads / Epad;
  const int e = tid & (Epad - 1), gi = tid / Epad;
  const int seg = (nch + Gp - 1) / Gp;
  const int c0 = min(nch, gi * seg), c1 = min(nch, c0 + seg);
  // global reads that do not depend on the support step, issued before it: the flags, the
  // fresh-list counts, the slot list of an unchanged support, and (all-expert routing, up to
  // kPre chunks per thread) both per-chunk pair counts
  constexpr int kPre = 4;
  const int pre_cf = tid < nch ? W.chunk_fresh[tid] : 0;
  const int pre_ex = tid < E ? L.S_list[tid] : 0;  // entries at and past S_size unused
  const bool pre_cnt = !s.restricted && seg <= kPre;
  int cv_f[kPre], cv_a[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const bool in = pre_cnt && e < E && c0 + k < c1;
    cv_f[k] = in ? W.cnt_f[(size_t)(c0 + k) * E + e] : 0;
    cv_a[k] = in ? W.cnt_a[(size_t)(c0 + k) * E + e] : 0;
  }
  // the fused placement's rows (one chunk per wave: position t = tid), read with the routing
  // a restricted shape usually takes (inside the support) and read again if it takes the other
  RowRouting row;
  const bool placer = FUSED_PLACE && (tid >> 6) < nch;
  if (placer) load_row_routing(tid, s.M, s.K, s.Kext, s.restricted, W, row);
  const PlanState ps = load_plan_state(L, W);
  const bool anomaly = ps.anomaly != 0;
  const int pre_nS = ps.s_size;
  const int sp = support_phase(s, iter, L, W, ps, sh);
  const bool route_r = (sp & 1) != 0;
  if (placer && route_r != row.inside) load_row_routing(tid, s.M, s.K, s.Kext, route_r, W, row);
  __syncthreads();

  const int32_t* cnt = route_r ? (anomaly ? W.cnt_ar : W.cnt_fr) : (anomaly ? W.cnt_a : W.cnt_f);
  auto count = [&](int c) {  // pairs of expert e in chunk c (c in [c0, c1))
    if (pre_cnt) {
      int v = 0;
#pragma unroll
      for (int k = 0; k < kPre; ++k)
        if (c == c0 + k) v = anomaly ? cv_a[k] : cv_f[k];
      return v;
    }
    return cnt[(size_t)c * E + e];
  };
  // longer chunk ranges: kBatch loads in flight, then the batch's stores (a load issued after
  // a store waits for it, so loads and stores alternate by batch, not by chunk)
  constexpr int kBatch = 8;
  int local = 0;
  if (e < E) {
    if (pre_cnt) {
      for (int c = c0; c < c1; ++c) local += count(c);
    } else {
      for (int cb = c0; cb < c1; cb += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = cb + j < c1 ? cnt[(size_t)(cb + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) local += v[j];
      }
    }
  }
  part[tid] = local;
  __syncthreads();
  if (e < E) {
    int base = 0, total = 0;
    for (int j = 0; j < Gp; ++j) {
      const int v = part[j * Epad + e];
      if (j < gi) base += v;
      total += v;
    }
    if (gi == 0) tot[e] = total;
    int run = base;
    for (int cb = c0; cb < c1; cb += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = cb + j < c1 ? count(cb + j) : 0;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int c = cb + j;
        if (c < c1) {
          W.chunk_base[(size_t)c * E + e] = run;
          if (FUSED_PLACE) cbl[c * kFusedPlaceMaxExperts + e] = run;
          run += v[j];
          W.cnt_f[(size_t)c * E + e] = 0;  // consumed: clear for the next forward
          W.cnt_a[(size_t)c * E + e] = 0;
          if (s.restricted) {
            W.cnt_fr[(size_t)c * E + e] = 0;
            W.cnt_ar[(size_t)c * E + e] = 0;
          }
        }
      }
    }
  }
  __syncthreads();
  // The prefix sums of the step in one workgroup scan:
  //   [0] pair totals by expert (one expert per thread)      -> eoffs, P
  //   [1] pair totals by support slot (one slot per thread)   -> offs
  //   [2], [3] small and big tile counts by slot              -> tile tables, T, Tb
  //   [4] fresh positions by chunk (first kPlanThreads chunks) -> chunk_foff
  //   [5] touched experts (a count only)
  //   [6], [7] experts on big tiles and their pairs (counts only)
  //   [8] tall tile counts by slot                             -> the tall tile table
  // offs[j] equals eoffs[S_list[j]]: every expert with pairs has a slot (the router flags a
  // routed expert outside the support, and such a forward rebuilds the slots), so the experts
  // between two slots contribute nothing.  An expert with at least kBigRows pairs goes to the
  // compute-bound table when the shape enables it.
  const bool slots_new = (sp & 2) != 0;
  const int nS = slots_new ? sh.size : pre_nS;
  const int my_tot = tid < E ? tot[tid] : 0;
  int slot_tot = 0, my_tiles = 0, my_tall = 0, my_big = 0;
  if (tid < nS) {
    slot_tot = tot[slots_new ? sh.slist[tid] : pre_ex];
    if (s.big_routed && slot_tot >= kBigRows) {
      my_big = (slot_tot + kBigTile - 1) / kBigTile;
    } else {
      my_tiles = (slot_tot + kTileRows - 1) / kTileRows;
      my_tall = (slot_tot + kTileRowsTall - 1) / kTileRowsTall;
    }
  }
  const int nf0 = tid < nch ? (anomaly ? min(kChunk, s.M - tid * kChunk) : pre_cf) : 0;
  int sc[9] = {my_tot, slot_tot, my_tiles, my_big, nf0, my_tot > 0 ? 1 : 0, my_big > 0 ? 1 : 0,
               my_big > 0 ? slot_tot : 0, my_tall};
  int stot[9];
  block_multi_scan(sc, msum, stot);
  // tall tiles when they are fewer: bf16 shapes without big tiles (the weight-stream kernel
  // beside the big tiles keeps short tiles, so that its workgroups fit beside theirs)
  const bool tall = s.bf16 && !s.big_routed && stot[8] < stot[2];
  const int P = stot[0], T = tall ? stot[8] : stot[2], Tb = stot[3], touched = stot[5];
  const int tile_rows_now = tall ? kTileRowsTall : kTileRows;
  if (tall) {
    sc[2] = sc[8];
    my_tiles = my_tall;
  }
  sh.scan[tid] = sc[0] - my_tot;  // read by the fused placement after the barrier below
  if (tid < E) W.eoffs[tid] = sc[0] - my_tot;
  if (tid == 0) {
    W.eoffs[E] = P;
    W.offs[nS] = P;
  }
  if (tid < nS) {
    const int my_off = sc[1] - slot_tot;
    W.offs[tid] = my_off;
    const int t0 = sc[2] - my_tiles;
    for (int i = 0; i < my_tiles; ++i) {
      W.tile_slot[t0 + i] = tid;
      W.tile_row0[t0 + i] = my_off + i * tile_rows_now;
    }
    const int b0 = sc[3] - my_big;
    for (int i = 0; i < my_big; ++i) {
      W.tile_slot_b[b0 + i] = tid;
      W.tile_row0_b[b0 + i] = my_off + i * kBigTile;
    }
  }
  // fresh-list offsets of the chunks: the first kPlanThreads from the scan above, the rest
  // (more than kPlanThreads * kChunk positions) kPlanThreads chunks per pass
  if (tid < nch) {
    W.chunk_foff[tid] = sc[4] - nf0;
    if (FUSED_PLACE) foffl[tid] = sc[4] - nf0;
    W.chunk_fresh[tid] = 0;
  }
  int carry = stot[4];
  for (int base = kPlanThreads; base < nch; base += kPlanThreads) {
    const int c = base + tid;
    const int nf = c < nch ? (anomaly ? min(kChunk, s.M - c * kChunk) : W.chunk_fresh[c]) : 0;
    int pass;
    const int incl = block_incl_scan(nf, sh.wsum, &pass);
    if (c < nch) {
      W.chunk_foff[c] = carry + incl - nf;
      W.chunk_fresh[c] = 0;
    }
    carry += pass;
  }
  if (tid == 0) {
    const int nfresh = carry;
    W.flags[FLAG_NFRESH] = nfresh;
    W.flags[FLAG_NPAIRS] = P;
    W.flags[FLAG_NTILES] = T;
    W.flags[FLAG_NTILES_BIG] = Tb;
    W.flags[FLAG_TILE_TALL] = tall ? 1 : 0;
    counter_add(L, EPOCH_CNT_FRESH_ROWS, nfresh);
    counter_add(L, EPOCH_CNT_PAIRS, P);
    counter_add(L, EPOCH_CNT_TOUCHED, touched);
    counter_add(L, EPOCH_CNT_BIG_EXPERTS, stot[6]);
    counter_add(L, EPOCH_CNT_BIG_PAIRS, stot[7]);
    counter_add(L, EPOCH_CNT_FORWARDS, 1);
    if (anomaly) counter_add(L, EPOCH_CNT_ANOMALY, 1);
    // every thread read MISS and ANOMALY before the barriers above
    W.flags[FLAG_FRESH_ALL] = anomaly ? 1 : 0;
    W.flags[FLAG_ROUTE_R] = route_r ? 1 : 0;
    W.flags[FLAG_MISS] = 0;
    W.flags[FLAG_ANOMALY] = 0;
    W.flags[FLAG_UNDER] = 0;
    W.flags[FLAG_SHORT] = 0;
  }
  if (FUSED_PLACE) {
    // the expert offsets, chunk bases and fresh-list offsets are in LDS (written above)
    __syncthreads();
    const int wave = tid >> 6;
    if (wave < nch)
      place_chunk(wave, s.M, E, s.K, anomaly, L, W, pmask[wave], sh.scan,
                  cbl + wave * kFusedPlaceMaxExperts, foffl[wave], row);
  }
}

// Placement as its own kernel (shapes with many chunks or experts): one wave per chunk.
__global__ __launch_bounds__(256) void k_place(int M, int E, int K, int Kext, int n_chunks,
                                               LayerState L, Scratch W) {
  __shared__ unsigned long long mask[4][kMaxExperts];
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 4 + wave;
  if (chunk >= n_chunks) return;
  RowRouting row;
  load_row_routing(chunk * kChunk + (threadIdx.x & 63), M, K, Kext, W.flags[FLAG_ROUTE_R] != 0, W,
                   row);
  place_chunk(chunk, M, E, K, W.flags[FLAG_FRESH_ALL] != 0, L, W, mask[wave], W.eoffs,
              W.chunk_base + (size_t)chunk * E, W.chunk_foff[chunk], row);
}

static bool fused_place(const Shape& s) {
  return s.E <= kFusedPlaceMaxExperts && s.n_chunks <= kFusedPlaceMaxChunks;
}

hipError_t launch_plan(const Shape& s, int iter, const LayerState& L, const Scratch& W,
                       hipStream_t st) {
  if (fused_place(s))
    launch(k_plan<true>, dim3(1), dim3(kPlanThreads), 0, st, s, iter, L, W);
  else
    launch(k_plan<false>, dim3(1), dim3(kPlanThreads), 0, st, s, iter, L, W);
  return hipGetLastError();
}

hipError_t launch_place(const Shape& s, const LayerState& L, const Scratch& W, hipStream_t st) {
  if (!fused_place(s))
    launch(k_place, dim3((s.n_chunks + 3) / 4), dim3(256), 0, st, s.M, s.E, s.K,
                       s.Kext, s.n_chunks, L, W);
  return hipGetLastError();
}

}  // namespace epoch
