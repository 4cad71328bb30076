// Block-clock and bookkeeping kernels: plan init, Expert Atlas support build, fresh set,
// expert-grouped worklist compaction and the cache commit (gfx950).
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
  }
  if (i < E) {
    L.inS[i] = 0;
    L.slot_of[i] = -1;
    L.S_list[i] = 0;
  }
  if (i < EPOCH_NUM_COUNTERS) L.counters[i] = 0;
  if (i == 0) {
    *L.S_size = 0;
    *L.S_valid = 0;
  }
}

hipError_t launch_init_layer(const Shape& s, const LayerState& L, hipStream_t st) {
  const int n = max(max(s.M, s.E), (int)EPOCH_NUM_COUNTERS);
  hipLaunchKernelGGL(k_init_layer, dim3((n + 255) / 256), dim3(256), 0, st, s.M, s.E, L);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- support build
// Expert Atlas (teardown, Expert Atlas section, steps one and two, coverage goal
// |U| <= (1 - q) N; "cold / hot-update / hot-skip" for when it runs).  One workgroup.
// Planner weights are the integers q_{t,j} (units of 2^-16), alpha / q / beta are rationals,
// so every sum is an exact integer and the result does not depend on the order of the
// atomics.  Runs when the layer has no support yet (cold) or when the router found a routed
// expert outside it (hot-update); otherwise counts a hot-skip and exits.
constexpr int kSupThreads = 1024;

__device__ __forceinline__ void coverage_pass(const int32_t* __restrict__ ids,
                                              const int32_t* __restrict__ q,
                                              const uint8_t* inS_sh, int M, int K, int Kext,
                                              int an, int ad, int32_t* __restrict__ Crow,
                                              int32_t* __restrict__ Rrow, int* nU_sh) {
  int local = 0;
  for (int t = threadIdx.x; t < M; t += kSupThreads) {
    const int32_t* it = ids + (size_t)t * Kext;
    const int32_t* qt = q + (size_t)t * Kext;
    int64_t r = 0, c = 0;
    for (int j = 0; j < Kext; ++j) {
      if (j < K) r += qt[j];
      if (inS_sh[it[j]]) c += qt[j];
    }
    Rrow[t] = (int32_t)r;
    Crow[t] = (int32_t)c;
    local += ((int64_t)ad * c < (int64_t)an * r);
  }
  if (local) atomicAdd(nU_sh, local);
}

__global__ __launch_bounds__(kSupThreads) void k_support_build(
    int M, int E, int K, int Kext, int B, int c, int an, int ad, int qn, int qd, int bn, int bd,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ q, int32_t* __restrict__ Crow,
    int32_t* __restrict__ Rrow, LayerState L, int32_t* __restrict__ flags) {
  __shared__ unsigned long long p_sh[kMaxExperts];
  __shared__ unsigned long long G_sh[kMaxExperts];
  __shared__ int32_t H_sh[kMaxExperts];
  __shared__ uint8_t inS_sh[kMaxExperts];
  __shared__ uint8_t pick_sh[kMaxExperts];
  __shared__ int32_t scan_sh[kMaxExperts];
  __shared__ int nU_sh, added_sh;
  const int tid = threadIdx.x;
  const bool valid = *L.S_valid != 0;
  const bool miss = flags[FLAG_MISS] != 0;
  if (valid && !miss) {
    if (tid == 0) {
      L.counters[EPOCH_CNT_HOT_SKIP] += 1;
      flags[FLAG_REBUILT] = 0;
    }
    return;
  }
  const long long Q = 65536;
  // (i) popularity p_e = sum_{t,j: I_{t,j} = e} W_{t,j}
  for (int e = tid; e < E; e += kSupThreads) p_sh[e] = 0;
  if (tid == 0) nU_sh = 0;
  __syncthreads();
  const int n = M * Kext;
  for (int i = tid; i < n; i += kSupThreads)
    atomicAdd(&p_sh[ids[i]], (unsigned long long)(long long)q[i]);
  __syncthreads();
  // initial support: experts with p_e > 0 whose rank by (p desc, id asc) is below B
  for (int e = tid; e < E; e += kSupThreads) {
    const unsigned long long pe = p_sh[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (p_sh[f] > pe) || (p_sh[f] == pe && f < e);
    inS_sh[e] = (pe > 0 && rank < B) ? 1 : 0;
  }
  __syncthreads();
  coverage_pass(ids, q, inS_sh, M, K, Kext, an, ad, Crow, Rrow, &nU_sh);
  __syncthreads();
  int rounds = 0, unmet = 0;
  // (ii) greedy repair while |U| > (1 - q) M
  while ((long long)qd * nU_sh > (long long)(qd - qn) * M) {
    for (int e = tid; e < E; e += kSupThreads) {
      G_sh[e] = 0;
      H_sh[e] = 0;
      pick_sh[e] = 0;
    }
    if (tid == 0) added_sh = 0;
    __syncthreads();
    for (int t = tid; t < M; t += kSupThreads) {
      const long long R = Rrow[t], C = Crow[t];
      if (!((long long)ad * C < (long long)an * R)) continue;
      const long long gap = (long long)an * R - (long long)ad * C;
      const int32_t* it = ids + (size_t)t * Kext;
      const int32_t* qt = q + (size_t)t * Kext;
      for (int j = 0; j < Kext; ++j) {
        const int e = it[j];
        if (inS_sh[e]) continue;
        const long long v = (long long)ad * qt[j];
        atomicAdd(&G_sh[e], (unsigned long long)(v < gap ? v : gap));
        if ((long long)ad * (C + qt[j]) >= (long long)an * R) atomicAdd(&H_sh[e], 1);
      }
    }
    __syncthreads();
    // score_e = H_e + beta G_e, scaled by alpha_den * Q * beta_den; add the best c positive
    for (int e = tid; e < E; e += kSupThreads) {
      if (inS_sh[e]) continue;
      const long long se = (long long)bd * H_sh[e] * ad * Q + (long long)bn * (long long)G_sh[e];
      if (se <= 0) continue;
      int rank = 0;
      for (int f = 0; f < E; ++f) {
        if (inS_sh[f]) continue;
        const long long sf = (long long)bd * H_sh[f] * ad * Q + (long long)bn * (long long)G_sh[f];
        rank += (sf > se) || (sf == se && f < e);
      }
      if (rank < c) {
        pick_sh[e] = 1;
        atomicAdd(&added_sh, 1);
      }
    }
    __syncthreads();
    if (added_sh == 0) {
      unmet = 1;
      break;
    }
    for (int e = tid; e < E; e += kSupThreads)
      if (pick_sh[e]) inS_sh[e] = 1;
    ++rounds;
    if (tid == 0) nU_sh = 0;
    __syncthreads();
    coverage_pass(ids, q, inS_sh, M, K, Kext, an, ad, Crow, Rrow, &nU_sh);
    __syncthreads();
  }
  const int nU_final = nU_sh;
  // (iii) closure: every routed expert of the current iteration gets a slot
  for (int i = tid; i < M * K; i += kSupThreads) {
    const int t = i / K, k = i - t * K;
    inS_sh[ids[(size_t)t * Kext + k]] = 1;
  }
  __syncthreads();
  // (iv) slots in expert-id order: inclusive scan of membership
  for (int e = tid; e < kMaxExperts; e += kSupThreads) scan_sh[e] = (e < E) ? inS_sh[e] : 0;
  __syncthreads();
  for (int off = 1; off < kMaxExperts; off <<= 1) {
    int v[kMaxExperts / kSupThreads];
#pragma unroll
    for (int u = 0; u < kMaxExperts / kSupThreads; ++u) {
      const int e = tid + u * kSupThreads;
      v[u] = (e >= off) ? scan_sh[e - off] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxExperts / kSupThreads; ++u) scan_sh[tid + u * kSupThreads] += v[u];
    __syncthreads();
  }
  for (int e = tid; e < E; e += kSupThreads) {
    const int incl = scan_sh[e];
    L.inS[e] = inS_sh[e];
    if (inS_sh[e]) {
      L.slot_of[e] = incl - 1;
      L.S_list[incl - 1] = e;
    } else {
      L.slot_of[e] = -1;
    }
  }
  if (tid == 0) {
    const int size = scan_sh[E - 1];
    *L.S_size = size;
    *L.S_valid = 1;
    L.counters[valid ? EPOCH_CNT_HOT_UPDATE : EPOCH_CNT_COLD] += 1;
    L.counters[EPOCH_CNT_UNMET] += unmet;
    L.counters[EPOCH_CNT_SUPPORT_SIZE] = size;
    L.counters[EPOCH_CNT_U_FINAL] = nU_final;
    L.counters[EPOCH_CNT_REPAIR_ROUNDS] += rounds;
    flags[FLAG_REBUILT] = 1;
  }
}

hipError_t launch_support(const Shape& s, const LayerState& L, const Scratch& W, hipStream_t st) {
  hipLaunchKernelGGL(k_support_build, dim3(1), dim3(kSupThreads), 0, st, s.M, s.E, s.K, s.Kext,
                     s.B, s.c, s.an, s.ad, s.qn, s.qd, s.bn, s.bd, W.ids, W.q, W.Crow, W.Rrow, L,
                     W.flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- fresh set + counts
// Fresh set (teardown, LSP: Z_i = D_i ∩ D_{i-1}; F_i = all on a cache miss or when refresh
// is due, else not Z_i; refresh period: reuse only while the age is at most R - 1; a
// liveness anomaly falls back to a full fresh pass).  One wave per chunk of 64 positions;
// also counts the chunk's fresh pairs per support slot for the stable compaction.
__global__ __launch_bounds__(256) void k_fresh_count(int M, int E, int K, int Kext, int R,
                                                     int iter, int n_chunks,
                                                     const uint8_t* __restrict__ D,
                                                     const uint8_t* __restrict__ force,
                                                     LayerState L, Scratch W) {
  __shared__ int32_t hist[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wave;
  const int t = chunk * kChunk + lane;
  const bool in = chunk < n_chunks && t < M;
  for (int e = lane; e < E; e += 64) hist[wave][e] = 0;
  bool fresh = false, forced = false, due = false;
  if (in) {
    const bool anomaly = W.flags[FLAG_ANOMALY] != 0;
    forced = force ? force[t] != 0 : false;
    const bool stable = D[t] && L.prev_D[t];
    const bool miss = !L.valid[t];
    due = (long long)iter - (long long)L.last_fresh[t] >= (long long)R;
    fresh = anomaly || forced || miss || !stable || due;
    L.fresh[t] = fresh ? 1 : 0;
  }
  __syncthreads();
  if (fresh) {
    const int32_t* it = W.ids + (size_t)t * Kext;
    for (int k = 0; k < K; ++k) {
      const int sl = L.slot_of[it[k]];  // the support's closure gives every routed expert a slot
      if (sl >= 0) atomicAdd(&hist[wave][sl], 1);
    }
  }
  const uint64_t fb = ballot64(fresh);
  const uint64_t forced_b = ballot64(in && forced);
  const uint64_t due_b = ballot64(in && due && L.valid[t]);
  __syncthreads();
  if (chunk < n_chunks) {
    for (int e = lane; e < E; e += 64) W.chunk_cnt[(size_t)chunk * E + e] = hist[wave][e];
    if (lane == 0) {
      W.chunk_fresh[chunk] = __popcll(fb);
      if (forced_b) atomicAdd((unsigned long long*)&L.counters[EPOCH_CNT_FORCED_ROWS],
                              (unsigned long long)__popcll(forced_b));
      if (due_b) atomicAdd((unsigned long long*)&L.counters[EPOCH_CNT_DUE_ROWS],
                           (unsigned long long)__popcll(due_b));
    }
  }
}

// Per-slot exclusive offsets of every chunk, slot offsets, chunk offsets of the fresh list and
// the grouped-GEMM tile table (one tile = up to kTileRows consecutive pairs of one slot).
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void k_scan(int M, int E, int K, int n_chunks,
                                                       LayerState L, Scratch W) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t tiles[kMaxExperts];
  __shared__ int32_t scan_a[kMaxExperts];
  __shared__ int32_t scan_b[kMaxExperts];
  const int tid = threadIdx.x;
  const int nS = *L.S_size;
  for (int s = tid; s < kMaxExperts; s += kScanThreads) {
    int run = 0;
    if (s < nS) {
      for (int c = 0; c < n_chunks; ++c) {
        W.chunk_base[(size_t)c * E + s] = run;
        run += W.chunk_cnt[(size_t)c * E + s];
      }
    }
    tot[s] = run;
    tiles[s] = (run + kTileRows - 1) / kTileRows;
    scan_a[s] = run;
    scan_b[s] = tiles[s];
  }
  __syncthreads();
  for (int off = 1; off < kMaxExperts; off <<= 1) {
    int va[kMaxExperts / kScanThreads], vb[kMaxExperts / kScanThreads];
#pragma unroll
    for (int u = 0; u < kMaxExperts / kScanThreads; ++u) {
      const int s = tid + u * kScanThreads;
      va[u] = s >= off ? scan_a[s - off] : 0;
      vb[u] = s >= off ? scan_b[s - off] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxExperts / kScanThreads; ++u) {
      scan_a[tid + u * kScanThreads] += va[u];
      scan_b[tid + u * kScanThreads] += vb[u];
    }
    __syncthreads();
  }
  // scan_* are inclusive; exclusive = inclusive - own
  for (int s = tid; s < nS; s += kScanThreads) {
    const int off = scan_a[s] - tot[s];
    W.offs[s] = off;
    const int t0 = scan_b[s] - tiles[s];
    for (int i = 0; i < tiles[s]; ++i) {
      W.tile_slot[t0 + i] = s;
      W.tile_row0[t0 + i] = off + i * kTileRows;
    }
  }
  if (tid == 0) {
    const int P = nS > 0 ? scan_a[nS - 1] : 0;
    const int T = nS > 0 ? scan_b[nS - 1] : 0;
    W.offs[nS] = P;
    int run = 0;
    for (int c = 0; c < n_chunks; ++c) {
      W.chunk_foff[c] = run;
      run += W.chunk_fresh[c];
    }
    W.flags[FLAG_NFRESH] = run;
    W.flags[FLAG_NPAIRS] = P;
    W.flags[FLAG_NTILES] = T;
    int touched = 0;
    for (int s = 0; s < nS; ++s) touched += tot[s] > 0;
    L.counters[EPOCH_CNT_FRESH_ROWS] += run;
    L.counters[EPOCH_CNT_PAIRS] += P;
    L.counters[EPOCH_CNT_TOUCHED] += touched;
    L.counters[EPOCH_CNT_FORWARDS] += 1;
    if (W.flags[FLAG_ANOMALY]) L.counters[EPOCH_CNT_ANOMALY] += 1;
  }
}

// Stable placement (teardown, FreshLane pack: fresh rows with their owner positions and
// routing metadata in a contiguous buffer; here grouped by expert for the expert kernel).
// Pair (t, k) of expert e lands at offs[slot] + base[chunk][slot] + rank, where rank counts
// the chunk's earlier positions routed to the same expert (a 64-bit mask per slot).
__global__ __launch_bounds__(256) void k_place(int M, int E, int K, int Kext, int n_chunks,
                                               LayerState L, Scratch W) {
  __shared__ unsigned long long mask[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + wave;
  const int t = chunk * kChunk + lane;
  const bool in = chunk < n_chunks && t < M;
  for (int e = lane; e < E; e += 64) mask[wave][e] = 0ull;
  const bool fresh = in && L.fresh[t];
  __syncthreads();
  const int32_t* it = W.ids + (size_t)(in ? t : 0) * Kext;
  if (fresh) {
    for (int k = 0; k < K; ++k) {
      const int sl = L.slot_of[it[k]];
      if (sl >= 0) atomicOr(&mask[wave][sl], 1ull << lane);
    }
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (fresh) {
    for (int k = 0; k < K; ++k) {
      const int s = L.slot_of[it[k]];
      if (s < 0) continue;
      const int rank = __popcll(mask[wave][s] & below);
      const int p = W.offs[s] + W.chunk_base[(size_t)chunk * E + s] + rank;
      W.wl_pos[p] = t;
      W.wl_k[p] = k;
      W.wl_w[p] = W.w[(size_t)t * K + k];
      W.inv[(size_t)t * K + k] = p;
    }
  } else if (in) {
    for (int k = 0; k < K; ++k) W.inv[(size_t)t * K + k] = -1;
  }
  const uint64_t fb = ballot64(fresh);
  if (fresh) W.fresh_list[W.chunk_foff[chunk] + __popcll(fb & below)] = t;
}

hipError_t launch_worklist(const Shape& s, int iter, const uint8_t* D, const uint8_t* force,
                           const LayerState& L, const Scratch& W, hipStream_t st) {
  const int wgs = (s.n_chunks + 3) / 4;
  hipLaunchKernelGGL(k_fresh_count, dim3(wgs), dim3(256), 0, st, s.M, s.E, s.K, s.Kext, s.R, iter,
                     s.n_chunks, D, force, L, W);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, st, s.M, s.E, s.K, s.n_chunks, L, W);
  hipLaunchKernelGGL(k_place, dim3(wgs), dim3(256), 0, st, s.M, s.E, s.K, s.Kext, s.n_chunks, L,
                     W);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- commit
// Cache commit (teardown, LSP state machine: fresh output -> cache update; refresh period:
// the age restarts at a fresh write; D_i becomes the D_{i-1} of the next iteration).
__global__ void k_commit(int M, int iter, LayerState L, const uint8_t* __restrict__ fresh,
                         const uint8_t* __restrict__ Dcopy) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < M) {
    if (fresh[t]) {
      L.valid[t] = 1;
      L.last_fresh[t] = iter;
    }
    L.prev_D[t] = Dcopy[t];
  }
  if (t == 0) L.counters[EPOCH_CNT_COMMITS] += 1;
}

hipError_t launch_commit(const Shape& s, int iter, const LayerState& L, const Scratch& W,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_commit, dim3((s.M + 255) / 256), dim3(256), 0, st, s.M, iter, L, L.fresh,
                     L.Dcur);
  return hipGetLastError();
}

}  // namespace epoch
