// Router: gate logits over every position, per-position top-k, and the fresh-set inputs
// of the worklist (gfx950).
//
// Gate logits G = x W_g^T + b are recomputed for all M positions every iteration
// (Epoch abstract; teardown, Expert Atlas: G in R^{N x E}, top-k over sigma(G) with
// K_ext = K + m candidates for the planner).  Products of a bf16 (or fp32) activation
// and an fp32 weight are exact in double, and the sums run on the fp64 MFMA pipe, so the
// fp32-rounded logit is the correctly rounded value in all but vanishingly rare cases.
// That makes the top-k ids and the planner's integer weights reproducible bit for bit.
#include "device_common.h"
#include "epoch_internal.h"

namespace epoch {

// ---------------------------------------------------------------------------- gate logits
// A workgroup of `ksplit` waves owns a BT x BT tile of (positions x experts); wave w sums the
// k-range [w H / ksplit, (w + 1) H / ksplit) on v_mfma_f64_16x16x4 (BT / 16 blocks per side),
// the partial tiles meet in LDS and are added in wave order, then the bias, then one rounding
// to fp32.  The contraction index is permuted: in each 64-wide k step, lane group g = l / 16
// owns k in [16 g, 16 g + 16) and feeds them to 16 successive MFMA steps, for the activation
// and the weight alike, so every product pairs x[t,k] with W[e,k].  Each lane loads its
// 16 values of each operand as whole 16-byte vectors, two steps ahead of the MFMAs.
template <typename T>
struct RouterRaw;
template <>
struct RouterRaw<uint16_t> {
  u32x4 v[2];  // 16 bf16
  __device__ __forceinline__ void load(const uint16_t* p) {
    v[0] = reinterpret_cast<const u32x4*>(p)[0];
    v[1] = reinterpret_cast<const u32x4*>(p)[1];
  }
  __device__ __forceinline__ double get(int m) const {
    const uint32_t w = v[m >> 3][(m >> 1) & 3];
    return (double)__uint_as_float((m & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct RouterRaw<float> {
  u32x4 v[4];  // 16 fp32
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const u32x4*>(p)[i];
  }
  __device__ __forceinline__ double get(int m) const {
    return (double)__uint_as_float(v[m >> 2][m & 3]);
  }
};

// ---------------------------------------------------------------------------- top-k + fresh inputs
// One wave per position.  Per position: the K_ext candidates in key order (logit desc, expert
// id asc), the gate scores in double (softmax over all E, or sigmoid), the routing weights of
// the first K, the planner weight q = floor(s * 2^16 + 1/2); the support-miss flag (a routed
// expert outside the current support) and the liveness-anomaly flag (decoded -> live).  The
// fresh test of the position before the anomaly override (teardown, LSP: fresh = not
// (D_i and D_{i-1}), a cache miss, or refresh due; forced rows), and per-chunk per-expert
// counts of the routed pairs of fresh positions and of all positions (integer atomics, so
// their order does not matter), the inputs of the stable worklist placement.
//
// Selection: every (logit, expert) pair gets a unique 42-bit key, the order-preserving bits of
// the fp32 logit above the inverted expert id, so "larger key" is exactly the key order
// above.  A bitwise radix search with wave ballots finds the K_ext-th largest key; the K_ext
// keys at or above it are ranked by comparing against each other (a readlane loop).
// Everything the top-k of a position reads besides the logits.
struct RouteArgs {
  LayerState L;
  Scratch W;
  const uint8_t* D;
  const uint8_t* force;
  int E, K, Kext, gate_sigmoid, norm_topk, R, iter;
  int restricted, an, ad;  // support-restricted routing; coverage floor alpha = an / ad
  int n_group, topk_group;  // group-limited top-k (n_group = 0: off)
  // logits split over kw workgroups (kw > 1): the fp64 partials [kw][M][E] (the first with
  // the bias added), summed here in order, then one rounding to fp32 (also stored to G)
  const double* Gp;
  int kw, M;
};

// The router's k split over workgroups (partial logits summed by the top-k) is used only with
// at most 64 experts (one per lane) and at most this many parts.
constexpr int kRouterMaxKw = 4;

// LDS of one wave's top-k: candidate scores (K_ext), in-support scores (K), group maxima and
// kept-group flags, in doubles
constexpr int kRouteLds = 2 * kMaxKext + kMaxGroups + 8;

__device__ __forceinline__ uint64_t sel_key(float g, int e) {
  uint32_t u = __float_as_uint(g);
  if (u == 0x80000000u) u = 0u;  // -0 and +0 compare equal as floats: one key for both
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 10) | (uint64_t)(1023 - e);
}

// lc: the workgroup's LDS counters of the position's chunk ([E] routed pairs of all positions,
// [E] of fresh positions, the same two for the in-support routing, then the fresh positions and
// the under-covered positions), flushed to global memory by the caller: a position updates
// them with LDS atomics only.
template <int NPER>
__device__ __forceinline__ void route_row(int t, const float* __restrict__ G, const RouteArgs& ra,
                                          double* s_buf, int32_t* lc) {
  const LayerState& L = ra.L;
  const Scratch& W = ra.W;
  const uint8_t* __restrict__ D = ra.D;
  const uint8_t* __restrict__ force = ra.force;
  const int E = ra.E, K = ra.K, Kext = ra.Kext, gate_sigmoid = ra.gate_sigmoid;
  const int norm_topk = ra.norm_topk, R = ra.R, iter = ra.iter;
  const int lane = threadIdx.x & 63;
  // restricted mode with a support in place: also route inside the support (the plan step
  // decides which routing the forward uses)
  const bool r_on = ra.restricted && L.A_state[0] != 0;
  // prologue: every global read of the position at once.  No load sits under a lane mask
  // (lanes past E read expert E - 1 and drop it afterwards): a masked load makes the compiler
  // wait for it before the next one is issued.
  // workgroups per logit (router k split): up to 4, and only with one expert per lane
  constexpr int kMaxKw = NPER == 1 ? kRouterMaxKw : 1;
  float gv[NPER];
  uint8_t in_s[NPER], in_a[NPER];
  double part[NPER][kMaxKw];
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int e = lane + 64 * j, ec = e < E ? e : E - 1;
    gv[j] = G[(size_t)t * E + ec];  // not yet written when kw > 1 (replaced below)
#pragma unroll
    for (int z = 0; z < kMaxKw; ++z)  // (a one-element buffer when kw = 1)
      part[j][z] = ra.Gp[z < ra.kw && ra.kw > 1 ? ((size_t)z * ra.M + t) * E + ec : 0];
    in_s[j] = L.inS[ec];
    in_a[j] = L.inA[ec];
  }
  const uint8_t d = D[t], pd = L.prev_D[t];
  const bool valid = L.valid[t] != 0;
  const int32_t last = L.last_fresh[t];
  const bool forced = force ? force[t] != 0 : false;
  const bool s_valid = *L.S_valid != 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const int e = lane + 64 * j;
    if (ra.kw > 1) {
      // the parts in workgroup order (the first one carries the bias), then one rounding
      double sum = 0.0;
#pragma unroll
      for (int z = 0; z < kMaxKw; ++z)
        if (z < ra.kw) sum += part[j][z];
      gv[j] = (float)sum;
      if (e < E) W.G[(size_t)t * E + e] = gv[j];
    }
    if (e >= E) gv[j] = -INFINITY;
    in_s[j] = e < E ? in_s[j] : 0;
    in_a[j] = (r_on && e < E) ? in_a[j] : 0;
  }
  uint64_t key[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) key[j] = (lane + 64 * j < E) ? sel_key(gv[j], lane + 64 * j) : 0ull;
  // the n largest of the keys kk (0 = excluded): membership masks and ranks
  auto select = [&](const uint64_t* kk, int n, uint64_t* selm, int* rank) {
    // largest threshold T with #{key >= T} >= n: the n-th largest key.  Keys are unique (the
    // expert id is in the low bits), so once exactly n keys lie at or above a candidate they
    // are the n largest and the lower bits cannot change the set: stop there.
    uint64_t T = 0;
    for (int b = 41; b >= 0; --b) {
      const uint64_t cand = T | (1ull << b);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < NPER; ++j) cnt += __popcll(ballot64(kk[j] >= cand));
      if (cnt >= n) T = cand;
      if (cnt == n) break;
    }
    // rank of each selected key among the selected ones
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      rank[j] = 0;
      selm[j] = ballot64(kk[j] >= T && kk[j] != 0ull);
    }
#pragma unroll
    for (int jj = 0; jj < NPER; ++jj) {
      uint64_t m = selm[jj];
      while (m) {
        const int src = __ffsll((long long)m) - 1;
        m &= m - 1;
        const uint64_t kb = ((uint64_t)__builtin_amdgcn_readlane((int)(kk[jj] >> 32), src) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kk[jj], src);
#pragma unroll
        for (int j = 0; j < NPER; ++j) rank[j] += (kb > kk[j]);
      }
    }
  };
  // group-limited rule: keep the keys of the experts of this position's topk_group best
  // groups, a group ranking by its best key (largest key among its non-zero ones)
  const int ng = ra.n_group, gsz = ng ? E / ng : 1;
  auto group_keep = [&](const uint64_t* kk, uint64_t* out) {
    unsigned long long* gmax = reinterpret_cast<unsigned long long*>(s_buf + 2 * kMaxKext);
    uint8_t* keep = reinterpret_cast<uint8_t*>(s_buf + 2 * kMaxKext + kMaxGroups);
    if (lane < ng) gmax[lane] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < NPER; ++j)
      if (kk[j]) atomicMax(&gmax[(lane + 64 * j) / gsz], (unsigned long long)kk[j]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint64_t gk = lane < ng ? gmax[lane] : 0ull;
    int grank = 0;
    for (int g2 = 0; g2 < ng; ++g2) {
      const uint64_t o = ((uint64_t)__builtin_amdgcn_readlane((int)(gk >> 32), g2) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gk, g2);
      grank += o > gk;
    }
    if (lane < ng) keep[lane] = (gk != 0ull && grank < ra.topk_group) ? 1 : 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int j = 0; j < NPER; ++j) out[j] = (kk[j] && keep[(lane + 64 * j) / gsz]) ? kk[j] : 0ull;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int rank[NPER];
  uint64_t selm[NPER];
  if (ng) {
    uint64_t kg[NPER];
    group_keep(key, kg);
    select(kg, Kext, selm, rank);
  } else {
    select(key, Kext, selm, rank);
  }
  // softmax normaliser over all E (max = the best key's logit); the exponentials are kept for
  // the scores of the candidates
  double zmax = 0.0, z = 0.0;
  double ex[NPER];
  if (!gate_sigmoid) {
    double m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPER; ++j)
      if (lane + 64 * j < E) m = fmax(m, (double)gv[j]);
    zmax = wave_max(m);
    double part = 0.0;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      ex[j] = exp((double)gv[j] - zmax);
      if (lane + 64 * j < E) part += ex[j];
    }
    z = wave_sum(part);
  }
  // the fresh test before the anomaly override
  const bool due = (long long)iter - (long long)last >= (long long)R;
  const bool fresh = forced || !valid || !(d && pd) || due;
  // the candidates in rank order, candidate r on lane r (through the group-maxima LDS, free
  // after the selection): the scores, planner weights, stores and counts then take one pass
  // over K_ext lanes instead of one per expert slot of a lane
  double* cval = s_buf + 2 * kMaxKext;                                      // [K_ext]
  int32_t* cmeta = reinterpret_cast<int32_t*>(s_buf + 2 * kMaxKext + kMaxKext);  // [K_ext]
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    if (!((selm[j] >> lane) & 1ull)) continue;
    const int rk = rank[j];
    cval[rk] = gate_sigmoid ? (double)gv[j] : ex[j];
    cmeta[rk] = (lane + 64 * j) | (in_s[j] ? 1 << 16 : 0) | (in_a[j] ? 1 << 17 : 0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bool miss = false;
  int q_routed = 0, q_in_a = 0;  // R_t and C_t(A) of the Atlas coverage test, this lane's part
  if (lane < Kext) {
    const double v = cval[lane];
    const int meta = cmeta[lane], e = meta & 0xffff;
    const double sc = gate_sigmoid ? 1.0 / (1.0 + exp(-v)) : v / z;
    const int32_t qv = (int32_t)floor(sc * 65536.0 + 0.5);
    W.ids[(size_t)t * Kext + lane] = e;
    W.scores[(size_t)t * Kext + lane] = (float)sc;
    W.q[(size_t)t * Kext + lane] = qv;
    s_buf[lane] = sc;
    if (meta & (1 << 17)) q_in_a += qv;
    if (lane < K) {
      q_routed += qv;
      miss |= s_valid && !(meta & (1 << 16));
      atomicAdd(&lc[e], 1);
      if (fresh) atomicAdd(&lc[E + e], 1);
    }
  }
  if (r_on) {
    // coverage of this position by the support: under-covered when alpha_den C < alpha_num R
    const int Rt = wave_sum(q_routed), Ct = wave_sum(q_in_a);
    if (lane == 0 && (long long)ra.ad * Ct < (long long)ra.an * Rt)
      atomicAdd(&lc[4 * E + 1], 1);
    // top-K inside the support (scores keep their definition over all E)
    uint64_t kr[NPER];
#pragma unroll
    for (int j = 0; j < NPER; ++j) kr[j] = in_a[j] ? key[j] : 0ull;
    if (ng) group_keep(kr, kr);  // the model's rule with the selectable experts in the support
    int n_sel = 0;
#pragma unroll
    for (int j = 0; j < NPER; ++j) n_sel += __popcll(ballot64(kr[j] != 0ull));
    if (n_sel < K && lane == 0) W.flags[FLAG_SHORT] = 1;  // this forward takes the full path
    int rrank[NPER];
    uint64_t rsel[NPER];
    select(kr, K, rsel, rrank);
    double* r_buf = s_buf + kMaxKext;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int e = lane + 64 * j;
      if (!((rsel[j] >> lane) & 1ull) || rrank[j] >= K) continue;
      const int rk = rrank[j];
      const double sc = gate_sigmoid ? 1.0 / (1.0 + exp(-(double)gv[j])) : exp((double)gv[j] - zmax) / z;
      W.rids[(size_t)t * K + rk] = e;
      r_buf[rk] = sc;
      atomicAdd(&lc[2 * E + e], 1);
      if (fresh) atomicAdd(&lc[3 * E + e], 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // fewer than K experts in the support leaves slots unset: the plan step then rebuilds
    // and this routing is not used
    if (lane < K) {
      double denom = 0.0;
      if (norm_topk)
        for (int k = 0; k < K; ++k) denom += r_buf[k];
      const double sk = r_buf[lane];
      W.rw[(size_t)t * K + lane] = (float)(norm_topk ? sk / denom : sk);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < K) {
    double denom = 0.0;
    if (norm_topk)
      for (int k = 0; k < K; ++k) denom += s_buf[k];  // rank order
    const double sk = s_buf[lane];
    W.w[(size_t)t * K + lane] = (float)(norm_topk ? sk / denom : sk);
  }
  if (ballot64(miss) != 0 && lane == 0) W.flags[FLAG_MISS] = 1;
  if (lane == 0) {
    L.Dcur[t] = d;
    if (pd && !d) W.flags[FLAG_ANOMALY] = 1;
    // bit 0: fresh before the anomaly override; bits 1, 2: forced, refresh due (counted per
    // chunk by the placement: one atomic per chunk rather than per position on one address)
    W.fpre[t] = (fresh ? 1 : 0) | (forced ? 2 : 0) | ((due && valid) ? 4 : 0);
    if (fresh) atomicAdd(&lc[4 * E], 1);
  }
}

// The top-k as its own kernel: one wave per position, WAVES positions per workgroup, all of
// one chunk (kChunk is a multiple of WAVES).  The per-chunk pair counts and the fresh /
// under-covered counts are summed in LDS and added to global memory once per workgroup: with
// popular experts, one global atomic per position and expert piles up dozens of same-address
// atomics per chunk in the L2.  Many positions take 16-wave workgroups (16 times fewer global
// atomics); few take 4-wave ones (more workgroups to spread over the CUs).
constexpr int kRouteRowsBigM = 4096;

template <int NPER, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_route_rows(const float* __restrict__ G,
                                                           RouteArgs ra, int M) {
  constexpr int kWaves = WAVES;
  static_assert(kChunk % kWaves == 0, "a workgroup's positions lie in one chunk");
  __shared__ double s_buf[kWaves][kRouteLds];
  __shared__ int32_t lc[4 * kMaxExperts + 2];
  const int E = ra.E;
  for (int i = threadIdx.x; i < 4 * E + 2; i += blockDim.x) lc[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kWaves + wave;
  if (t < M) route_row<NPER>(t, G, ra, s_buf[wave], lc);
  __syncthreads();
  const Scratch& W = ra.W;
  const size_t chunk = (size_t)blockIdx.x * kWaves / kChunk;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const size_t i = chunk * E + e;
    if (lc[e]) atomicAdd(&W.cnt_a[i], lc[e]);
    if (lc[E + e]) atomicAdd(&W.cnt_f[i], lc[E + e]);
    if (lc[2 * E + e]) atomicAdd(&W.cnt_ar[i], lc[2 * E + e]);
    if (lc[3 * E + e]) atomicAdd(&W.cnt_fr[i], lc[3 * E + e]);
  }
  if (threadIdx.x == 0) {
    if (lc[4 * E]) atomicAdd(&W.chunk_fresh[chunk], lc[4 * E]);
    if (lc[4 * E + 1]) atomicAdd(&W.flags[FLAG_UNDER], lc[4 * E + 1]);
  }
}

template <typename T, int BT>
__global__ __launch_bounds__(BT == 32 ? 256 : 1024) void k_router(
    const T* __restrict__ x, const float* __restrict__ Wg, const float* __restrict__ bias,
    float* __restrict__ G, double* __restrict__ Gp, int M, int H, int E, int ksplit, int kw) {
  constexpr int NB = BT / 16;
  extern __shared__ double red[];  // [ksplit][BT * BT]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e0 = blockIdx.x * BT, t0 = blockIdx.y * BT;
  // workgroup blockIdx.z of kw sums its k range; its waves split it further
  const int klen = H / (ksplit * kw), kbeg = (blockIdx.z * ksplit + wave) * klen;
  const int nsteps = klen / 64;
  const int r = lane & 15, g = lane >> 4;
  // rows past M or E read row 0 (always present): they only feed logits that are never
  // stored, so every lane loads with no branch around it (a load under a lane mask would make
  // the compiler wait for the prefetched step too before multiplying the current one)
  const T* xr[NB];
  const float* wr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int t = t0 + 16 * b + r, e = e0 + 16 * b + r;
    xr[b] = x + (size_t)(t < M ? t : 0) * H + kbeg + 16 * g;
    wr[b] = Wg + (size_t)(e < E ? e : 0) * H + kbeg + 16 * g;
  }
  f64x4 acc[NB][NB];
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f64x4{0, 0, 0, 0};
  RouterRaw<T> xa[2][NB];
  RouterRaw<float> wa[2][NB];
  // a step's loads issue as one group, ahead of the MFMAs of the step before (the scheduling
  // barriers keep the compiler from sinking them between those MFMAs, where each would be
  // waited for at once)
  auto load = [&](int step, int buf) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      xa[buf][b].load(xr[b] + 64 * step);
      wa[buf][b].load(wr[b] + 64 * step);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      double A[NB], B[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        A[b] = xa[buf][b].get(m);
        B[b] = wa[buf][b].get(m);
      }
#pragma unroll
      for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(A[a], B[b], acc[a][b], 0, 0, 0);
    }
  };
  // two steps in flight: a buffer is refilled with the step after next as soon as its MFMAs
  // are issued.  The refills are unconditional (past the end they re-read the last step): a
  // load under a branch, even a uniform one, leaves the compiler unable to count it, and it
  // then waits for every load before the MFMAs of the current step.
  load(0, 0);
  load(min(1, nsteps - 1), 1);
  for (int st = 0; st < nsteps; st += 2) {
    mma(0);
    load(min(st + 2, nsteps - 1), 0);
    if (st + 1 >= nsteps) break;
    mma(1);
    load(min(st + 3, nsteps - 1), 1);
  }
  // f64 16x16x4 output layout: D[i][j] sits in lane (j + 16 * (i % 4)), register i / 4
  double* mine = red + (size_t)wave * BT * BT;
#pragma unroll
  for (int a = 0; a < NB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[(16 * a + 4 * i + g) * BT + 16 * b + r] = acc[a][b][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < BT * BT; idx += blockDim.x) {
    const int t = t0 + idx / BT, e = e0 + idx % BT;
    if (t >= M || e >= E) continue;
    double s = 0.0;
    for (int w = 0; w < ksplit; ++w) s += red[(size_t)w * BT * BT + idx];
    if (kw > 1) {
      if (bias && blockIdx.z == 0) s += (double)bias[e];
      Gp[((size_t)blockIdx.z * M + t) * E + e] = s;  // the top-k kernel adds the parts
    } else {
      if (bias) s += (double)bias[e];
      G[(size_t)t * E + e] = (float)s;
    }
  }
}

template <typename T, int BT>
static void launch_k_router(const Shape& s, const void* x, const float* Wg, const float* bias,
                            const Scratch& W, hipStream_t st) {
  const size_t lds = (size_t)s.ksplit * BT * BT * sizeof(double);
  const dim3 grid((s.E + BT - 1) / BT, (s.M + BT - 1) / BT, s.router_kw), block(64 * s.ksplit);
  launch((k_router<T, BT>), grid, block, lds, st, static_cast<const T*>(x), Wg, bias,
                     W.G, W.Gp, s.M, s.H, s.E, s.ksplit, s.router_kw);
}

template <int NP>
static void launch_route_rows(const Shape& s, const Scratch& W, const RouteArgs& ra,
                              hipStream_t st) {
  if constexpr (NP <= 8) {
    if (s.M >= kRouteRowsBigM) {
      launch(k_route_rows<NP, 16>, dim3((s.M + 15) / 16), dim3(1024), 0, st, W.G, ra, s.M);
      return;
    }
  }
  launch(k_route_rows<NP, 4>, dim3((s.M + 3) / 4), dim3(256), 0, st, W.G, ra, s.M);
}

hipError_t launch_router(const Shape& s, const void* x, const float* Wg, const float* bias,
                         const uint8_t* D, const uint8_t* force, int iter, const LayerState& L,
                         const Scratch& W, hipStream_t st) {
  // The logits go through memory between the two kernels.  Handing a row group's logits to its
  // last-finishing tile inside one kernel needs a device-scope release / acquire per workgroup,
  // which on this chip writes back the XCD's L2 each time: slower than the second launch.
  if (s.router_bt == 32) {
    if (s.bf16)
      launch_k_router<uint16_t, 32>(s, x, Wg, bias, W, st);
    else
      launch_k_router<float, 32>(s, x, Wg, bias, W, st);
  } else {
    if (s.bf16)
      launch_k_router<uint16_t, 16>(s, x, Wg, bias, W, st);
    else
      launch_k_router<float, 16>(s, x, Wg, bias, W, st);
  }
  const RouteArgs ra{L,         W,   D,    force,        s.E,  s.K,  s.Kext,    s.gate_sigmoid,
                     s.norm_topk, s.R, iter, s.restricted, s.an, s.ad, s.n_group, s.topk_group,
                     W.Gp,        s.router_kw, s.M};
  const int nper = (s.E + 63) / 64;
  if (nper <= 1)
    launch_route_rows<1>(s, W, ra, st);
  else if (nper <= 2)
    launch_route_rows<2>(s, W, ra, st);
  else if (nper <= 4)
    launch_route_rows<4>(s, W, ra, st);
  else if (nper <= 8)
    launch_route_rows<8>(s, W, ra, st);
  else
    launch_route_rows<16>(s, W, ra, st);
  return hipGetLastError();
}

}  // namespace epoch
