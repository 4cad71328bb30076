// Router: gate logits over every position and the per-position top-k (gfx950).
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

// ---------------------------------------------------------------------------- partial logits
// One wave computes a 32-position x 32-expert tile over one k-range with 2 x 2 blocks of
// v_mfma_f64_16x16x4.  The contraction index is permuted so that each lane feeds four
// consecutive k values (one 8- or 16-byte load) to four successive MFMA steps; A and B use
// the same permutation, so every product pairs x[t,k] with W[e,k].
template <typename T>
__device__ __forceinline__ void load4_as_f64(const T* p, bool ok, double out[4]);

template <>
__device__ __forceinline__ void load4_as_f64<uint16_t>(const uint16_t* p, bool ok, double out[4]) {
  uint2 v = ok ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
  out[0] = (double)__uint_as_float(v.x << 16);
  out[1] = (double)__uint_as_float(v.x & 0xffff0000u);
  out[2] = (double)__uint_as_float(v.y << 16);
  out[3] = (double)__uint_as_float(v.y & 0xffff0000u);
}

template <>
__device__ __forceinline__ void load4_as_f64<float>(const float* p, bool ok, double out[4]) {
  float4 v = ok ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
  out[0] = v.x;
  out[1] = v.y;
  out[2] = v.z;
  out[3] = v.w;
}

template <typename T>
__global__ __launch_bounds__(64) void k_router_partial(const T* __restrict__ x,
                                                       const float* __restrict__ Wg,
                                                       double* __restrict__ Gpart, int M, int H,
                                                       int E, int kchunk,
                                                       int32_t* __restrict__ flags) {
  const int lane = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && lane < FLAG_WORDS)
    flags[lane] = 0;  // per-forward flags start clear; later kernels of this forward set them
  const int e0 = blockIdx.x * 32, t0 = blockIdx.y * 32, split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int kend = min(H, kbeg + kchunk);
  const int r = lane & 15, g = lane >> 4;
  const int ta = t0 + r, tb = t0 + 16 + r, ea = e0 + r, eb = e0 + 16 + r;
  const bool vta = ta < M, vtb = tb < M, vea = ea < E, veb = eb < E;
  const T* xa = x + (size_t)(vta ? ta : 0) * H;
  const T* xb = x + (size_t)(vtb ? tb : 0) * H;
  const float* wa = Wg + (size_t)(vea ? ea : 0) * H;
  const float* wb = Wg + (size_t)(veb ? eb : 0) * H;
  f64x4 acc00 = {0, 0, 0, 0}, acc01 = acc00, acc10 = acc00, acc11 = acc00;
  for (int k = kbeg; k < kend; k += 16) {
    const int kk = k + 4 * g;
    double A0[4], A1[4], B0[4], B1[4];
    load4_as_f64<T>(xa + kk, vta, A0);
    load4_as_f64<T>(xb + kk, vtb, A1);
    load4_as_f64<float>(wa + kk, vea, B0);
    load4_as_f64<float>(wb + kk, veb, B1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc00 = __builtin_amdgcn_mfma_f64_16x16x4f64(A0[j], B0[j], acc00, 0, 0, 0);
      acc01 = __builtin_amdgcn_mfma_f64_16x16x4f64(A0[j], B1[j], acc01, 0, 0, 0);
      acc10 = __builtin_amdgcn_mfma_f64_16x16x4f64(A1[j], B0[j], acc10, 0, 0, 0);
      acc11 = __builtin_amdgcn_mfma_f64_16x16x4f64(A1[j], B1[j], acc11, 0, 0, 0);
    }
  }
  // f64 16x16x4 output layout: D[i][j] sits in lane (j + 16 * (i % 4)), register i / 4
  double* out = Gpart + (size_t)split * M * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + g;
    const int t_lo = t0 + row, t_hi = t0 + 16 + row;
    if (t_lo < M) {
      if (vea) out[(size_t)t_lo * E + ea] = acc00[i];
      if (veb) out[(size_t)t_lo * E + eb] = acc01[i];
    }
    if (t_hi < M) {
      if (vea) out[(size_t)t_hi * E + ea] = acc10[i];
      if (veb) out[(size_t)t_hi * E + eb] = acc11[i];
    }
  }
}

// ---------------------------------------------------------------------------- top-k select
// One wave per position: sums the k-split partials and the bias, rounds to fp32, selects the
// K_ext candidates in key order (logit desc, expert id asc), computes the gate scores in
// double (softmax over all E or sigmoid), the routing weights of the first K, and the
// planner weight q = floor(s * 2^16 + 1/2).  Also raises the support-miss flag (a routed
// expert outside the current support) and the liveness-anomaly flag (decoded -> live).
constexpr int kSelPerLane = kMaxExperts / kWave;

__global__ __launch_bounds__(256) void k_route_select(
    const double* __restrict__ Gpart, int splits, const float* __restrict__ bias,
    const uint8_t* __restrict__ D, const uint8_t* __restrict__ prevD,
    const uint8_t* __restrict__ inS, const int32_t* __restrict__ S_valid, int M, int E, int K,
    int Kext, int gate_sigmoid, int norm_topk, float* __restrict__ G, int32_t* __restrict__ ids,
    float* __restrict__ scores, int32_t* __restrict__ qout, float* __restrict__ wout,
    uint8_t* __restrict__ Dcopy, int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= M) return;
  const int nper = (E + 63) >> 6;
  float gv[kSelPerLane];
#pragma unroll
  for (int j = 0; j < kSelPerLane; ++j) {
    gv[j] = -INFINITY;
    const int e = lane + 64 * j;
    if (j < nper && e < E) {
      double acc = 0.0;
      for (int s = 0; s < splits; ++s) acc += Gpart[((size_t)s * M + t) * E + e];
      if (bias) acc += (double)bias[e];
      gv[j] = (float)acc;
      G[(size_t)t * E + e] = gv[j];
    }
  }
  uint32_t taken = 0;
  int my_id = 0;
  float my_g = 0.f;
  for (int r = 0; r < Kext; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j) {
      const int e = lane + 64 * j;
      if (j < nper && e < E && !((taken >> j) & 1u) && (gv[j] > bv || (gv[j] == bv && e < bi))) {
        bv = gv[j];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == r) {
      my_id = bi;
      my_g = bv;
    }
  }
  double zmax = -INFINITY, z = 0.0;
  if (!gate_sigmoid) {
    double m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (j < nper && lane + 64 * j < E) m = fmax(m, (double)gv[j]);
    zmax = wave_max(m);
    double part = 0.0;
#pragma unroll
    for (int j = 0; j < kSelPerLane; ++j)
      if (j < nper && lane + 64 * j < E) part += exp((double)gv[j] - zmax);
    z = wave_sum(part);
  }
  double s = 0.0;
  if (lane < Kext) s = gate_sigmoid ? 1.0 / (1.0 + exp(-(double)my_g)) : exp((double)my_g - zmax) / z;
  const double denom = wave_sum(lane < K ? s : 0.0);
  if (lane < Kext) {
    ids[(size_t)t * Kext + lane] = my_id;
    scores[(size_t)t * Kext + lane] = (float)s;
    qout[(size_t)t * Kext + lane] = (int32_t)floor(s * 65536.0 + 0.5);
  }
  if (lane < K) wout[(size_t)t * K + lane] = (float)(norm_topk ? s / denom : s);
  const bool miss = (*S_valid != 0) && lane < K && !inS[my_id];
  if (ballot64(miss) != 0 && lane == 0) flags[FLAG_MISS] = 1;
  if (lane == 0) {
    const uint8_t d = D[t];
    Dcopy[t] = d;
    if (prevD[t] && !d) flags[FLAG_ANOMALY] = 1;
  }
}

hipError_t launch_router(const Shape& s, const void* x, const float* Wg, const float* bias,
                         const uint8_t* D, const LayerState& L, const Scratch& W, hipStream_t st) {
  const int kchunk = ((s.H + s.splits - 1) / s.splits + 15) / 16 * 16;
  dim3 grid((s.E + 31) / 32, (s.M + 31) / 32, s.splits);
  if (s.bf16)
    hipLaunchKernelGGL(k_router_partial<uint16_t>, grid, dim3(64), 0, st,
                       static_cast<const uint16_t*>(x), Wg, W.Gpart, s.M, s.H, s.E, kchunk,
                       W.flags);
  else
    hipLaunchKernelGGL(k_router_partial<float>, grid, dim3(64), 0, st,
                       static_cast<const float*>(x), Wg, W.Gpart, s.M, s.H, s.E, kchunk, W.flags);
  hipLaunchKernelGGL(k_route_select, dim3((s.M + 3) / 4), dim3(256), 0, st, W.Gpart, s.splits,
                     bias, D, L.prev_D, L.inS, L.S_valid, s.M, s.E, s.K, s.Kext, s.gate_sigmoid,
                     s.norm_topk, W.G, W.ids, W.scores, W.q, W.w, L.Dcur, W.flags);
  return hipGetLastError();
}

}  // namespace epoch
