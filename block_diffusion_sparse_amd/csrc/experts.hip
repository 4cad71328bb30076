// Expert compute on the fresh worklist, the shared expert, and the combine / stale merge /
// dense restore (gfx950).
//
// Routed experts (teardown, MoE-bottleneck equation; FreshLane: the same fused expert math
// run on a smaller worklist, invalid slots load no weights): the worklist is grouped by
// expert, so a tile of up to kTileRows pairs of one expert streams that expert's weights once
// for all of its rows.  The contraction is a dense bf16 GEMM and runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  The shared expert (untouched by the
// liveness split, teardown LSP section) is the same kernel over all M positions.
#include "device_common.h"
#include "epoch_internal.h"
#include "expert_gemm.h"

namespace epoch {

// Weight-stream tiles (k_expert_stream), three chunk buffers.  Routed experts: tiles of 64 rows
// or, when the plan step finds them fewer, 128 (an expert with 65..128 fresh pairs then streams
// its weights once, not twice), eight waves (128 gate/up or 256 down columns share each staged
// activation chunk), one workgroup per CU.  The shared expert, only used here below
// kBigTileMinRows positions: 64-row tiles and four waves, two workgroups per CU, which gives it
// four times the work items.  Both measured best at the benchmark shapes.
constexpr int kStreamBuffers = 3;
constexpr int kLdsPerCu = 160 * 1024;
// dense (shared-expert) layers of at least this many positions use the compute-bound
// 128 x 128 kernel; below it the weight-stream kernel has more workgroups to spread
constexpr int kBigTileMinRows = 2048;
constexpr int kBig256MinBlocks = 512;  // 256-row tiles only when two workgroups per CU remain
// waves of the compute-bound routed tiles (kBigTile rows x 32 kBigWaves weight rows): four, two
// workgroups per CU.  Eight (256 x 256 tiles, one workgroup per CU) measured no faster at the
// 8192-position shape, where these tiles run beside the weight-stream kernel and the larger
// workgroup no longer fits in the LDS it leaves free; nor did k_gemm_w4's one wave per SIMD,
// which takes whole CUs from that kernel (1038 -> 1006 us per layer-iteration at full
// freshness, 755 -> 768 us at half).
constexpr int kBigWaves = 4;

// Workgroups of k_expert_stream with lds bytes each that fit on the device at once, at most
// per_cu per CU, as a multiple of 8 (one per XCD lane).
static int stream_slots(int lds, int per_cu) {
  const int n_cu = device_cu_count();
  const int fit = kLdsPerCu / lds;
  return ((n_cu * (fit < per_cu ? fit : per_cu)) / 8) * 8;
}

template <bool GATEUP, bool ROUTED, int WAVES, int BMAX>
static void launch_gemm_w(int tiles, int per_cu, hipStream_t st, int Kdim, const uint16_t* A,
                          const uint16_t* B0, const uint16_t* B1, const Scratch& W,
                          const int32_t* S_list, uint16_t* out, int M, int Ndim) {
  constexpr int cbw = (GATEUP ? 16 : 32) * WAVES;  // output columns per work item
  constexpr int lds = kStreamBuffers * (BMAX * 64 + 32 * WAVES * 64) * 2;
  const int n_cb = (Ndim + cbw - 1) / cbw;
  // persistent grid: as many workgroups as fit at once, never more than the work items (tile
  // slots rounded up to a multiple of 8, times the column blocks)
  const int slots = stream_slots(lds, per_cu);
  const int items = ((tiles + 7) / 8) * 8 * n_cb;
  launch((k_expert_stream<GATEUP, ROUTED, kStreamBuffers, WAVES, BMAX>),
         dim3(items < slots ? items : slots), dim3(64 * WAVES), 0, st, A, B0, B1, W.flags,
         W.tile_slot, W.tile_row0, W.offs, S_list, W.wl_pos, W.wl_w, out, M, Kdim, Ndim,
         LmPartials{});
}

// Routed experts run eight waves per workgroup, the shared expert four.  When the compute-bound
// big tiles run concurrently on another stream, the routed stream kernel takes four waves and
// one workgroup per CU, leaving LDS for one big-tile workgroup beside it (measured: the two
// kernels slow each other down, but less than they take one after the other).
template <bool GATEUP, bool ROUTED>
static void launch_gemm(int tiles, hipStream_t st, int Kdim, const uint16_t* A, const uint16_t* B0,
                        const uint16_t* B1, const Scratch& W, const int32_t* S_list,
                        uint16_t* out, int M, int Ndim, bool beside_big = false) {
  if constexpr (!ROUTED)
    launch_gemm_w<GATEUP, ROUTED, 4, kDenseTileRows>(tiles, 2, st, Kdim, A, B0, B1, W, S_list,
                                                     out, M, Ndim);
  else if (beside_big)  // short tiles only (the plan step never makes tall ones here)
    launch_gemm_w<GATEUP, ROUTED, 4, kTileRows>(tiles, 1, st, Kdim, A, B0, B1, W, S_list, out,
                                                M, Ndim);
  else
    launch_gemm_w<GATEUP, ROUTED, 8, kTileRowsTall>(tiles, 1, st, Kdim, A, B0, B1, W, S_list,
                                                    out, M, Ndim);
}

// ---------------------------------------------------------------------------- fp32 variant
// fp32 activations and weights (small layers): one thread per output element, sequential fp32
// FMA over the contraction.  Same tiling of rows as the MFMA kernels.
template <bool ROUTED>
__global__ __launch_bounds__(256) void k_gateup_f32(
    const float* __restrict__ x, const float* __restrict__ W1, const float* __restrict__ W3,
    const int32_t* __restrict__ flags, const int32_t* __restrict__ tile_slot,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ S_list, const int32_t* __restrict__ wl_pos,
    float* __restrict__ h, int M, int H, int I) {
  const TileRows tr = tile_rows(ROUTED, blockIdx.x, ROUTED ? kTileRows : kDenseTileRows,
                                ROUTED ? flags[FLAG_NTILES] : 0,
                                tile_slot, tile_row0, offs, M);
  if (!tr.active) return;
  const int e = ROUTED ? S_list[tr.slot] : 0;
  const int i0 = blockIdx.y * kGateUpCols;
  const int ncol = min(kGateUpCols, I - i0);
  const int nrow = tr.row_end - tr.row0;
  for (int idx = threadIdx.x; idx < nrow * ncol; idx += blockDim.x) {
    const int rr = idx / ncol, i = i0 + idx % ncol;
    const int p = tr.row0 + rr;
    const int t = ROUTED ? wl_pos[p] : p;
    const float* xr = x + (size_t)t * H;
    const float* a = W1 + ((size_t)e * I + i) * H;
    const float* b = W3 + ((size_t)e * I + i) * H;
    float gv = 0.f, uv = 0.f;
    for (int k = 0; k < H; ++k) {
      gv = fmaf(xr[k], a[k], gv);
      uv = fmaf(xr[k], b[k], uv);
    }
    h[(size_t)p * I + i] = gv / (1.0f + expf(-gv)) * uv;
  }
}

template <bool ROUTED>
__global__ __launch_bounds__(256) void k_down_f32(
    const float* __restrict__ hbuf, const float* __restrict__ W2, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const float* __restrict__ wl_w, float* __restrict__ out, int M, int H, int I) {
  const TileRows tr = tile_rows(ROUTED, blockIdx.x, ROUTED ? kTileRows : kDenseTileRows,
                                ROUTED ? flags[FLAG_NTILES] : 0,
                                tile_slot, tile_row0, offs, M);
  if (!tr.active) return;
  const int e = ROUTED ? S_list[tr.slot] : 0;
  const int j0 = blockIdx.y * kDownCols;
  const int ncol = min(kDownCols, H - j0);
  const int nrow = tr.row_end - tr.row0;
  for (int idx = threadIdx.x; idx < nrow * ncol; idx += blockDim.x) {
    const int rr = idx / ncol, j = j0 + idx % ncol;
    const int p = tr.row0 + rr;
    const float* hr = hbuf + (size_t)p * I;
    const float* b = W2 + ((size_t)e * H + j) * I;
    float acc = 0.f;
    for (int k = 0; k < I; ++k) acc = fmaf(hr[k], b[k], acc);
    out[(size_t)p * H + j] = (ROUTED ? wl_w[p] : 1.0f) * acc;
  }
}

hipError_t launch_routed_gateup(const Shape& s, const void* x, const void* w1, const void* w3,
                                const LayerState& L, const Scratch& W, hipStream_t st) {
  if (s.bf16)
    launch_gemm<true, true>(s.T_max, st, s.H, static_cast<const uint16_t*>(x),
                            static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3), W,
                            L.S_list, static_cast<uint16_t*>(W.h), s.M, s.I, s.big_routed);
  else
    launch(k_gateup_f32<true>, dim3(s.T_max, (s.I + kGateUpCols - 1) / kGateUpCols), dim3(256),
           0, st, static_cast<const float*>(x), static_cast<const float*>(w1),
           static_cast<const float*>(w3), W.flags, W.tile_slot, W.tile_row0, W.offs, L.S_list,
           W.wl_pos, static_cast<float*>(W.h), s.M, s.H, s.I);
  return hipGetLastError();
}

hipError_t launch_routed_gateup_big(const Shape& s, const void* x, const void* w1,
                                    const void* w3, const LayerState& L, const Scratch& W,
                                    hipStream_t st) {
  // experts with many fresh rows: compute-bound kBigTile-row tiles
  launch((k_gemm_big<true, true, kBigTile>),
         dim3(((s.T_big_max + 7) / 8) * 8 * ((s.I + 16 * kBigWaves - 1) / (16 * kBigWaves))),
         dim3(64 * kBigWaves), 0, st,
         static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w1),
         static_cast<const uint16_t*>(w3), W.flags, W.tile_slot_b, W.tile_row0_b, W.offs,
         L.S_list, W.wl_pos, W.wl_w, static_cast<uint16_t*>(W.h), s.M, s.H, s.I);
  return hipGetLastError();
}

hipError_t launch_routed_down(const Shape& s, const void* w2, const LayerState& L,
                              const Scratch& W, hipStream_t st) {
  if (s.bf16)
    launch_gemm<false, true>(s.T_max, st, s.I, static_cast<const uint16_t*>(W.h),
                             static_cast<const uint16_t*>(w2), nullptr, W, L.S_list,
                             static_cast<uint16_t*>(W.y_pair), s.M, s.H, s.big_routed);
  else
    launch(k_down_f32<true>, dim3(s.T_max, (s.H + kDownCols - 1) / kDownCols), dim3(256), 0, st,
           static_cast<const float*>(W.h), static_cast<const float*>(w2), W.flags, W.tile_slot,
           W.tile_row0, W.offs, L.S_list, W.wl_w, static_cast<float*>(W.y_pair), s.M, s.H, s.I);
  return hipGetLastError();
}

hipError_t launch_routed_down_big(const Shape& s, const void* w2, const LayerState& L,
                                  const Scratch& W, hipStream_t st) {
  launch((k_gemm_big<false, true, kBigTile>),
         dim3(((s.T_big_max + 7) / 8) * 8 * ((s.H + 32 * kBigWaves - 1) / (32 * kBigWaves))),
         dim3(64 * kBigWaves), 0, st,
         static_cast<const uint16_t*>(W.h), static_cast<const uint16_t*>(w2), nullptr, W.flags,
         W.tile_slot_b, W.tile_row0_b, W.offs, L.S_list, W.wl_pos, W.wl_w,
         static_cast<uint16_t*>(W.y_pair), s.M, s.I, s.H);
  return hipGetLastError();
}

hipError_t launch_shared(const Shape& s, const void* x, const void* sw1, const void* sw3,
                         const void* sw2, const Scratch& W, hipStream_t st) {
  dim3 g1(s.T_dense, (s.Is + kGateUpCols - 1) / kGateUpCols);
  dim3 g2(s.T_dense, (s.H + kDownCols - 1) / kDownCols);
  if (s.bf16 && s.M >= kBigTileMinRows) {
    // many rows: compute-bound tiles with both operands copied into LDS; 256-row tiles when
    // they still give every CU two workgroups, else 128-row tiles
    const int t128 = (s.M + 127) / 128, t256 = (s.M + 255) / 256;
    const int ncu = s.Is / 64, ncd = (s.H + 127) / 128;
    auto grid = [](int tiles, int n_cb) { return dim3(((tiles + 7) / 8) * 8 * n_cb); };
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* hs = static_cast<const uint16_t*>(W.hs);
    uint16_t* hs_out = static_cast<uint16_t*>(W.hs);
    uint16_t* S_out = static_cast<uint16_t*>(W.S);
    const uint16_t* w1b = static_cast<const uint16_t*>(sw1);
    const uint16_t* w3b = static_cast<const uint16_t*>(sw3);
    const uint16_t* w2b = static_cast<const uint16_t*>(sw2);
    // one-wave-per-SIMD 256 x 256 tiles once they give every CU a tile
    const int n_cu = device_cu_count();
    const int w4u = (s.Is + 127) / 128, w4d = (s.H + 255) / 256;
    if (t256 * w4u >= n_cu)
      launch((k_gemm_w4<true, false>), dim3(gemm_w4_dense_grid(s.M, w4u)), dim3(256), 0, st, xb,
             w1b, w3b, W.flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, hs_out, s.M,
             s.H, s.Is);
    else if (t256 * ncu >= kBig256MinBlocks)
      launch((k_gemm_big<true, false, 256>), grid(t256, ncu), dim3(256), 0, st, xb, w1b,
             w3b, W.flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, hs_out, s.M, s.H,
             s.Is);
    else
      launch((k_gemm_big<true, false>), grid(t128, ncu), dim3(256), 0, st, xb, w1b, w3b, W.flags,
             nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, hs_out, s.M, s.H, s.Is);
    if (t256 * w4d >= n_cu)
      launch((k_gemm_w4<false, false>), dim3(gemm_w4_dense_grid(s.M, w4d)), dim3(256), 0, st, hs,
             w2b, nullptr, W.flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, S_out,
             s.M, s.Is, s.H);
    else if (t256 * ncd >= kBig256MinBlocks)
      launch((k_gemm_big<false, false, 256>), grid(t256, ncd), dim3(256), 0, st, hs, w2b,
             nullptr, W.flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, S_out, s.M,
             s.Is, s.H);
    else
      launch((k_gemm_big<false, false>), grid(t128, ncd), dim3(256), 0, st, hs, w2b, nullptr,
             W.flags, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, S_out, s.M, s.Is, s.H);
  } else if (s.bf16) {
    launch_gemm<true, false>(s.T_dense, st, s.H, static_cast<const uint16_t*>(x),
                             static_cast<const uint16_t*>(sw1), static_cast<const uint16_t*>(sw3),
                             W, nullptr, static_cast<uint16_t*>(W.hs), s.M, s.Is);
    launch_gemm<false, false>(s.T_dense, st, s.Is,
                              static_cast<const uint16_t*>(W.hs), static_cast<const uint16_t*>(sw2),
                              nullptr, W, nullptr, static_cast<uint16_t*>(W.S), s.M, s.H);
  } else {
    launch(k_gateup_f32<false>, g1, dim3(256), 0, st, static_cast<const float*>(x),
                       static_cast<const float*>(sw1), static_cast<const float*>(sw3), W.flags,
                       nullptr, nullptr, nullptr, nullptr, nullptr, static_cast<float*>(W.hs),
                       s.M, s.H, s.Is);
    launch(k_down_f32<false>, g2, dim3(256), 0, st, static_cast<const float*>(W.hs),
                       static_cast<const float*>(sw2), W.flags, nullptr, nullptr, nullptr, nullptr,
                       nullptr, static_cast<float*>(W.S), s.M, s.H, s.Is);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------- combine / merge
// Weighted combine, stale merge and dense restore (teardown, LSP: Y[F] = Y_F,
// Y[not F] = C_l[not F]; FreshLane combine and scatter/merge; the layer epilogue sees the
// full dense tensor).  One workgroup per position, 8 columns per thread per step.
//   fresh t:  R_t = act(sum_{k<K} y_pair[inv[t,k]]) (fp32, k order); C_l[t] = R_t
//   stable t: R_t = C_l[t], copied bitwise
//   Y_t = act(R_t + S_t) with the shared expert, else R_t.
template <typename T>
struct Vec8 {
  T v[8];
};

template <typename T>
__device__ __forceinline__ void load8(const T* p, float out[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const T v[8]) {
  if constexpr (sizeof(T) == 2) {
    uint4 u;
    u.x = (uint32_t)v[0] | ((uint32_t)v[1] << 16);
    u.y = (uint32_t)v[2] | ((uint32_t)v[3] << 16);
    u.z = (uint32_t)v[4] | ((uint32_t)v[5] << 16);
    u.w = (uint32_t)v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<uint4*>(p) = u;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <typename T>
__device__ __forceinline__ void copy8(const T* src, T v[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (T)(w[i] & 0xffffu);
      v[2 * i + 1] = (T)(w[i] >> 16);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// KT: the number of pairs per position when fixed at compile time (all K loads of a column
// block issued before the first add), 0 for any K (one pair at a time)
template <typename T, int KT>
__global__ __launch_bounds__(256) void k_combine(int M, int H, int K, int has_shared, int iter,
                                                 LayerState L, const int32_t* __restrict__ inv,
                                                 const T* __restrict__ y_pair,
                                                 const T* __restrict__ S, T* __restrict__ y,
                                                 T* __restrict__ y_routed) {
  const int t = blockIdx.x;
  const bool f = L.fresh[t] != 0;
  T* __restrict__ cache = static_cast<T*>(L.cache);
  if (threadIdx.x == 0) {
    // the commit of this forward, into the next copy of the position's state (teardown, LSP
    // state machine: a fresh output enters the cache and restarts the age; D_i becomes the
    // D_{i-1} of the next iteration); it takes effect when the caller commits
    L.valid_n[t] = (L.valid[t] || f) ? 1 : 0;
    L.last_fresh_n[t] = f ? iter : L.last_fresh[t];
    L.prev_D_n[t] = L.Dcur[t];
  }
  for (int j = threadIdx.x * 8; j < H; j += blockDim.x * 8) {
    T rb[8];
    if (f) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (KT > 0) {
        float v[KT][8];
#pragma unroll
        for (int k = 0; k < KT; ++k) load8<T>(y_pair + (size_t)inv[(size_t)t * KT + k] * H + j, v[k]);
#pragma unroll
        for (int k = 0; k < KT; ++k)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += v[k][i];
      } else {
        for (int k = 0; k < K; ++k) {
          const int p = inv[(size_t)t * K + k];
          float v[8];
          load8<T>(y_pair + (size_t)p * H + j, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) rb[i] = from_f32<T>(acc[i]);
      store8<T>(cache + (size_t)t * H + j, rb);
    } else {
      copy8<T>(cache + (size_t)t * H + j, rb);
    }
    if (y_routed) store8<T>(y_routed + (size_t)t * H + j, rb);
    T yo[8];
    if (has_shared) {
      float sv[8];
      load8<T>(S + (size_t)t * H + j, sv);
#pragma unroll
      for (int i = 0; i < 8; ++i) yo[i] = from_f32<T>(to_f32<T>(rb[i]) + sv[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) yo[i] = rb[i];
    }
    store8<T>(y + (size_t)t * H + j, yo);
  }
}

hipError_t launch_combine(const Shape& s, int iter, const LayerState& L, const Scratch& W,
                          void* y, void* y_routed, hipStream_t st) {
  if (s.bf16 && s.K == 8)
    launch(k_combine<uint16_t, 8>, dim3(s.M), dim3(256), 0, st, s.M, s.H, s.K,
                       s.n_shared, iter, L, W.inv, static_cast<const uint16_t*>(W.y_pair),
                       static_cast<const uint16_t*>(W.S), static_cast<uint16_t*>(y),
                       static_cast<uint16_t*>(y_routed));
  else if (s.bf16)
    launch(k_combine<uint16_t, 0>, dim3(s.M), dim3(256), 0, st, s.M, s.H, s.K,
                       s.n_shared, iter, L, W.inv, static_cast<const uint16_t*>(W.y_pair),
                       static_cast<const uint16_t*>(W.S), static_cast<uint16_t*>(y),
                       static_cast<uint16_t*>(y_routed));
  else
    launch(k_combine<float, 0>, dim3(s.M), dim3(256), 0, st, s.M, s.H, s.K, s.n_shared,
                       iter, L, W.inv, static_cast<const float*>(W.y_pair),
                       static_cast<const float*>(W.S), static_cast<float*>(y),
                       static_cast<float*>(y_routed));
  return hipGetLastError();
}

}  // namespace epoch
