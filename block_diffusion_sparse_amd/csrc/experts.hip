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

namespace epoch {

// A 16-byte fragment: 8 consecutive bf16 of one row.
__device__ __forceinline__ bf16x8 ld_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 zero_frag() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

// Row source of a tile: routed tiles gather activations through the worklist; dense (shared
// expert) tiles take positions in order.
struct TileRows {
  int row0, row_end, slot;
  bool active;
};

__device__ __forceinline__ TileRows tile_rows(bool routed, int tile, const int32_t* flags,
                                              const int32_t* tile_slot,
                                              const int32_t* tile_row0, const int32_t* offs,
                                              int M) {
  TileRows r;
  if (routed) {
    r.active = tile < flags[FLAG_NTILES];
    if (!r.active) return r;
    r.slot = tile_slot[tile];
    r.row0 = tile_row0[tile];
    r.row_end = min(offs[r.slot + 1], r.row0 + kTileRows);
  } else {
    r.active = true;
    r.slot = 0;
    r.row0 = tile * kTileRows;
    r.row_end = min(M, r.row0 + kTileRows);
  }
  return r;
}

// ---------------------------------------------------------------------------- gate/up + SwiGLU
// Workgroup = 4 waves over one tile (32 rows) x 64 intermediate columns; wave w owns columns
// [16w, 16w + 16) of both W1 and W3, full K.  Lane l feeds A row (l % 16) and B column
// (l % 16) with the same 8 consecutive k values (k-group l / 16), so every product pairs
// x[t, k] with W[i, k].  Epilogue: h = bf16(silu(g) * u), silu(z) = z / (1 + e^-z).
template <bool ROUTED>
__global__ __launch_bounds__(256) void k_gateup_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W3, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, uint16_t* __restrict__ h, int M, int H, int I) {
  const TileRows tr = tile_rows(ROUTED, blockIdx.x, flags, tile_slot, tile_row0, offs, M);
  if (!tr.active) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e = ROUTED ? S_list[tr.slot] : 0;
  const int i0 = blockIdx.y * kGateUpCols + wave * 16;
  const size_t wofs = (size_t)e * I * H;
  const uint16_t* w1r = W1 + wofs + (size_t)(i0 + r) * H + 8 * g;
  const uint16_t* w3r = W3 + wofs + (size_t)(i0 + r) * H + 8 * g;
  const int p0 = tr.row0 + r, p1 = tr.row0 + 16 + r;
  const bool v0 = p0 < tr.row_end, v1 = p1 < tr.row_end;
  const int x0 = v0 ? (ROUTED ? wl_pos[p0] : p0) : 0;
  const int x1 = v1 ? (ROUTED ? wl_pos[p1] : p1) : 0;
  const uint16_t* xr0 = x + (size_t)x0 * H + 8 * g;
  const uint16_t* xr1 = x + (size_t)x1 * H + 8 * g;
  f32x4 g0 = {0, 0, 0, 0}, g1 = g0, u0 = g0, u1 = g0;
#pragma unroll 4
  for (int k = 0; k < H; k += 32) {
    const bf16x8 a0 = v0 ? ld_frag(xr0 + k) : zero_frag();
    const bf16x8 a1 = v1 ? ld_frag(xr1 + k) : zero_frag();
    const bf16x8 b1 = ld_frag(w1r + k);
    const bf16x8 b3 = ld_frag(w3r + k);
    g0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b1, g0, 0, 0, 0);
    g1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, g1, 0, 0, 0);
    u0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b3, u0, 0, 0, 0);
    u1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b3, u1, 0, 0, 0);
  }
  // D[i][j] of a 16x16 block: lane j + 16 * (i / 4), register i % 4
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row_a = tr.row0 + 4 * g + q, row_b = row_a + 16;
    if (row_a < tr.row_end) {
      const float gv = g0[q], uv = u0[q];
      h[(size_t)row_a * I + i0 + r] = f32_to_bf16(gv / (1.0f + expf(-gv)) * uv);
    }
    if (row_b < tr.row_end) {
      const float gv = g1[q], uv = u1[q];
      h[(size_t)row_b * I + i0 + r] = f32_to_bf16(gv / (1.0f + expf(-gv)) * uv);
    }
  }
}

// ---------------------------------------------------------------------------- down projection
// Workgroup = 4 waves over one tile x 64 output columns; wave w owns columns [16w, 16w + 16).
// Routed: y_pair[p] = bf16(w_p * (W2_e h_p)); dense: out[t] = bf16(W2 h_t).
template <bool ROUTED>
__global__ __launch_bounds__(256) void k_down_bf16(
    const uint16_t* __restrict__ hbuf, const uint16_t* __restrict__ W2,
    const int32_t* __restrict__ flags, const int32_t* __restrict__ tile_slot,
    const int32_t* __restrict__ tile_row0, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ S_list, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int H, int I) {
  const TileRows tr = tile_rows(ROUTED, blockIdx.x, flags, tile_slot, tile_row0, offs, M);
  if (!tr.active) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int e = ROUTED ? S_list[tr.slot] : 0;
  const int j0 = blockIdx.y * kDownCols + wave * 16;
  const uint16_t* w2r = W2 + (size_t)e * H * I + (size_t)(j0 + r) * I + 8 * g;
  const int p0 = tr.row0 + r, p1 = tr.row0 + 16 + r;
  const bool v0 = p0 < tr.row_end, v1 = p1 < tr.row_end;
  const uint16_t* hr0 = hbuf + (size_t)(v0 ? p0 : 0) * I + 8 * g;
  const uint16_t* hr1 = hbuf + (size_t)(v1 ? p1 : 0) * I + 8 * g;
  f32x4 c0 = {0, 0, 0, 0}, c1 = c0;
#pragma unroll 4
  for (int k = 0; k < I; k += 32) {
    const bf16x8 a0 = v0 ? ld_frag(hr0 + k) : zero_frag();
    const bf16x8 a1 = v1 ? ld_frag(hr1 + k) : zero_frag();
    const bf16x8 b = ld_frag(w2r + k);
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, c1, 0, 0, 0);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row_a = tr.row0 + 4 * g + q, row_b = row_a + 16;
    if (row_a < tr.row_end) {
      const float s = ROUTED ? wl_w[row_a] : 1.0f;
      out[(size_t)row_a * H + j0 + r] = f32_to_bf16(s * c0[q]);
    }
    if (row_b < tr.row_end) {
      const float s = ROUTED ? wl_w[row_b] : 1.0f;
      out[(size_t)row_b * H + j0 + r] = f32_to_bf16(s * c1[q]);
    }
  }
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
  const TileRows tr = tile_rows(ROUTED, blockIdx.x, flags, tile_slot, tile_row0, offs, M);
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
  const TileRows tr = tile_rows(ROUTED, blockIdx.x, flags, tile_slot, tile_row0, offs, M);
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
  dim3 grid(s.T_max, (s.I + kGateUpCols - 1) / kGateUpCols);
  if (s.bf16)
    hipLaunchKernelGGL(k_gateup_bf16<true>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w1),
                       static_cast<const uint16_t*>(w3), W.flags, W.tile_slot, W.tile_row0,
                       W.offs, L.S_list, W.wl_pos, static_cast<uint16_t*>(W.h), s.M, s.H, s.I);
  else
    hipLaunchKernelGGL(k_gateup_f32<true>, grid, dim3(256), 0, st, static_cast<const float*>(x),
                       static_cast<const float*>(w1), static_cast<const float*>(w3), W.flags,
                       W.tile_slot, W.tile_row0, W.offs, L.S_list, W.wl_pos,
                       static_cast<float*>(W.h), s.M, s.H, s.I);
  return hipGetLastError();
}

hipError_t launch_routed_down(const Shape& s, const void* w2, const LayerState& L,
                              const Scratch& W, hipStream_t st) {
  dim3 grid(s.T_max, (s.H + kDownCols - 1) / kDownCols);
  if (s.bf16)
    hipLaunchKernelGGL(k_down_bf16<true>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(W.h), static_cast<const uint16_t*>(w2),
                       W.flags, W.tile_slot, W.tile_row0, W.offs, L.S_list, W.wl_w,
                       static_cast<uint16_t*>(W.y_pair), s.M, s.H, s.I);
  else
    hipLaunchKernelGGL(k_down_f32<true>, grid, dim3(256), 0, st, static_cast<const float*>(W.h),
                       static_cast<const float*>(w2), W.flags, W.tile_slot, W.tile_row0, W.offs,
                       L.S_list, W.wl_w, static_cast<float*>(W.y_pair), s.M, s.H, s.I);
  return hipGetLastError();
}

hipError_t launch_shared(const Shape& s, const void* x, const void* sw1, const void* sw3,
                         const void* sw2, const Scratch& W, hipStream_t st) {
  dim3 g1(s.T_dense, (s.Is + kGateUpCols - 1) / kGateUpCols);
  dim3 g2(s.T_dense, (s.H + kDownCols - 1) / kDownCols);
  if (s.bf16) {
    hipLaunchKernelGGL(k_gateup_bf16<false>, g1, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(sw1),
                       static_cast<const uint16_t*>(sw3), W.flags, nullptr, nullptr, nullptr,
                       nullptr, nullptr, static_cast<uint16_t*>(W.hs), s.M, s.H, s.Is);
    hipLaunchKernelGGL(k_down_bf16<false>, g2, dim3(256), 0, st,
                       static_cast<const uint16_t*>(W.hs), static_cast<const uint16_t*>(sw2),
                       W.flags, nullptr, nullptr, nullptr, nullptr, nullptr,
                       static_cast<uint16_t*>(W.S), s.M, s.H, s.Is);
  } else {
    hipLaunchKernelGGL(k_gateup_f32<false>, g1, dim3(256), 0, st, static_cast<const float*>(x),
                       static_cast<const float*>(sw1), static_cast<const float*>(sw3), W.flags,
                       nullptr, nullptr, nullptr, nullptr, nullptr, static_cast<float*>(W.hs),
                       s.M, s.H, s.Is);
    hipLaunchKernelGGL(k_down_f32<false>, g2, dim3(256), 0, st, static_cast<const float*>(W.hs),
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

template <typename T>
__global__ __launch_bounds__(256) void k_combine(int M, int H, int K, int has_shared,
                                                 const uint8_t* __restrict__ fresh,
                                                 const int32_t* __restrict__ inv,
                                                 const T* __restrict__ y_pair,
                                                 const T* __restrict__ S, T* __restrict__ cache,
                                                 T* __restrict__ y, T* __restrict__ y_routed) {
  const int t = blockIdx.x;
  const bool f = fresh[t] != 0;
  for (int j = threadIdx.x * 8; j < H; j += blockDim.x * 8) {
    T rb[8];
    if (f) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int k = 0; k < K; ++k) {
        const int p = inv[(size_t)t * K + k];
        float v[8];
        load8<T>(y_pair + (size_t)p * H + j, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
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

hipError_t launch_combine(const Shape& s, const LayerState& L, const Scratch& W, void* y,
                          void* y_routed, hipStream_t st) {
  if (s.bf16)
    hipLaunchKernelGGL(k_combine<uint16_t>, dim3(s.M), dim3(256), 0, st, s.M, s.H, s.K,
                       s.n_shared, L.fresh, W.inv, static_cast<const uint16_t*>(W.y_pair),
                       static_cast<const uint16_t*>(W.S), static_cast<uint16_t*>(L.cache),
                       static_cast<uint16_t*>(y), static_cast<uint16_t*>(y_routed));
  else
    hipLaunchKernelGGL(k_combine<float>, dim3(s.M), dim3(256), 0, st, s.M, s.H, s.K, s.n_shared,
                       L.fresh, W.inv, static_cast<const float*>(W.y_pair),
                       static_cast<const float*>(W.S), static_cast<float*>(L.cache),
                       static_cast<float*>(y), static_cast<float*>(y_routed));
  return hipGetLastError();
}

}  // namespace epoch
