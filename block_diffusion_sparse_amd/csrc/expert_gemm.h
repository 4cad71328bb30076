// Grouped bf16 expert GEMM of the SwiGLU experts (gfx950, v_mfma_f32_16x16x32_bf16).
#pragma once
#include "device_common.h"
#include "epoch_internal.h"

namespace epoch {

// Row source of a tile: routed tiles gather activations through the worklist; dense (shared
// expert) tiles take positions in order.
struct TileRows {
  int row0, row_end, slot;
  bool active;
};

__device__ __forceinline__ TileRows tile_rows(bool routed, int tile, int tile_rows_max,
                                              int ntiles, const int32_t* tile_slot,
                                              const int32_t* tile_row0, const int32_t* offs,
                                              int M) {
  TileRows r;
  if (routed) {
    r.active = tile < ntiles;
    if (!r.active) return r;
    r.slot = tile_slot[tile];
    r.row0 = tile_row0[tile];
    r.row_end = min(offs[r.slot + 1], r.row0 + tile_rows_max);
  } else {
    r.row0 = tile * tile_rows_max;
    r.active = r.row0 < M;
    r.slot = 0;
    r.row_end = min(M, r.row0 + tile_rows_max);
  }
  return r;
}


constexpr float kLog2e = 1.4426950408889634f;

// SwiGLU's silu(g) = g / (1 + e^-g) as v_exp_f32 and v_rcp_f32 (both about 1 ulp): relative error
// about 1e-6 for |g| up to 20, far below the bf16 rounding of h that follows; for g below -88
// e^-g overflows to inf and the result is the correctly signed 0.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * kLog2e));
}

// Output of the LM-head kernels (k_expert_stream's LM mode, k_lm_head_w4): the rows are live
// positions (gathered through live_list, n_live of them), the columns vocabulary tokens, and
// instead of the logits the kernels write, per row and per block of tokens, the largest logit,
// its token (lower id on ties) and the sum of exp(logit - largest) over the block; n_p per row:
// vocab / 32 from k_expert_stream (one wave's columns), vocab / 256 rounded up from k_lm_head_w4
// (one tile's columns).
struct LmPartials {
  const int32_t* live_list;
  const int32_t* n_live;
  float* pmax;
  int32_t* parg;
  float* psum;
  int n_p;
};

// Wait until at most N of this wave's vector-memory operations are outstanding and all of its
// LDS operations have completed (s_waitcnt: vmcnt N, lgkmcnt 0, expcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// One 16-byte copy per lane from global memory into LDS (global_load_lds_dwordx4): lane l's
// bytes land at lds_dst + 16 l, where lds_dst is the same for the whole wave.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// The same copy with the non-temporal policy (nt), for operands streamed once per launch (the
// expert weights): whole 128-byte lines read this way sustain a higher HBM rate on gfx950.
__device__ __forceinline__ void copy16_to_lds_stream(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 2);
}

// Weight-stream grouped GEMM of both projections of the SwiGLU expert (v_mfma_f32_16x16x32_bf16,
// fp32 accumulation), for tiles of up to BM rows of one expert: the rows (fresh pairs, gathered
// through the worklist for routed gate/up; positions in order for the shared expert) are few,
// so the expert's weights, read once per tile, dominate the traffic.  A work item is one tile
// against 32 WAVES weight rows (a column block):
//   gate/up: wave w owns intermediate columns 16 w .. 16 w + 15 of the block's 16 WAVES and
//            holds those rows of W1 and of W3; epilogue h = bf16(silu(g) * u);
//   down:    wave w owns output columns 32 w .. 32 w + 31 of the block's 32 WAVES rows of W2;
//            epilogue y = bf16(w_p * acc) (routed) or bf16(acc) (shared expert).
// Every wave multiplies all rows of the tile; 16-row blocks past the tile's last row are
// skipped (no fragment reads, no MFMAs), so a short tile costs only its weight stream.
// K runs in chunks of 64 bf16, so a row of a chunk is one 128-byte line and one copy
// instruction (global_load_lds_dwordx4, lane l's 16 bytes landing at the wave's LDS base +
// 16 l) moves eight whole lines.  Every wave copies its own 32 weight rows with the
// non-temporal policy (whole lines streamed that way sustain a higher HBM rate) and its share
// of the activation rows with the cached one (the tile's other column blocks read them again).
// LDS rows of 128 bytes hold k-segment slot ^ (row & 7) in 16-byte slot `slot`: ds_read_b128
// is served eight lanes at a time, 128 bytes a cycle, and the eight rows those lanes read then
// sit in eight different slots, i.e. on distinct banks (no bank conflicts).
//
// Synchronisation (NB chunk buffers): step q waits for its own copies of chunk q (vmcnt; the
// NB - 2 chunks after it may stay in flight), meets the barrier (every wave's copies of chunk q
// have landed, every wave has finished reading chunk q - 1), copies chunk q + NB - 1 into the
// buffer of chunk q - 1, then reads chunk q's fragments (inline ds_read_b128, with an explicit
// lgkmcnt wait that names them, since the compiler cannot tell chunk buffers apart and would
// otherwise wait for every copy in flight) and multiplies.  NB - 1 chunks are in flight during
// the MFMAs.
//
// Persistent workgroups: the grid (a multiple of 8, about one workgroup per CU slot) walks the
// work items i = blockIdx.x + k gridDim.x, and the chunks of consecutive items form one
// stream, so the next item's first chunks are already in flight while the current one is
// multiplied and stored (no pipeline fill or drain per item).  Item i is column block
// (i / 8) % n_col_blocks of tile 8 ((i / 8) / n_col_blocks) + i % 8: the hardware hands
// workgroups to the 8 XCDs in turn, so every column block of a tile runs on one XCD and the
// tile's activation rows are fetched into one L2 only.  Everything an item needs that lives in
// memory (tile table, offsets, expert id, gathered row ids, routing weights) is read with
// uniform addresses, i.e. scalar loads, and spread to the lanes by selects: a vector load here
// would make the wait for it also wait for every copy in flight.
// The kernel body for tiles of BM rows; As / Bs: NB chunk buffers of BM x 64 and 32 WAVES x 64
// bf16 in LDS.
// The LM-head mode's per-row, per-wave partials of one work item, for the combine of the
// item's waves (an LDS array only in the kernels that use it).
struct LmPart {
  float mx;
  int arg;
  float se;
};
template <int N>
__device__ __forceinline__ LmPart* lm_part_lds() {
  __shared__ LmPart part[N];
  return part;
}

template <bool GATEUP, bool ROUTED, int NB, int WAVES, int BM, bool LMHEAD>
__device__ __forceinline__ void expert_stream_body(
    uint16_t* As, uint16_t* Bs, const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int Kdim, int Ndim, const LmPartials& lp) {
  static_assert(NB >= 2, "one chunk in flight while another is multiplied");
  static_assert(!LMHEAD || (!GATEUP && !ROUTED), "the LM head is a plain gathered product");
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves");
  static_assert(BM == 64 || BM == 128 || BM == 256, "tiles of 64, 128 or 256 rows");
  constexpr int KC = 64, WR = 32 * WAVES;
  constexpr int CBW = GATEUP ? 16 * WAVES : 32 * WAVES;  // output columns per item
  constexpr int MB = BM / 16;
  constexpr int NAW = BM / 8 / WAVES;     // activation copies per wave and chunk (8 rows each)
  constexpr int NBW = 4;                  // weight copies per wave and chunk (its 32 rows)
  constexpr int CPW = NAW + NBW;
  constexpr int ABUF = BM * KC, BBUF = WR * KC;  // elements per chunk buffer
  const int n_cb = (Ndim + CBW - 1) / CBW;
  // LM head: the live rows, this kernel's only when there are at most kLmStreamMaxRows
  const int rows = LMHEAD ? *lp.n_live : M;
  const int ntiles = ROUTED   ? flags[FLAG_NTILES]
                     : LMHEAD ? (rows <= kLmStreamMaxRows ? (rows + BM - 1) / BM : 0)
                              : (M + BM - 1) / BM;
  // this workgroup's items: position (blockIdx.x / 8) + k G8 along the tile-major order of
  // its XCD lane, active while the tile 8 (position / n_cb) + lane8 exists.  LM head: the
  // column blocks blockIdx.x + j gridDim.x, each with all its row tiles back to back (the
  // decoding call gives it no more live rows than one tile holds, so each vocabulary slab is
  // read once).
  const int lane8 = blockIdx.x & 7, pos0 = blockIdx.x >> 3, G8 = gridDim.x >> 3;
  int nitems;
  if (LMHEAD) {
    const int ncb_w = (int)blockIdx.x < n_cb ? (n_cb - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    nitems = ncb_w * ntiles;
  } else {
    const int T8 = ntiles > lane8 ? (ntiles - lane8 + 7) >> 3 : 0;
    const int span = T8 * n_cb - pos0;
    nitems = span > 0 ? (span + G8 - 1) / G8 : 0;
  }
  if (nitems == 0) return;
  const int nch = Kdim / KC;
  const int Q = nitems * nch;  // chunks in this workgroup's stream
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const size_t estride = (size_t)Ndim * Kdim;
  const int lrow = lane >> 3, pslot = lane & 7;  // copies: lane l moves slot l % 8 of row l / 8

  struct Item {
    int row0, row_end, col0, rot;
    size_t e;
    bool wact;
  };
  auto item = [&](int k) {
    int pos, cb, tile;
    if (LMHEAD) {
      const int j = k / ntiles;
      tile = k - j * ntiles;
      cb = blockIdx.x + j * gridDim.x;
      pos = cb;
    } else {
      pos = pos0 + k * G8;
      cb = pos % n_cb;
      tile = 8 * (pos / n_cb) + lane8;
    }
    const TileRows tr = tile_rows(ROUTED, tile, BM, ntiles, tile_slot, tile_row0, offs, rows);
    Item it;
    it.row0 = tr.row0;
    it.row_end = tr.row_end;
    it.e = ROUTED ? (size_t)S_list[tr.slot] : 0;
    it.col0 = cb * CBW + (GATEUP ? 16 : 32) * wave;
    // Ndim is a multiple of 64, so a wave's columns are all inside or all outside; a wave
    // outside copies stand-in rows (the first 32 of the expert), skips its MFMAs and stores,
    // and still copies its share of the activations and meets every barrier
    it.wact = it.col0 < Ndim;
    // items start their walk over K at different chunks and wrap around, so that at any
    // moment the weight rows being read sit at different offsets within their rows
    it.rot = pos % nch;
    return it;
  };

  // issue side: the item whose chunks are being copied, its copy sources, the next chunk
  const uint16_t* asrc[NAW];
  const uint16_t* bsrc[NBW];
  int ik = 0, ic = 0, irot = 0;
  auto sources = [&](const Item& it) {
#pragma unroll
    for (int j = 0; j < NAW; ++j) {
      const int row0 = 8 * (NAW * wave + j);
      const int row = row0 + lrow;
      const int lslot = pslot ^ (row & 7);
      int src_row;
      if ((ROUTED && GATEUP) || LMHEAD) {
        // the eight gathered rows of this copy (rows past the tile repeat its last row)
        src_row = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int v = wl_pos[min(it.row0 + row0 + t, it.row_end - 1)];
          src_row = lrow == t ? v : src_row;
        }
      } else {
        src_row = min(it.row0 + row, it.row_end - 1);
      }
      asrc[j] = A + (size_t)src_row * Kdim + lslot * 8;
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int row = 8 * j + lrow;  // within the wave's 32 rows; (32 w + row) & 7 == row & 7
      const int lslot = pslot ^ (row & 7);
      int wrow;
      const uint16_t* base;
      if (GATEUP) {
        wrow = it.col0 + (row & 15);
        base = row < 16 ? B0 : B1;
      } else {
        wrow = it.col0 + row;
        base = B0;
      }
      if (!it.wact) wrow = row;
      bsrc[j] = base + it.e * estride + (size_t)wrow * Kdim + lslot * 8;
    }
    irot = it.rot;
  };
  // copy the next chunk of the stream into chunk buffer buf (moving to the next item when the
  // current one is done; the caller keeps the stream within its Q chunks)
  auto issue_next = [&](int buf) {
    if (ic == nch) {
      ++ik;
      ic = 0;
      sources(item(ik));
    }
    const int cc = ic + irot < nch ? ic + irot : ic + irot - nch;
#pragma unroll
    for (int j = 0; j < NAW; ++j)
      copy16_to_lds(asrc[j] + (size_t)cc * KC, &As[buf * ABUF + 8 * (NAW * wave + j) * KC]);
#pragma unroll
    for (int j = 0; j < NBW; ++j)
      copy16_to_lds_stream(bsrc[j] + (size_t)cc * KC, &Bs[buf * BBUF + (32 * wave + 8 * j) * KC]);
    ++ic;
  };

  f32x4 c0[MB], c1[MB];
  // fragments: k-step s of a chunk is k-segment 4 s + g for lane (r, g), held in slot
  // (4 s + g) ^ (r & 7) of LDS rows 16 m + r (activations) and 32 w + r, 32 w + 16 + r
  // (weights)
  const int key = r & 7;
  const int off0 = (g ^ key) * 8, off1 = ((4 + g) ^ key) * 8;
  // activation fragments are read FG row blocks at a time (all of them up to 8 blocks, else in
  // groups of 4, which keeps a 256-row tile's registers within two waves per SIMD)
  constexpr int FG = MB <= 8 ? MB : 4;
  u32x4 fa[2][FG], fb[2][2];
  // the weight fragments of chunk buffer buf, and the activation fragments of row blocks
  // g0 .. g0 + FG - 1 below mlive; complete on return
  auto read_frags = [&](int buf, int g0, int mlive, bool with_b) {
    const uint32_t a0 = (uint32_t)(uintptr_t)&As[buf * ABUF + (16 * g0 + r) * KC + off0];
    const uint32_t a1 = (uint32_t)(uintptr_t)&As[buf * ABUF + (16 * g0 + r) * KC + off1];
    if (with_b) {
      const uint32_t b0 = (uint32_t)(uintptr_t)&Bs[buf * BBUF + (32 * wave + r) * KC + off0];
      const uint32_t b1 = (uint32_t)(uintptr_t)&Bs[buf * BBUF + (32 * wave + r) * KC + off1];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fb[0][n]) : "v"(b0), "i"(n * 16 * KC * 2));
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fb[1][n]) : "v"(b1), "i"(n * 16 * KC * 2));
      }
    }
#pragma unroll
    for (int m = 0; m < FG; ++m) {
      if (g0 + m < mlive) {
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fa[0][m]) : "v"(a0), "i"(m * 16 * KC * 2));
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fa[1][m]) : "v"(a1), "i"(m * 16 * KC * 2));
      }
    }
    if constexpr (FG == 8)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[0][2]), "+v"(fa[0][3]),
                     "+v"(fa[0][4]), "+v"(fa[0][5]), "+v"(fa[0][6]), "+v"(fa[0][7]),
                     "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fa[1][2]), "+v"(fa[1][3]),
                     "+v"(fa[1][4]), "+v"(fa[1][5]), "+v"(fa[1][6]), "+v"(fa[1][7]),
                     "+v"(fb[0][0]), "+v"(fb[0][1]), "+v"(fb[1][0]), "+v"(fb[1][1]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[0][2]), "+v"(fa[0][3]),
                     "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fa[1][2]), "+v"(fa[1][3]),
                     "+v"(fb[0][0]), "+v"(fb[0][1]), "+v"(fb[1][0]), "+v"(fb[1][1]));
  };
  // weights as the left operand: lane (r, g) of block m ends up with row 16 m + r and the four
  // consecutive columns 4 g .. 4 g + 3 (one 8-byte store in the epilogue)
  auto mma = [&](int g0, int mlive) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int m = 0; m < FG; ++m) {
        if (g0 + m < mlive) {
          const bf16x8 f = __builtin_bit_cast(bf16x8, fa[s][m]);
          c0[g0 + m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fb[s][0]), f, c0[g0 + m], 0, 0, 0);
          c1[g0 + m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fb[s][1]), f, c1[g0 + m], 0, 0, 0);
        }
      }
  };
  auto pack4 = [](const float* v) {
    return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  };
  auto epilogue = [&](const Item& it) {
    if constexpr (LMHEAD) {
      // per row: the 32 logits of this wave's token block sit in the 4 lanes with the same r
      // (tokens 4 g .. 4 g + 3 and 16 + 4 g .. + 3); reduce (max, lower token on ties), then
      // the sum of exp(logit - max); the item's WAVES waves then meet in LDS and one
      // (max, token, sum) per row and item (CBW tokens) is written.  Every wave runs this
      // (a wave past the vocabulary contributes (-inf, -, 0)), so its barrier is uniform.
      LmPart* part = lm_part_lds<BM * WAVES>();  // [row][wave]
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (it.row0 + 16 * m >= it.row_end) continue;
        float mx = c0[m][0];
        int arg = it.col0 + 4 * g;
#pragma unroll
        for (int i = 1; i < 4; ++i)
          if (c0[m][i] > mx) {
            mx = c0[m][i];
            arg = it.col0 + 4 * g + i;
          }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c1[m][i] > mx) {
            mx = c1[m][i];
            arg = it.col0 + 16 + 4 * g + i;
          }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
          const float om = __shfl_xor(mx, o, 64);
          const int oa = __shfl_xor(arg, o, 64);
          if (om > mx || (om == mx && oa < arg)) {
            mx = om;
            arg = oa;
          }
        }
        // exp(v - mx) as one v_exp_f32 of v log2(e) - mx log2(e), as in k_lm_head_w4
        const float nm = -mx * kLog2e;
        float se = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          se += __builtin_amdgcn_exp2f(fmaf(c0[m][i], kLog2e, nm)) +
                __builtin_amdgcn_exp2f(fmaf(c1[m][i], kLog2e, nm));
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) se += __shfl_xor(se, o, 64);
        if (g == 0)
          part[(16 * m + r) * WAVES + wave] =
              it.wact ? LmPart{mx, arg, se} : LmPart{-INFINITY, 0x7fffffff, 0.0f};
      }
      // the partials of every wave are in LDS (the next item's writes follow at least one
      // more barrier of the chunk loop, after these reads)
      asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
      const int blk = it.col0 / CBW;  // col0 = CBW blk + 32 wave
      for (int rr = tid; rr < BM; rr += 64 * WAVES) {
        const int li = it.row0 + rr;
        if (li >= it.row_end) continue;
        LmPart best = part[rr * WAVES];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
          const LmPart q = part[rr * WAVES + w];
          if (q.mx > best.mx) best = q;
        }
        const float nm = -best.mx * kLog2e;
        float se = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
          const LmPart q = part[rr * WAVES + w];
          se += q.se * __builtin_amdgcn_exp2f(fmaf(q.mx, kLog2e, nm));
        }
        const size_t idx = (size_t)li * lp.n_p + blk;
        lp.pmax[idx] = best.mx;
        lp.parg[idx] = best.arg;
        lp.psum[idx] = se;
      }
      return;
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (it.row0 + 16 * m >= it.row_end) continue;  // uniform: a block past the tile's rows
      float sc = 1.0f;
      if (ROUTED && !GATEUP) {  // routing weights of rows 16 m .. 16 m + 15
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const float v = wl_w[min(it.row0 + 16 * m + t, it.row_end - 1)];
          sc = r == t ? v : sc;
        }
      }
      const int row = it.row0 + 16 * m + r;
      if (row >= it.row_end) continue;
      float v[4];
      if (GATEUP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = silu(c0[m][i]) * c1[m][i];
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + it.col0 + 4 * g) = pack4(v);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = sc * c0[m][i];
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + it.col0 + 4 * g) = pack4(v);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = sc * c1[m][i];
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + it.col0 + 16 + 4 * g) = pack4(v);
      }
    }
  };

  static_assert(CPW * (NB - 2) < 64, "vmcnt range");
  constexpr int kAfter = CPW * (NB - 2);  // copies of the chunks after chunk q
  // prologue: chunks 0 .. NB - 2 of the stream in flight
  sources(item(0));
#pragma unroll
  for (int x = 0; x < NB - 1; ++x)
    if (x < Q) issue_next(x);
  int ck = 0, cc = 0;  // item and chunk of the chunk being multiplied
  Item cur = item(0);
  int mlive = (cur.row_end - cur.row0 + 15) >> 4;
  for (int q = 0; q < Q; ++q) {
    // every chunk up to q + NB - 2 has been issued: while all NB - 2 after q exist, they may
    // stay in flight, else wait for everything
    if (q + NB - 2 < Q)
      wait_vm_lds<kAfter>();
    else
      wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    if (q + NB - 1 < Q) issue_next((q + NB - 1) % NB);
    if (cc == 0) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        c0[m] = f32x4{0, 0, 0, 0};
        c1[m] = f32x4{0, 0, 0, 0};
      }
    }
    if (cur.wact) {
#pragma unroll
      for (int g0 = 0; g0 < MB; g0 += FG) {
        if (g0 < mlive) {
          read_frags(q % NB, g0, mlive, g0 == 0);
          mma(g0, mlive);
        }
      }
    }
    if (++cc == nch) {
      if (LMHEAD || cur.wact) epilogue(cur);
      ++ck;
      cc = 0;
      if (ck < nitems) {
        cur = item(ck);
        mlive = (cur.row_end - cur.row0 + 15) >> 4;
      }
    }
  }
}

// Routed tiles: the plan step's tile table holds kTileRows- or kTileRowsTall-row tiles
// (FLAG_TILE_TALL; never tall for shapes with big tiles); shared-expert tiles: kDenseTileRows
// rows; LM head (LMHEAD: rows gathered through lp.live_list, lp.n_live of them, the epilogue
// writing lp's partials): BMAX-row tiles.  BMAX = the tallest tile the instance handles, which
// sizes its LDS.
template <bool GATEUP, bool ROUTED, int NB, int WAVES, int BMAX, bool LMHEAD = false>
__global__ __launch_bounds__(64 * WAVES) void k_expert_stream(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int Kdim, int Ndim, LmPartials lp) {
  __shared__ __attribute__((aligned(16))) uint16_t As[NB * BMAX * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NB * 32 * WAVES * 64];
  if constexpr (ROUTED && BMAX == kTileRowsTall) {
    if (flags[FLAG_TILE_TALL]) {
      expert_stream_body<GATEUP, ROUTED, NB, WAVES, kTileRowsTall, false>(
          As, Bs, A, B0, B1, flags, tile_slot, tile_row0, offs, S_list, wl_pos, wl_w, out, M,
          Kdim, Ndim, lp);
      return;
    }
    expert_stream_body<GATEUP, ROUTED, NB, WAVES, kTileRows, false>(
        As, Bs, A, B0, B1, flags, tile_slot, tile_row0, offs, S_list, wl_pos, wl_w, out, M, Kdim,
        Ndim, lp);
  } else {
    expert_stream_body<GATEUP, ROUTED, NB, WAVES, BMAX, LMHEAD>(
        As, Bs, A, B0, B1, flags, tile_slot, tile_row0, offs, S_list, wl_pos, wl_w, out, M, Kdim,
        Ndim, lp);
  }
}

// Compute-bound variant for tiles with many rows on two waves per SIMD (routed experts with
// many fresh pairs, which run beside the weight-stream kernel, and shared-expert layers with
// too few 256 x 256 tiles for k_gemm_w4): a BR-row x 128-weight-row output tile per workgroup
// of four waves, two along the rows and two along the weight rows, each wave accumulating a
// (BR / 2) x 64 sub-tile with v_mfma_f32_16x16x32_bf16 (BR / 32 x 4 blocks); two workgroups
// per CU.
// K runs in chunks of KC = 32.  Both operands of a chunk go from global memory straight into
// LDS (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base + 16 x lane),
// NB chunk buffers deep, NB - 2 chunks in flight while a chunk is multiplied.  LDS rows of
// KC = 32 bf16 (64 bytes, four 16-byte slots) hold k-segment slot ^ ((row >> 1) & 3) in slot
// `slot`: a lane fetches the segment its slot must hold.  ds_read_b128 is served eight lanes
// (eight consecutive rows of a fragment, two per 128 bytes) at a time, and with this key those
// eight rows occupy eight distinct 16-byte bank groups, so fragment reads have no bank
// conflicts.  Rows past the tile (and weight rows past N) load a stand-in row of the same
// operand: they only feed outputs that are never stored.
// Synchronisation is explicit: before each barrier a wave waits for its own copies of the next
// chunk (vmcnt) and for its LDS reads (lgkmcnt); the fragment reads are inline ds_read_b128,
// because the compiler, which cannot tell chunk buffers apart, would otherwise wait for every
// copy in flight before any LDS read.  Gate/up: the BC staged weight rows are groups of 32 rows
// alternating W1 and W3 ([W1 i0..i0+32, W3 i0..i0+32, W1 i0+32..i0+64, ...]), so each wave
// holds g and u of the same 32 columns and the SwiGLU epilogue stays in registers; down: BC
// rows of W2.  Grid as k_expert_stream (XCD-grouped, 1-D): BC / 2 (gate/up) or BC (down)
// columns per block.
template <bool GATEUP, bool ROUTED, int BR = 128>
__global__ __launch_bounds__(256, 2) void k_gemm_big(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int Kdim, int Ndim) {
  static_assert(BR == 128 || BR == 256, "row tiles of 128 or 256");
  constexpr int WAVES = 4, KC = 32, WN = WAVES / 2, BC = 64 * WN;
  constexpr int MB = BR / 32;                                   // 16-row blocks per wave
  constexpr int NB = BR == 256 ? 3 : 4;                         // LDS chunk buffers
  constexpr int NA = BR / (16 * WAVES), NBI = BC / (16 * WAVES);  // copies per wave and chunk
  constexpr int CBW = GATEUP ? BC / 2 : BC;                     // output columns per block
  __shared__ __attribute__((aligned(16))) uint16_t As[NB][BR * KC];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NB][BC * KC];
  const int n_cb = (Ndim + CBW - 1) / CBW;
  const int pos = blockIdx.x >> 3;
  const int tile = ((pos / n_cb) << 3) + (blockIdx.x & 7), cb = pos % n_cb;
  // routed big tiles come from their own table, counted in FLAG_NTILES_BIG
  const TileRows tr = tile_rows(ROUTED, tile, BR, ROUTED ? flags[FLAG_NTILES_BIG] : 0, tile_slot,
                                tile_row0, offs, M);
  if (!tr.active) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const size_t estride = (size_t)Ndim * Kdim;
  const size_t e = ROUTED ? (size_t)S_list[tr.slot] : 0;
  // copy sources: copy j of wave w fills LDS rows [16 (WAVES j + w), +16) of a chunk buffer,
  // lane l slot l % 4 of row 16 (WAVES j + w) + l / 4
  const uint16_t* asrc[NA];
  const uint16_t* bsrc[NBI];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int row = 16 * (WAVES * j + wave) + (lane >> 2);
    const int c8 = (lane & 3) ^ ((row >> 1) & 3);
    const int p = tr.row0 + row < tr.row_end ? tr.row0 + row : tr.row0;
    const int src_row = (ROUTED && GATEUP) ? wl_pos[p] : p;
    asrc[j] = A + (size_t)src_row * Kdim + c8 * 8;
  }
#pragma unroll
  for (int j = 0; j < NBI; ++j) {
    const int row = 16 * (WAVES * j + wave) + (lane >> 2);
    const int c8 = (lane & 3) ^ ((row >> 1) & 3);
    int wrow;
    const uint16_t* base;
    if (GATEUP) {
      const int q = row >> 5;  // groups of 32 staged rows: W1, W3, W1, W3, ...
      wrow = cb * CBW + (q >> 1) * 32 + (row & 31);
      base = (q & 1) ? B1 : B0;
    } else {
      wrow = cb * BC + row;
      base = B0;
    }
    bsrc[j] = base + e * estride + (size_t)(wrow < Ndim ? wrow : 0) * Kdim + c8 * 8;
  }
  auto issue = [&](int c, int buf) {
#pragma unroll
    for (int j = 0; j < NA; ++j)
      copy16_to_lds(asrc[j] + (size_t)c * KC, &As[buf][16 * (WAVES * j + wave) * KC]);
#pragma unroll
    for (int j = 0; j < NBI; ++j)
      copy16_to_lds(bsrc[j] + (size_t)c * KC, &Bs[buf][16 * (WAVES * j + wave) * KC]);
  };
  f32x4 acc[MB][4];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};
  // fragments of one chunk: lane (r, g) reads slot g ^ ((r >> 1) & 3) of rows 16 m + r; two
  // register sets, so that chunk c + 1 is read from LDS while c is multiplied
  const int swz = (g ^ ((r >> 1) & 3)) * 8;
  u32x4 fa[2][MB], fb[2][4];
  auto read_frags = [&](int buf, int set) {
    const uint32_t ab = (uint32_t)(uintptr_t)&As[buf][(BR / 2 * wm + r) * KC + swz];
    const uint32_t bb = (uint32_t)(uintptr_t)&Bs[buf][(64 * wn + r) * KC + swz];
#pragma unroll
    for (int m = 0; m < MB; ++m)
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fa[set][m]) : "v"(ab), "i"(m * 16 * KC * 2));
#pragma unroll
    for (int n = 0; n < 4; ++n)
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(fb[set][n]) : "v"(bb), "i"(n * 16 * KC * 2));
  };
  // a set's fragments are complete once this wave's LDS reads are: the wait names them as
  // operands, so no use of them can be scheduled before it (it adds no wait of its own when
  // the wait before the barrier already covered the reads)
  auto frags_ready = [&](int set) {
    if constexpr (MB == 8)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(fa[set][0]), "+v"(fa[set][1]), "+v"(fa[set][2]), "+v"(fa[set][3]),
                     "+v"(fa[set][4]), "+v"(fa[set][5]), "+v"(fa[set][6]), "+v"(fa[set][7]),
                     "+v"(fb[set][0]), "+v"(fb[set][1]), "+v"(fb[set][2]), "+v"(fb[set][3]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(fa[set][0]), "+v"(fa[set][1]), "+v"(fa[set][2]), "+v"(fa[set][3]),
                     "+v"(fb[set][0]), "+v"(fb[set][1]), "+v"(fb[set][2]), "+v"(fb[set][3]));
  };
  // The operands go in swapped (weights as the 16 x 32 left operand), so that a block holds its
  // outputs transposed: lane (r, g) gets four consecutive columns 4 g .. 4 g + 3 of row r,
  // stored with one 8-byte store.
  auto mma = [&](int set) {
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, fb[set][n]), __builtin_bit_cast(bf16x8, fa[set][m]),
            acc[m][n], 0, 0, 0);
  };
  constexpr int kInFlight = (NA + NBI) * (NB - 2);  // copies after chunk c + 1's
  const int nch = Kdim / KC;
  // prologue: chunks 0 .. NB - 2 in flight, chunk 0 landed, its fragments read
#pragma unroll
  for (int x = 0; x < NB - 1; ++x)
    if (x < nch) issue(x, x);
  if (nch >= NB - 1)
    wait_vm_lds<(NA + NBI) * (NB - 2)>();
  else
    wait_vm_lds<0>();
  __builtin_amdgcn_s_barrier();
  read_frags(0, 0);
  // step c: copy chunk c + NB - 1 into the buffer of chunk c - 1 (every wave read it before
  // the previous barrier), wait for chunk c + 1, barrier, read its fragments, multiply chunk c
  int c = 0;
  for (; c + NB - 1 < nch; c += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = c + u;
      if (cc + NB - 1 < nch) {
        issue(cc + NB - 1, (cc + NB - 1) % NB);
        wait_vm_lds<kInFlight>();
      } else {
        wait_vm_lds<0>();
      }
      __builtin_amdgcn_s_barrier();
      frags_ready(u & 1);
      read_frags((cc + 1) % NB, (u + 1) & 1);
      mma(u & 1);
    }
  }
  for (; c < nch; c += 2) {  // the last chunks: nothing more to copy
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = c + u;
      if (cc < nch) {
        wait_vm_lds<0>();
        __builtin_amdgcn_s_barrier();
        frags_ready(u & 1);
        if (cc + 1 < nch) read_frags((cc + 1) % NB, (u + 1) & 1);
        mma(u & 1);
      }
    }
  }
  // transposed blocks: lane (r, g) holds row 16 m + r, columns 16 n + 4 g .. + 3
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = tr.row0 + BR / 2 * wm + 16 * m + r;
    if (row >= tr.row_end) continue;
    if (GATEUP) {
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int col = cb * CBW + 32 * wn + 16 * n + 4 * g;
        if (col >= Ndim) continue;
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu(acc[m][n][i]) * acc[m][n + 2][i];
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + col) =
            make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      }
    } else {
      const float sc = ROUTED ? wl_w[row] : 1.0f;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int col = cb * BC + 64 * wn + 16 * n + 4 * g;
        if (col >= Ndim) continue;
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + col) =
            make_uint2(pack_bf16x2(sc * acc[m][n][0], sc * acc[m][n][1]),
                       pack_bf16x2(sc * acc[m][n][2], sc * acc[m][n][3]));
      }
    }
  }
}

// Compute-bound tiles on one wave per SIMD: a 256 x 256 output tile per workgroup of four
// waves, each wave accumulating 128 x 128 (8 x 8 blocks of v_mfma_f32_16x16x32_bf16, 256 fp32
// accumulators per lane held in AGPRs), so that a wave reads a third fewer operand bytes from
// LDS per MFMA than the two-waves-per-SIMD tiles of k_gemm_big.  Same operand roles, staged row
// layouts (gate/up: groups of 64 rows alternating W1 and W3, so a wave holds g and u of the same
// 64 columns) and epilogues as k_gemm_big; used where the grid has at least one tile per CU
// (the LM head's persistent variant is k_lm_head_w4).
// K runs in chunks of 64 bf16: a chunk row is one 128-byte line, and one copy instruction
// (global_load_lds_dwordx4) moves eight whole lines straight into LDS, half the cache-line
// requests of 64-byte rows.  Two chunk buffers of 64 KB: while the second half of chunk c is
// multiplied, chunk c + 2 is copied into chunk c's buffer (whose fragments have all been read)
// and chunk c + 1, which has landed, is read.  LDS rows hold k-segment slot ^ (row & 7) in 16-byte
// slot `slot`, so that the eight lanes a ds_read_b128 serves at once hit distinct banks.
// Each chunk is multiplied as two halves of K = 32 with fragment register sets 0 and 1: the
// fragments of the next half are read from LDS (two ds_read_b128 per four MFMAs in the first
// half of the half) while the current half is multiplied, and have landed by its end.  One barrier per chunk, before the second half: every wave's
// copies of chunk c + 1 have landed and every wave has read all of chunk c, whose buffer the
// second half refills.  Every step issues the same copies and reads (past the last chunk they
// repeat the last one into a buffer nobody reads again), so the loop has no tail.
// The MFMAs are inline asm with AGPR accumulators ("+a"): the compiler, which otherwise keeps
// MFMA results in VGPRs and spills them to AGPRs around every use, cannot insert the wait
// states an MFMA result needs before a VALU reads it, so the epilogue starts after 48 idle
// cycles.
// Grid: dense tiles in XCD supertiles: workgroup 8 i + x runs on XCD x, and the 32
// workgroups an XCD holds at once cover 4 row tiles x 8 column blocks, so each XCD's L2 serves
// a 4 x 8 block of tiles; routed tiles as in k_gemm_big (the big-tile table).
template <bool GATEUP, bool ROUTED>
__global__ __launch_bounds__(256, 1) void k_gemm_w4(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int Kdim, int Ndim) {
  constexpr int BR = 256, BC = 256, KC = 64, WAVES = 4, MB = 8, NBK = 8;
  constexpr int NA = BR / (8 * WAVES), NBI = BC / (8 * WAVES);  // copies per wave and chunk
  constexpr int CPC = NA + NBI;
  constexpr int CBW = GATEUP ? BC / 2 : BC;  // output columns per block
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BR * KC];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BC * KC];
  const int n_cb = (Ndim + CBW - 1) / CBW;
  int tile, cb;
  if (!ROUTED) {
    const int T = (M + BR - 1) / BR, nsc = (n_cb + 7) / 8;
    const int within = blockIdx.x >> 3, s = (within >> 5) * 8 + (blockIdx.x & 7);
    tile = (s / nsc) * 4 + ((within & 31) >> 3);
    cb = (s % nsc) * 8 + (within & 7);
    if (tile >= T || cb >= n_cb) return;
  } else {
    const int pos = blockIdx.x >> 3;
    tile = ((pos / n_cb) << 3) + (blockIdx.x & 7);
    cb = pos % n_cb;
  }
  const TileRows tr = tile_rows(ROUTED, tile, BR, ROUTED ? flags[FLAG_NTILES_BIG] : 0, tile_slot,
                                tile_row0, offs, M);
  if (!tr.active) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const size_t estride = (size_t)Ndim * Kdim;
  const size_t e = ROUTED ? (size_t)S_list[tr.slot] : 0;
  // copy j of wave w fills LDS rows [8 (WAVES j + w), +8) of a chunk buffer: lane l slot l % 8
  // of row 8 (WAVES j + w) + l / 8, i.e. k-segment (l % 8) ^ (row & 7) of that row.  Activation
  // rows by pointer, weight rows by 32-bit byte offset from their column block's first row (at
  // most 256 rows of at most 16384 elements); rows past the tile or past N load a stand-in row
  // of the operand: they only feed outputs that are never stored
  const char* asrc[NA];
  uint32_t boff[NBI];
  const uint16_t* bbase[NBI];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int row = 8 * (WAVES * j + wave) + (lane >> 3);
    const int seg = (lane & 7) ^ (row & 7);
    const int p = tr.row0 + row < tr.row_end ? tr.row0 + row : tr.row0;
    const int src_row = (ROUTED && GATEUP) ? wl_pos[p] : p;
    asrc[j] = reinterpret_cast<const char*>(A + (size_t)src_row * Kdim + seg * 8);
  }
#pragma unroll
  for (int j = 0; j < NBI; ++j) {
    const int row = 8 * (WAVES * j + wave) + (lane >> 3);
    const int seg = (lane & 7) ^ (row & 7);
    int first, wrow;  // the column block's first row of this operand, the staged row's row
    const uint16_t* base;
    if (GATEUP) {
      // groups of 64 staged rows: W1, W3, W1, W3; copy j's rows 32 j + [0, 32) lie in group j / 2
      const int q = j >> 1;
      first = cb * CBW;
      wrow = first + (q >> 1) * 64 + (row & 63);
      base = (q & 1) ? B1 : B0;
    } else {
      first = cb * BC;
      wrow = first + row;
      base = B0;
    }
    bbase[j] = base + e * estride + (size_t)first * Kdim;
    const int lrow = wrow < Ndim ? wrow - first : 0;
    boff[j] = ((uint32_t)lrow * (uint32_t)Kdim + seg * 8) * 2u;
  }
  auto issue = [&](int j, int c, int buf) {
    if (j < NA)
      copy16_to_lds(asrc[j] + (size_t)c * (KC * 2), &As[buf][8 * (WAVES * j + wave) * KC]);
    else
      copy16_to_lds(reinterpret_cast<const char*>(bbase[j - NA]) + (size_t)c * (KC * 2) +
                        boff[j - NA],
                    &Bs[buf][8 * (WAVES * (j - NA) + wave) * KC]);
  };
  f32x4 acc[MB][NBK];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NBK; ++b) acc[a][b] = f32x4{0, 0, 0, 0};
  // fragments of half h: lane (r, g) reads row 16 i + r, k-segment 4 h + g, which sits in slot
  // (4 h + g) ^ (r & 7)
  u32x4 fa[2][MB], fb[2][NBK];
  const uint32_t a_l = (uint32_t)(uintptr_t)&As[0][(128 * wm + r) * KC];
  const uint32_t b_l = (uint32_t)(uintptr_t)&Bs[0][(128 * wn + r) * KC];
  const uint32_t sw0 = (g ^ (r & 7)) * 16, sw1 = ((4 + g) ^ (r & 7)) * 16;
  auto read = [&](int buf, int half, int set, int i) {
    const uint32_t sw = half ? sw1 : sw0;
    if (i < MB)
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(fa[set][i]) : "v"(a_l + buf * (BR * KC * 2) + sw), "i"(i * 16 * KC * 2));
    else
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(fb[set][i - MB])
                   : "v"(b_l + buf * (BC * KC * 2) + sw), "i"((i - MB) * 16 * KC * 2));
  };
  // a set's fragments are complete once this wave's LDS reads are; the wait names them as
  // operands, so no MFMA using them is placed before it
  auto frags_ready = [&](int set) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(fa[set][0]), "+v"(fa[set][1]), "+v"(fa[set][2]), "+v"(fa[set][3]),
                   "+v"(fa[set][4]), "+v"(fa[set][5]), "+v"(fa[set][6]), "+v"(fa[set][7]),
                   "+v"(fb[set][0]), "+v"(fb[set][1]), "+v"(fb[set][2]), "+v"(fb[set][3]),
                   "+v"(fb[set][4]), "+v"(fb[set][5]), "+v"(fb[set][6]), "+v"(fb[set][7]));
  };
  // operands swapped as in k_gemm_big: lane (r, g) of block (m, n) gets columns 16 n + 4 g ..
  // + 3 of row 16 m + r
  auto mma = [&](int set, int idx) {
    const int m = idx / NBK, n = idx % NBK;
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
        : "+a"(acc[m][n]) : "v"(fb[set][n]), "v"(fa[set][m]));
  };
  // one half: 64 MFMAs on `set`; the 16 fragment reads of (rbuf, rhalf) into the other set,
  // two per group of four MFMAs in the first eight groups, so that they have landed by the
  // half's end; when `copy`, the CPC copies of chunk cp into buffer cbuf, one per group
  auto half_step = [&](int set, int rbuf, int rhalf, bool copy, int cp, int cbuf) {
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) {
      if (grp < 8) {
        read(rbuf, rhalf, set ^ 1, 2 * grp);
        read(rbuf, rhalf, set ^ 1, 2 * grp + 1);
      }
      mma(set, 4 * grp + 0);
      mma(set, 4 * grp + 1);
      if (copy) issue(grp, cp, cbuf);
      mma(set, 4 * grp + 2);
      mma(set, 4 * grp + 3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int nch = Kdim / KC;
  auto src_chunk = [&](int c) { return c < nch ? c : nch - 1; };
#pragma unroll
  for (int j = 0; j < CPC; ++j) issue(j, 0, 0);
#pragma unroll
  for (int j = 0; j < CPC; ++j) issue(j, src_chunk(1), 1);
  wait_vm_lds<CPC>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 16; ++i) read(0, 0, 0, i);
  frags_ready(0);
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    half_step(0, buf, 1, false, 0, 0);
    wait_vm_lds<0>();
    frags_ready(1);
    __builtin_amdgcn_s_barrier();
    half_step(1, buf ^ 1, 0, true, src_chunk(c + 2), buf);
    // the next chunk's first-half fragments have landed before the loop's back edge, where the
    // compiler may copy registers
    frags_ready(0);
    // the wait states before the accumulators are read, inside the loop: the compiler, which
    // does not know that the asm MFMAs' results arrive late, places the copies and spills of
    // the accumulators that the epilogue needs where the loop exits
    if (c == nch - 1) asm volatile("s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
  }
  // the last step's surplus copies land before anything else uses LDS
  wait_vm_lds<0>();
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int row = tr.row0 + 128 * wm + 16 * m + r;
    if (row >= tr.row_end) continue;
    if (GATEUP) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int col = cb * CBW + 64 * wn + 16 * n + 4 * g;
        if (col >= Ndim) continue;
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = silu(acc[m][n][i]) * acc[m][n + 4][i];
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + col) =
            make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
      }
    } else {
      const float sc = ROUTED ? wl_w[row] : 1.0f;
#pragma unroll
      for (int n = 0; n < NBK; ++n) {
        const int col = cb * BC + 128 * wn + 16 * n + 4 * g;
        if (col >= Ndim) continue;
        *reinterpret_cast<uint2*>(out + (size_t)row * Ndim + col) =
            make_uint2(pack_bf16x2(sc * acc[m][n][0], sc * acc[m][n][1]),
                       pack_bf16x2(sc * acc[m][n][2], sc * acc[m][n][3]));
      }
    }
  }
}

// Grid of k_gemm_w4 for a dense GEMM of `rows` rows and n_cb column blocks: whole
// XCD supertiles of 4 x 8 tiles, 32 workgroups each, supertiles dealt to the 8 XCDs in turn.
inline int gemm_w4_dense_grid(int rows, int n_cb) {
  const int supertiles = ((rows + 255) / 256 + 3) / 4 * ((n_cb + 7) / 8);
  return (supertiles + 7) / 8 * 8 * 32;
}

}  // namespace epoch
