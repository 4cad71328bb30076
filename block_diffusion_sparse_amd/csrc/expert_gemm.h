// Grouped bf16 expert GEMM of the SwiGLU experts (gfx950, v_mfma_f32_16x16x32_bf16).
#pragma once
#include "device_common.h"
#include "epoch_internal.h"

namespace epoch {

// A 16-byte fragment: 8 consecutive bf16 of one row.
__device__ __forceinline__ bf16x8 ld_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

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

// One kernel for both projections of the SwiGLU expert.
// Workgroup = 4 waves over one tile (up to BM rows of one expert) and 4 x 32 weight rows:
//   gate/up: wave w owns intermediate columns [16w, 16w + 16) of a 64-column block and reads
//            those rows of W1 and of W3 (32 weight rows); epilogue h = bf16(silu(g) * u);
//   down:    wave w owns output columns [32w, 32w + 32) of a 128-column block of W2;
//            epilogue y = bf16(w_p * acc) (routed) or bf16(acc) (shared expert).
// The contraction runs in chunks of KC.  The tile's activation rows (gathered through the
// worklist for routed gate/up) are staged per chunk in LDS (double-buffered) and shared by
// the four waves; every wave streams its weight rows straight into a ring of NST register
// stages, so NST - 1 chunks of weights are in flight while a chunk's MFMAs run.  Lane l
// feeds A row (l % 16) and B row (l % 16) with the same 8 consecutive k values (k-group
// l / 16), so every product pairs an activation with the weight of the same k.
//
// Grid: one-dimensional, n_col_blocks * (tile slots rounded up to a multiple of 8).  The
// hardware hands consecutive workgroups to the 8 XCDs in turn; workgroup L runs column block
// (L / 8) % NB of tile 8 * ((L / 8) / NB) + L % 8, so every column block of a tile lands on
// the same XCD and the tile's activation rows are fetched into one L2 only.
template <int BM, int KC, int NST, bool GATEUP, bool ROUTED, int WAVES = 4>
__global__ __launch_bounds__(64 * WAVES) void k_expert_gemm(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int Kdim, int Ndim) {
  constexpr int NTH = 64 * WAVES;
  constexpr int CBW = GATEUP ? 16 * WAVES : 32 * WAVES;  // columns per workgroup
  const int n_cb = (Ndim + CBW - 1) / CBW;
  const int pos = blockIdx.x >> 3;
  const int tile = ((pos / n_cb) << 3) + (blockIdx.x & 7);
  const int cb = pos % n_cb;
  constexpr int MB = BM / 16;        // 16-row MFMA blocks per tile
  constexpr int KS = KC / 32;        // MFMA k-steps per chunk
  constexpr int LDA = KC + 8;        // LDS row pitch (bf16), breaks bank aliasing
  constexpr int SEGS = BM * KC / 8;  // 16-byte segments of one activation chunk
  constexpr int ASEG = SEGS / NTH;   // per thread
  static_assert(SEGS % NTH == 0, "activation chunk must split evenly over the threads");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];

  const TileRows tr = tile_rows(ROUTED, tile, BM, ROUTED ? flags[FLAG_NTILES] : 0, tile_slot,
                                tile_row0, offs, M);
  if (!tr.active) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const size_t estride = (size_t)Ndim * Kdim;
  const size_t e = ROUTED ? (size_t)S_list[tr.slot] : 0;
  int col0;
  const uint16_t *bp0, *bp1;
  if (GATEUP) {
    col0 = cb * CBW + wave * 16;
    bp0 = B0 + e * estride + (size_t)(col0 + r) * Kdim + 8 * g;
    bp1 = B1 + e * estride + (size_t)(col0 + r) * Kdim + 8 * g;
  } else {
    col0 = cb * CBW + wave * 32;
    bp0 = B0 + e * estride + (size_t)(col0 + r) * Kdim + 8 * g;
    bp1 = bp0 + (size_t)16 * Kdim;
  }
  // Ndim is a multiple of 64, so a wave's 16 or 32 columns are all inside or all outside;
  // a wave outside streams a valid stand-in (the first columns of the expert), skips the MFMA
  // work and the stores, and meets every barrier
  const bool wact = col0 < Ndim;
  if (!wact) {
    bp0 = B0 + e * estride + (size_t)r * Kdim + 8 * g;
    bp1 = GATEUP ? B1 + e * estride + (size_t)r * Kdim + 8 * g : bp0;
  }
  // activation segments this thread stages: row = seg / (KC / 8), 8 columns each; a segment
  // past the tile's last row reads row 0 (always present) and is replaced by zeros
  const uint16_t* asrc[ASEG];
  int adst[ASEG];
  bool aok[ASEG];
#pragma unroll
  for (int j = 0; j < ASEG; ++j) {
    const int seg = tid + NTH * j;
    const int row = seg / (KC / 8), c8 = seg % (KC / 8);
    const int p = tr.row0 + row;
    aok[j] = p < tr.row_end;
    const int src_row = aok[j] ? ((ROUTED && GATEUP) ? wl_pos[p] : p) : 0;
    asrc[j] = A + (size_t)src_row * Kdim + c8 * 8;
    adst[j] = row * LDA + c8 * 8;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int nch = Kdim / KC;
  // Workgroups start their walk over K at different chunks (rot, by column block and tile
  // position) and wrap around, so that at any moment the weight rows being read sit at
  // different offsets within their rows rather than all at the same one.
  const int rot = pos % nch;
  auto kchunk = [&](int c) { return c + rot < nch ? c + rot : c + rot - nch; };

  u32x4 areg[ASEG];
  bf16x8 bx[NST][KS], by[NST][KS];
  f32x4 c0[MB], c1[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    c0[m] = f32x4{0, 0, 0, 0};
    c1[m] = f32x4{0, 0, 0, 0};
  }

  // Every global load below is issued by every lane, with no branch around it: the hardware
  // counts outstanding loads in issue order, and a load under a lane-dependent branch makes the
  // compiler wait for all of them at the next use.  With activations issued before the weight
  // chunk of the same step, staging the activations waits only for themselves and the weight
  // ring keeps NST - 1 chunks in flight across the barrier.
  auto load_a = [&](int c) {
#pragma unroll
    for (int j = 0; j < ASEG; ++j)
      areg[j] = *reinterpret_cast<const u32x4*>(asrc[j] + (size_t)kchunk(c) * KC);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int j = 0; j < ASEG; ++j)
      *reinterpret_cast<u32x4*>(&As[buf][adst[j]]) = aok[j] ? areg[j] : zero;
  };
  auto load_b = [&](int c_, bf16x8* x0, bf16x8* x1) {
    const int c = kchunk(c_);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      x0[s] = ld_frag(bp0 + (size_t)c * KC + 32 * s);
      x1[s] = ld_frag(bp1 + (size_t)c * KC + 32 * s);
    }
  };
  auto compute = [&](int buf, const bf16x8* x0, const bf16x8* x1) {
    const uint16_t* ab = &As[buf][r * LDA + 8 * g];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const bf16x8 f =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ab + m * 16 * LDA + 32 * s));
        c0[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, x0[s], c0[m], 0, 0, 0);
        c1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f, x1[s], c1[m], 0, 0, 0);
      }
    }
  };

  // one step: stage the activations of chunk c + 1 and fetch weight chunk c + NST - 1 into the
  // ring slot freed by chunk c - 1, multiply chunk c, then publish chunk c + 1's activations
  auto step = [&](int c, int u, bool next_a, bool pre_b) {
    if (next_a) load_a(c + 1);
    if (pre_b) load_b(c + NST - 1, bx[(u + NST - 1) % NST], by[(u + NST - 1) % NST]);
    if (wact) compute(c & 1, bx[u], by[u]);
    if (next_a) store_a((c + 1) & 1);
    __syncthreads();
  };
  load_a(0);
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < nch) load_b(st, bx[st], by[st]);
  store_a(0);
  __syncthreads();
  // steady state, NST steps per trip with every prefetch in range: no branch around a load
  int kb = 0;
  for (; kb + 2 * NST - 2 < nch; kb += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) step(kb + u, u, true, true);
  }
  // the last NST to 2 NST - 2 chunks (uniform conditions)
#pragma unroll
  for (int u = 0; u < 2 * NST - 1; ++u) {
    const int c = kb + u;
    if (c < nch) step(c, u % NST, c + 1 < nch, c + NST - 1 < nch);
  }

  if (!wact) return;
  // D[i][j] of a 16x16 block: lane j + 16 * (i / 4), register i % 4
#pragma unroll
  for (int m = 0; m < MB; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = tr.row0 + 16 * m + 4 * g + q;
      if (row >= tr.row_end) continue;
      const float v0 = c0[m][q], v1 = c1[m][q];
      if (GATEUP) {
        out[(size_t)row * Ndim + col0 + r] = f32_to_bf16(v0 / (1.0f + expf(-v0)) * v1);
      } else {
        const float sc = ROUTED ? wl_w[row] : 1.0f;
        out[(size_t)row * Ndim + col0 + r] = f32_to_bf16(sc * v0);
        out[(size_t)row * Ndim + col0 + 16 + r] = f32_to_bf16(sc * v1);
      }
    }
  }
}

}  // namespace epoch

namespace epoch {

// Output of the LM-head mode of k_gemm_big: the rows are live positions (gathered through
// live_list, n_live of them), the columns vocabulary tokens, and instead of the logits each wave
// writes, per row and per block of 64 tokens, the largest logit, its token (lower id on ties)
// and the sum of exp(logit - largest) over the block; n_p = vocab / 64 blocks per row.
struct LmPartials {
  const int32_t* live_list;
  const int32_t* n_live;
  float* pmax;
  int32_t* parg;
  float* psum;
  int n_p;
};

// Compute-bound variant for tiles with many rows (the shared expert over all M positions,
// routed experts with many fresh pairs): a 128-row x 128-weight-row output tile per
// workgroup, four waves in a 2 x 2 arrangement, each accumulating a 64 x 64 sub-tile with
// v_mfma_f32_16x16x32_bf16 (4 x 4 blocks).  K runs in chunks of KC = 32: both operands of a
// chunk are staged through LDS (double-buffered), and chunk loads from global memory run NR - 1
// steps ahead in a register ring, so that NR - 2 chunks stay in flight while a chunk is
// multiplied (one chunk is ~256 MFMA cycles per wave, far shorter than a memory round trip).
// Every global load is issued by every lane with no branch around it (rows past the tile read
// a valid stand-in, replaced by zeros when stored to LDS).  Gate/up: the 128 staged weight rows
// are [W1 i0..i0+32, W3 i0..i0+32, W1 i0+32..i0+64, W3 i0+32..i0+64], so each wave holds g
// and u of the same 32 columns and the SwiGLU epilogue stays in registers; down: 128 rows of
// W2.  Grid as k_expert_gemm (XCD-grouped, 1-D): 64 (gate/up) or 128 (down) columns per block.
template <bool GATEUP, bool ROUTED, bool LMHEAD = false>
__global__ __launch_bounds__(256, 2) void k_gemm_big(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const int32_t* __restrict__ flags,
    const int32_t* __restrict__ tile_slot, const int32_t* __restrict__ tile_row0,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ S_list,
    const int32_t* __restrict__ wl_pos, const float* __restrict__ wl_w,
    uint16_t* __restrict__ out, int M, int Kdim, int Ndim, LmPartials lp) {
  static_assert(!LMHEAD || (!GATEUP && !ROUTED), "the LM head is a plain gathered GEMM");
  constexpr int BR = 128, KC = 32, SEG_ROW = KC / 8;
  constexpr int NSEG = BR * SEG_ROW / 256;  // 16-byte segments per thread per operand and chunk
  constexpr int NR = 4;                     // register ring depth (chunks), even
  constexpr int NB = 3;                     // LDS buffers (chunks)
  constexpr int CBW = GATEUP ? 64 : 128;
  // LDS rows of KC = 32 bf16 (64 bytes, four 16-byte segments), no padding: segment c8 of row
  // `row` sits at slot c8 ^ ((row >> 2) & 3), so that the 16 rows of an MFMA fragment read and
  // the four segments of the rows a wave stores both fall on distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t As[NB][BR * KC];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NB][BR * KC];
  const int n_cb = (Ndim + CBW - 1) / CBW;
  int tile, cb;
  if (LMHEAD) {
    // few row tiles, many token blocks: token blocks go round the 8 XCDs and every row tile
    // of a block runs on the block's XCD (its W_v rows enter one L2); M bounds the row tiles
    const int T = (M + BR - 1) / BR, within = blockIdx.x >> 3;
    cb = 8 * (within / T) + (blockIdx.x & 7);
    tile = within % T;
    if (cb >= n_cb) return;
  } else {
    const int pos = blockIdx.x >> 3;
    tile = ((pos / n_cb) << 3) + (blockIdx.x & 7);
    cb = pos % n_cb;
  }
  // routed big tiles come from their own table, counted in FLAG_NTILES_BIG
  const TileRows tr = tile_rows(ROUTED, tile, BR, ROUTED ? flags[FLAG_NTILES_BIG] : 0, tile_slot,
                                tile_row0, offs, LMHEAD ? *lp.n_live : M);
  if (!tr.active) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const size_t estride = (size_t)Ndim * Kdim;
  const size_t e = ROUTED ? (size_t)S_list[tr.slot] : 0;
  // staging: NSEG activation and NSEG weight segments of 16 bytes per thread per chunk
  const uint16_t* asrc[NSEG];
  const uint16_t* bsrc[NSEG];
  bool aok[NSEG], bok[NSEG];
  int dst[NSEG];
#pragma unroll
  for (int j = 0; j < NSEG; ++j) {
    const int seg = tid + 256 * j;
    const int row = seg / SEG_ROW, c8 = seg % SEG_ROW;
    dst[j] = row * KC + ((c8 ^ ((row >> 2) & 3)) * 8);
    const int p = tr.row0 + row;
    aok[j] = p < tr.row_end;
    const int src_row =
        aok[j] ? ((ROUTED && GATEUP) ? wl_pos[p] : (LMHEAD ? lp.live_list[p] : p)) : 0;
    asrc[j] = A + (size_t)src_row * Kdim + c8 * 8;
    int wrow;
    const uint16_t* base;
    if (GATEUP) {
      const int q = row >> 5;  // quarter: W1, W3, W1, W3
      wrow = cb * 64 + (q >> 1) * 32 + (row & 31);
      base = (q & 1) ? B1 : B0;
    } else {
      wrow = cb * 128 + row;
      base = B0;
    }
    bok[j] = wrow < Ndim;
    bsrc[j] = base + e * estride + (size_t)(bok[j] ? wrow : 0) * Kdim + c8 * 8;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 ra[NR][NSEG], rb[NR][NSEG];  // chunk x waits in slot x % NR from its load to its store
  auto load = [&](int c, int slot) {
#pragma unroll
    for (int j = 0; j < NSEG; ++j) {
      ra[slot][j] = *reinterpret_cast<const u32x4*>(asrc[j] + (size_t)c * KC);
      rb[slot][j] = *reinterpret_cast<const u32x4*>(bsrc[j] + (size_t)c * KC);
    }
  };
  auto store = [&](int buf, int slot) {
#pragma unroll
    for (int j = 0; j < NSEG; ++j) {
      *reinterpret_cast<u32x4*>(&As[buf][dst[j]]) = aok[j] ? ra[slot][j] : zero;
      *reinterpret_cast<u32x4*>(&Bs[buf][dst[j]]) = bok[j] ? rb[slot][j] : zero;
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};
  // fragments of one chunk: lane (r, g) reads segment g of rows 16 m + r, whose slot depends
  // on r only; two register sets, so that chunk c + 1 is read from LDS while c is multiplied
  const int swz = (g ^ ((r >> 2) & 3)) * 8;
  bf16x8 fa[2][4], fb[2][4];
  auto read_frags = [&](int buf, int set) {
    const uint16_t* ab = &As[buf][(64 * wm + r) * KC + swz];
    const uint16_t* bb = &Bs[buf][(64 * wn + r) * KC + swz];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      fa[set][m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ab + m * 16 * KC));
      fb[set][m] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bb + m * 16 * KC));
    }
  };
  auto mma = [&](int set) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[set][m], fb[set][n], acc[m][n], 0, 0, 0);
  };
  static_assert(KC == 32, "one MFMA k-step per chunk");
  static_assert(NR % 2 == 0, "fragment sets alternate with the chunk parity");
  // Chunk x: fetched from global into ring slot x % NR at step x - NR (in the prologue for
  // x < NR), stored to LDS buffer x % NB at step x - 2, read into fragment set x & 1 at step
  // x - 1, multiplied at step x.  A buffer is rewritten two barriers after the step that last
  // read it; a ring slot is refilled after its chunk went to LDS.
  auto step = [&](int c, int u, bool pre, bool rd, bool st) {
    if (pre) load(c + NR, u % NR);
    __builtin_amdgcn_sched_barrier(0);  // keep the fetch ahead of the multiply
    if (rd) read_frags((c + 1) % NB, (u + 1) & 1);
    mma(u & 1);
    if (st) store((c + 2) % NB, (u + 2) % NR);
    __syncthreads();
  };
  const int nch = Kdim / KC;
#pragma unroll
  for (int x = 0; x < NR; ++x)
    if (x < nch) load(x, x);
  store(0, 0);
  if (nch > 1) store(1, 1);
  __syncthreads();
  read_frags(0, 0);
  // steady state: NR steps per trip (kb a multiple of NR, so slot and set follow u), every
  // fetch, read and store in range
  int kb = 0;
  for (; kb + 2 * NR - 1 < nch; kb += NR) {
#pragma unroll
    for (int u = 0; u < NR; ++u) step(kb + u, u, true, true, true);
  }
#pragma unroll
  for (int u = 0; u < 2 * NR - 1; ++u) {
    const int c = kb + u;
    if (c < nch) step(c, u, c + NR < nch, c + 1 < nch, c + 2 < nch);
  }
  // D[i][j] of a 16x16 block: lane j + 16 * (i / 4), register i % 4
  if (LMHEAD) {
    // per row: the 64 logits of this wave's token block sit in the 16 lanes with the same g,
    // four per lane; reduce (max, lower token on ties) and then sum exp(logit - max)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = tr.row0 + 64 * wm + 16 * m + 4 * g + q;
        const int col0 = cb * 128 + 64 * wn + r;
        float mx = acc[m][0][q];
        int arg = col0;
#pragma unroll
        for (int n = 1; n < 4; ++n)
          if (acc[m][n][q] > mx) {
            mx = acc[m][n][q];
            arg = col0 + 16 * n;
          }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          const float om = __shfl_xor(mx, o, 64);
          const int oa = __shfl_xor(arg, o, 64);
          if (om > mx || (om == mx && oa < arg)) {
            mx = om;
            arg = oa;
          }
        }
        float se = 0.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) se += expf(acc[m][n][q] - mx);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) se += __shfl_xor(se, o, 64);
        if (r == 0 && row < tr.row_end) {
          const size_t idx = (size_t)row * lp.n_p + 2 * cb + wn;
          lp.pmax[idx] = mx;
          lp.parg[idx] = arg;
          lp.psum[idx] = se;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = tr.row0 + 64 * wm + 16 * m + 4 * g + q;
      if (row >= tr.row_end) continue;
      if (GATEUP) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int col = cb * 64 + 32 * wn + 16 * n + r;
          const float gv = acc[m][n][q], uv = acc[m][n + 2][q];
          if (col < Ndim) out[(size_t)row * Ndim + col] = f32_to_bf16(gv / (1.0f + expf(-gv)) * uv);
        }
      } else {
        const float sc = ROUTED ? wl_w[row] : 1.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int col = cb * 128 + 64 * wn + 16 * n + r;
          if (col < Ndim) out[(size_t)row * Ndim + col] = f32_to_bf16(sc * acc[m][n][q]);
        }
      }
    }
  }
}

}  // namespace epoch
