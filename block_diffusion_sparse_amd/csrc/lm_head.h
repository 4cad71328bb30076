// LM head over the live rows of one decoding step on the compute-bound tiles, persistent
// (gfx950, v_mfma_f32_16x16x32_bf16).
#pragma once
#include "expert_gemm.h"

namespace epoch {

// LM head over the live rows with a fixed grid (k_lm_head_w4): the logits of 256 live rows x
// 256 tokens per tile on k_gemm_w4's compute-bound tiles (four waves of 128 x 128 outputs, one
// wave per SIMD, accumulators in AGPRs, K in chunks of 64 through two LDS buffers), reduced in
// the epilogue to (largest logit, its token, sum of exp(logit - largest)) per row and tile.
// Each workgroup walks a sequence of tiles, and its copy cursor runs two chunks ahead of the
// multiplication across tile boundaries: the last two chunks of a tile copy the first two of
// the next one, which land while the epilogue reduces the tile.  The start of a tile
// (activation row lookups, the first two chunks' latency, a workgroup launch) is thus paid
// once per workgroup instead of once per tile.
// Walk: the tiles in supertile order (row supertiles of 4 row tiles; in each, supertiles of
// 4 row tiles x 8 token blocks, row-major; the last row or token supertile narrower when the
// counts are not multiples of 4 and 8), dealt in rounds of G = 8 P tiles: in round k workgroup
// 8 i + x (on XCD x) takes tile k G + P x + i.  So every workgroup gets the same number of
// tiles, give or take one, whatever the row and token counts; each XCD takes P consecutive
// tiles per round, with P = 32 one whole supertile, of which workgroup i keeps slot i (row
// tile i / 8, token block i % 8), so that its row tile changes only at a new row supertile.
// Accumulators start from zero through the first half-chunk's MFMAs (inline constant C = 0).
// Epilogue per row: the lane's largest logit is a max tree and its token the first equal
// logit (so the lowest token on ties), then the row's four lanes and two waves combine with
// the lower token on ties; the sum of exp(logit - largest) is summed in a fixed order.
__global__ __launch_bounds__(256, 1) void k_lm_head_w4(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ W, int Kdim,
                                                       int V, LmPartials lp) {
  constexpr int BR = 256, BC = 256, KC = 64, WAVES = 4, WN = 2, MB = 8, NBK = 8;
  constexpr int NA = BR / (8 * WAVES), NBI = BC / (8 * WAVES);  // copies per wave and chunk
  constexpr int CPC = NA + NBI;
  struct Part {
    float mx;
    int arg;
    float se;
  };
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BR * KC];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BC * KC];
  __shared__ Part part[BR * WN];  // [row][wave column half]
  const int rows = *lp.n_live;
  if (rows <= kLmStreamMaxRows) return;  // the streamed LM head covered them
  const int T = (rows + BR - 1) / BR, n_cb = (V + BC - 1) / BC, NV = T * n_cb;
  const int G = gridDim.x, P = G >> 3;
  const int nch = Kdim / KC;
  // tile v of the walk order: row supertiles of four row tiles (the last one R < 4 when T is
  // not a multiple of 4), each in supertiles of R row tiles x 8 token blocks (the last one
  // C < 8 blocks wide), each supertile row-major
  auto tile_of = [&](int v, int& tile, int& cb) __attribute__((always_inline)) {
    const int full_rs = T >> 2, per_rs = 4 * n_cb;
    int rs, w, R;
    if (v < full_rs * per_rs) {
      rs = v / per_rs;
      w = v - rs * per_rs;
      R = 4;
    } else {
      rs = full_rs;
      w = v - full_rs * per_rs;
      R = T - 4 * full_rs;
    }
    const int ncs = n_cb >> 3, full = 8 * R * ncs;
    int cs, o, C;
    if (w < full) {
      cs = w / (8 * R);
      o = w - cs * 8 * R;
      C = 8;
    } else {
      cs = ncs;
      o = w - full;
      C = n_cb - 8 * ncs;
    }
    tile = 4 * rs + o / C;
    cb = 8 * cs + o % C;
  };
  // walk position u of this workgroup: tile u G + P (blockIdx.x % 8) + blockIdx.x / 8, so that
  // each round of G tiles gives every XCD P consecutive tiles of the order; false at the end
  const int wg_off = P * (int)(blockIdx.x & 7) + (int)(blockIdx.x >> 3);
  auto locate = [&](int u, int& tile, int& cb) __attribute__((always_inline)) -> bool {
    const int v = u * G + wg_off;
    if (v >= NV) return false;
    tile_of(v, tile, cb);
    return true;
  };
  int cu_u = 0, cu_tile = 0, cu_cb = 0, cu_c = 0;  // copy cursor
  if (!locate(cu_u, cu_tile, cu_cb)) return;
  int co_u = cu_u, co_tile = cu_tile, co_cb = cu_cb;  // the tile being multiplied
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  // copy j of wave w fills LDS rows 32 j + 8 w + [0, 8) of a chunk buffer, lane l slot l % 8
  // of row 32 j + 8 w + l / 8, i.e. k-segment seg = (l % 8) ^ (l / 8): activation rows by
  // pointer (gathered through the live list; rows past the live count load the tile's first
  // row), token rows as the block's first token row (a scalar base), plus 32 j rows (scalar),
  // plus the lane's row and segment (one 32-bit offset for all j).  A block with only 128
  // tokens left in the vocabulary (its size is a multiple of 128) loads its first 128 rows again
  // for the second 128; those stand-ins only feed outputs that are never used
  const int rbase = 8 * wave + (lane >> 3), seg = (lane & 7) ^ (lane >> 3);
  const uint32_t boff = ((uint32_t)rbase * (uint32_t)Kdim + seg * 8) * 2u;
  const char* asrc[NA];
  const char* bbase = nullptr;
  bool bhalf = false;
  auto set_rows = [&](int tile) __attribute__((always_inline)) {
    const int row0 = tile * BR, row_end = min(rows, row0 + BR);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int p = row0 + 32 * j + rbase < row_end ? row0 + 32 * j + rbase : row0;
      asrc[j] = reinterpret_cast<const char*>(A + (size_t)lp.live_list[p] * Kdim + seg * 8);
    }
  };
  auto set_cols = [&](int cb) __attribute__((always_inline)) {
    bbase = reinterpret_cast<const char*>(W + (size_t)cb * BC * Kdim);
    bhalf = V - cb * BC < BC;
  };
  // the cursor's next chunk: the next chunk of its tile, else the first of the walk's next
  // tile; past the walk's end it stays on the last chunk (copies nobody reads)
  auto advance = [&]() __attribute__((always_inline)) {
    if (++cu_c < nch) return;
    const int u = cu_u + 1;
    int t = 0, cb = 0;
    if (!locate(u, t, cb)) {
      cu_c = nch - 1;
      return;
    }
    cu_c = 0;
    cu_u = u;
    if (t != cu_tile) {
      cu_tile = t;
      set_rows(t);
    }
    if (cb != cu_cb) {
      cu_cb = cb;
      set_cols(cb);
    }
  };
  auto issue = [&](int j, int buf) __attribute__((always_inline)) {
    if (j < NA)
      copy16_to_lds(asrc[j] + (size_t)cu_c * (KC * 2), &As[buf][8 * (WAVES * j + wave) * KC]);
    else {
      const int jb = j - NA, jr = bhalf && jb >= NBI / 2 ? jb - NBI / 2 : jb;
      copy16_to_lds(bbase + (size_t)jr * (32 * 2) * Kdim + (boff + (uint32_t)cu_c * (KC * 2)),
                    &Bs[buf][8 * (WAVES * jb + wave) * KC]);
    }
  };
  f32x4 acc[MB][NBK];
  // fragments of half h: lane (r, g) reads row 16 i + r, k-segment 4 h + g, in slot
  // (4 h + g) ^ (r & 7)
  u32x4 fa[2][MB], fb[2][NBK];
  const uint32_t a_l = (uint32_t)(uintptr_t)&As[0][(128 * wm + r) * KC];
  const uint32_t b_l = (uint32_t)(uintptr_t)&Bs[0][(128 * wn + r) * KC];
  const uint32_t sw0 = (g ^ (r & 7)) * 16, sw1 = ((4 + g) ^ (r & 7)) * 16;
  auto read = [&](int buf, int half, int set, int i) __attribute__((always_inline)) {
    const uint32_t sw = half ? sw1 : sw0;
    if (i < MB)
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(fa[set][i]) : "v"(a_l + buf * (BR * KC * 2) + sw), "i"(i * 16 * KC * 2));
    else
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(fb[set][i - MB])
                   : "v"(b_l + buf * (BC * KC * 2) + sw), "i"((i - MB) * 16 * KC * 2));
  };
  auto frags_ready = [&](int set) __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(fa[set][0]), "+v"(fa[set][1]), "+v"(fa[set][2]), "+v"(fa[set][3]),
                   "+v"(fa[set][4]), "+v"(fa[set][5]), "+v"(fa[set][6]), "+v"(fa[set][7]),
                   "+v"(fb[set][0]), "+v"(fb[set][1]), "+v"(fb[set][2]), "+v"(fb[set][3]),
                   "+v"(fb[set][4]), "+v"(fb[set][5]), "+v"(fb[set][6]), "+v"(fb[set][7]));
  };
  // lane (r, g) of block (m, n) gets tokens 16 n + 4 g .. + 3 of row 16 m + r
  auto mma = [&](int set, int idx, bool zero) __attribute__((always_inline)) {
    const int m = idx / NBK, n = idx % NBK;
    if (zero)
      asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
          : "=a"(acc[m][n]) : "v"(fb[set][n]), "v"(fa[set][m]));
    else
      asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
          : "+a"(acc[m][n]) : "v"(fb[set][n]), "v"(fa[set][m]));
  };
  // one half: 64 MFMAs on `set` (from C = 0 when `zero`); when `rd`, the 16 fragment reads of
  // (rbuf, rhalf) into the other set, two per group of four MFMAs in the first eight groups, so
  // that they have landed by the half's end; when `copy`, the cursor's CPC copies into buffer
  // cbuf, one per group
  auto half_step = [&](int set, int rbuf, int rhalf, bool zero, bool rd, bool copy,
                       int cbuf) __attribute__((always_inline)) {
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) {
      if (rd && grp < 8) {
        read(rbuf, rhalf, set ^ 1, 2 * grp);
        read(rbuf, rhalf, set ^ 1, 2 * grp + 1);
      }
      mma(set, 4 * grp + 0, zero);
      mma(set, 4 * grp + 1, zero);
      if (copy) issue(grp, cbuf);
      mma(set, 4 * grp + 2, zero);
      mma(set, 4 * grp + 3, zero);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One chunk in buffer buf, its first half's fragments in set 0: the second half refills buf
  // with the cursor's chunk and, except in a tile's last chunk, reads the first half of the
  // next chunk (buffer buf ^ 1) into set 0.  Every read has landed by the end of the step
  // (frags_ready), so no fragment register is in flight where steps meet: the compiler, which
  // takes an asm output as written at once, may copy registers at those joins.  A tile's last
  // chunk leaves its read until after the epilogue, whose registers it would otherwise hold.
  auto step = [&](int buf, bool first, bool last) __attribute__((always_inline)) {
    half_step(0, buf, 1, first, true, false, 0);
    wait_vm_lds<0>();
    frags_ready(1);
    asm volatile("s_barrier" ::: "memory");
    half_step(1, buf ^ 1, 0, false, !last, true, buf);
    if (!last) frags_ready(0);
    advance();
  };
  // The row's four lanes (lane bits 4 and 5) combine in two rounds of pairs (lanes 16, then 32
  // apart) on the VALU: v_permlane16_swap / v_permlane32_swap with both operands one register
  // leave the two lanes of every pair holding both pair values, one in each result, so a
  // symmetric combine of the two results is the pair's combine in both of its lanes.  The
  // best of two is the larger logit, the lower token on ties; sums add the two values, which
  // gives both lanes the same bits
  auto swap_pair = [](uint32_t v, bool far) __attribute__((always_inline)) {
    return far ? __builtin_amdgcn_permlane32_swap(v, v, false, false)
               : __builtin_amdgcn_permlane16_swap(v, v, false, false);
  };
  auto pair_best = [&](float& mx, int& arg, bool far) __attribute__((always_inline)) {
    const auto pm = swap_pair(__float_as_uint(mx), far);
    const auto pa = swap_pair((uint32_t)arg, far);
    const float m0 = __uint_as_float(pm[0]), m1 = __uint_as_float(pm[1]);
    const int a0 = (int)pa[0], a1 = (int)pa[1];
    const bool one = (m1 > m0) | ((m1 == m0) & (a1 < a0));
    mx = one ? m1 : m0;
    arg = one ? a1 : a0;
  };
  auto pair_sum = [&](float& v, bool far) __attribute__((always_inline)) {
    const auto p = swap_pair(__float_as_uint(v), far);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  };
  set_rows(cu_tile);
  set_cols(cu_cb);
#pragma unroll
  for (int j = 0; j < CPC; ++j) issue(j, 0);
  advance();
#pragma unroll
  for (int j = 0; j < CPC; ++j) issue(j, 1);
  advance();
  wait_vm_lds<CPC>();
  __builtin_amdgcn_s_barrier();
  int buf = 0;  // the buffer of the tile's first chunk, landed and visible to every wave
  for (;;) {
#pragma unroll
    for (int i = 0; i < 16; ++i) read(buf, 0, 0, i);
    frags_ready(0);
    if (nch == 1) {
      step(buf, true, true);
      buf ^= 1;
    } else {
      step(buf, true, false);
      buf ^= 1;
      for (int c = 1; c < nch - 1; ++c) {
        step(buf, false, false);
        buf ^= 1;
      }
      step(buf, false, true);
      buf ^= 1;
    }
    // the wait states before the accumulators are read
    asm volatile("s_nop 15\n s_nop 15\n s_nop 15" ::: "memory");
    // Per row, over the tile's 256 tokens: lane (r, g) of row block m holds tokens
    // 16 n + 4 g + i (n < 8, i < 4) of its wave's 128-token half for row 16 m + r; the lane's
    // (max, first token), then across the four lanes of the row (lane bits 4 and 5, lower token
    // on ties), then the sum of exp(logit - max) likewise; the two waves of a row meet in LDS.
    // A wave whose tokens lie past the vocabulary contributes (-inf, -, 0).  exp(v - mx) is one
    // v_exp_f32 of v log2(e) - mx log2(e) (one fma)
    {
      const int row0 = co_tile * BR, row_end = min(rows, row0 + BR);
      const bool wlive = co_cb * BC + 128 * wn < V;
      const int tok0 = co_cb * BC + 128 * wn + 4 * g;
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        // the block's accumulators are read from here on, not all blocks' at the epilogue's start
        asm volatile(""
                     : "+a"(acc[m][0]), "+a"(acc[m][1]), "+a"(acc[m][2]), "+a"(acc[m][3]),
                       "+a"(acc[m][4]), "+a"(acc[m][5]), "+a"(acc[m][6]), "+a"(acc[m][7])
                     :
                     : "memory");
        float mx = acc[m][0][0];
#pragma unroll
        for (int k = 1; k < 4 * NBK; ++k) mx = fmaxf(mx, acc[m][k >> 2][k & 3]);
        // first equal logit, from two independent scans over halves of the lane's tokens
        int k0 = 4 * NBK, k1 = 0;
#pragma unroll
        for (int k = 2 * NBK - 1; k >= 0; --k) {
          k0 = acc[m][k >> 2][k & 3] == mx ? k : k0;
          k1 = acc[m][(k + 2 * NBK) >> 2][k & 3] == mx ? k + 2 * NBK : k1;
        }
        const int k = k0 < 4 * NBK ? k0 : k1;
        int arg = tok0 + 16 * (k >> 2) + (k & 3);
        pair_best(mx, arg, false);
        pair_best(mx, arg, true);
        const float nm = -mx * kLog2e;
        float se = 0.0f;
#pragma unroll
        for (int n = 0; n < NBK; ++n)
          se += (__builtin_amdgcn_exp2f(fmaf(acc[m][n][0], kLog2e, nm)) +
                 __builtin_amdgcn_exp2f(fmaf(acc[m][n][1], kLog2e, nm))) +
                (__builtin_amdgcn_exp2f(fmaf(acc[m][n][2], kLog2e, nm)) +
                 __builtin_amdgcn_exp2f(fmaf(acc[m][n][3], kLog2e, nm)));
        pair_sum(se, false);
        pair_sum(se, true);
        if (g == 0)
          part[(128 * wm + 16 * m + r) * WN + wn] =
              wlive ? Part{mx, arg, se} : Part{-INFINITY, 0x7fffffff, 0.0f};
        // one row block at a time: the registers of one block's 32 logits suffice
        __builtin_amdgcn_sched_barrier(0);
      }
      // the partials of both waves of every row are in LDS (the next write of part follows
      // at least one more barrier of the loop, after these reads)
      asm volatile("s_waitcnt lgkmcnt(0)\n s_barrier" ::: "memory");
      const int row = row0 + tid;
      if (row < row_end) {
        Part best = part[tid * WN];
#pragma unroll
        for (int w = 1; w < WN; ++w) {
          const Part q = part[tid * WN + w];
          if (q.mx > best.mx) best = q;
        }
        const float nm = -best.mx * kLog2e;
        float se = 0.0f;
#pragma unroll
        for (int w = 0; w < WN; ++w) {
          const Part q = part[tid * WN + w];
          se += q.se * __builtin_amdgcn_exp2f(fmaf(q.mx, kLog2e, nm));
        }
        const size_t idx = (size_t)row * lp.n_p + co_cb;
        lp.pmax[idx] = best.mx;
        lp.parg[idx] = best.arg;
        lp.psum[idx] = se;
      }
    }
    ++co_u;
    if (!locate(co_u, co_tile, co_cb)) break;
  }
  // the surplus copies land before the workgroup's LDS is released
  wait_vm_lds<0>();
}

// Grid of k_lm_head_w4: one workgroup per CU, a multiple of the 8 XCDs (at least one per XCD).
inline int lm_head_grid(int n_cu) { return n_cu >= 16 ? n_cu / 8 * 8 : 8; }

}  // namespace epoch
