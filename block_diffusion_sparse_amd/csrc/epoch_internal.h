// Internal declarations shared by the HIP translation units of libepoch (gfx950 only).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/epoch.h"

namespace epoch {

// Timing events of the kernel group being launched on this host thread (none: not timed).
// The group's first launch carries `start`, every launch carries `stop`, so the pair spans the
// group from its first kernel's start to its last kernel's end, stamped by the dispatches
// themselves: timing adds no packets between kernels.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;  // a launch has taken `start`
};
LaunchEvents& launch_events();

// Every kernel launch of the library goes through here.
template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t st, Args... args) {
  LaunchEvents& ev = launch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev.used ? nullptr : ev.start, ev.stop, 0u,
                        args...);
  if (ev.stop) ev.used = true;
}

constexpr int kWave = 64;
constexpr int kChunk = 64;        // positions per compaction chunk (one wave)
constexpr int kMaxKext = 32;      // candidates per position the wave top-k keeps
constexpr int kMaxExperts = 1024;
// Routed weight-stream tiles: kTileRows rows, or kTileRowsTall when the plan step finds that
// taller tiles need fewer of them (experts with more than kTileRows fresh pairs stream their
// weights once per tile); FLAG_TILE_TALL tells the expert kernel which.
constexpr int kTileRows = 64;
constexpr int kTileRowsTall = 128;
constexpr int kDenseTileRows = 64;  // rows per shared-expert weight-stream tile
// live-only decoding: up to this many live rows the LM head streams the vocabulary
// (k_expert_stream, one 128-row tile per token block), beyond it the compute-bound tiles of
// k_lm_head_w4 take it: from about this many rows up they are faster even with most of a
// 256-row tile empty, since every wave of the streamed head reads every live row's
// fragments from LDS
constexpr int kLmStreamMaxRows = 128;
constexpr int kBigTile = 256;     // rows per compute-bound routed tile
// experts with at least this many fresh rows use the compute-bound tiles (on shapes that enable
// them): beside those tiles the weight stream keeps 64-row tiles, so an expert with more rows
// would stream its weights once per 64 rows there, but once per 256 rows here (measured on the
// 8192-position shape: 64 to 128 best, 768 up to 10% slower)
constexpr int kBigRows = 128;
constexpr int kGateUpCols = 64;   // intermediate columns per gate/up workgroup
constexpr int kDownCols = 64;     // output columns per down workgroup

// per-forward flag words (int32) in the scratch area
// MISS and ANOMALY are raised by the router and cleared by the plan step once read (FRESH_ALL
// keeps the anomaly decision for the placement); the rest are written by the plan step.
// UNDER (restricted mode: positions under-covered by the Atlas support, counted by the router)
// is cleared by the plan step too; ROUTE_R (1 = this forward routes inside the support) is
// written by the plan step for the placement.
enum { FLAG_MISS = 0, FLAG_ANOMALY = 1, FLAG_NFRESH = 2, FLAG_NPAIRS = 3, FLAG_NTILES = 4,
       FLAG_NTILES_BIG = 5, FLAG_FRESH_ALL = 6, FLAG_UNDER = 7, FLAG_ROUTE_R = 8,
       FLAG_SHORT = 9, FLAG_TILE_TALL = 10, FLAG_WORDS = 16 };
// SHORT (restricted mode): some position has fewer than K selectable support experts; set by
// the router, cleared by the plan step.
// TILE_TALL (written by the plan step): the routed tile table holds kTileRowsTall-row tiles.
constexpr int kMaxGroups = 64;

// Device-side view of one layer's persistent state.
// valid / last_fresh / prev_D exist twice: the forward reads the current copy and writes the
// next one (combine), and a commit makes the next copy current (host side, no launch).
struct LayerState {
  void* cache;          // [M x H] act
  uint8_t* valid;       // [M] current
  int32_t* last_fresh;  // [M] current
  uint8_t* prev_D;      // [M] current
  uint8_t* valid_n;     // [M] next
  int32_t* last_fresh_n;// [M] next
  uint8_t* prev_D_n;    // [M] next
  uint8_t* inS;         // [E]
  int32_t* slot_of;     // [E]
  int32_t* S_list;      // [E]
  int32_t* S_size;      // [1]
  int32_t* S_valid;     // [1]
  int64_t* counters;    // [EPOCH_NUM_COUNTERS]
  uint8_t* fresh;       // [M] fresh flags of the layer's latest forward
  uint8_t* Dcur;        // [M] D_i seen by the layer's latest forward
  uint8_t* inA;         // [E] restricted mode: the Atlas support (no closure)
  int32_t* A_state;     // [4] restricted mode: valid flag, iteration of the latest build, size
};

// Device-side view of the per-forward scratch.
struct Scratch {
  float* G;             // [M x E]
  double* Gp;           // [router_kw x M x E] per-workgroup partial logits (router_kw > 1)
  int32_t* ids;         // [M x Kext]
  float* scores;        // [M x Kext]
  int32_t* q;           // [M x Kext]
  float* w;             // [M x K]
  int32_t* flags;       // [FLAG_WORDS]
  uint8_t* fpre;        // [M] bit 0 fresh test before the anomaly override, 1 forced, 2 due
  int32_t* rids;        // [M x K] restricted mode: top-K inside the support
  float* rw;            // [M x K] and its weights
  int32_t* routed_ids;  // [M x K] the routing the worklist used
  float* routed_w;      // [M x K]
  // cnt_f, cnt_a, cnt_fr, cnt_ar, chunk_fresh: carved back to back (one clearing range)
  int32_t* cnt_f;       // [n_chunks x E] routed pairs of fresh positions per chunk and expert
  int32_t* cnt_a;       // [n_chunks x E] routed pairs of all positions per chunk and expert
  int32_t* cnt_fr;      // [n_chunks x E] the same for the in-support routing (restricted mode)
  int32_t* cnt_ar;      // [n_chunks x E]
  int32_t* chunk_fresh; // [n_chunks]
  int32_t* chunk_base;  // [n_chunks x E]
  int32_t* chunk_foff;  // [n_chunks]
  int32_t* offs;        // [E + 1] per support slot
  int32_t* eoffs;       // [E + 1] per expert
  int32_t* wl_pos;      // [P_max]
  int32_t* wl_k;        // [P_max]
  float* wl_w;          // [P_max]
  int32_t* inv;         // [M x K]
  int32_t* fresh_list;  // [M]
  int32_t* tile_slot;   // [T_max]
  int32_t* tile_row0;   // [T_max]
  int32_t* tile_slot_b; // [T_big_max] tiles of kBigTile rows (experts with >= kBigRows pairs)
  int32_t* tile_row0_b; // [T_big_max]
  int32_t* Crow;        // [M] support-build coverage
  int32_t* Rrow;        // [M]
  void* h;              // [P_max x I] act
  void* y_pair;         // [P_max x H] act
  void* hs;             // [M x Is] act
  void* S;              // [M x H] act (shared expert output)
};

struct Shape {
  int M, H, E, K, Kext, I, Is, n_shared, R, gate_sigmoid, norm_topk, bf16;
  int n_chunks, ksplit, router_bt, router_kw, T_max, T_dense, T_big_max, big_routed;
  int restricted, atlas_period, n_group, topk_group;  // n_group <= 1: no grouping
  int B, c, an, ad, qn, qd, bn, bd;
};

// Compute units of the current device (read once per device; 256 if the query fails).
int device_cu_count();

// launchers (stream-ordered, no host sync); each returns hipGetLastError()
hipError_t launch_init_layer(const Shape& s, const LayerState& L, hipStream_t st);
hipError_t launch_init_scratch(const Shape& s, const Scratch& W, hipStream_t st);
hipError_t launch_router(const Shape& s, const void* x, const float* Wg, const float* bias,
                         const uint8_t* D, const uint8_t* force, int iter, const LayerState& L,
                         const Scratch& W, hipStream_t st);
hipError_t launch_plan(const Shape& s, int iter, const LayerState& L, const Scratch& W,
                       hipStream_t st);
hipError_t launch_place(const Shape& s, const LayerState& L, const Scratch& W, hipStream_t st);
// routed experts: the weight-stream tiles, and (shapes with big_routed) the compute-bound
// 256-row tiles of experts with many fresh pairs, which the forward runs on another stream
hipError_t launch_routed_gateup(const Shape& s, const void* x, const void* w1, const void* w3,
                                const LayerState& L, const Scratch& W, hipStream_t st);
hipError_t launch_routed_gateup_big(const Shape& s, const void* x, const void* w1,
                                    const void* w3, const LayerState& L, const Scratch& W,
                                    hipStream_t st);
hipError_t launch_routed_down(const Shape& s, const void* w2, const LayerState& L,
                              const Scratch& W, hipStream_t st);
hipError_t launch_routed_down_big(const Shape& s, const void* w2, const LayerState& L,
                                  const Scratch& W, hipStream_t st);
hipError_t launch_shared(const Shape& s, const void* x, const void* sw1, const void* sw3,
                         const void* sw2, const Scratch& W, hipStream_t st);
hipError_t launch_combine(const Shape& s, int iter, const LayerState& L, const Scratch& W,
                          void* y, void* y_routed, hipStream_t st);

}  // namespace epoch
