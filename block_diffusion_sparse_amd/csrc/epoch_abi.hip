// C ABI of libepoch: descriptor validation, workspace carving, the per-iteration launch
// sequence on the caller's stream, and the plan lifecycle.  No device allocation, no host
// synchronisation on the forward path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "epoch_internal.h"

using namespace epoch;

namespace {

constexpr size_t kAlign = 256;

struct Layout {
  std::vector<LayerState> layers;
  Scratch scratch;
  size_t bytes = 0;
};

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t n) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += std::max<size_t>(n, 1) * sizeof(T);
    return p;
  }
  void* take_bytes(size_t n) { return take<char>(n); }
};

int32_t check_desc(const epoch_desc* d) {
  if (!d) return EPOCH_E_NULL;
  if (d->act_dtype != EPOCH_DTYPE_BF16 && d->act_dtype != EPOCH_DTYPE_F32) return EPOCH_E_DTYPE;
  if (d->gate != EPOCH_GATE_SOFTMAX && d->gate != EPOCH_GATE_SIGMOID) return EPOCH_E_DTYPE;
  if (d->flags != 0) return EPOCH_E_SHAPE;
  if (d->routing != EPOCH_ROUTING_EXACT && d->routing != EPOCH_ROUTING_RESTRICTED)
    return EPOCH_E_SHAPE;
  if (d->atlas_period < 0 || (d->routing == EPOCH_ROUTING_EXACT && d->atlas_period != 0))
    return EPOCH_E_SHAPE;
  if (d->n_layers < 1 || d->hidden < 1 || d->hidden > 16384) return EPOCH_E_SHAPE;
  if (d->n_experts < 1 || d->n_experts > kMaxExperts) return EPOCH_E_SHAPE;
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->n_experts) return EPOCH_E_SHAPE;
  if (d->inter < 1 || d->batch < 1 || d->block < 1) return EPOCH_E_SHAPE;
  if ((long long)d->batch * d->block > (1 << 20)) return EPOCH_E_SHAPE;
  if (d->n_shared != 0 && d->n_shared != 1) return EPOCH_E_SHAPE;
  if (d->n_shared && d->shared_inter < 1) return EPOCH_E_SHAPE;
  if (d->staleness_R < 1) return EPOCH_E_SHAPE;
  if (d->atlas_m < 0 || d->atlas_B < 0 || d->atlas_c < 1) return EPOCH_E_SHAPE;
  if (d->alpha_num < 0 || d->alpha_den < 1 || d->q_num < 0 || d->q_den < 1 ||
      d->q_num > d->q_den || d->beta_num < 0 || d->beta_den < 1)
    return EPOCH_E_SHAPE;
  const int kext = std::min(d->top_k + d->atlas_m, d->n_experts);
  if (kext > kMaxKext) return EPOCH_E_SHAPE;
  if (d->n_group < 0) return EPOCH_E_SHAPE;
  if (d->n_group > 1) {
    if (d->n_group > kMaxGroups || d->n_experts % d->n_group) return EPOCH_E_SHAPE;
    if (d->topk_group < 1 || d->topk_group > d->n_group) return EPOCH_E_SHAPE;
    if ((long long)d->topk_group * (d->n_experts / d->n_group) < kext) return EPOCH_E_SHAPE;
  }
  if (d->hidden % 64) return EPOCH_E_SHAPE;
  if (d->act_dtype == EPOCH_DTYPE_BF16) {
    if (d->inter % 64) return EPOCH_E_SHAPE;
    if (d->n_shared && d->shared_inter % 64) return EPOCH_E_SHAPE;
  }
  return EPOCH_OK;
}

Shape make_shape(const epoch_desc* d) {
  Shape s{};
  s.M = d->batch * d->block;
  s.H = d->hidden;
  s.E = d->n_experts;
  s.K = d->top_k;
  s.Kext = std::min(d->top_k + d->atlas_m, d->n_experts);
  s.I = d->inter;
  s.n_shared = d->n_shared;
  s.Is = d->n_shared ? d->shared_inter : 0;
  s.R = d->staleness_R;
  s.gate_sigmoid = d->gate == EPOCH_GATE_SIGMOID;
  s.norm_topk = d->norm_topk != 0;
  s.bf16 = d->act_dtype == EPOCH_DTYPE_BF16;
  s.n_chunks = (s.M + kChunk - 1) / kChunk;
  // router: 32 x 32 tiles when that gives at least 512 workgroups, else 16 x 16; the k range
  // is split over the waves of a workgroup until about 2048 waves run (H / ksplit stays a
  // multiple of 64; the LDS reduction stays within 32 KB)
  const int tiles32 = ((s.M + 31) / 32) * ((s.E + 31) / 32);
  s.router_bt = tiles32 >= 512 ? 32 : 16;
  const int tiles = ((s.M + s.router_bt - 1) / s.router_bt) * ((s.E + s.router_bt - 1) / s.router_bt);
  const int max_split = s.router_bt == 32 ? 4 : 16;
  s.ksplit = 1;
  while (s.ksplit < max_split && tiles * s.ksplit < 2048 && s.H % (128 * s.ksplit) == 0)
    s.ksplit *= 2;
  // few logit tiles: part of that split goes to workgroups instead of waves (router_kw of them
  // per tile, their fp64 partial sums added in order by the top-k kernel) so that about 256
  // workgroups share the fp64 MFMA work
  s.router_kw = 1;
  while (s.E <= 64 && s.router_kw < 4 && s.router_kw < s.ksplit && tiles * s.router_kw < 256)
    s.router_kw *= 2;  // (the top-k kernel holds up to 4 parts per lane, one expert per lane)
  s.ksplit /= s.router_kw;  // waves per workgroup
  const long long P_max = (long long)s.M * s.K;
  s.T_max = (int)((P_max + kTileRows - 1) / kTileRows) + s.E;
  s.T_dense = (s.M + kDenseTileRows - 1) / kDenseTileRows;
  // experts with at least kBigRows fresh pairs take compute-bound 128-row tiles; enabled only
  // for shapes whose iterations can hold far more pairs than the weight-stream tiles cover
  // well (with fewer pairs per iteration the extra launch costs more than it saves)
  s.big_routed = s.bf16 && P_max >= 32768;
  s.T_big_max = s.big_routed ? (int)((P_max + kBigTile - 1) / kBigTile + P_max / kBigRows + 1) : 0;
  s.B = d->atlas_B;
  s.c = d->atlas_c;
  s.an = d->alpha_num;
  s.ad = d->alpha_den;
  s.qn = d->q_num;
  s.qd = d->q_den;
  s.bn = d->beta_num;
  s.bd = d->beta_den;
  s.restricted = d->routing == EPOCH_ROUTING_RESTRICTED;
  s.atlas_period = d->atlas_period;
  s.n_group = d->n_group > 1 ? d->n_group : 0;
  s.topk_group = d->n_group > 1 ? d->topk_group : 0;
  return s;
}

Layout carve(const epoch_desc* d, const Shape& s, void* base) {
  Layout lay;
  Carver c{static_cast<char*>(base)};
  const size_t act = s.bf16 ? 2 : 4;
  const size_t M = s.M, H = s.H, E = s.E, K = s.K, Kext = s.Kext;
  for (int l = 0; l < d->n_layers; ++l) {
    LayerState L{};
    L.cache = c.take_bytes(M * H * act);
    L.valid = c.take<uint8_t>(M);
    L.last_fresh = c.take<int32_t>(M);
    L.prev_D = c.take<uint8_t>(M);
    L.valid_n = c.take<uint8_t>(M);
    L.last_fresh_n = c.take<int32_t>(M);
    L.prev_D_n = c.take<uint8_t>(M);
    L.inS = c.take<uint8_t>(E);
    L.slot_of = c.take<int32_t>(E);
    L.S_list = c.take<int32_t>(E);
    L.S_size = c.take<int32_t>(1);
    L.S_valid = c.take<int32_t>(1);
    L.counters = c.take<int64_t>(EPOCH_NUM_COUNTERS);
    L.fresh = c.take<uint8_t>(M);
    L.Dcur = c.take<uint8_t>(M);
    L.inA = c.take<uint8_t>(E);
    L.A_state = c.take<int32_t>(4);
    lay.layers.push_back(L);
  }
  const size_t P_max = M * K;
  Scratch& W = lay.scratch;
  W.G = c.take<float>(M * E);
  W.Gp = c.take<double>(s.router_kw > 1 ? (size_t)s.router_kw * M * E : 1);
  W.ids = c.take<int32_t>(M * Kext);
  W.scores = c.take<float>(M * Kext);
  W.q = c.take<int32_t>(M * Kext);
  W.w = c.take<float>(M * K);
  W.flags = c.take<int32_t>(FLAG_WORDS);
  W.fpre = c.take<uint8_t>(M);
  W.rids = c.take<int32_t>(M * K);
  W.rw = c.take<float>(M * K);
  W.routed_ids = c.take<int32_t>(M * K);
  W.routed_w = c.take<float>(M * K);
  // cnt_f, cnt_a, cnt_fr, cnt_ar, chunk_fresh: carved back to back (cleared as one range)
  W.cnt_f = c.take<int32_t>((size_t)s.n_chunks * E);
  W.cnt_a = c.take<int32_t>((size_t)s.n_chunks * E);
  W.cnt_fr = c.take<int32_t>((size_t)s.n_chunks * E);
  W.cnt_ar = c.take<int32_t>((size_t)s.n_chunks * E);
  W.chunk_fresh = c.take<int32_t>(s.n_chunks);
  W.chunk_base = c.take<int32_t>((size_t)s.n_chunks * E);
  W.chunk_foff = c.take<int32_t>(s.n_chunks);
  W.offs = c.take<int32_t>(E + 1);
  W.eoffs = c.take<int32_t>(E + 1);
  W.wl_pos = c.take<int32_t>(P_max);
  W.wl_k = c.take<int32_t>(P_max);
  W.wl_w = c.take<float>(P_max);
  W.inv = c.take<int32_t>(M * K);
  W.fresh_list = c.take<int32_t>(M);
  W.tile_slot = c.take<int32_t>(s.T_max);
  W.tile_row0 = c.take<int32_t>(s.T_max);
  W.tile_slot_b = c.take<int32_t>(std::max(s.T_big_max, 1));
  W.tile_row0_b = c.take<int32_t>(std::max(s.T_big_max, 1));
  W.Crow = c.take<int32_t>(M);
  W.Rrow = c.take<int32_t>(M);
  W.h = c.take_bytes(P_max * s.I * act);
  W.y_pair = c.take_bytes(P_max * H * act);
  W.hs = c.take_bytes(M * std::max(s.Is, 1) * act);
  W.S = c.take_bytes(M * H * act);
  lay.bytes = (c.off + kAlign - 1) / kAlign * kAlign;
  return lay;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

namespace epoch {
LaunchEvents& launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // 0 = not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}
}  // namespace epoch

// The side stream of the current device: one per device for the whole process, created at its
// first use (default priority, non-blocking) and never destroyed, so that building a plan
// creates no stream and every plan of a device forks onto the same queue.
hipStream_t device_side_stream() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static hipStream_t streams[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!streams[dev] && hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking) != hipSuccess)
    streams[dev] = nullptr;
  return streams[dev];
}

struct TimedPair {
  int group;
  hipEvent_t a, b;
};

// Process-wide pool of timing events, so that a timed region reuses events created earlier.
std::mutex g_event_mu;
std::vector<hipEvent_t> g_free_events;

hipEvent_t pool_event() {
  {
    std::lock_guard<std::mutex> lk(g_event_mu);
    if (!g_free_events.empty()) {
      hipEvent_t e = g_free_events.back();
      g_free_events.pop_back();
      return e;
    }
  }
  // timing only: no system-scope fence (cache writeback and invalidate) at each record, which
  // would otherwise stall the work after it; elapsed times are still exact
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

void pool_release(hipEvent_t e) {
  std::lock_guard<std::mutex> lk(g_event_mu);
  g_free_events.push_back(e);
}

struct epoch_plan {
  epoch_desc d;
  Shape s;
  std::vector<epoch_layer_weights> w;
  Layout lay;
  std::vector<int32_t> iter;
  std::vector<uint8_t> pending;
  std::vector<uint8_t> parity;  // which copy of the commit state is current, per layer
  int last_layer = -1;
  uint32_t timing_mask = 0;
  // Work that does not depend on the rest of the forward runs on the device's side stream,
  // forked after the caller's earlier work and joined before the combine: the shared expert
  // (it depends only on x) from the start of the forward, and the compute-bound big-tile routed
  // experts (they depend on the plan step) beside the light tiles' weight stream.  Null when
  // the layer has neither.  The events are the plan's own.
  hipStream_t side = nullptr;
  bool joined = false;  // `join` has been recorded at least once
  hipEvent_t fork = nullptr, fork_big = nullptr, join = nullptr;
  std::vector<TimedPair> pairs;
  double ms[EPOCH_TIMING_GROUPS] = {};
  int64_t launches[EPOCH_TIMING_GROUPS] = {};
};

namespace {

// Times one kernel group when timing is on: the group's launches carry an event pair (see
// launch()), kept for epoch_plan_timing if some kernel of the group ran.
struct GroupTimer {
  epoch_plan* p;
  int group;
  hipEvent_t a = nullptr, b = nullptr;
  GroupTimer(epoch_plan* p_, hipStream_t, int g) : p(p_), group(g) {
    if (!((p->timing_mask >> g) & 1u)) return;
    a = pool_event();
    b = a ? pool_event() : nullptr;
    if (!b) {
      if (a) pool_release(a);
      a = nullptr;
      return;
    }
    launch_events() = LaunchEvents{a, b, false};
  }
  void done() {
    if (!b) return;
    if (launch_events().used) {
      p->pairs.push_back({group, a, b});
    } else {
      pool_release(a);
      pool_release(b);
    }
    launch_events() = LaunchEvents{};
    a = b = nullptr;
  }
  ~GroupTimer() { done(); }
};

}  // namespace

namespace {

// The layer's state with the current copy of the commit state in front.
LayerState state_now(const epoch_plan* p, int layer) {
  LayerState L = p->lay.layers[layer];
  if (p->parity[layer]) {
    std::swap(L.valid, L.valid_n);
    std::swap(L.last_fresh, L.last_fresh_n);
    std::swap(L.prev_D, L.prev_D_n);
  }
  return L;
}

}  // namespace

extern "C" {

int32_t epoch_plan_workspace_bytes(const epoch_desc* d, size_t* out_bytes) {
  if (!out_bytes) return EPOCH_E_NULL;
  const int32_t rc = check_desc(d);
  if (rc) return rc;
  const Shape s = make_shape(d);
  *out_bytes = carve(d, s, nullptr).bytes;
  return EPOCH_OK;
}

int32_t epoch_block_plan_build(const epoch_desc* d, const epoch_layer_weights* weights,
                               void* workspace, size_t workspace_bytes, void* stream,
                               epoch_plan** out_plan) {
  if (!out_plan || !weights || !workspace) return EPOCH_E_NULL;
  *out_plan = nullptr;
  int32_t rc = check_desc(d);
  if (rc) return rc;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return EPOCH_E_WORKSPACE;
  const Shape s = make_shape(d);
  for (int l = 0; l < d->n_layers; ++l) {
    const epoch_layer_weights& w = weights[l];
    if (!w.router_w || !w.w1 || !w.w3 || !w.w2) return EPOCH_E_NULL;
    if (d->n_shared && (!w.sw1 || !w.sw3 || !w.sw2)) return EPOCH_E_NULL;
    if (!aligned16(w.router_w) || !aligned16(w.w1) || !aligned16(w.w3) || !aligned16(w.w2))
      return EPOCH_E_ALIGN;
    if (d->n_shared && (!aligned16(w.sw1) || !aligned16(w.sw3) || !aligned16(w.sw2)))
      return EPOCH_E_ALIGN;
  }
  Layout lay = carve(d, s, workspace);
  if (workspace_bytes < lay.bytes) return EPOCH_E_WORKSPACE;
  epoch_plan* p = new (std::nothrow) epoch_plan();
  if (!p) return EPOCH_E_NULL;
  p->d = *d;
  p->s = s;
  p->w.assign(weights, weights + d->n_layers);
  p->lay = std::move(lay);
  p->iter.assign(d->n_layers, 0);
  p->pending.assign(d->n_layers, 0);
  p->parity.assign(d->n_layers, 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d->n_shared || s.big_routed) {
    p->side = device_side_stream();
    if (!p->side ||
        hipEventCreateWithFlags(&p->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&p->fork_big, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&p->join, hipEventDisableTiming) != hipSuccess) {
      epoch_block_plan_destroy(p);
      return EPOCH_E_HIP;
    }
  }
  for (int l = 0; l < d->n_layers; ++l) {
    if (launch_init_layer(s, p->lay.layers[l], st) != hipSuccess) {
      epoch_block_plan_destroy(p);
      return EPOCH_E_HIP;
    }
  }
  if (launch_init_scratch(s, p->lay.scratch, st) != hipSuccess) {
    epoch_block_plan_destroy(p);
    return EPOCH_E_HIP;
  }
  *out_plan = p;
  return EPOCH_OK;
}

int32_t epoch_moe_fresh_forward(epoch_plan* p, int32_t layer, const void* x,
                                const uint8_t* decoded, const uint8_t* force_fresh, void* y,
                                void* y_routed, void* stream) {
  if (!p || !x || !decoded || !y) return EPOCH_E_NULL;
  if (layer < 0 || layer >= p->d.n_layers) return EPOCH_E_LAYER;
  if (!aligned16(x) || !aligned16(y) || (y_routed && !aligned16(y_routed))) return EPOCH_E_ALIGN;
  const Shape& s = p->s;
  const LayerState L = state_now(p, layer);
  const Scratch& W = p->lay.scratch;
  const epoch_layer_weights& w = p->w[layer];
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (s.n_shared) {
    if (hipEventRecord(p->fork, st) != hipSuccess ||
        hipStreamWaitEvent(p->side, p->fork, 0) != hipSuccess)
      return EPOCH_E_HIP;
    GroupTimer tm(p, p->side, 5);
    e = launch_shared(s, x, w.sw1, w.sw3, w.sw2, W, p->side);
    tm.done();
    if (e != hipSuccess) return EPOCH_E_HIP;
  }
  {
    GroupTimer tm(p, st, 0);
    e = launch_router(s, x, w.router_w, w.router_b, decoded, force_fresh, p->iter[layer], L, W, st);
    tm.done();
  }
  if (e != hipSuccess) return EPOCH_E_HIP;
  {
    GroupTimer tm(p, st, 1);
    e = launch_plan(s, p->iter[layer], L, W, st);
    tm.done();
  }
  if (e != hipSuccess) return EPOCH_E_HIP;
  {
    GroupTimer tm(p, st, 2);
    e = launch_place(s, L, W, st);
    tm.done();
  }
  if (e != hipSuccess) return EPOCH_E_HIP;
  // the big tiles depend on the plan step: forked onto the side stream from here
  if (s.big_routed && (hipEventRecord(p->fork_big, st) != hipSuccess ||
                       hipStreamWaitEvent(p->side, p->fork_big, 0) != hipSuccess))
    return EPOCH_E_HIP;
  {
    GroupTimer tm(p, st, 3);
    e = launch_routed_gateup(s, x, w.w1, w.w3, L, W, st);
    tm.done();
  }
  if (e != hipSuccess) return EPOCH_E_HIP;
  if (s.big_routed) {
    GroupTimer tm(p, p->side, 7);
    e = launch_routed_gateup_big(s, x, w.w1, w.w3, L, W, p->side);
    tm.done();
    if (e != hipSuccess) return EPOCH_E_HIP;
  }
  {
    GroupTimer tm(p, st, 4);
    e = launch_routed_down(s, w.w2, L, W, st);
    tm.done();
  }
  if (e != hipSuccess) return EPOCH_E_HIP;
  if (s.big_routed) {
    GroupTimer tm(p, p->side, 8);
    e = launch_routed_down_big(s, w.w2, L, W, p->side);
    tm.done();
    if (e != hipSuccess) return EPOCH_E_HIP;
  }
  if (p->side) {
    if (hipEventRecord(p->join, p->side) != hipSuccess ||
        hipStreamWaitEvent(st, p->join, 0) != hipSuccess)
      return EPOCH_E_HIP;
    p->joined = true;
  }
  {
    GroupTimer tm(p, st, 6);
    e = launch_combine(s, p->iter[layer], L, W, y, y_routed, st);
    tm.done();
  }
  if (e != hipSuccess) return EPOCH_E_HIP;
  p->pending[layer] = 1;
  p->last_layer = layer;
  return EPOCH_OK;
}

int32_t epoch_cache_update(epoch_plan* p, int32_t layer, void* stream) {
  if (!p) return EPOCH_E_NULL;
  if (layer < 0 || layer >= p->d.n_layers) return EPOCH_E_LAYER;
  if (!p->pending[layer]) return EPOCH_E_STATE;
  (void)stream;  // the forward already wrote the committed state into the next copy
  p->parity[layer] ^= 1;
  p->pending[layer] = 0;
  p->iter[layer] += 1;
  return EPOCH_OK;
}

int32_t epoch_plan_inspect(const epoch_plan* p, int32_t layer, epoch_inspect* out) {
  if (!p || !out) return EPOCH_E_NULL;
  if (layer < 0 || layer >= p->d.n_layers) return EPOCH_E_LAYER;
  const Scratch& W = p->lay.scratch;
  const LayerState L = state_now(p, layer);
  std::memset(out, 0, sizeof(*out));
  out->logits = W.G;
  out->ids = W.ids;
  out->scores = W.scores;
  out->atlas_q = W.q;
  out->weights = W.w;
  out->fresh = L.fresh;
  out->fresh_list = W.fresh_list;
  out->n_fresh = W.flags + FLAG_NFRESH;
  out->n_pairs = W.flags + FLAG_NPAIRS;
  out->wl_pos = W.wl_pos;
  out->wl_k = W.wl_k;
  out->wl_w = W.wl_w;
  out->offs = W.offs;
  out->inv = W.inv;
  out->routed_ids = W.routed_ids;
  out->routed_w = W.routed_w;
  out->in_support = L.inS;
  out->slot_of = L.slot_of;
  out->support = L.S_list;
  out->support_size = L.S_size;
  out->atlas = L.inA;
  out->cache = L.cache;
  out->valid = L.valid;
  out->last_fresh = L.last_fresh;
  out->prev_decoded = L.prev_D;
  out->counters = L.counters;
  out->k_ext = p->s.Kext;
  out->iteration = p->iter[layer];
  out->last_forward_layer = p->last_layer;
  return EPOCH_OK;
}

int32_t epoch_block_plan_destroy(epoch_plan* p) {
  if (!p) return EPOCH_OK;
  for (auto& tp : p->pairs) {
    (void)hipEventSynchronize(tp.b);
    pool_release(tp.a);
    pool_release(tp.b);
  }
  // the side stream is the device's; the plan's last work on it precedes its join event
  if (p->joined) (void)hipEventSynchronize(p->join);
  if (p->fork) (void)hipEventDestroy(p->fork);
  if (p->fork_big) (void)hipEventDestroy(p->fork_big);
  if (p->join) (void)hipEventDestroy(p->join);
  delete p;
  return EPOCH_OK;
}

const char* epoch_status_string(int32_t status) {
  switch (status) {
    case EPOCH_OK: return "ok";
    case EPOCH_E_NULL: return "a required pointer is NULL";
    case EPOCH_E_SHAPE: return "descriptor value out of the supported range";
    case EPOCH_E_DTYPE: return "unknown dtype or gate";
    case EPOCH_E_WORKSPACE: return "workspace too small or misaligned";
    case EPOCH_E_LAYER: return "layer index out of range";
    case EPOCH_E_STATE: return "commit without a preceding forward of that layer";
    case EPOCH_E_HIP: return "a kernel launch failed";
    case EPOCH_E_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case EPOCH_E_SCRATCH:
      return "the shape needs more scratch than the library's static device array holds";
    default: return "unknown status";
  }
}

int32_t epoch_plan_set_timing(epoch_plan* p, int32_t enabled) {
  if (!p) return EPOCH_E_NULL;
  p->timing_mask = static_cast<uint32_t>(enabled) & ((1u << EPOCH_TIMING_GROUPS) - 1u);
  for (int g = 0; g < EPOCH_TIMING_GROUPS; ++g) {
    p->ms[g] = 0.0;
    p->launches[g] = 0;
  }
  return EPOCH_OK;
}

int32_t epoch_plan_timing(epoch_plan* p, float* ms, int64_t* launches, int32_t n) {
  if (!p) return EPOCH_E_NULL;
  for (auto& tp : p->pairs) {
    if (hipEventSynchronize(tp.b) != hipSuccess) return EPOCH_E_HIP;
    float dt = 0.f;
    if (hipEventElapsedTime(&dt, tp.a, tp.b) != hipSuccess) return EPOCH_E_HIP;
    p->ms[tp.group] += dt;
    p->launches[tp.group] += 1;
    pool_release(tp.a);
    pool_release(tp.b);
  }
  p->pairs.clear();
  for (int g = 0; g < std::min<int>(n, EPOCH_TIMING_GROUPS); ++g) {
    if (ms) ms[g] = (float)p->ms[g];
    if (launches) launches[g] = p->launches[g];
  }
  return EPOCH_OK;
}

}  // extern "C"
