// Live-only output decoding of one refinement step (gfx950): the LM-head logits of the live
// positions only, their top token and confidence, and the threshold commit that produces the
// next decoded mask (teardown, evaluation setup: greedy threshold decoding with commit
// threshold tau = 0.95, at most 64 refinement steps per block, early exit; LSP section: only
// live positions reach the output decoding, and a position's commit / no-commit decision
// depends on its live logits).
//
// Five launches, no host synchronisation:
//   k_live_compact  one workgroup: the live positions (D = 0) in ascending order, their count,
//                   and each position's index in that list;
//   k_expert_stream LM-head mode, when at most kLmStreamMaxRows positions are live: the
//                   vocabulary streamed through LDS once, 256 or 128 tokens per work item,
//                   the epilogue reducing each row's logits of a work item to (max, argmax,
//                   sum exp), the item's waves combined in LDS;
//   k_lm_head_w4    when more are live: tiles of 256 live rows x 256 tokens on the compute-bound
//                   MFMA tiles, one workgroup per CU walking its tiles with the next tile's
//                   first chunks copied during the current one's last chunks and epilogue, one
//                   (max, argmax, sum exp) per row and 256-token block (the tile's two column
//                   waves combined in LDS);
//   k_decode_rows   one workgroup per position: the partials of each live row combined in double
//                   (confidence = 1 / sum_v exp(z_v - z_max)) with its top token;
//   k_decode_final  one workgroup per sequence: the commits.
// The live count is known on the device only, so both LM-head kernels are launched and the one
// that does not own it exits at once (the compute-bound one is not launched for batches of at
// most kLmStreamMaxRows positions).
#include "device_common.h"
#include "epoch_internal.h"
#include "expert_gemm.h"
#include "lm_head.h"

#include <mutex>
#include <new>

namespace epoch {

constexpr int kCompactThreads = 1024;
// the streamed LM head: one 128-row tile (a single pass over the vocabulary, its rows streamed
// with the non-temporal policy), eight waves of 32 tokens with three chunk buffers (3 x 48 KB
// of LDS, two chunks in flight), or four waves with four (4 x 32 KB) when the vocabulary has
// fewer 256-token blocks than the device has CUs
constexpr int kLmStreamBuffers = 3;
constexpr int kLmStreamBuffers4 = 4;
constexpr int kLmStreamTileRows = 128;
static_assert(kLmStreamTileRows >= kLmStreamMaxRows, "one pass over the vocabulary");
// beyond kLmStreamMaxRows live rows: compute-bound tiles of 256 live rows x 256 tokens
// (k_lm_head_w4: four waves of 128 x 128 outputs, one workgroup per CU)
constexpr int kLmBigTileCols = 256;

__global__ __launch_bounds__(kCompactThreads) void k_live_compact(int M,
                                                                  const uint8_t* __restrict__ D,
                                                                  int32_t* __restrict__ live_list,
                                                                  int32_t* __restrict__ live_idx,
                                                                  int32_t* __restrict__ n_live) {
  __shared__ int32_t wcount[kCompactThreads / 64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int carry = 0;
  for (int base = 0; base < M; base += kCompactThreads) {
    const int t = base + tid;
    const bool live = t < M && D[t] == 0;
    const unsigned long long bal = ballot64(live);
    if (lane == 0) wcount[wave] = __popcll(bal);
    __syncthreads();
    int before = carry, total = 0;
    for (int w = 0; w < kCompactThreads / 64; ++w) {
      if (w < wave) before += wcount[w];
      total += wcount[w];
    }
    const int idx = before + __popcll(bal & below);
    if (t < M) live_idx[t] = live ? idx : -1;
    if (live) live_list[idx] = t;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) *n_live = carry;
}

// One workgroup per position: a live position's partials combined in double, the confidence
// of its top token 1 / sum_v exp(z_v - z_max) and that token (the lowest id among equal
// maxima); a decoded position gets confidence -1 and token -1.  The partials are n_p_stream
// per row when the streamed LM head ran (at most kLmStreamMaxRows live), else n_p_big.
template <bool CACHED>
__global__ __launch_bounds__(256) void k_decode_rows(int n_p_stream, int n_p_big,
                                                     const int32_t* __restrict__ n_live,
                                                     const int32_t* __restrict__ live_idx,
                                                     const float* __restrict__ pmax,
                                                     const int32_t* __restrict__ parg,
                                                     const float* __restrict__ psum,
                                                     double* __restrict__ conf_pos,
                                                     int32_t* __restrict__ top_pos) {
  __shared__ float sm[4];
  __shared__ int sa[4];
  __shared__ double sz[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  const int li = live_idx[t];
  if (li < 0) {
    if (threadIdx.x == 0) {
      conf_pos[t] = -1.0;
      top_pos[t] = -1;
    }
    return;
  }
  const int n_p = *n_live <= kLmStreamMaxRows ? n_p_stream : n_p_big;
  const size_t row = (size_t)li * n_p;
  // CACHED (launched for batches of at most kLmStreamMaxRows positions, whose partials the
  // streamed head wrote, 128- or 256-token blocks): up to kRowCache partials per thread stay
  // in registers between the two passes (every vocabulary the call accepts), so the row is
  // read from memory once.  The registers this takes would halve the workgroups per CU of a
  // large batch's launch, so other batches read their (fewer, 256-token) partials twice.
  constexpr int kRowCache = 16;
  const bool cached = CACHED && n_p <= 256 * kRowCache;
  float cm[kRowCache], cs[kRowCache];
  float m = -INFINITY;
  int a = 0x7fffffff;
  if (cached) {
#pragma unroll
    for (int k = 0; k < kRowCache; ++k) {
      const int j = threadIdx.x + 256 * k;
      cm[k] = -INFINITY;
      cs[k] = 0.0f;
      if (j < n_p) {
        cm[k] = pmax[row + j];
        cs[k] = psum[row + j];
        const int pa = parg[row + j];
        if (cm[k] > m || (cm[k] == m && pa < a)) {
          m = cm[k];
          a = pa;
        }
      }
    }
  } else {
    for (int j = threadIdx.x; j < n_p; j += 256) {
      const float pm = pmax[row + j];
      const int pa = parg[row + j];
      if (pm > m || (pm == m && pa < a)) {
        m = pm;
        a = pa;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int oa = __shfl_xor(a, o, 64);
    if (om > m || (om == m && oa < a)) {
      m = om;
      a = oa;
    }
  }
  if (lane == 0) {
    sm[wave] = m;
    sa[wave] = a;
  }
  __syncthreads();
  m = sm[0];
  a = sa[0];
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (sm[w] > m || (sm[w] == m && sa[w] < a)) {
      m = sm[w];
      a = sa[w];
    }
  double z = 0.0;
  if (cached) {
#pragma unroll
    for (int k = 0; k < kRowCache; ++k)
      if (threadIdx.x + 256 * k < n_p) z += (double)cs[k] * exp((double)cm[k] - (double)m);
  } else {
    for (int j = threadIdx.x; j < n_p; j += 256)
      z += (double)psum[row + j] * exp((double)pmax[row + j] - (double)m);
  }
  z = wave_sum(z);
  if (lane == 0) sz[wave] = z;
  __syncthreads();
  if (threadIdx.x == 0) {
    conf_pos[t] = 1.0 / (((sz[0] + sz[1]) + sz[2]) + sz[3]);
    top_pos[t] = a;
  }
}

// One workgroup per sequence (block positions): the commit rule.  Every live position with
// confidence >= tau commits, and a sequence none of whose live positions reaches tau commits
// its most confident one (lower position on ties).
__global__ __launch_bounds__(256) void k_decode_final(int block, double tau,
                                                      const uint8_t* __restrict__ D,
                                                      const double* __restrict__ conf_pos,
                                                      const int32_t* __restrict__ top_pos,
                                                      uint8_t* __restrict__ D_next,
                                                      int32_t* __restrict__ tokens,
                                                      float* __restrict__ conf_out) {
  extern __shared__ double conf_s[];  // [block], then int top_s[block]
  int32_t* top_s = reinterpret_cast<int32_t*>(conf_s + block);
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int p = threadIdx.x; p < block; p += blockDim.x) {
    conf_s[p] = conf_pos[(size_t)b * block + p];
    top_s[p] = top_pos[(size_t)b * block + p];
  }
  __syncthreads();
  int hit = 0;
  for (int p = threadIdx.x; p < block; p += blockDim.x) hit |= conf_s[p] >= tau;
  const bool any = __syncthreads_or(hit) != 0;
  // most confident live position (wave 0), used only when none reaches tau
  __shared__ int fallback;
  if (wave == 0) {
    double bc = -1.0;
    int bp = -1;
    for (int p = lane; p < block; p += 64)
      if (conf_s[p] > bc) {  // ascending p per lane: the first maximum is the lowest position
        bc = conf_s[p];
        bp = p;
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double oc = __shfl_xor(bc, o, 64);
      const int op = __shfl_xor(bp, o, 64);
      if (oc > bc || (oc == bc && op >= 0 && (bp < 0 || op < bp))) {
        bc = oc;
        bp = op;
      }
    }
    if (lane == 0) fallback = bc >= 0.0 ? bp : -1;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < block; p += blockDim.x) {
    const int t = b * block + p;
    const bool live = top_s[p] >= 0;
    const bool commit = live && (any ? conf_s[p] >= tau : p == fallback);
    D_next[t] = (D[t] || commit) ? 1 : 0;
    if (commit) tokens[t] = top_s[p];
    if (conf_out) conf_out[t] = live ? (float)conf_s[p] : 0.0f;
  }
}

namespace {

struct DecodeLayout {
  int32_t *live_list, *live_idx, *n_live, *parg, *top_pos;
  float *pmax, *psum;
  double* conf_pos;
  size_t bytes;
};

// The partials hold the streamed LM head's (at most kLmStreamMaxRows rows of vocab / 128
// blocks at most) or the compute-bound tiles' (all M rows of vocab / 256 blocks, rounded up).
DecodeLayout decode_carve(const epoch_decode_desc* d, void* base) {
  const size_t M = (size_t)d->batch * d->block;
  const size_t n_stream = (M < (size_t)kLmStreamMaxRows ? M : (size_t)kLmStreamMaxRows) *
                          ((size_t)d->vocab / 128);
  const size_t n_big = M * (((size_t)d->vocab + kLmBigTileCols - 1) / kLmBigTileCols);
  const size_t n_part = n_stream > n_big ? n_stream : n_big;
  size_t off = 0;
  char* b = static_cast<char*>(base);
  auto take = [&](size_t n) {
    off = (off + 255) / 256 * 256;
    void* p = b ? b + off : nullptr;
    off += n;
    return p;
  };
  DecodeLayout L;
  L.live_list = static_cast<int32_t*>(take(M * 4));
  L.live_idx = static_cast<int32_t*>(take(M * 4));
  L.n_live = static_cast<int32_t*>(take(4));
  L.pmax = static_cast<float*>(take(n_part * 4));
  L.parg = static_cast<int32_t*>(take(n_part * 4));
  L.psum = static_cast<float*>(take(n_part * 4));
  L.conf_pos = static_cast<double*>(take(M * 8));
  L.top_pos = static_cast<int32_t*>(take(M * 4));
  L.bytes = (off + 255) / 256 * 256;
  return L;
}

int32_t check_decode_desc(const epoch_decode_desc* d) {
  if (!d) return EPOCH_E_NULL;
  if (d->act_dtype != EPOCH_DTYPE_BF16) return EPOCH_E_DTYPE;
  if (d->flags != 0) return EPOCH_E_SHAPE;
  if (d->batch < 1 || d->block < 1 || d->block > 1024) return EPOCH_E_SHAPE;
  if ((long long)d->batch * d->block > (1 << 20)) return EPOCH_E_SHAPE;
  if (d->hidden < 64 || d->hidden % 64 || d->hidden > 16384) return EPOCH_E_SHAPE;
  if (d->vocab < 128 || d->vocab % 128 || d->vocab > (1 << 20)) return EPOCH_E_SHAPE;
  if (!(d->tau > 0.0 && d->tau <= 1.0)) return EPOCH_E_SHAPE;
  return EPOCH_OK;
}

int32_t check_decode_args(const epoch_decode_desc* d, const void* h, const void* w_vocab,
                          const uint8_t* decoded, const uint8_t* decoded_next,
                          const int32_t* tokens) {
  const int32_t rc = check_decode_desc(d);
  if (rc) return rc;
  if (!h || !w_vocab || !decoded || !decoded_next || !tokens) return EPOCH_E_NULL;
  if ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(w_vocab)) & 15u)
    return EPOCH_E_ALIGN;
  return EPOCH_OK;
}

// The launch sequence of one decoding step on the buffers of L.  Every scratch buffer is
// written before it is read (live list and index for all M positions, partials for the live
// rows the row kernel reads, confidences and tokens for all positions), so nothing needs to
// start at zero and a scratch area that holds an earlier call's contents is fine.
int32_t decode_enqueue(const epoch_decode_desc* d, const void* h, const void* w_vocab,
                       const uint8_t* decoded, uint8_t* decoded_next, int32_t* tokens, float* conf,
                       const DecodeLayout& L, hipStream_t st) {
  const int M = d->batch * d->block;
  launch(k_live_compact, dim3(1), dim3(kCompactThreads), 0, st, M, decoded,
                     L.live_list, L.live_idx, L.n_live);
  // the streamed head's partials: one per row and work item (256 or 128 tokens)
  int n_p = 0;
  // few live rows: the streamed LM head, one workgroup per CU walking token blocks
  // blockIdx.x + j gridDim.x (256 tokens, or 128 when that is needed to give every CU one)
  {
    const int n_cu = device_cu_count();
    const uint16_t* hb = static_cast<const uint16_t*>(h);
    const uint16_t* wv = static_cast<const uint16_t*>(w_vocab);
    if (d->vocab / 256 < n_cu) {
      const int n_cb = d->vocab / 128;
      n_p = n_cb;
      const LmPartials lp{L.live_list, L.n_live, L.pmax, L.parg, L.psum, n_p};
      launch((k_expert_stream<false, false, kLmStreamBuffers4, 4, kLmStreamTileRows, true>),
             dim3(n_cb < n_cu ? n_cb : n_cu), dim3(256), 0, st, hb, wv, nullptr, nullptr, nullptr,
             nullptr, nullptr, nullptr, L.live_list, nullptr, nullptr, M, d->hidden, d->vocab, lp);
    } else {
      const int n_cb = (d->vocab + 255) / 256;  // the last block may be half (vocab % 256 = 128)
      n_p = n_cb;
      const LmPartials lp{L.live_list, L.n_live, L.pmax, L.parg, L.psum, n_p};
      launch((k_expert_stream<false, false, kLmStreamBuffers, 8, kLmStreamTileRows, true>),
             dim3(n_cb < n_cu ? n_cb : n_cu), dim3(512), 0, st, hb, wv, nullptr, nullptr, nullptr,
             nullptr, nullptr, nullptr, L.live_list, nullptr, nullptr, M, d->hidden, d->vocab, lp);
    }
  }
  // one workgroup per CU, eight per XCD group (a walk per XCD); blocks of kLmBigTileCols tokens
  // (the last one half when the vocabulary is an odd multiple of 128)
  // (not launched when the batch has no more positions than the streamed head takes)
  const int n_cb = (d->vocab + kLmBigTileCols - 1) / kLmBigTileCols;
  const LmPartials lp_big{L.live_list, L.n_live, L.pmax, L.parg, L.psum, n_cb};
  if (M > kLmStreamMaxRows)
    launch(k_lm_head_w4, dim3(lm_head_grid(device_cu_count())), dim3(256), 0, st,
           static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(w_vocab), d->hidden,
           d->vocab, lp_big);
  const size_t lds = (size_t)d->block * (sizeof(double) + sizeof(int32_t));
  if (M <= kLmStreamMaxRows)
    launch(k_decode_rows<true>, dim3(M), dim3(256), 0, st, n_p, n_cb, L.n_live, L.live_idx,
           L.pmax, L.parg, L.psum, L.conf_pos, L.top_pos);
  else
    launch(k_decode_rows<false>, dim3(M), dim3(256), 0, st, n_p, n_cb, L.n_live, L.live_idx,
           L.pmax, L.parg, L.psum, L.conf_pos, L.top_pos);
  launch(k_decode_final, dim3(d->batch), dim3(256), lds, st, d->block, d->tau, decoded,
         L.conf_pos, L.top_pos, decoded_next, tokens, conf);
  return hipGetLastError() == hipSuccess ? EPOCH_OK : EPOCH_E_HIP;
}

// Scratch of epoch_live_decode_static, for callers that cannot allocate device memory: one
// array per device, kept by the loaded library until the process ends.  Host code never uses
// the array's name as an address (on the host it names a stand-in, not device memory); it uses
// the device address looked up below.
constexpr size_t kDecodeStaticScratchBytes = EPOCH_DECODE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

// The device address of `scratch` on the current device, looked up once per device (the first
// static call on it) and kept; null if the lookup fails.
void* static_scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

}  // namespace
}  // namespace epoch

using namespace epoch;

extern "C" {

int32_t epoch_decode_workspace_bytes(const epoch_decode_desc* d, size_t* out_bytes) {
  if (!out_bytes) return EPOCH_E_NULL;
  const int32_t rc = check_decode_desc(d);
  if (rc) return rc;
  *out_bytes = decode_carve(d, nullptr).bytes;
  return EPOCH_OK;
}

int32_t epoch_live_decode(const epoch_decode_desc* d, const void* h, const void* w_vocab,
                          const uint8_t* decoded, uint8_t* decoded_next, int32_t* tokens,
                          float* conf, void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t rc = check_decode_args(d, h, w_vocab, decoded, decoded_next, tokens);
  if (rc) return rc;
  if (!workspace) return EPOCH_E_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return EPOCH_E_WORKSPACE;
  const DecodeLayout L = decode_carve(d, workspace);
  if (workspace_bytes < L.bytes) return EPOCH_E_WORKSPACE;
  return decode_enqueue(d, h, w_vocab, decoded, decoded_next, tokens, conf, L,
                        static_cast<hipStream_t>(stream));
}

int32_t epoch_live_decode_static(const epoch_decode_desc* d, const void* h, const void* w_vocab,
                                 const uint8_t* decoded, uint8_t* decoded_next, int32_t* tokens,
                                 float* conf, void* stream) {
  const int32_t rc = check_decode_args(d, h, w_vocab, decoded, decoded_next, tokens);
  if (rc) return rc;
  if (decode_carve(d, nullptr).bytes > kDecodeStaticScratchBytes) return EPOCH_E_SCRATCH;
  void* base = static_scratch_address();
  if (!base) return EPOCH_E_HIP;
  return decode_enqueue(d, h, w_vocab, decoded, decoded_next, tokens, conf,
                        decode_carve(d, base), static_cast<hipStream_t>(stream));
}

}  // extern "C"
