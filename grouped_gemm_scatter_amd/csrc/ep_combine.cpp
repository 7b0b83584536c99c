// Host side of the C ABI declared in include/ep_combine.h: argument
// validation, handle state, tile-configuration choice and kernel launches.
// No device memory is allocated here; every buffer belongs to the caller,
// except the small library-held counter array of the allocation-free GEMM
// entry point below.
#include "ep_combine.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>

#include "combine_common.h"
#include "ep_kernels.h"

// Counters of ep_grouped_gemm_scatter_noalloc: R election counters, then E_l
// per-expert tile counters (the roles of ep_combine_buffers.rank_counter and
// .tile_counter), at most EP_MAX_RANKS + EP_MAX_LOCAL_EXPERTS words.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code this name is not a device address: kernels and copies get the address
// that hipGetSymbolAddress returned for the current device (scratch_on()).
constexpr int kScratchWords = EP_MAX_RANKS + EP_MAX_LOCAL_EXPERTS;
static __device__ __align__(256) int32_t scratch[kScratchWords];

struct ep_combine_handle {
  ep_combine_params p;
  ep_combine_buffers b;
  int device;
  int num_cus;
  int tile;                 // ep::GemmTile used for this geometry
};

namespace {

constexpr int64_t kDefaultSpinLimit = int64_t(1) << 22;

// Device address of `scratch` on each device, looked up once per device by
// ep_combine_init with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch[kMaxDevices];

// Looks up (once) the address of `scratch` on device `dev`, which must be the
// current device.  Returns EP_OK or EP_ERR_HIP.
int resolve_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return EP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return EP_OK;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EP_ERR_HIP;
  g_scratch[dev] = static_cast<int32_t*>(p);
  return EP_OK;
}

int32_t* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch[dev];
}

// Zeroes n words (a kernel, not a memset node: callers may capture the
// allocation-free entry point in a graph).
__global__ void zero_words_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}
// at most this many rows per local expert on average: bf16 GEMMs use the
// decode tile below
constexpr int kDecodeRowsPerExpert = 48;
constexpr int kDecodeTile = ep::kTileDecode64x128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_params(const ep_combine_params* p) {
  if (!p) return EP_ERR_INVALID_ARG;
  if (p->n_ranks < 1 || p->n_ranks > EP_MAX_RANKS) return EP_ERR_INVALID_ARG;
  // Only ranks reachable by direct stores are supported (no SHMEM path).
  if (p->p2p_world_size != p->n_ranks) return EP_ERR_UNSUPPORTED;
  if (p->my_rank < 0 || p->my_rank >= p->n_ranks) return EP_ERR_INVALID_ARG;
  if (p->top_k < 1 || p->top_k > 64) return EP_ERR_INVALID_ARG;
  if (p->n_experts_per_device < 1 || p->n_experts_per_device > EP_MAX_LOCAL_EXPERTS)
    return EP_ERR_INVALID_ARG;
  if (p->max_tokens_per_rank < 1) return EP_ERR_INVALID_ARG;
  if (p->hidden_k < 1 || p->hidden_n < 1) return EP_ERR_INVALID_ARG;
  if (p->msg_bytes < 2 * p->hidden_n || p->msg_bytes % 16) return EP_ERR_INVALID_ARG;
  if (p->hidden_n % 128) return EP_ERR_UNSUPPORTED;
  if (p->dtype == EP_DTYPE_BF16) {
    if (p->hidden_k % 64) return EP_ERR_UNSUPPORTED;
  } else if (p->dtype == EP_DTYPE_FP8_E4M3_B128) {
    if (p->hidden_k % 128) return EP_ERR_UNSUPPORTED;
  } else {
    return EP_ERR_UNSUPPORTED;
  }
  if (p->flags &
      ~uint32_t(EP_FLAG_SYSTEM_SCOPE | EP_FLAG_PER_EXPERT_RELEASE | EP_FLAG_EPILOGUE_ONLY |
                EP_FLAG_TRACE | EP_FLAG_W_SLICE_MAJOR | EP_FLAG_DEVICE_EPOCH |
                EP_FLAG_SEND_TILE))
    return EP_ERR_INVALID_ARG;
  if ((p->flags & EP_FLAG_W_SLICE_MAJOR) && p->dtype != EP_DTYPE_BF16) return EP_ERR_UNSUPPORTED;
  if (p->send_waves != 0 && p->send_waves != 4) return EP_ERR_INVALID_ARG;
  if (p->send_waves || (p->flags & EP_FLAG_SEND_TILE)) {
    // the send-wave kernel: bf16, no measurement modes
    if (p->dtype != EP_DTYPE_BF16) return EP_ERR_UNSUPPORTED;
    if (p->flags & (EP_FLAG_EPILOGUE_ONLY | EP_FLAG_TRACE)) return EP_ERR_UNSUPPORTED;
  }
  if (p->flag_spin_limit < 0) return EP_ERR_INVALID_ARG;
  // 32-bit element offsets inside the kernels
  const uint64_t wbytes = uint64_t(p->n_experts_per_device) * p->hidden_n * p->hidden_k *
                          (p->dtype == EP_DTYPE_BF16 ? 2 : 1);
  if (wbytes >= (uint64_t(1) << 32)) return EP_ERR_UNSUPPORTED;
  return EP_OK;
}

ep::SinkState sink_state(const ep_combine_handle* h, uint64_t epoch) {
  ep::SinkState s{};
  for (int i = 0; i < EP_MAX_RANKS; ++i)
    s.recv[i] = i < h->p.n_ranks ? static_cast<uint8_t*>(h->b.recv_buf[i]) : nullptr;
  s.words = h->b.recv_count;
  s.rank_counter = h->b.rank_counter;
  s.tile_counter = h->b.tile_counter;
  s.err = h->b.error_word;
  s.epoch_ptr = (h->p.flags & EP_FLAG_DEVICE_EPOCH) ? h->b.epoch_word : nullptr;
  s.epoch = epoch;
  s.n_ranks = h->p.n_ranks;
  s.n_experts = h->p.n_experts_per_device;
  s.top_k = h->p.top_k;
  s.msg_bytes = h->p.msg_bytes;
  s.max_tokens = h->p.max_tokens_per_rank;
  s.system_scope = (h->p.flags & EP_FLAG_SYSTEM_SCOPE) ? 1 : 0;
  s.per_expert = (h->p.flags & EP_FLAG_PER_EXPERT_RELEASE) ? 1 : 0;
  return s;
}

// A step's epoch is nonzero.  With per-expert completion the count words
// carry its low 32 bits as their tag and start out zero, so those bits must be
// nonzero as well (epochs then only need to differ modulo 2^32).  A handle
// that keeps the epoch in device memory takes 0 here: the kernels read the word.
bool epoch_ok(const ep_combine_handle* h, uint64_t epoch) {
  if (h->p.flags & EP_FLAG_DEVICE_EPOCH) return epoch == 0;
  if (epoch == 0) return false;
  if ((h->p.flags & EP_FLAG_PER_EXPERT_RELEASE) && (epoch & 0xffffffffull) == 0) return false;
  return true;
}

// Checks and fills the consumer combine's arguments (ep_combine_reduce and the
// consumer side of ep_grouped_gemm_scatter_combine).  tokens_per_rank > 0.
int combine_args(const ep_combine_handle* h, const int32_t* topk_ids, const float* topk_w,
                 int32_t tokens_per_rank, void* out, uint64_t epoch, ep::CombineArgs* a) {
  if (!topk_ids || !topk_w || !out || !aligned16(out)) return EP_ERR_INVALID_ARG;
  *a = ep::CombineArgs{};
  a->topk_ids = topk_ids;
  a->topk_w = topk_w;
  a->out = static_cast<uint8_t*>(out);
  a->flags = h->b.recv_count + size_t(h->p.n_experts_per_device) * h->p.n_ranks;
  for (int i = 0; i < EP_MAX_RANKS; ++i)
    a->recv[i] = i < h->p.n_ranks ? static_cast<uint8_t*>(h->b.recv_buf[i]) : nullptr;
  a->err = h->b.error_word;
  a->epoch = epoch;
  a->epoch_ptr = (h->p.flags & EP_FLAG_DEVICE_EPOCH) ? h->b.epoch_word : nullptr;
  a->spin_limit = h->p.flag_spin_limit;
  a->n_ranks = h->p.n_ranks;
  a->tokens = tokens_per_rank;
  a->top_k = h->p.top_k;
  a->N = h->p.hidden_n;
  a->msg_bytes = h->p.msg_bytes;
  a->expert_lo = h->p.my_rank * h->p.n_experts_per_device;
  a->n_experts = h->p.n_experts_per_device;
  a->system_scope = (h->p.flags & EP_FLAG_SYSTEM_SCOPE) ? 1 : 0;
  a->per_expert = (h->p.flags & EP_FLAG_PER_EXPERT_RELEASE) ? 1 : 0;
  a->words = h->b.recv_count;
  return EP_OK;
}

int pick_tile(const ep_combine_params* p) {
  if (p->dtype == EP_DTYPE_FP8_E4M3_B128)
    return (p->hidden_n % 256 == 0) ? ep::kTile256x256 : ep::kTile256x128;
  if (p->send_waves) return ep::kTileSend128x128;
  if (p->flags & EP_FLAG_SEND_TILE) return ep::kTileSendNone128x128;
  return (p->hidden_n % 256 == 0) ? ep::kTile256x256 : ep::kTile128x128;
}

// Tile of one grouped-GEMM call: small row groups (decode: a few dozen rows
// per local expert) stream W_e with the decode tile, which keeps several K
// slices in flight.
int call_tile(const ep_combine_handle* h, int32_t m_total) {
  const bool fp8 = h->p.dtype == EP_DTYPE_FP8_E4M3_B128;
  return (!fp8 && h->tile == ep::kTile256x256 &&
          int64_t(m_total) <= int64_t(kDecodeRowsPerExpert) * h->p.n_experts_per_device)
             ? kDecodeTile
             : h->tile;
}

}  // namespace

extern "C" {

int ep_combine_version(void) { return 100; }

const char* ep_combine_strerror(int code) {
  switch (code) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument";
    case EP_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_ERR_SLOT_OOB: return "device: receive slot out of bounds";
    case EP_ERR_FLAG_TIMEOUT: return "device: timed out waiting for a rank flag";
    case EP_ERR_BAD_GROUP: return "device: inconsistent group offsets or signal coordinates";
    default: return code > 0 ? "device: several error bits" : "unknown error";
  }
}

int ep_combine_init(const ep_combine_params* params, const ep_combine_buffers* bufs,
                    ep_combine_t* out) {
  if (!out) return EP_ERR_INVALID_ARG;
  *out = nullptr;
  int rc = validate_params(params);
  if (rc != EP_OK) return rc;
  if (!bufs || !bufs->recv_count || !bufs->rank_counter || !bufs->tile_counter ||
      !bufs->error_word)
    return EP_ERR_INVALID_ARG;
  for (int i = 0; i < params->n_ranks; ++i)
    if (!bufs->recv_buf[i] || !aligned16(bufs->recv_buf[i])) return EP_ERR_INVALID_ARG;
  if ((params->flags & EP_FLAG_TRACE) &&
      (!bufs->trace || !aligned16(bufs->trace) || bufs->trace_records <= 0))
    return EP_ERR_INVALID_ARG;
  if ((params->flags & EP_FLAG_DEVICE_EPOCH) &&
      (!bufs->epoch_word || reinterpret_cast<uintptr_t>(bufs->epoch_word) % 8))
    return EP_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return EP_ERR_HIP;
  // the allocation-free GEMM's counters on this device; a failed lookup only
  // makes that one entry point unavailable (it then returns EP_ERR_HIP)
  (void)resolve_scratch(dev);
  auto* h = new (std::nothrow) ep_combine_handle;
  if (!h) return EP_ERR_INVALID_ARG;
  h->p = *params;
  if (h->p.flag_spin_limit == 0) h->p.flag_spin_limit = kDefaultSpinLimit;
  h->b = *bufs;
  h->device = dev;
  h->num_cus = cus > 0 ? cus : 256;
  h->tile = pick_tile(params);
  *out = h;
  return EP_OK;
}

void ep_combine_destroy(ep_combine_t h) { delete h; }

}  // extern "C"

namespace {

// ep_grouped_gemm_scatter with its election and tile counters at
// rank_counter / tile_counter (the caller's, or the library's scratch).
int gemm_scatter(ep_combine_t h, const void* x, const void* w, const float* x_scale,
                 const float* w_scale, const int32_t* offsets, const int32_t* src_info,
                 int32_t m_total, int32_t p3_control, void* c_local, uint64_t epoch,
                 void* stream, int32_t* rank_counter, int32_t* tile_counter,
                 const ep::CombineArgs* comb = nullptr) {
  if (!h || !w || !offsets) return EP_ERR_INVALID_ARG;
  if (m_total < 0) return EP_ERR_INVALID_ARG;
  if (m_total > 0 && (!x || !src_info)) return EP_ERR_INVALID_ARG;
  const bool sink_on = p3_control >= 0;
  if (!sink_on && m_total > 0 && (!c_local || !aligned16(c_local))) return EP_ERR_INVALID_ARG;
  if (sink_on && !epoch_ok(h, epoch)) return EP_ERR_INVALID_ARG;
  const bool fp8 = h->p.dtype == EP_DTYPE_FP8_E4M3_B128;
  if (fp8 && ((m_total > 0 && !x_scale) || !w_scale)) return EP_ERR_INVALID_ARG;
  const int elt = fp8 ? 1 : 2;
  if (uint64_t(m_total) * h->p.hidden_k * elt >= (uint64_t(1) << 32)) return EP_ERR_UNSUPPORTED;
  if ((x && !aligned16(x)) || !aligned16(w)) return EP_ERR_INVALID_ARG;

  ep::GemmArgs a{};
  a.x = static_cast<const uint8_t*>(x);
  a.w = static_cast<const uint8_t*>(w);
  a.x_scale = x_scale;
  a.w_scale = w_scale;
  a.offsets = offsets;
  a.src_info = src_info;
  a.c_local = static_cast<uint8_t*>(c_local);
  a.m_total = m_total;
  a.K = h->p.hidden_k;
  a.N = h->p.hidden_n;
  a.sink_on = sink_on ? 1 : 0;
  a.epilogue_only = (h->p.flags & EP_FLAG_EPILOGUE_ONLY) ? 1 : 0;
  a.w_slice_major = (h->p.flags & EP_FLAG_W_SLICE_MAJOR) ? 1 : 0;
  a.s = sink_state(h, epoch);
  a.s.rank_counter = rank_counter;
  a.s.tile_counter = tile_counter;
  if ((h->p.flags & EP_FLAG_TRACE) && !a.epilogue_only) {
    a.trace = h->b.trace;
    a.trace_records = h->b.trace_records;
  }

  const int El = h->p.n_experts_per_device;
  const int tile = call_tile(h, m_total);
  const int bm = ep::gemm_tile_rows(tile), bn = ep::gemm_tile_cols(tile);
  const int64_t nt = h->p.hidden_n / bn;
  const int64_t items = (int64_t(m_total) / bm + El) * nt + El;     // upper bound
  const int64_t resident = int64_t(h->num_cus) * ep::gemm_blocks_per_cu(tile);
  int64_t grid = std::min(items, resident);
  grid = (grid + 7) / 8 * 8;
  if (comb) {
    // fused launch: every workgroup turns consumer after its tiles, and a
    // consumer waits for workgroups that are still producing, so the whole grid
    // must be resident at once: at most `resident` workgroups, a multiple of 8
    if (a.epilogue_only || a.trace || !sink_on || tile >= ep::kTileSend128x128)
      return EP_ERR_UNSUPPORTED;
    grid = std::max<int64_t>(8, resident / 8 * 8);   // the launcher sizes it from occupancy
    a.fused = 1;
    a.num_cus = h->num_cus;
    a.comb = *comb;
    int tpr = 0, rpr = 0;
    // about four runs per workgroup
    ep::combine_split(comb->n_ranks, comb->tokens, 4 * grid, &tpr, &rpr);
    a.comb_tokens_per_run = tpr;
    a.comb_runs_per_rank = rpr;
    a.comb_chunks = ep::combine_chunks(comb->N);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = fp8 ? ep::launch_gemm_fp8(a, tile, int(grid), st)
                  : tile >= ep::kTileSend128x128
                      ? ep::launch_gemm_send(a, tile == ep::kTileSend128x128 ? 4 : 0, int(grid), st)
                      : ep::launch_gemm_bf16(a, tile, int(grid), st);
  return err == hipSuccess ? EP_OK : (err == hipErrorNotSupported ? EP_ERR_UNSUPPORTED : EP_ERR_HIP);
}

}  // namespace

extern "C" {

int ep_grouped_gemm_scatter(ep_combine_t h, const void* x, const void* w, const float* x_scale,
                            const float* w_scale, const int32_t* offsets,
                            const int32_t* src_info, int32_t m_total, int32_t p3_control,
                            void* c_local, uint64_t epoch, void* stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  return gemm_scatter(h, x, w, x_scale, w_scale, offsets, src_info, m_total, p3_control,
                      c_local, epoch, stream, h->b.rank_counter, h->b.tile_counter);
}

int ep_grouped_gemm_scatter_noalloc(ep_combine_t h, const void* x, const void* w,
                                    const float* x_scale, const float* w_scale,
                                    const int32_t* offsets, const int32_t* src_info,
                                    int32_t m_total, int32_t p3_control, void* c_local,
                                    uint64_t epoch, void* stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  const int R = h->p.n_ranks, El = h->p.n_experts_per_device;
  if (R > EP_MAX_RANKS || El > EP_MAX_LOCAL_EXPERTS || R + El > kScratchWords)
    return EP_ERR_UNSUPPORTED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
  int32_t* ws = scratch_on(dev);
  if (!ws) return EP_ERR_HIP;        // no handle was initialised on this device
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p3_control >= 0) {
    // the counters start each call at zero, whatever an earlier call left
    const int n = R + El;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, st, ws, n);
    if (hipGetLastError() != hipSuccess) return EP_ERR_HIP;
  }
  return gemm_scatter(h, x, w, x_scale, w_scale, offsets, src_info, m_total, p3_control,
                      c_local, epoch, stream, ws, ws + R);
}

int ep_gemm_tile(ep_combine_t h, int32_t m_total, int32_t* tile_rows, int32_t* tile_cols) {
  if (!h || m_total < 0 || !tile_rows || !tile_cols) return EP_ERR_INVALID_ARG;
  const int tile = call_tile(h, m_total);
  const bool fp8 = h->p.dtype == EP_DTYPE_FP8_E4M3_B128;
  // the bf16 256-column tile takes up to nine 32-row blocks (rows spread
  // evenly over an expert's tiles)
  *tile_rows = (!fp8 && tile == ep::kTile256x256) ? 288 : ep::gemm_tile_rows(tile);
  *tile_cols = ep::gemm_tile_cols(tile);
  return tile;
}

int ep_group_local_picks(ep_combine_t h, const int32_t* topk_ids, int32_t tokens_per_rank,
                         int32_t* offsets, int32_t* src_info, void* stream) {
  if (!h || !offsets) return EP_ERR_INVALID_ARG;
  if (tokens_per_rank < 0 || tokens_per_rank > h->p.max_tokens_per_rank) return EP_ERR_INVALID_ARG;
  if (tokens_per_rank > 0 && (!topk_ids || !src_info)) return EP_ERR_INVALID_ARG;
  const int R = h->p.n_ranks, El = h->p.n_experts_per_device;
  // row indices and src_info word offsets stay in 32 bits
  if (int64_t(2) * R * tokens_per_rank * h->p.top_k >= (int64_t(1) << 31)) return EP_ERR_UNSUPPORTED;
  ep::GroupArgs a{};
  a.topk_ids = topk_ids;
  a.offsets = offsets;
  a.src_info = src_info;
  a.n_ranks = R;
  a.n_experts = El;
  a.expert_lo = h->p.my_rank * El;
  a.tokens = tokens_per_rank;
  a.top_k = h->p.top_k;
  const hipError_t err = ep::launch_grouping(a, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_dispatch_rows(ep_combine_t h, const void* tokens_x, int32_t tokens_per_rank,
                     int32_t row_bytes, const int32_t* offsets, const int32_t* src_info,
                     int32_t m_total, void* x_out, void* stream) {
  if (!h || !offsets || m_total < 0) return EP_ERR_INVALID_ARG;
  if (tokens_per_rank < 0 || tokens_per_rank > h->p.max_tokens_per_rank) return EP_ERR_INVALID_ARG;
  if (row_bytes < 16 || row_bytes % 16) return EP_ERR_INVALID_ARG;
  if (m_total == 0) return EP_OK;
  if (!tokens_x || !src_info || !x_out || !aligned16(tokens_x) || !aligned16(x_out))
    return EP_ERR_INVALID_ARG;
  ep::DispatchArgs a{};
  a.tokens_x = static_cast<const uint8_t*>(tokens_x);
  a.offsets = offsets;
  a.src_info = src_info;
  a.x_out = static_cast<uint8_t*>(x_out);
  a.err = h->b.error_word;
  a.m_total = m_total;
  a.row_bytes = row_bytes;
  a.tokens = tokens_per_rank;
  a.n_ranks = h->p.n_ranks;
  a.n_experts = h->p.n_experts_per_device;
  const hipError_t err = ep::launch_dispatch(a, h->num_cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_pack_weights(ep_combine_t h, const void* w, void* w_out, void* stream) {
  if (!h || !w || !w_out || !aligned16(w) || !aligned16(w_out)) return EP_ERR_INVALID_ARG;
  if (h->p.dtype != EP_DTYPE_BF16) return EP_ERR_UNSUPPORTED;
  const uint64_t bytes =
      uint64_t(h->p.n_experts_per_device) * h->p.hidden_n * h->p.hidden_k * 2;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_out);
  if (a < b + bytes && b < a + bytes) return EP_ERR_INVALID_ARG;
  const hipError_t err = ep::launch_pack_slice_major(
      static_cast<const uint8_t*>(w), static_cast<uint8_t*>(w_out), h->p.n_experts_per_device,
      h->p.hidden_n, h->p.hidden_k, h->num_cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_grouped_gemm_swiglu(ep_combine_t h, const void* x1, const void* w1,
                           const int32_t* offsets, int32_t m_total, void* h_out, void* stream) {
  if (!h || !w1 || !offsets || m_total < 0) return EP_ERR_INVALID_ARG;
  if (m_total > 0 && (!x1 || !h_out)) return EP_ERR_INVALID_ARG;
  if ((x1 && !aligned16(x1)) || !aligned16(w1) || (h_out && !aligned16(h_out)))
    return EP_ERR_INVALID_ARG;
  if (h->p.dtype != EP_DTYPE_BF16) return EP_ERR_UNSUPPORTED;
  const int hidden = h->p.hidden_n, inter = h->p.hidden_k;
  // 2I GEMM columns in whole 256-column tiles; 32-bit offsets inside X1 and W1_e
  if (inter % 128) return EP_ERR_UNSUPPORTED;
  if (uint64_t(m_total) * hidden * 2 >= (uint64_t(1) << 32)) return EP_ERR_UNSUPPORTED;
  if (uint64_t(2) * inter * hidden * 2 >= (uint64_t(1) << 32)) return EP_ERR_UNSUPPORTED;

  ep::GemmArgs a{};
  a.x = static_cast<const uint8_t*>(x1);
  a.w = static_cast<const uint8_t*>(w1);
  a.offsets = offsets;
  a.c_local = static_cast<uint8_t*>(h_out);
  a.m_total = m_total;
  a.K = hidden;
  a.N = 2 * inter;
  a.sink_on = 0;
  a.s = sink_state(h, 1);     // rank / expert counts and the error word only

  const int El = h->p.n_experts_per_device;
  const int64_t nt = a.N / ep::gemm_tile_cols(ep::kTile256x256);
  const int64_t items = (int64_t(m_total) / ep::gemm_tile_rows(ep::kTile256x256) + El) * nt + El;
  const int64_t resident = int64_t(h->num_cus) * ep::gemm_blocks_per_cu(ep::kTile256x256);
  int64_t grid = std::min(items, resident);
  grid = (grid + 7) / 8 * 8;
  hipError_t err = ep::launch_swiglu_bf16(a, int(grid), static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_grouped_gemm_swiglu_fp8(ep_combine_t h, const void* x1, const float* x1_scale,
                               const void* w1, const float* w1_scale, const int32_t* offsets,
                               int32_t m_total, void* h_out, float* h_scale, void* stream) {
  if (!h || !w1 || !w1_scale || !offsets || m_total < 0) return EP_ERR_INVALID_ARG;
  if (m_total > 0 && (!x1 || !x1_scale || !h_out || !h_scale)) return EP_ERR_INVALID_ARG;
  if ((x1 && !aligned16(x1)) || !aligned16(w1) || (h_out && !aligned16(h_out)))
    return EP_ERR_INVALID_ARG;
  if (h->p.dtype != EP_DTYPE_FP8_E4M3_B128) return EP_ERR_UNSUPPORTED;
  const int hidden = h->p.hidden_n, inter = h->p.hidden_k;
  // the handle's fp8 rules give hidden and I multiples of 128: 2I GEMM columns in
  // whole 256-column tiles; 32-bit offsets inside X1 and W1_e
  if (uint64_t(m_total) * hidden >= (uint64_t(1) << 32)) return EP_ERR_UNSUPPORTED;
  if (uint64_t(2) * inter * hidden >= (uint64_t(1) << 32)) return EP_ERR_UNSUPPORTED;

  ep::GemmArgs a{};
  a.x = static_cast<const uint8_t*>(x1);
  a.w = static_cast<const uint8_t*>(w1);
  a.x_scale = x1_scale;
  a.w_scale = w1_scale;
  a.offsets = offsets;
  a.c_local = static_cast<uint8_t*>(h_out);
  a.c_scale = h_scale;
  a.m_total = m_total;
  a.K = hidden;
  a.N = 2 * inter;
  a.sink_on = 0;
  a.s = sink_state(h, 1);     // rank / expert counts and the error word only

  const int El = h->p.n_experts_per_device;
  const int64_t nt = a.N / ep::gemm_tile_cols(ep::kTile256x256);
  const int64_t items = (int64_t(m_total) / ep::gemm_tile_rows(ep::kTile256x256) + El) * nt + El;
  const int64_t resident = int64_t(h->num_cus) * ep::gemm_blocks_per_cu(ep::kTile256x256);
  int64_t grid = std::min(items, resident);
  grid = (grid + 7) / 8 * 8;
  hipError_t err = ep::launch_swiglu_fp8(a, int(grid), static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_signal_completion(ep_combine_t h, const int32_t* expert, const int32_t* dst_rank,
                         const uint64_t* signal, int32_t n, uint64_t epoch, void* stream) {
  if (!h || n < 0 || !epoch_ok(h, epoch)) return EP_ERR_INVALID_ARG;
  if (n == 0) return EP_OK;
  if (!expert || !dst_rank || !signal) return EP_ERR_INVALID_ARG;
  hipError_t err = ep::launch_signal(sink_state(h, epoch), expert, dst_rank, signal, n,
                                     static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_combine_reduce(ep_combine_t h, const int32_t* topk_ids, const float* topk_w,
                      int32_t tokens_per_rank, void* out, uint64_t epoch, void* stream) {
  if (!h || !epoch_ok(h, epoch)) return EP_ERR_INVALID_ARG;
  if (tokens_per_rank < 0 || tokens_per_rank > h->p.max_tokens_per_rank) return EP_ERR_INVALID_ARG;
  if (tokens_per_rank == 0) return EP_OK;
  ep::CombineArgs a{};
  const int rc = combine_args(h, topk_ids, topk_w, tokens_per_rank, out, epoch, &a);
  if (rc != EP_OK) return rc;
  hipError_t err = ep::launch_combine(a, h->num_cus, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_grouped_gemm_scatter_combine(ep_combine_t h, const void* x, const void* w,
                                    const float* x_scale, const float* w_scale,
                                    const int32_t* offsets, const int32_t* src_info,
                                    int32_t m_total, const int32_t* topk_ids,
                                    const float* topk_w, int32_t tokens_per_rank, void* out,
                                    uint64_t epoch, void* stream) {
  if (!h || !epoch_ok(h, epoch)) return EP_ERR_INVALID_ARG;
  if (tokens_per_rank < 1 || tokens_per_rank > h->p.max_tokens_per_rank) return EP_ERR_INVALID_ARG;
  if (h->p.flags & (EP_FLAG_EPILOGUE_ONLY | EP_FLAG_TRACE)) return EP_ERR_UNSUPPORTED;
  ep::CombineArgs c{};
  const int rc = combine_args(h, topk_ids, topk_w, tokens_per_rank, out, epoch, &c);
  if (rc != EP_OK) return rc;
  return gemm_scatter(h, x, w, x_scale, w_scale, offsets, src_info, m_total, 0, nullptr, epoch,
                      stream, h->b.rank_counter, h->b.tile_counter, &c);
}

int ep_advance_epoch(ep_combine_t h, void* stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  if (!(h->p.flags & EP_FLAG_DEVICE_EPOCH)) return EP_ERR_UNSUPPORTED;
  const hipError_t err = ep::launch_advance_epoch(h->b.epoch_word, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? EP_OK : EP_ERR_HIP;
}

int ep_combine_query_error(ep_combine_t h, void* stream) {
  if (!h) return EP_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, h->b.error_word, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess)
    return EP_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return EP_ERR_HIP;
  if (v != 0) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(h->b.error_word, &zero, sizeof(zero), hipMemcpyHostToDevice, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return EP_ERR_HIP;
  }
  return v;
}

}  // extern "C"
