// combine: a grid of about four workgroups per CU; each workgroup owns a
// contiguous run of tokens of one source rank rk, so it acquires rk's
// rank-completion flag exactly once (one thread, bounded wait) before reading
// any slot ("ep_signal_completion", description: a fused consumer acquires
// once per source rank); in per-expert completion mode its first E_l threads
// acquire the rank's E_l tagged count words instead.  Each wave reduces one token at a time: the lanes
// holding picks find the local ones (ballot); then every lane issues the
// loads of up to CH chunks of its share of each local slot row at once (chunks of
// 16 bytes, "P3PeerSendConfig" slot formula), accumulates w_k * slot_k in fp32
// in ascending k, and stores the bf16 row.  The next token's picks and
// weights are fetched while the current one is reduced.  The pass is a pure
// HBM stream (slot reads + output writes), written for coalesced 16-byte
// accesses with many bytes in flight per wave.
#include "ep_kernels.h"

namespace ep {

namespace {

constexpr int kCombineThreads = 512;
constexpr int kCombineWaves = kCombineThreads / 64;
// CH = 16-byte chunks in flight per lane per pass: the launcher picks the
// smallest of 4, 8 and 14 that covers a row in one pass (14: a 7168-wide row),
// so no lane carries masked loads it does not need; wider rows take more passes.
template <int CH>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a, int tokens_per_wg,
                                                                 int wg_per_rank) {
  __shared__ int s_ok;
  const int rk = blockIdx.x / wg_per_rank;
  const int tbeg = (blockIdx.x % wg_per_rank) * tokens_per_wg;
  const int tend = min(a.tokens, tbeg + tokens_per_wg);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tbeg >= tend) return;
  if (a.per_expert) {
    // per-expert completion: thread e acquires count word (e, rk)
    if (tid == 0) s_ok = 1;
    __syncthreads();
    if (tid < a.n_experts &&
        !acquire_count(a.words + count_index(tid, rk, a.n_ranks), a.epoch, a.spin_limit,
                       a.system_scope))
      s_ok = 0;
    __syncthreads();
    if (!s_ok) {
      if (tid == 0) latch_error(a.err, kErrFlagTimeout);
      return;
    }
  } else {
    if (tid == 0) {
      bool ok = acquire_flag(a.flags + rk, a.epoch, a.spin_limit, a.system_scope);
      if (!ok) latch_error(a.err, kErrFlagTimeout);
      s_ok = ok;
    }
    __syncthreads();
    if (!s_ok) return;
  }

  uint8_t* recv = nullptr;
#pragma unroll
  for (int i = 0; i < kMaxRanks; ++i)
    if (i == rk) recv = a.recv[i];

  const int nchunks = a.N / 8;                  // 16-byte chunks per row
  auto load_picks = [&](int t, int& g, float& wk) {
    g = -1;
    wk = 0.f;
    if (t < tend && lane < a.top_k) {
      const size_t p = ((size_t)rk * a.tokens + t) * a.top_k + lane;
      g = a.topk_ids[p];
      wk = a.topk_w[p];
    }
  };
  int g_next;
  float w_next;
  load_picks(tbeg + wave, g_next, w_next);
  for (int t = tbeg + wave; t < tend; t += kCombineWaves) {
    const int g = g_next;
    const float wk = w_next;
    load_picks(t + kCombineWaves, g_next, w_next);
    const bool is_local = g >= a.expert_lo && g < a.expert_lo + a.n_experts;
    const uint64_t mask = __ballot(is_local);
    const uint8_t* slots = recv + slot_offset(t, 0, a.top_k, a.msg_bytes);
    uint8_t* orow = a.out + ((size_t)rk * a.tokens + t) * a.N * 2;
    for (int c0 = 0; c0 < nchunks; c0 += 64 * CH) {
      float acc[CH][8];
#pragma unroll
      for (int u = 0; u < CH; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
      uint64_t mm = mask;
      while (mm) {
        const int k = __builtin_ctzll(mm);
        mm &= mm - 1;
        const float wgt = __shfl(wk, k);
        const uint8_t* src = slots + (size_t)k * a.msg_bytes;
        u32x4 v[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          const int c = c0 + u * 64 + lane;
          v[u] = c < nchunks ? load16_nt(src + (size_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < CH; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u][2 * q] = __builtin_fmaf(wgt, bf16_lo(v[u][q]), acc[u][2 * q]);
            acc[u][2 * q + 1] = __builtin_fmaf(wgt, bf16_hi(v[u][q]), acc[u][2 * q + 1]);
          }
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nchunks) {
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
          store16_nt(orow + (size_t)c * 16, o);
        }
      }
    }
  }
}

__global__ void signal_kernel(SinkState s, const int32_t* expert, const int32_t* dst_rank,
                              const uint64_t* signal, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = expert[i], rk = dst_rank[i];
  if (e < 0 || e >= s.n_experts || rk < 0 || rk >= s.n_ranks) {
    latch_error(s.err, kErrBadGroup);
    return;
  }
  if (s.per_expert) publish_count_release(s, e, rk, signal[i]);
  else signal_rank(s, e, rk, signal[i]);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int num_cus, hipStream_t st) {
  // about four workgroups per CU, each a run of one rank's tokens (a multiple of
  // the wave count), so every workgroup acquires one flag
  const int64_t target = 4 * (int64_t)num_cus;
  const int64_t total = (int64_t)a.n_ranks * a.tokens;
  int tokens_per_wg = (int)((total + target - 1) / target);
  tokens_per_wg = (tokens_per_wg + kCombineWaves - 1) / kCombineWaves * kCombineWaves;
  tokens_per_wg = tokens_per_wg < kCombineWaves ? kCombineWaves : tokens_per_wg;
  const int wg_per_rank = (a.tokens + tokens_per_wg - 1) / tokens_per_wg;
  const dim3 grid(a.n_ranks * wg_per_rank), block(kCombineThreads);
  const int per_lane = (a.N / 8 + 63) / 64;     // 16-byte chunks of a row per lane
  if (per_lane <= 4)
    hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, st, a, tokens_per_wg, wg_per_rank);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, st, a, tokens_per_wg, wg_per_rank);
  else
    hipLaunchKernelGGL(combine_kernel<14>, grid, block, 0, st, a, tokens_per_wg, wg_per_rank);
  return hipGetLastError();
}

hipError_t launch_signal(const SinkState& s, const int32_t* expert, const int32_t* dst_rank,
                         const uint64_t* signal, int n, hipStream_t st) {
  const int threads = 64;
  hipLaunchKernelGGL(signal_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0, st, s,
                     expert, dst_rank, signal, n);
  return hipGetLastError();
}

}  // namespace ep
