// Consumer side of the EP-combine step and the standalone completion signal.
//
// combine: one workgroup per (source rank rk, block of tokens).  One thread
// acquires rk's rank-completion flag once (bounded wait), after which the
// workgroup reads the slots of its tokens ("ep_signal_completion",
// description: a fused consumer acquires once per source rank).  Each wave
// reduces one token at a time: the lanes holding picks find which picks are
// local, then every lane streams 16-byte chunks of the local slots
// ("P3PeerSendConfig", description: slot formula), accumulates
// w_k * slot_k in fp32 in ascending k, and stores the bf16 row.  The pass is a
// pure stream over HBM (slot reads + output writes), so it is written for
// coalesced 16-byte accesses with several chunks in flight per lane.
#include "ep_kernels.h"

namespace ep {

namespace {

constexpr int kCombineThreads = 256;
constexpr int kTokensPerWave = 4;
constexpr int kUnroll = 4;              // 16-byte chunks in flight per lane per pick

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  __shared__ int s_ok;
  const int rk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    bool ok = acquire_flag(a.flags + rk, a.epoch, a.spin_limit, a.system_scope);
    if (!ok) latch_error(a.err, kErrFlagTimeout);
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) return;

  uint8_t* recv = nullptr;
#pragma unroll
  for (int i = 0; i < kMaxRanks; ++i)
    if (i == rk) recv = a.recv[i];

  const int nchunks = a.N / 8;                  // 16-byte chunks per row
  const int t0 = (blockIdx.x * (kCombineThreads / 64) + wave) * kTokensPerWave;
  for (int tt = 0; tt < kTokensPerWave; ++tt) {
    const int t = t0 + tt;
    if (t >= a.tokens) break;
    const size_t pick0 = ((size_t)rk * a.tokens + t) * a.top_k;
    int g = -1;
    float wk = 0.f;
    if (lane < a.top_k) {
      g = a.topk_ids[pick0 + lane];
      wk = a.topk_w[pick0 + lane];
    }
    const bool is_local = g >= a.expert_lo && g < a.expert_lo + a.n_experts;
    const uint64_t mask = __ballot(is_local);
    const uint8_t* slots = recv + slot_offset(t, 0, a.top_k, a.msg_bytes);
    uint8_t* orow = a.out + ((size_t)rk * a.tokens + t) * a.N * 2;

    for (int c0 = 0; c0 < nchunks; c0 += 64 * kUnroll) {
      float acc[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = 0.f;
      uint64_t mm = mask;
      while (mm) {
        const int k = __builtin_ctzll(mm);
        mm &= mm - 1;
        const float wgt = __shfl(wk, k);
        const uint8_t* src = slots + (size_t)k * a.msg_bytes;
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < nchunks) v[u] = load16_nt(src + (size_t)c * 16);
          else v[u] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[u][2 * q] = __builtin_fmaf(wgt, bf16_lo(v[u][q]), acc[u][2 * q]);
            acc[u][2 * q + 1] = __builtin_fmaf(wgt, bf16_hi(v[u][q]), acc[u][2 * q + 1]);
          }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
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
  signal_rank(s, e, rk, signal[i]);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int num_cus, hipStream_t st) {
  (void)num_cus;
  const int tokens_per_block = (kCombineThreads / 64) * kTokensPerWave;
  dim3 grid((a.tokens + tokens_per_block - 1) / tokens_per_block, a.n_ranks);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(kCombineThreads), 0, st, a);
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
