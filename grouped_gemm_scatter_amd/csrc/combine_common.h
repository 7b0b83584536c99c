// The consumer combine of one run of tokens of one source rank, shared by the
// standalone combine kernel and the grouped-GEMM kernels that run the
// combine in the same launch after their tiles.
//
// The run's workgroup first acquires rank rk's completion ("ep_signal_completion",
// description: a fused consumer acquires once per source rank): one thread
// waits, bounded, for the rank flag to carry the step's epoch; in per-expert
// completion mode its first E_l threads wait for the E_l tagged count words of
// the rank instead.  A timeout latches EP_ERR_FLAG_TIMEOUT and leaves the
// run's outputs untouched.  Then each wave reduces one token at a time, or
// one of `parts` column ranges of it (the standalone combine splits every row
// over two waves; the consumer inside the GEMM's grid takes whole rows): the
// lanes holding picks find the local ones (ballot); every lane issues the
// loads of up to CH 16-byte chunks of its share of each local slot row at once
// ("P3PeerSendConfig", description: the slot formula), accumulates
// w_k * slot_k with one fused multiply-add per pick in ascending k in fp32, and
// stores the bf16 values.  The next token's picks and weights are fetched while
// the current one is reduced.
#pragma once

#include "ep_kernels.h"

namespace ep {

constexpr int kCombineThreads = 512;
constexpr int kCombineWaves = kCombineThreads / 64;

// Acquires rank rk's completion for this workgroup (all threads call it;
// s_ok is an LDS word).  Returns false after a timeout (error latched once).
__device__ __forceinline__ bool combine_acquire(const CombineArgs& a, int rk, int* s_ok) {
  const int tid = threadIdx.x;
  const uint64_t epoch = a.epoch_ptr ? *a.epoch_ptr : a.epoch;   // the step's epoch
  if (a.per_expert) {
    // per-expert completion: the threads acquire the E_l count words (e, rk)
    if (tid == 0) *s_ok = 1;
    __syncthreads();
    for (int e = tid; e < a.n_experts; e += blockDim.x)
      if (!acquire_count(a.words + count_index(e, rk, a.n_ranks), epoch, a.spin_limit,
                         a.system_scope))
        *s_ok = 0;
  } else if (tid == 0) {
    *s_ok = acquire_flag(a.flags + rk, epoch, a.spin_limit, a.system_scope);
  }
  __syncthreads();
  const bool ok = *s_ok;
  __syncthreads();        // every thread has read s_ok before it is written again
  if (!ok && tid == 0) latch_error(a.err, kErrFlagTimeout);
  return ok;
}

// Combines tokens [tbeg, tend) of rank rk (rank completion already acquired)
// over the workgroup's waves (whatever their number): `parts` (1, 2 or 4,
// dividing the wave count) consecutive waves share a token, wave w taking
// column range w % parts of it, so waves / parts tokens are in flight.
// CH = 16-byte chunks in flight per lane per pass: the caller picks the
// smallest of 4, 8 and 14 that covers a range in one pass (14: a 7168-wide
// row), so no lane carries masked loads it does not need; wider rows take more
// passes.  g_first / w_first: this lane's pick (global expert id, -1 for none)
// and weight of the wave's first token, loaded by the caller.
template <int CH>
__device__ __forceinline__ void combine_run(const CombineArgs& a, int rk, int tbeg, int tend,
                                            int g_first, float w_first, int parts) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int waves = (blockDim.x >> 6) / parts;   // tokens in flight
  uint8_t* recv = nullptr;
#pragma unroll
  for (int i = 0; i < kMaxRanks; ++i)
    if (i == rk) recv = a.recv[i];

  const int nchunks = a.N / 8;                  // 16-byte chunks per row
  const int per_part = (nchunks + parts - 1) / parts;
  const int cbeg = (wave % parts) * per_part;
  const int cend = min(nchunks, cbeg + per_part);
  auto load_picks = [&](int t, int& g, float& wk) {
    g = -1;
    wk = 0.f;
    if (t < tend && lane < a.top_k) {
      const size_t p = ((size_t)rk * a.tokens + t) * a.top_k + lane;
      g = a.topk_ids[p];
      wk = a.topk_w[p];
    }
  };
  int g_next = g_first;
  float w_next = w_first;
  for (int t = tbeg + wave / parts; t < tend; t += waves) {
    const int g = g_next;
    const float wk = w_next;
    load_picks(t + waves, g_next, w_next);
    const bool is_local = g >= a.expert_lo && g < a.expert_lo + a.n_experts;
    const uint64_t mask = __ballot(is_local);
    const uint8_t* slots = recv + slot_offset(t, 0, a.top_k, a.msg_bytes);
    uint8_t* orow = a.out + ((size_t)rk * a.tokens + t) * a.N * 2;
    for (int c0 = cbeg; c0 < cend; c0 += 64 * CH) {
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
          v[u] = c < cend ? load16_nt(src + (size_t)c * 16) : u32x4{0u, 0u, 0u, 0u};
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
        if (c < cend) {
          u32x4 o;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[u][2 * q], acc[u][2 * q + 1]);
          store16_nt(orow + (size_t)c * 16, o);
        }
      }
    }
  }
}

// 16-byte chunks per lane per pass for column ranges of rows of N bf16
// values split in `parts`: 4, 8 or 14.
inline int combine_chunks(int N, int parts = 1) {
  const int per_lane = ((N / 8 + parts - 1) / parts + 63) / 64;
  return per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : 14;
}

// Split of R * tokens tokens into runs of one rank each, about `target` runs
// in all; each run is a multiple of `unit` tokens (the tokens a workgroup has
// in flight).
inline void combine_split(int n_ranks, int tokens, int64_t target, int* tokens_per_run,
                          int* runs_per_rank, int unit = kCombineWaves) {
  const int64_t total = (int64_t)n_ranks * tokens;
  int tpr = (int)((total + target - 1) / target);
  tpr = (tpr + unit - 1) / unit * unit;
  tpr = tpr < unit ? unit : tpr;
  *tokens_per_run = tpr;
  *runs_per_rank = (tokens + tpr - 1) / tpr;
}

// Every run u = ru0, ru0 + step, ... of the combine: acquire the run's rank,
// then combine its tokens (the consumer side of a launch; CH by range width,
// `parts` waves per token).
template <int CH>
__device__ __forceinline__ void combine_runs_ch(const CombineArgs& a, int ru0, int step,
                                                int tokens_per_run, int runs_per_rank,
                                                int* s_ok, int parts = 1) {
  const int runs = a.n_ranks * runs_per_rank;
  for (int u = ru0; u < runs; u += step) {
    const int rk = u / runs_per_rank;
    const int tbeg = (u % runs_per_rank) * tokens_per_run;
    const int tend = min(a.tokens, tbeg + tokens_per_run);
    if (tbeg >= tend) continue;
    // this wave's first token's picks and weights (inputs of the step, not
    // published by the producers): their loads overlap the acquire
    const int lane = threadIdx.x & 63, t0 = tbeg + (threadIdx.x >> 6) / parts;
    int g = -1;
    float wk = 0.f;
    if (t0 < tend && lane < a.top_k) {
      const size_t p = ((size_t)rk * a.tokens + t0) * a.top_k + lane;
      g = a.topk_ids[p];
      wk = a.topk_w[p];
    }
    if (!combine_acquire(a, rk, s_ok)) continue;
    combine_run<CH>(a, rk, tbeg, tend, g, wk, parts);
  }
}

}  // namespace ep
