// combine: a grid of up to sixteen workgroups per CU; each workgroup owns a
// contiguous run of tokens of one source rank rk, so it acquires rk's
// rank-completion flag exactly once (one thread, bounded wait) before reading
// any slot ("ep_signal_completion", description: a fused consumer acquires
// once per source rank); in per-expert completion mode its first E_l threads
// acquire the rank's E_l tagged count words instead.  Two waves share each
// token, one column range each: the lanes holding picks find the local ones
// (ballot); then every lane issues the loads of up to CH chunks of its share
// of each local slot row at once (chunks of 16 bytes, "P3PeerSendConfig" slot
// formula), accumulates w_k * slot_k in fp32 in ascending k, and stores the
// bf16 values.  The next token's picks and weights are fetched while the
// current one is reduced.  The pass is a pure
// HBM stream (slot reads + output writes), written for coalesced 16-byte
// accesses with many bytes in flight per wave.
#include "combine_common.h"

namespace ep {

namespace {

template <int CH>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a,
                                                                 int tokens_per_wg,
                                                                 int wg_per_rank, int parts) {
  __shared__ int s_ok;
  combine_runs_ch<CH>(a, blockIdx.x, gridDim.x, tokens_per_wg, wg_per_rank, &s_ok, parts);
}

// One step forward of a device-resident epoch (a single thread; stream order
// puts it between the previous step's consumer and the next step's producers).
// Values whose low 32 bits are zero are skipped: the per-expert tag of a
// count word is those bits, and zero is the words' initial content.
__global__ void advance_epoch_kernel(uint64_t* word) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    uint64_t e = *word + 1;
    if ((e & 0xffffffffull) == 0) ++e;
    *word = e;
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
  // two waves per token, each a column range of it (the 8-chunk form for
  // 7168-wide rows, 138 VGPRs): against one wave per token, 183.8 -> 176.4 us
  // at the prefill shape, 118.6 -> 112.3 at the skewed fp8 shape, 16.6 -> 15.0
  // at decode, the Qwen3 shape unchanged; four waves per token (82 VGPRs,
  // three workgroups resident per CU) took 44.8 against 33.8 us at Qwen3.
  // A grid of up to sixteen workgroups per CU (one resident per CU at a time),
  // each a run of one rank's tokens (a multiple of the four tokens a workgroup
  // has in flight), so every workgroup acquires one flag: short runs keep the
  // launch's last workgroups short (with one wave per token, 4 per CU took
  // 193 us at the prefill shape, 8 took 186, 16 took 184)
  const int parts = 2;
  int tokens_per_wg = 0, wg_per_rank = 0;
  combine_split(a.n_ranks, a.tokens, 16 * (int64_t)num_cus, &tokens_per_wg, &wg_per_rank,
                kCombineWaves / parts);
  const dim3 grid(a.n_ranks * wg_per_rank), block(kCombineThreads);
  switch (combine_chunks(a.N, parts)) {
    case 4:
      hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, st, a, tokens_per_wg, wg_per_rank,
                         parts);
      break;
    case 8:
      hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, st, a, tokens_per_wg, wg_per_rank,
                         parts);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel<14>, grid, block, 0, st, a, tokens_per_wg, wg_per_rank,
                         parts);
  }
  return hipGetLastError();
}

hipError_t launch_advance_epoch(uint64_t* word, hipStream_t st) {
  hipLaunchKernelGGL(advance_epoch_kernel, dim3(1), dim3(64), 0, st, word);
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
