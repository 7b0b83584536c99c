// combine: a grid of up to sixteen workgroups per CU; each workgroup owns a
// contiguous run of tokens of one source rank rk, so it acquires rk's
// rank-completion flag exactly once (one thread, bounded wait) before reading
// any slot ("ep_signal_completion", description: a fused consumer acquires
// once per source rank); in per-expert completion mode its first E_l threads
// acquire the rank's E_l tagged count words instead.  Each wave reduces one
// token at a time: the lanes holding picks find the local ones (ballot); then
// every lane issues the loads of up to CH chunks of its share of each local
// slot row at once (chunks of 16 bytes, "P3PeerSendConfig" slot formula),
// accumulates w_k * slot_k in fp32
// in ascending k, and stores the bf16 row.  The next token's picks and
// weights are fetched while the current one is reduced.  The pass is a pure
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
  // a grid of up to sixteen workgroups per CU (one token per wave at the
  // prefill shape; with two waves per SIMD resident, one workgroup per CU runs
  // at a time), each a run of one rank's tokens (a multiple of the tokens a
  // workgroup has in flight), so every workgroup acquires one flag: short runs
  // keep the launch's last workgroups short (4 per CU took 193 us at the
  // prefill shape, 8 took 186, 16 took 184)
  // with fewer tokens than 8 waves per CU (decode: 1024 tokens), a token's row
  // is split over 2 (or 4) waves: 16.6 -> 15.0 us at the decode shape (15.4
  // with 4); splitting rows at the Qwen3 shape (8192 tokens) changed nothing
  const int64_t total = (int64_t)a.n_ranks * a.tokens;
  int parts = 1;
  while (parts < 4 && total * parts < 8 * (int64_t)num_cus) parts *= 2;
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
