// Local grouping of the routing: the dispatch layout the grouped GEMM
// consumes.  A pick (rk, t, k) whose global expert g lies in this GPU's slice
// [lo, lo + E_l) becomes a row of group e = g - lo ("EpiloguePeerSink",
// send_tile argument expert_id); rows are ordered by (e, rk, t, k), so that
// group e's run of rank rk starts at offsets[e*R + rk] ("P3PeerSendConfig",
// description: the e*n_ranks + rk count layout), and src_info[m] = (t, k)
// ("P3PeerSendConfig", field src_info_ptr).  Integer work only; every result
// is fixed, so the kernels use no atomics.
//   1. count: one workgroup per (e, rk); its 8 waves take contiguous eighths of
//      rank rk's T*top_k picks, each lane four consecutive picks per chunk of
//      256 and four chunks per pass (sixteen loads in flight), and count the
//      matches; offsets[e*R + rk + 1] = the count.
//   2. scan: one wave turns the counts into offsets (exclusive prefix).
//   3. place: the count workgroups again, each wave starting at its group's
//      offset plus the matches of the eighths before it; in a chunk, a
//      match's row is that base plus the matches of the lanes below it (one
//      ballot per pick position) plus its lane's earlier matches.

#include "ep_kernels.h"

namespace ep {
namespace {

constexpr int kGroupThreads = 512;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kScanPerLane = 32;   // the scan wave covers 64 * 32 = 2048 groups
constexpr int kChunk = 256;        // picks per wave and chunk: four per lane
constexpr int kChunksPerPass = 4;

// Picks [beg, end) of one wave: an eighth of the rank's picks, in whole
// chunks except the last.
__device__ __forceinline__ void wave_range(int n, int wave, int& beg, int& end) {
  const int per = ((n + kGroupWaves - 1) / kGroupWaves + kChunk - 1) / kChunk * kChunk;
  beg = min(n, wave * per);
  end = min(n, beg + per);
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

template <bool PLACE>
__global__ __launch_bounds__(kGroupThreads) void group_kernel(GroupArgs a) {
  __shared__ int s_cnt[kGroupWaves];
  const int g = blockIdx.x;
  const int e = g / a.n_ranks, rk = g % a.n_ranks;
  const int want = a.expert_lo + e;
  const int n = a.tokens * a.top_k;
  const int32_t* ids = a.topk_ids + (size_t)rk * n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int beg, end;
  wave_range(n, wave, beg, end);

  // pick q of chunk c in a pass starting at i: q = i + c*kChunk + 4*lane + j
  auto load_pass = [&](int i, int (&v)[kChunksPerPass][4]) {
#pragma unroll
    for (int c = 0; c < kChunksPerPass; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = i + c * kChunk + 4 * lane + j;
        v[c][j] = q < end ? ids[q] : -1;
      }
  };
  int cnt = 0;
  for (int i = beg; i < end; i += kChunksPerPass * kChunk) {
    int v[kChunksPerPass][4];
    load_pass(i, v);
#pragma unroll
    for (int c = 0; c < kChunksPerPass; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) cnt += v[c][j] == want;
  }
  cnt = wave_sum(cnt);
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  if constexpr (!PLACE) {
    if (threadIdx.x == 0) {
      int total = 0;
      for (int w = 0; w < kGroupWaves; ++w) total += s_cnt[w];
      a.offsets[g + 1] = total;
    }
    return;
  }
  int base = a.offsets[g];
  for (int w = 0; w < wave; ++w) base += s_cnt[w];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i = beg; i < end; i += kChunksPerPass * kChunk) {
    int v[kChunksPerPass][4];
    load_pass(i, v);
#pragma unroll
    for (int c = 0; c < kChunksPerPass; ++c) {
      // rows of this chunk, in pick order: the lanes below, then this lane's
      // earlier positions
      int row = base;
      int total = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint64_t m = __ballot(v[c][j] == want);
        row += __popcll(m & below);
        total += __popcll(m);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (v[c][j] == want) {
          const int q = i + c * kChunk + 4 * lane + j;
          a.src_info[2 * (size_t)row] = q / a.top_k;
          a.src_info[2 * (size_t)row + 1] = q % a.top_k;
          ++row;
        }
      base += total;
    }
  }
}

// offsets[1..n] hold counts on entry; on exit offsets[i] = sum of counts of
// groups below i.  Lane L takes groups [32L, 32L + 32).
__global__ __launch_bounds__(64) void group_scan_kernel(int32_t* offsets, int n) {
  const int lane = threadIdx.x;
  int v[kScanPerLane];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kScanPerLane; ++j) {
    const int i = lane * kScanPerLane + j;
    v[j] = i < n ? offsets[i + 1] : 0;
    sum += v[j];
  }
  // exclusive prefix of the lanes' sums
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  int run = incl - sum;
#pragma unroll
  for (int j = 0; j < kScanPerLane; ++j) {
    const int i = lane * kScanPerLane + j;
    run += v[j];
    if (i < n) offsets[i + 1] = run;
  }
  if (lane == 0) offsets[0] = 0;
}

}  // namespace

hipError_t launch_grouping(const GroupArgs& a, hipStream_t st) {
  const int groups = a.n_experts * a.n_ranks;
  if (groups > 64 * kScanPerLane) return hipErrorInvalidValue;
  hipLaunchKernelGGL(group_kernel<false>, dim3(groups), dim3(kGroupThreads), 0, st, a);
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(64), 0, st, a.offsets, groups);
  hipLaunchKernelGGL(group_kernel<true>, dim3(groups), dim3(kGroupThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ep
