// Dispatch side of the expert FFN on one GPU's share: every grouped row m (a
// local pick (rk, t, k), rows ordered by (e, rk, t, k)) receives the hidden
// row of token t of source rank rk, the row the up-projection consumes.  In a
// multi-GPU layer the token's owner would send that row to this GPU; here the
// R source ranks are R logical token arrays in this GPU's memory, and the
// copy is made from the receiving side.  A pure HBM copy: each wave resolves
// a row's source (its expert group, rank run and token) and copies the row with
// 16-byte loads and nontemporal 16-byte stores, rows spread over the waves.
#include <algorithm>

#include "ep_kernels.h"

namespace ep {

namespace {

constexpr int kDispatchThreads = 256;

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(DispatchArgs a) {
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (kDispatchThreads / 64);
  const int wave = blockIdx.x * (kDispatchThreads / 64) + (threadIdx.x >> 6);
  const int chunks = a.row_bytes / 16;
  // source row of grouped row m: its expert is the group holding m, its rank
  // the run of that group holding m, its token src_info[m][0]; null (and the
  // error latched by the caller) for a token index outside the source arrays
  auto source = [&](int m) -> const uint8_t* {
    int lo = 0, hi = a.n_experts;                 // expert: largest e with offsets[e*R] <= m
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid * a.n_ranks] <= m) lo = mid; else hi = mid;
    }
    int rk = 0;
    for (int r = 1; r < a.n_ranks; ++r)
      if (a.offsets[lo * a.n_ranks + r] <= m) rk = r;
    const int t = a.src_info[2 * (size_t)m];
    if (t < 0 || t >= a.tokens) return nullptr;
    return a.tokens_x + ((size_t)rk * a.tokens + t) * a.row_bytes;
  };
  for (int m = wave; m < a.m_total; m += waves) {
    const uint8_t* src = source(m);
    uint8_t* dst = a.x_out + (size_t)m * a.row_bytes;
    if (!src) {
      if (lane == 0) latch_error(a.err, kErrBadGroup);
      continue;
    }
    for (int c = lane; c < chunks; c += 64) store16_nt(dst + (size_t)c * 16, load16(src + (size_t)c * 16));
  }
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, int num_cus, hipStream_t st) {
  const int64_t waves_needed = a.m_total;
  int64_t grid = std::min<int64_t>((waves_needed + 3) / 4, 8 * (int64_t)num_cus);
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(dispatch_kernel, dim3((int)grid), dim3(kDispatchThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ep
