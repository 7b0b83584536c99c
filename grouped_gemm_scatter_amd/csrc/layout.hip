// Weight layout for the decode-shaped down-projection: a bf16 stack W
// [E_l][N][K] re-laid as [E_l][K/64][N][64], so that the 64-element K slice
// of a block of rows, which one copy step of the GEMM moves, is one contiguous
// run of HBM instead of one 128-byte piece per row.  A one-time transform of
// static weights, made once per weight load; the GEMM reads either layout.
// Each thread moves 16-byte pieces in output order: the writes are contiguous
// and the reads come in 128-byte runs, one per (row, slice).
#include <algorithm>

#include "ep_kernels.h"

namespace ep {

namespace {

constexpr int kPackThreads = 256;

__global__ __launch_bounds__(kPackThreads) void pack_slice_major_kernel(const uint8_t* w,
                                                                       uint8_t* out,
                                                                       int64_t pieces, int N,
                                                                       int K) {
  const int64_t expert_bytes = (int64_t)N * K * 2;
  const int64_t slice_bytes = (int64_t)N * 128;
  const int64_t stride = (int64_t)gridDim.x * kPackThreads;
  for (int64_t i = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; i < pieces; i += stride) {
    const int64_t o = i * 16;                    // output byte offset
    const int64_t e = o / expert_bytes;
    const int64_t r = o - e * expert_bytes;      // within the expert: [K/64][N][128 bytes]
    const int64_t s = r / slice_bytes;
    const int64_t q = r - s * slice_bytes;
    const int64_t n = q >> 7, c = q & 127;
    const int64_t src = e * expert_bytes + n * (int64_t)K * 2 + s * 128 + c;
    store16_nt(out + o, load16(w + src));
  }
}

}  // namespace

hipError_t launch_pack_slice_major(const uint8_t* w, uint8_t* out, int64_t experts, int N, int K,
                                   int num_cus, hipStream_t st) {
  const int64_t pieces = experts * (int64_t)N * K * 2 / 16;
  if (pieces == 0) return hipSuccess;
  const int64_t grid = std::max<int64_t>(
      1, std::min<int64_t>((pieces + kPackThreads - 1) / kPackThreads, 16 * (int64_t)num_cus));
  hipLaunchKernelGGL(pack_slice_major_kernel, dim3((int)grid), dim3(kPackThreads), 0, st, w, out,
                     pieces, N, K);
  return hipGetLastError();
}

}  // namespace ep
