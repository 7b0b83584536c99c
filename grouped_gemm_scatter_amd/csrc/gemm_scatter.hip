// Grouped GEMM with the receive-buffer sink epilogue, bf16 in, fp32
// accumulate, bf16 rows out, for gfx950.
//
// Work decomposition.  Every local expert e owns the row group
// [offsets[e*R], offsets[(e+1)*R]) of X; its output C_e = X_e * W_e is cut into
// BM x BN tiles.  An expert with no rows still gets one work item, which only
// publishes its zero counts, so that every rank's election completes
// ("ep_signal_completion", parameter n_experts_per_device: the election bound).
// The grid is persistent; items are handed out so that each XCD (workgroups
// are dispatched round-robin over the 8 XCDs) walks a contiguous range of
// items, which keeps the X rows and W_e slabs of neighbouring tiles in that
// XCD's L2.
//
// Main loop.  4 waves in a 2 x 2 arrangement; each wave owns a (BM/2) x (BN/2)
// sub-tile as 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16).  W_e feeds the
// MFMA's first operand and X its second, so each lane's accumulator holds four
// consecutive output columns of one row, which packs into one 8-byte LDS store
// in the epilogue.  A and B K-slices (64 wide) are double-buffered in LDS with
// a 16-byte-chunk XOR swizzle.
//
// Epilogue ("EpiloguePeerSink", send_tile: the finished tile replaces the
// local store).  The bf16 tile is staged in LDS; each row's destination is
// resolved once (owner rank from the offsets, slot from src_info with the
// "P3PeerSendConfig" slot formula and bounds check) and then rows are written
// with coalesced 16-byte nontemporal stores.  Every wave releases its stores
// at agent (or system) scope; one thread then counts the tile on the expert's
// tile counter, and the expert's last tile publishes the counts and runs the
// rank election.
#include "ep_kernels.h"

namespace ep {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;               // bf16 elements per K slice = 128 bytes per row
constexpr int kRowBytes = kBK * 2;

template <int BM, int BN>
struct Bf16Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int AC = BM * 8 / kThreads;     // 16-byte chunks per thread per slice
  static constexpr int BC = BN * 8 / kThreads;
  static constexpr int C_PITCH = BN * 2 + 16;      // bytes per staged output row
  static constexpr int LDS_MAIN = 2 * STAGE;
  static constexpr int LDS_C = BM * C_PITCH;
  static constexpr int LDS = LDS_MAIN > LDS_C ? LDS_MAIN : LDS_C;
  static_assert(AC * kThreads == BM * 8 && BC * kThreads == BN * 8, "tile/threads");
};

// Expert that owns work item `item`: largest e with base[e] <= item.
__device__ __forceinline__ int find_expert(const int* base, int n_experts, int item) {
  int lo = 0, hi = n_experts;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (base[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// Per-workgroup setup shared by the GEMM kernels: validates the offsets and
// builds the prefix of work items per expert.  Returns false (and latches
// EP_ERR_BAD_GROUP once) when the offsets are inconsistent.
template <int BM>
__device__ bool build_work_table(const GemmArgs& a, int nt, int* s_base, int* s_bad) {
  const int tid = threadIdx.x;
  const int R = a.s.n_ranks, El = a.s.n_experts;
  if (tid == 0) *s_bad = 0;
  __syncthreads();
  for (int i = tid; i <= El * R; i += kThreads) {
    int v = a.offsets[i];
    bool bad = v < 0 || v > a.m_total || (i == 0 && v != 0) ||
               (i == El * R && v != a.m_total) || (i > 0 && v < a.offsets[i - 1]);
    if (bad) *s_bad = 1;
  }
  __syncthreads();
  if (*s_bad) {
    if (tid == 0 && blockIdx.x == 0) latch_error(a.s.err, kErrBadGroup);
    return false;
  }
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < El; ++e) {
      s_base[e] = acc;
      int me = a.offsets[(e + 1) * R] - a.offsets[e * R];
      acc += me ? ((me + BM - 1) / BM) * nt : 1;
    }
    s_base[El] = acc;
  }
  __syncthreads();
  return true;
}

// Destination of row m of expert e's group for this tile (0 = not sent).
__device__ __forceinline__ uint64_t row_destination(const GemmArgs& a, uint8_t* const* s_recv,
                                                    int e, int m) {
  if (!a.sink_on) return (uint64_t)(a.c_local + (size_t)m * a.N * 2);
  const int R = a.s.n_ranks;
  const int32_t* grp = a.offsets + e * R;
  int rk = 0;
  for (int r = 1; r < R; ++r)
    if (grp[r] <= m) rk = r;
  const int t = a.src_info[2 * (size_t)m];
  const int k = a.src_info[2 * (size_t)m + 1];
  if (t < 0 || t >= a.s.max_tokens || k < 0 || k >= a.s.top_k) {
    latch_error(a.s.err, kErrSlotOob);
    return 0;
  }
  return (uint64_t)(s_recv[rk] + slot_offset(t, k, a.s.top_k, a.s.msg_bytes));
}

// Completion of one tile of expert e: release this wave's row stores, count
// the tile; the expert's last tile publishes the counts and joins the rank
// elections.
__device__ __forceinline__ void finish_tile(const GemmArgs& a, int e, int tiles_of_e) {
  release_fence(a.s.system_scope);
  __syncthreads();
  if (threadIdx.x == 0) {
    int old = __hip_atomic_fetch_add(a.s.tile_counter + e, 1, __ATOMIC_ACQ_REL,
                                     __HIP_MEMORY_SCOPE_AGENT);
    if (old == tiles_of_e - 1) {
      __hip_atomic_store(a.s.tile_counter + e, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int R = a.s.n_ranks;
      for (int rk = 0; rk < R; ++rk) {
        uint64_t rows = (uint64_t)(a.offsets[e * R + rk + 1] - a.offsets[e * R + rk]);
        signal_rank(a.s, e, rk, rows);
      }
    }
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_scatter_bf16_kernel(GemmArgs a) {
  using T = Bf16Tile<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[T::LDS];
  __shared__ uint64_t s_rowdst[BM];
  __shared__ int s_base[kMaxLocalExperts + 1];
  __shared__ uint8_t* s_recv[kMaxRanks];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int K = a.K, N = a.N;
  const int nt = N / BN;
  const int R = a.s.n_ranks, El = a.s.n_experts;

  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) s_recv[i] = a.s.recv[i];
  }
  if (!build_work_table<BM>(a, nt, s_base, &s_bad)) return;
  const int total = s_base[El];

  const int G = gridDim.x;                  // a multiple of 8
  const int per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  // per-thread constant parts of the global->LDS copy
  const int crow = tid >> 3, ckc = tid & 7;
  const int lds_off = crow * kRowBytes + ((ckc ^ (crow & 7)) << 4);
  // fragment read offsets: lane reads row (lane & 31) of a 32-row block,
  // 16-byte chunk (2*s + lane/32) of the 128-byte K slice
  const int frow = lane & 31, fhalf = lane >> 5;

  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= total) break;
    const int e = find_expert(s_base, El, item);
    const int g0 = a.offsets[e * R], g1 = a.offsets[(e + 1) * R];
    const int me = g1 - g0;
    if (me == 0) {
      if (a.sink_on && tid == 0)
        for (int rk = 0; rk < R; ++rk) signal_rank(a.s, e, rk, 0);
      continue;
    }
    const int mt = (me + BM - 1) / BM;
    const int local = item - s_base[e];
    const int mb = local % mt, nb = local / mt;
    const int m_abs = g0 + mb * BM, n_abs = nb * BN;

    const uint8_t* xg = a.x;
    const uint8_t* wg = a.w + (size_t)e * N * K * 2;
    uint32_t a_src[T::AC], b_src[T::BC];
#pragma unroll
    for (int i = 0; i < T::AC; ++i) {
      int m = min(m_abs + crow + i * 32, g1 - 1);   // rows past m_end re-read a valid row
      a_src[i] = (uint32_t)((size_t)m * K * 2 + ckc * 16);
    }
#pragma unroll
    for (int i = 0; i < T::BC; ++i)
      b_src[i] = (uint32_t)((size_t)(n_abs + crow + i * 32) * K * 2 + ckc * 16);

    f32x16 acc[T::TN][T::TM];
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
      for (int j = 0; j < T::TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    u32x4 ra[T::AC], rb[T::BC];
    const int KT = K / kBK;
    auto gload = [&](int kt) {
      const size_t kb = (size_t)kt * kRowBytes;
#pragma unroll
      for (int i = 0; i < T::AC; ++i) ra[i] = load16(xg + a_src[i] + kb);
#pragma unroll
      for (int i = 0; i < T::BC; ++i) rb[i] = load16(wg + b_src[i] + kb);
    };
    auto lstore = [&](int stage) {
      uint8_t* sa = smem + stage * T::STAGE;
      uint8_t* sb = sa + T::A_BYTES;
#pragma unroll
      for (int i = 0; i < T::AC; ++i)
        *reinterpret_cast<u32x4*>(sa + lds_off + i * 32 * kRowBytes) = ra[i];
#pragma unroll
      for (int i = 0; i < T::BC; ++i)
        *reinterpret_cast<u32x4*>(sb + lds_off + i * 32 * kRowBytes) = rb[i];
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) gload(kt + 1);
      const uint8_t* sa = smem + (kt & 1) * T::STAGE;
      const uint8_t* sb = sa + T::A_BYTES;
#pragma unroll
      for (int s = 0; s < kBK / 16; ++s) {
        const int chunk = ((2 * s + fhalf) ^ (frow & 7)) << 4;
        bf16x8 fw[T::TN], fx[T::TM];
#pragma unroll
        for (int i = 0; i < T::TN; ++i)
          fw[i] = *reinterpret_cast<const bf16x8*>(sb + (wn * T::WN + i * 32 + frow) * kRowBytes + chunk);
#pragma unroll
        for (int j = 0; j < T::TM; ++j)
          fx[j] = *reinterpret_cast<const bf16x8*>(sa + (wm * T::WM + j * 32 + frow) * kRowBytes + chunk);
#pragma unroll
        for (int i = 0; i < T::TN; ++i)
#pragma unroll
          for (int j = 0; j < T::TM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fx[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) lstore((kt + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue: stage the bf16 tile, resolve row destinations, send rows
    if (tid < BM) {
      const int m = m_abs + tid;
      s_rowdst[tid] = m < g1 ? row_destination(a, s_recv, e, m) : 0;
    }
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
#pragma unroll
      for (int j = 0; j < T::TM; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = wn * T::WN + i * 32 + 8 * g + 4 * fhalf;
          const int m = wm * T::WM + j * 32 + frow;
          u32x2 v;
          v[0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          v[1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<u32x2*>(smem + m * T::C_PITCH + n * 2) = v;
        }
    __syncthreads();
    constexpr int TPR = BN * 2 / 16;          // threads per row
    constexpr int RPP = kThreads / TPR;       // rows per pass
    const int rows = min(BM, g1 - m_abs);
    const int cr = tid / TPR, cc = tid % TPR;
    for (int r0 = 0; r0 < rows; r0 += RPP) {
      const int r = r0 + cr;
      if (r < rows) {
        const uint64_t dst = s_rowdst[r];
        if (dst) {
          u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * T::C_PITCH + cc * 16);
          store16_nt(reinterpret_cast<uint8_t*>(dst) + (size_t)n_abs * 2 + cc * 16, v);
        }
      }
    }
    if (a.sink_on) finish_tile(a, e, mt * nt);
    __syncthreads();
  }
}

template <int BM, int BN>
hipError_t launch_bf16(const GemmArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((gemm_scatter_bf16_kernel<BM, BN>), dim3(grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_rows(int tile) { return tile == kTile128x128 ? 128 : 256; }
int gemm_tile_cols(int tile) { return tile == kTile256x256 ? 256 : 128; }
int gemm_blocks_per_cu(int tile, int dtype) {
  (void)dtype;
  return tile == kTile128x128 ? 2 : 1;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, int grid, hipStream_t st) {
  switch (tile) {
    case kTile256x256: return launch_bf16<256, 256>(a, grid, st);
    case kTile128x128: return launch_bf16<128, 128>(a, grid, st);
    case kTile256x128: return launch_bf16<256, 128>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ep
