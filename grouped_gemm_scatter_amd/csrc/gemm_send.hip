// Grouped GEMM + sink with dedicated send waves ("EpiloguePeerSink", comptime
// member SendWarps and the methods service, drain and shutdown), bf16 in,
// fp32 accumulate, bf16 rows out, for gfx950.
//
// SendWarps counts the waves the sink takes above the MFMA waves, or 0 to run
// inside them.  With SW = 4 the workgroup is 8 MFMA waves (2 x 4, 64 x 32 each,
// 32 x 32 MFMA blocks) plus 4 send waves.  The MFMA waves never store a row:
// at the end of tile t they stage its bf16 output in an LDS buffer of its own
// and go on to tile t + 1, while the send waves (service) read the staged
// tile and send its rows to their receive slots, then, once their stores are
// acknowledged, count the tile towards its expert's completion (drain: what
// the previous tile left pending).  After the last tile the send waves
// send and count it and publish the finished experts (shutdown).  Every wave
// takes part in every workgroup barrier: the send waves step through the same
// barriers as the MFMA waves' K loop, doing their work between them, so the
// arrivals always match.
//
// LDS: three 32 KB stages (two K slices in flight) plus the 34 KB staged tile;
// the 256 x 256 tile of the main kernel cannot hold a staged tile beside its
// stages (128 KB of stages and 132 KB of staged output in 160 KB), which is why
// this kernel works on 128 x 128 tiles, one workgroup per CU.  SW = 0 is the
// same kernel with the MFMA waves staging and sending their own tile after the
// K loop (the sink inside the output waves), for comparison.
#include "gemm_bf16.h"

namespace ep {

namespace {

using namespace gemm;

using SendTile = Bf16Tile<128, 128, 2, 4, 64, 3>;
constexpr int kSendTilePitch = SendTile::BN * 2 + 16;   // staged row: 16-byte skew

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left unconstrained: this wave's
// LDS reads and writes are complete.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// MFMA waves: the finished accumulators (32 x 32 blocks, lane holding 4
// consecutive columns of one row per group) as bf16 rows of the staged tile.
template <class T, int JV>
__device__ __forceinline__ void stage_tile(const f32x16 (&acc)[T::TN][T::TM], uint8_t* s_c,
                                           int wm, int wn, int lane) {
  const int frow = lane & 31, fhalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
      if (j < JV) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = wn * T::WN + i * 32 + 8 * g + 4 * fhalf;
          const int m = wm * T::WM + j * 32 + frow;
          u32x2 v;
          v[0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          v[1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<u32x2*>(s_c + m * kSendTilePitch + n * 2) = v;
        }
      }
}

// Send waves (service): the `rows` valid rows of the staged tile go to their
// destinations (s_rowdst, 0 = not sent) with 16-byte nontemporal stores,
// NT threads, BN*2/16 threads per row.
template <class T, int NT>
__device__ __forceinline__ void send_staged(const uint8_t* s_c, const uint64_t* s_rowdst,
                                            int rows, int n_abs, int stid) {
  constexpr int TPR = T::BN * 2 / 16, RPP = NT / TPR;
  const int cr = stid / TPR, cc = stid % TPR;
  for (int r0 = 0; r0 < rows; r0 += RPP) {
    const int r = r0 + cr;
    if (r < rows) {
      const uint64_t dst = s_rowdst[r];
      if (dst) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(s_c + r * kSendTilePitch + cc * 16);
        store16_nt(reinterpret_cast<uint8_t*>(dst) + (size_t)n_abs * 2 + cc * 16, v);
      }
    }
  }
}

// The K loop of the MFMA waves: S = 3 stages, two slices in flight.  The
// prologue's copies of slices 0 and 1 are issued by the caller.  Each step
// copies slice k + 2 into the stage the previous step freed, multiplies slice
// k, waits until slice k + 1 has landed and meets the workgroup barrier: KT
// barriers in all.
template <class T, int JV, bool WS>
__device__ __forceinline__ void k_loop_send(f32x16 (&acc)[T::TN][T::TM], uint8_t* smem,
                                            uint32_t lds0, const CopyPlan<T, WS>& c, int KT,
                                            int wm, int wn, int lane) {
  constexpr int S = T::STAGES;
  for (int kt = 0; kt < KT; kt += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int k = kt + u;
      if (k >= KT) break;
      const bool ahead = k + S - 1 < KT;
      if (ahead) copy_slice(lds0 + ((u + S - 1) % S) * T::STAGE, c, k + S - 1);
      if constexpr (JV > 0) mma_slice<T, JV>(acc, smem + u * T::STAGE, wm, wn, lane);
      if (ahead)
        wait_vm<T::IPW>();
      else
        wait_vm<0>();
      raw_barrier();
    }
  }
}

// One tile of an MFMA wave: the K loop, then the accumulators staged as bf16
// (both with JV, this wave's MFMA row blocks before m_end, as a constant).
template <class T, int JV, bool WS>
__device__ __forceinline__ void mfma_tile(uint8_t* smem, uint32_t lds0, const CopyPlan<T, WS>& c,
                                          int KT, int wm, int wn, int lane, uint8_t* s_c) {
  f32x16 acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  k_loop_send<T, JV, WS>(acc, smem, lds0, c, KT, wm, wn, lane);
  stage_tile<T, JV>(acc, s_c, wm, wn, lane);
}

template <class T, int J, bool WS>
__device__ __forceinline__ void mfma_tile_jv(int jv, uint8_t* smem, uint32_t lds0,
                                             const CopyPlan<T, WS>& c, int KT, int wm, int wn,
                                             int lane, uint8_t* s_c) {
  if constexpr (J > 0) {
    if (jv != J) {
      mfma_tile_jv<T, J - 1, WS>(jv, smem, lds0, c, KT, wm, wn, lane, s_c);
      return;
    }
  }
  mfma_tile<T, J, WS>(smem, lds0, c, KT, wm, wn, lane, s_c);
}

template <int SW, bool WS>
__global__ __launch_bounds__(64 * (SendTile::WAVES + SW)) void gemm_scatter_send_kernel(
    GemmArgs a) {
  using T = SendTile;
  constexpr int BM = T::BM, BN = T::BN;
  constexpr int THREADS = 64 * (T::WAVES + SW);
  constexpr int SEND_THREADS = 64 * SW;
  static_assert(SW == 0 || SW == 4, "send waves");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_MAIN];
  __shared__ __attribute__((aligned(16))) uint8_t s_c[BM * kSendTilePitch];
  __shared__ uint64_t s_rowdst[BM];
  __shared__ int s_base[kMaxLocalExperts + 1];
  __shared__ int s_gbeg[kMaxLocalExperts + 1];
  __shared__ uint8_t* s_recv[kMaxRanks];
  __shared__ int s_bad;
  __shared__ uint32_t s_done[kDoneWords];
  __shared__ int s_pend[kPendingMax];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves 0..SW-1 send (thread 0, which counts and publishes, is a sender);
  // the rest run the MFMAs
  const bool sender = wave < SW;
  const int mw = wave - SW;
  const int wm = mw / T::WAVES_N, wn = mw % T::WAVES_N;
  const int mtid = tid - SEND_THREADS;     // thread index among the MFMA waves
  const int K = a.K, N = a.N;
  const int El = a.s.n_experts;

  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) s_recv[i] = a.s.recv[i];
  }
  init_done(s_done);
  if (!build_work_table<BM, THREADS>(a, N / BN, s_base, s_gbeg, &s_bad)) return;
  const int total = s_base[El];
  const int G = gridDim.x;                  // a multiple of 8
  const int per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  PendingTiles pending;
  pending.done = s_done;
  pending.e = s_pend;
  pending.base = s_base;

  CopyPlan<T, WS> cp;
  cp.q0 = (sender ? 0 : mw) * T::IPW;
  const bool copies_a = cp.q0 < BM / T::ROWS_PER_COPY;
  if constexpr (WS) cp.kstride = copies_a ? (uint32_t)T::RB : (uint32_t)N * 128u;
  const int r0 = (copies_a ? cp.q0 : cp.q0 - BM / T::ROWS_PER_COPY) * T::ROWS_PER_COPY +
                 lane / T::CPR;
  const uint32_t lds0 = lds_addr(smem);
  const int KT = K / T::BK;

  TileWork prev{};                          // send waves: the tile staged in s_c
  bool have_prev = false;
  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= total) break;
    const TileWork t = tile_of<BM, BN>(a, s_base, s_gbeg, item);
    if (t.empty) {
      signal_empty_expert(a, t.e, pending);
      continue;
    }
    // rows of this tile: their coordinates load under the K loop
    const int rtid = SW ? tid : mtid;       // the BM threads that own one row each
    const RowInfo ri = (rtid >= 0 && rtid < BM) ? load_row_info(a, t.e, t.g1, t.m_abs + rtid)
                                                : RowInfo{-1, 0, 0};
    if (!sender) {
      cp.base = copies_a ? a.x
                         : a.w + (size_t)t.e * N * K * 2 + (WS ? (size_t)t.n_abs * 128 : 0);
      const int gr0 = (copies_a ? t.m_abs : (WS ? 0 : t.n_abs)) + r0;
      const int glim = copies_a ? t.g1 - 1 : 0x7fffffff;
      const uint32_t row_bytes = (WS && !copies_a) ? 128u : (uint32_t)(K * 2);
#pragma unroll
      for (int j = 0; j < T::IPW; ++j) {
        const int r = r0 + j * T::ROWS_PER_COPY;
        const uint32_t chunk = ((lane % T::CPR) ^ ((r >> T::SWZ_SHIFT) & (T::CPR - 1))) * 16;
        cp.voff[j] = (uint32_t)min(gr0 + j * T::ROWS_PER_COPY, glim) * row_bytes + chunk;
      }
      copy_slice(lds0, cp, 0);
      if (KT > 1) copy_slice(lds0 + T::STAGE, cp, 1);
      // SW = 0: a batch of earlier tiles is counted after this barrier, so
      // every earlier row store must be complete first
      if (KT > 1 && (SW > 0 || pending.n < kPendingMax))
        wait_vm<T::IPW>();
      else
        wait_vm<0>();
    } else if (have_prev) {
      // service: the previous tile's rows go out while the MFMA waves run
      // this one
      send_staged<T, SEND_THREADS>(s_c, s_rowdst, prev.rows, prev.n_abs, tid);
    }
    if constexpr (SW > 0) {
      wait_lds();                           // the staged tile and its rows are read
      raw_barrier();
    } else {
      prologue_barrier(a, pending);         // counts a full batch of earlier tiles
    }
    const int jv = min(T::TM, max(0, (t.rows - wm * T::WM + 31) / 32));
    if (!sender) {
      mfma_tile_jv<T, T::TM, WS>(jv, smem, lds0, cp, KT, wm, wn, lane, s_c);
    } else {
      for (int k = 0; k < KT; ++k) raw_barrier();   // the K loop's barriers
      if (have_prev) {
        // drain: the previous tile's stores are acknowledged; count it after
        // the barrier below
        wait_vm<0>();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      }
    }
    if constexpr (SW > 0) {
      // this tile's row destinations; then the staged tile is complete
      if (sender && tid < BM) s_rowdst[tid] = row_destination(a, s_recv, ri, t.m_abs + tid);
      wait_lds();
      raw_barrier();
      if (sender) {
        if (have_prev) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          if (tid == 0) pending.e[pending.n] = prev.e;
          ++pending.n;
          if (pending.n >= kPendingMax) complete_pending(a, pending);
        }
        prev = t;
        have_prev = true;
      }
    } else {
      // the sink inside the MFMA waves: rows sent right after staging
      if (mtid < BM) s_rowdst[mtid] = row_destination(a, s_recv, ri, t.m_abs + mtid);
      wait_lds();
      raw_barrier();
      // (the next tile's stage and row destinations are written after its K
      // loop's barriers, long after these reads)
      send_staged<T, THREADS>(s_c, s_rowdst, t.rows, t.n_abs, mtid);
      if (tid == 0) pending.e[pending.n] = t.e;
      ++pending.n;
    }
  }
  if constexpr (SW > 0) {
    // shutdown: the last staged tile goes out and is counted, with the
    // arrivals of the MFMA waves matched by one last barrier
    if (sender && have_prev) {
      send_staged<T, SEND_THREADS>(s_c, s_rowdst, prev.rows, prev.n_abs, tid);
      wait_vm<0>();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    }
    raw_barrier();
    if (!sender) return;
    if (have_prev) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (tid == 0) pending.e[pending.n] = prev.e;
      ++pending.n;
    }
    complete_pending(a, pending);
  }
  flush_pending(a, pending);   // SW > 0: nothing left to count, publication only
}

}  // namespace

hipError_t launch_gemm_send(const GemmArgs& a, int send_waves, int grid, hipStream_t st) {
  constexpr int W = SendTile::WAVES;
  if (send_waves == 4) {
    if (a.w_slice_major)
      hipLaunchKernelGGL((gemm_scatter_send_kernel<4, true>), dim3(grid), dim3(64 * (W + 4)), 0,
                         st, a);
    else
      hipLaunchKernelGGL((gemm_scatter_send_kernel<4, false>), dim3(grid), dim3(64 * (W + 4)), 0,
                         st, a);
  } else if (send_waves == 0) {
    if (a.w_slice_major)
      hipLaunchKernelGGL((gemm_scatter_send_kernel<0, true>), dim3(grid), dim3(64 * W), 0, st, a);
    else
      hipLaunchKernelGGL((gemm_scatter_send_kernel<0, false>), dim3(grid), dim3(64 * W), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ep
