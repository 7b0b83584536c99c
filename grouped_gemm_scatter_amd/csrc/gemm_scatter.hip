// Grouped GEMM with the receive-buffer sink epilogue, bf16 in, fp32
// accumulate, bf16 rows out, for gfx950.
//
// Work decomposition.  Every local expert e owns the row group
// [offsets[e*R], offsets[(e+1)*R]) of X; its output C_e = X_e * W_e is cut into
// tiles of BN columns and up to BM rows (the 256-column tile spreads an
// expert's 32-row blocks evenly over its row tiles, see row_tiles).  An expert
// with no rows still gets one work item, which only publishes its zero
// counts, so that every rank's election completes ("ep_signal_completion",
// parameter n_experts_per_device: the election bound).
// The grid is persistent; items are handed out so that each XCD (workgroups
// are dispatched round-robin over the 8 XCDs) walks a contiguous range of
// items, which keeps the X rows and W_e slabs of neighbouring tiles in that
// XCD's L2.
//
// Main loop.  WAVES_M x WAVES_N waves, two per SIMD for the large tile, so
// one wave's MFMAs cover the other's LDS and barrier waits.  Each wave owns a
// sub-tile of up to TM x TN 32 x 32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16).  W_e feeds the MFMA's first operand and X its
// second, so each lane's accumulator holds four consecutive output columns of
// one row, which packs into one 8-byte LDS store in the epilogue.  K slices of
// 64 are copied global -> LDS directly (global_load_lds_dwordx4, no register
// staging), double-buffered, in a 16-byte-chunk XOR swizzle that keeps the
// fragment reads conflict-free.  In the last tile of a ragged group, MFMA
// blocks whose 32 rows all lie past m_end are skipped.
//
// Epilogue ("EpiloguePeerSink", send_tile: the finished tile replaces the
// local store): see gemm_common.h.
#include <type_traits>

#include "gemm_bf16.h"

namespace ep {

namespace {

using namespace gemm;

// Copies of a tile whose X and W_e copies do not fall into whole waves (the
// up-projection's 256 x 128 half tile: 32 X copies and 16 W_e copies per
// slice): every wave moves A_PER_WAVE copies of X rows and B_PER_WAVE of W_e
// rows.
template <class T>
struct SplitPlan {
  static constexpr int A_COPIES = T::BM / T::ROWS_PER_COPY;
  static constexpr int A_PER_WAVE = A_COPIES / T::WAVES;
  static constexpr int B_PER_WAVE = T::BN / T::ROWS_PER_COPY / T::WAVES;
  static_assert(A_PER_WAVE * T::WAVES == A_COPIES &&
                B_PER_WAVE * T::WAVES * T::ROWS_PER_COPY == T::BN, "copy split");
  static_assert(T::RB == 128, "64-element K slices");
  const uint8_t* xa;          // X
  const uint8_t* wb;          // W_e
  uint32_t voff_a[A_PER_WAVE];
  uint32_t voff_b[B_PER_WAVE];
  int wave;
};

template <class T>
__device__ __forceinline__ void copy_slice(uint32_t st, const SplitPlan<T>& c, int kt) {
  using P = SplitPlan<T>;
  const size_t kb = (size_t)kt * T::RB;
  const uint8_t* xa = uniform_ptr(c.xa + kb);
  const uint8_t* wb = uniform_ptr(c.wb + kb);
#pragma unroll
  for (int j = 0; j < P::A_PER_WAVE; ++j)
    g2lds16s(xa, c.voff_a[j], st + (c.wave * P::A_PER_WAVE + j) * 1024);
#pragma unroll
  for (int j = 0; j < P::B_PER_WAVE; ++j)
    g2lds16s(wb, c.voff_b[j], st + (P::A_COPIES + c.wave * P::B_PER_WAVE + j) * 1024);
}

// Copies of the tall tile (288 x 256): waves 0-3 move X rows [64w, 64w + 64)
// (8 copies each), waves 4-7 W_e rows [64(w-4), 64(w-4) + 64) (8 copies each)
// and, in a tile of more than 256 rows, X rows [256 + 8(w-4), 264 + 8(w-4))
// (one copy each).  Every wave's copies of one operand share a wave-uniform
// base; `extra` is the same in every lane of a wave.
template <class T, bool WS>
struct TallPlan {
  static_assert(T::BM == 288 && T::BN == 256 && T::WAVES == 8 && T::RB == 128, "tall tile");
  const uint8_t* base;        // X (waves 0-3) or W_e (waves 4-7)
  const uint8_t* xbase;       // X, for the copy of rows 256..287
  uint32_t voff[8];
  uint32_t voff_x;
  uint32_t dst0;              // LDS offset of the wave's first copy inside a stage
  uint32_t dst_x;             // LDS offset of its copy of rows 256..287
  uint32_t kstride;           // WS: bytes from one K slice of `base` to the next
  bool extra;
};

template <class T, bool WS>
__device__ __forceinline__ void copy_slice(uint32_t st, const TallPlan<T, WS>& c, int kt) {
  const uint8_t* base = uniform_ptr(c.base + (size_t)kt * (WS ? c.kstride : T::RB));
#pragma unroll
  for (int j = 0; j < 8; ++j) g2lds16s(base, c.voff[j], st + c.dst0 + j * 1024);
  if (c.extra) g2lds16s(uniform_ptr(c.xbase + (size_t)kt * T::RB), c.voff_x, st + c.dst_x);
}

// The tall tile's copy plan for tile t (see TallPlan); rows past m_end
// re-read the group's last row.
template <class T, bool WS>
__device__ __forceinline__ void tall_plan(TallPlan<T, WS>& c, const GemmArgs& a,
                                          const TileWork& t, int wave, int lane) {
  const int K = a.K, N = a.N;
  const bool xw = wave < 4;
  const int sub = lane / T::CPR;
  auto chunk_of = [&](int r) {
    return (uint32_t)(((lane % T::CPR) ^ ((r >> T::SWZ_SHIFT) & (T::CPR - 1))) * 16);
  };
  c.base = xw ? a.x : a.w + (size_t)t.e * N * K * 2 + (WS ? (size_t)t.n_abs * 128 : 0);
  if constexpr (WS) c.kstride = xw ? (uint32_t)T::RB : (uint32_t)N * 128u;
  c.dst0 = xw ? (uint32_t)wave * 8 * 1024 : (uint32_t)(T::A_BYTES + (wave - 4) * 8 * 1024);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (xw) {
      const int r = wave * 64 + j * 8 + sub;
      c.voff[j] = (uint32_t)min(t.m_abs + r, t.g1 - 1) * (uint32_t)(K * 2) + chunk_of(r);
    } else {
      const int r = (wave - 4) * 64 + j * 8 + sub;
      c.voff[j] = (WS ? (uint32_t)r * 128u : (uint32_t)(t.n_abs + r) * (uint32_t)(K * 2)) +
                  chunk_of(r);
    }
  }
  c.xbase = a.x;
  {
    const int r = 256 + (xw ? 0 : wave - 4) * 8 + sub;
    c.voff_x = (uint32_t)min(t.m_abs + r, t.g1 - 1) * (uint32_t)(K * 2) + chunk_of(r);
    c.dst_x = (uint32_t)(32 + (xw ? 0 : wave - 4)) * 1024;
  }
  c.extra = __builtin_amdgcn_readfirstlane((int)(!xw && t.rows > 256)) != 0;
}

// The K loop of one tile, two LDS stages, one slice in flight.  Each step
// copies slice k + 1 into the stage freed by the previous step, multiplies
// slice k, waits for its own copies and synchronises the workgroup.  Steps go
// in pairs (stage 0, stage 1) so that every stage index is a constant and the
// loop has a single exit; an odd last slice gets a step of its own.  Only the
// first JV MFMA row blocks of this wave are computed (the others lie past
// m_end).  The previous tile's pending completion is done right after the
// prologue's barrier.
template <class T, int JV, int U, class P>
__device__ __forceinline__ void k_step(f32x16 (&acc)[T::TN][T::TM], uint8_t* smem,
                                       uint32_t lds0, const P& c, int k, bool next,
                                       int wm, int wn, int lane) {
  if (next) copy_slice(lds0 + (1 - U) * T::STAGE, c, k + 1);
  if constexpr (JV > 0) mma_slice<T, JV>(acc, smem + U * T::STAGE, wm, wn, lane);
  wait_vm<0>();
  raw_barrier();
}

template <class T, int JV, class P>
__device__ __forceinline__ void k_loop(f32x16 (&acc)[T::TN][T::TM], uint8_t* smem,
                                       uint32_t lds0, const P& c, int KT, int wm,
                                       int wn, int lane, const GemmArgs& a,
                                       PendingTiles& pending) {
  static_assert(T::STAGES == 2, "two-stage loop");
  copy_slice(lds0, c, 0);
  wait_vm<0>();
  // every wave's stores of the earlier tiles are now complete: count them
  prologue_barrier(a, pending);
  int k = 0;
  for (; k + 1 < KT; k += 2) {
    k_step<T, JV, 0>(acc, smem, lds0, c, k, true, wm, wn, lane);
    k_step<T, JV, 1>(acc, smem, lds0, c, k + 1, k + 2 < KT, wm, wn, lane);
  }
  if (k < KT) k_step<T, JV, 0>(acc, smem, lds0, c, k, false, wm, wn, lane);
}

// One tile: zeroed accumulators, the K loop, the sink epilogue.
template <class T, int JV, class P>
__device__ __forceinline__ void run_tile(const GemmArgs& a, uint8_t* smem, uint32_t lds0,
                                         const P& cp, int KT, int wm, int wn, int lane,
                                         const TileWork& t, const RowInfo& ri,
                                         uint64_t* s_rowdst, uint8_t* const* s_recv,
                                         PendingTiles& pending) {
  f32x16 acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  k_loop<T, JV>(acc, smem, lds0, cp, KT, wm, wn, lane, a, pending);
  send_tile<T::BM, T::BN, T::WM, T::WN, T::TM, T::TN, T::THREADS>(a, acc, smem, s_rowdst, s_recv,
                                                                   t, wm, wn, JV, ri, pending);
}

// Runs the tile with JV = jv, the count of this wave's 32-row MFMA blocks
// that hold rows before m_end (TM for every wave of a full tile), as a
// compile-time constant: each variant is branch-free in its K loop.  Waves of
// one workgroup may take different variants; all of them copy, wait and
// synchronise alike.
template <class T, int J, class P>
__device__ __forceinline__ void run_tile_jv(int jv, const GemmArgs& a, uint8_t* smem,
                                            uint32_t lds0, const P& cp, int KT, int wm,
                                            int wn, int lane, const TileWork& t,
                                            const RowInfo& ri, uint64_t* s_rowdst,
                                            uint8_t* const* s_recv, PendingTiles& pending) {
  if constexpr (J > 0) {
    if (jv != J) {
      run_tile_jv<T, J - 1>(jv, a, smem, lds0, cp, KT, wm, wn, lane, t, ri, s_rowdst, s_recv,
                            pending);
      return;
    }
  }
  run_tile<T, J>(a, smem, lds0, cp, KT, wm, wn, lane, t, ri, s_rowdst, s_recv, pending);
}

// The half tile of a 256-column tile (the up-projection's split last round).
template <class T>
using HalfTile = Bf16Tile<T::BM, T::BN / 2, T::WAVES_M, T::WAVES_N, T::BK, T::STAGES>;

template <class T, bool EPI, bool TRACE, bool FUSED, bool WS>
__global__ __launch_bounds__(T::THREADS) void gemm_scatter_bf16_kernel(GemmArgs a) {
  constexpr int BM = T::BM, BN = T::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
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
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int K = a.K, N = a.N;
  const int El = a.s.n_experts;

  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) s_recv[i] = a.s.recv[i];
  }
  init_done(s_done);
  if (!build_work_table<BM, T::THREADS, T::BAL>(a, N / BN, s_base, s_gbeg, &s_bad)) return;
  const int total = s_base[El];

  const int G = gridDim.x;                  // a multiple of 8
  const int per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  PendingTiles pending;
  pending.done = s_done;
  pending.e = s_pend;
  pending.base = s_base;
  if constexpr (EPI) {
    epilogue_only_loop<BM, BN, T::WM, T::WN, T::TM, T::TN, T::THREADS, T::TM0, T::BAL>(
        a, smem, s_rowdst, s_recv, s_base, s_gbeg, pending, xcd * per_xcd + slot, G, total, wm,
        wn);
    flush_pending(a, pending);
    return;
  }
  constexpr bool kTall = T::BAL > 0;
  using Plan = std::conditional_t<kTall, TallPlan<T, WS>, CopyPlan<T, WS>>;
  Plan cp;
  bool copies_a = false;
  int r0 = 0;
  if constexpr (!kTall) {
    cp.q0 = wave * T::IPW;
    copies_a = cp.q0 < BM / T::ROWS_PER_COPY;
    if constexpr (WS) cp.kstride = copies_a ? (uint32_t)T::RB : (uint32_t)N * 128u;
    // first tile row this lane copies, and its chunk: the swizzle of row
    // r0 + j*RPC depends on j only through j*RPC >> SWZ_SHIFT
    r0 = (copies_a ? cp.q0 : cp.q0 - BM / T::ROWS_PER_COPY) * T::ROWS_PER_COPY + lane / T::CPR;
  }
  const uint32_t lds0 = lds_addr(smem);

  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= total) break;
    const TileWork t = tile_of<BM, BN, 0, T::BAL>(a, s_base, s_gbeg, item);
    if (t.empty) {
      signal_empty_expert(a, t.e, pending);
      continue;
    }
    if constexpr (kTall) {
      tall_plan(cp, a, t, wave, lane);
    } else {
      // Lane L fills physical chunk L % CPR of row r = row0 + j*RPC + L / CPR,
      // which holds logical chunk (L % CPR) ^ swizzle(r).  Rows past m_end
      // re-read the group's last row.
      // (slice-major W: the base at the tile's first row, rows 128 bytes apart)
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
    }

    const RowInfo ri = tid < BM ? load_row_info(a, t.e, t.g1, t.m_abs + tid) : RowInfo{-1, 0, 0};
    const int KT = K / T::BK;
    const int jv = min(wm == 0 ? T::TM0 : T::TM, max(0, (t.rows - wm * T::WM + 31) / 32));
    if constexpr (TRACE) trace_start(a, item);
    run_tile_jv<T, T::TM>(jv, a, smem, lds0, cp, KT, wm, wn, lane, t, ri, s_rowdst, s_recv,
                          pending);
    if constexpr (TRACE) trace_end(a, item, t, BN);
  }
  flush_pending(a, pending);
  if constexpr (FUSED) fused_consume(a, &s_bad);
}

// ---------------------------------------------------------------------------
// Small row groups (decode): with a few dozen rows per expert the GEMM is a
// stream of W_e, so this tile keeps three K slices in flight instead of the
// big tile's one (two 64 KB stages fill the LDS there, half of each slice
// re-reads of the same few X rows).  64 x 128, 2 x 4 waves of 32 x 32, four
// 24 KB stages: every row of an expert with up to 64 rows lies in one item,
// so W_e is streamed once, and E_l * N / 128 items (1792 at N = 7168) divide
// evenly over a grid of 256 workgroups.
// Copies: the X rows of a slice are split into 1 KB copies by the first
// BM / 8 waves (a wave skips its copy when all its rows lie past m_end); each
// wave then moves BN / 8 / 8 copies of W_e rows.

using DecodeTile = Bf16Tile<64, 128, 2, 4, 64, 4>;

template <class T, bool WS = false>
struct DecodeCopies {
  static constexpr int A_COPIES = T::BM / T::ROWS_PER_COPY;
  static constexpr int B_PER_WAVE = T::BN / T::ROWS_PER_COPY / T::WAVES;
  static_assert(A_COPIES <= T::WAVES && B_PER_WAVE * T::ROWS_PER_COPY * T::WAVES == T::BN,
                "copy split");
  static_assert(T::TM == 1 && T::TN == 1 && T::WM == 32 && T::WN == 32, "32 x 32 per wave");
  static_assert(T::RB == 128, "64-element K slices");
  const uint8_t* xa;          // X
  const uint8_t* wb;          // W_e
  uint32_t voff_a;            // lane offset of the wave's X copy
  uint32_t voff_b[B_PER_WAVE];
  int wave;
  uint32_t wstride;           // WS: bytes from one K slice of W_e to the next
  bool has_a;                 // this wave copies X rows in this tile
};

template <class T, bool WS>
__device__ __forceinline__ void copy_slice_dec(uint32_t st, const DecodeCopies<T, WS>& c, int kt) {
  using C = DecodeCopies<T, WS>;
  const size_t kb = (size_t)kt * T::RB;
  if (c.has_a) g2lds16s(c.xa + kb, c.voff_a, st + c.wave * 1024);
  const uint8_t* wb = c.wb + (WS ? (size_t)kt * c.wstride : kb);
#pragma unroll
  for (int j = 0; j < C::B_PER_WAVE; ++j)
    g2lds16s(wb, c.voff_b[j], st + (C::A_COPIES + c.wave * C::B_PER_WAVE + j) * 1024);
}

// Waits until at most `n` slices of this wave's copies are in flight.
template <class T, bool WS>
__device__ __forceinline__ void wait_dec(const DecodeCopies<T, WS>& c, int n) {
  using C = DecodeCopies<T, WS>;
  if (c.has_a) wait_slices<C::B_PER_WAVE + 1, T::STAGES - 2>(n);
  else wait_slices<C::B_PER_WAVE, T::STAGES - 2>(n);
}

// K loop: each step copies slice k + S - 1 into the stage freed by the
// previous step, multiplies slice k, waits for slice k + 1 and synchronises.
template <class T, int JV, bool WS>
__device__ __forceinline__ void k_loop_dec(f32x16 (&acc)[1][1], uint8_t* smem, uint32_t lds0,
                                           const DecodeCopies<T, WS>& c, int KT, int wm, int wn,
                                           int lane, const GemmArgs& a, PendingTiles& pending) {
  constexpr int S = T::STAGES;
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KT) copy_slice_dec(lds0 + p * T::STAGE, c, p);
  wait_dec(c, min(S - 2, KT - 1));
  // every wave's stores of the earlier tiles are now complete: count them
  prologue_barrier(a, pending);
  for (int kt = 0; kt < KT; kt += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int k = kt + u;
      if (k >= KT) break;
      if (k + S - 1 < KT) copy_slice_dec(lds0 + ((u + S - 1) % S) * T::STAGE, c, k + S - 1);
      if constexpr (JV > 0) mma_slice<T, JV>(acc, smem + u * T::STAGE, wm, wn, lane);
      wait_dec(c, max(0, min(S - 2, KT - 2 - k)));
      raw_barrier();
    }
  }
}

template <class T, int JV, bool WS>
__device__ __forceinline__ void run_tile_dec(const GemmArgs& a, uint8_t* smem, uint32_t lds0,
                                             const DecodeCopies<T, WS>& c, int KT, int wm, int wn,
                                             int lane, const TileWork& t, const RowInfo& ri,
                                             uint64_t* s_rowdst, uint8_t* const* s_recv,
                                             PendingTiles& pending) {
  f32x16 acc[1][1];
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[0][0][r] = 0.f;
  k_loop_dec<T, JV, WS>(acc, smem, lds0, c, KT, wm, wn, lane, a, pending);
  send_tile<T::BM, T::BN, T::WM, T::WN, T::TM, T::TN, T::THREADS>(a, acc, smem, s_rowdst, s_recv,
                                                                   t, wm, wn, JV, ri, pending);
}

template <class T, bool EPI, bool TRACE, bool FUSED, bool WS>
__global__ __launch_bounds__(T::THREADS) void gemm_scatter_bf16_decode_kernel(GemmArgs a) {
  using C = DecodeCopies<T, WS>;
  constexpr int BM = T::BM, BN = T::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
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
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int K = a.K, N = a.N;
  const int El = a.s.n_experts;

  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) s_recv[i] = a.s.recv[i];
  }
  init_done(s_done);
  if (!build_work_table<BM, T::THREADS>(a, N / BN, s_base, s_gbeg, &s_bad)) return;
  const int total = s_base[El];

  const int G = gridDim.x;                  // a multiple of 8
  const int per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const uint32_t lds0 = lds_addr(smem);

  PendingTiles pending;
  pending.done = s_done;
  pending.e = s_pend;
  pending.base = s_base;
  if constexpr (EPI) {
    epilogue_only_loop<BM, BN, T::WM, T::WN, T::TM, T::TN, T::THREADS>(
        a, smem, s_rowdst, s_recv, s_base, s_gbeg, pending, xcd * per_xcd + slot, G, total, wm,
        wn);
    flush_pending(a, pending);
    return;
  }
  C c;
  c.wave = wave;
  c.xa = a.x;
  if constexpr (WS) c.wstride = (uint32_t)N * 128u;
  // lane L fills physical chunk L % 8 of row 8q + L / 8 (q: the copy's index
  // within its operand), which holds logical chunk (L % 8) ^ swizzle(row)
  const int sub = lane / T::CPR;
  auto chunk_of = [&](int r) {
    return (uint32_t)(((lane % T::CPR) ^ ((r >> T::SWZ_SHIFT) & (T::CPR - 1))) * 16);
  };
  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= total) break;
    const TileWork t = tile_of<BM, BN>(a, s_base, s_gbeg, item);
    if (t.empty) {
      signal_empty_expert(a, t.e, pending);
      continue;
    }
    c.wb = a.w + (size_t)t.e * N * K * 2 + (WS ? (size_t)t.n_abs * 128 : 0);
    c.has_a = wave < C::A_COPIES && wave * T::ROWS_PER_COPY < t.rows;
    {
      const int r = wave * T::ROWS_PER_COPY + sub;   // rows past m_end re-read the last row
      c.voff_a = (uint32_t)min(t.m_abs + r, t.g1 - 1) * (uint32_t)(K * 2) + chunk_of(r);
    }
#pragma unroll
    for (int j = 0; j < C::B_PER_WAVE; ++j) {
      const int r = (wave * C::B_PER_WAVE + j) * T::ROWS_PER_COPY + sub;
      c.voff_b[j] = (WS ? (uint32_t)r * 128u : (uint32_t)(t.n_abs + r) * (uint32_t)(K * 2)) +
                    chunk_of(r);
    }
    const RowInfo ri = tid < BM ? load_row_info(a, t.e, t.g1, t.m_abs + tid) : RowInfo{-1, 0, 0};
    const int KT = K / T::BK;
    // this wave's 32-row block holds rows of the tile, or none
    if constexpr (TRACE) trace_start(a, item);
    if (t.rows > wm * 32)
      run_tile_dec<T, 1, WS>(a, smem, lds0, c, KT, wm, wn, lane, t, ri, s_rowdst, s_recv, pending);
    else
      run_tile_dec<T, 0, WS>(a, smem, lds0, c, KT, wm, wn, lane, t, ri, s_rowdst, s_recv, pending);
    if constexpr (TRACE) trace_end(a, item, t, BN);
  }
  flush_pending(a, pending);
  if constexpr (FUSED) fused_consume(a, &s_bad);
}

// ---------------------------------------------------------------------------
// Up-projection with SwiGLU, the expert FFN's first GEMM, whose output is the
// X of the down-projection above:
//   H[m][i] = silu(X1[m] . Wg_e[i]) * (X1[m] . Wu_e[i]),  silu(g) = g / (1 + e^-g),
// for the rows m of expert e's group, with W1_e = [Wg_e; Wu_e] stored
// [2I][hidden] (K-contiguous).  Same tile, copies and K loop as the
// down-projection (K = hidden, 2I GEMM columns); the 256 B rows of a tile are
// permuted so that each wave's 64 columns are 32 gate rows followed by the 32
// matching up rows: every lane then holds the gate and up accumulators of the
// same output elements, and the activation runs on fp32 registers before the
// one bf16 rounding.  A tile yields 256 x 128 outputs, staged in LDS and
// stored as 256-byte row pieces.  No sink, no completion signalling.

// W1 row of GEMM column c of a tile whose output columns start at i0 and
// whose waves own WN columns each: WN / 2 gate rows, then the matching up rows.
template <int WN>
__device__ __forceinline__ int swiglu_w_row(int c, int i0, int I) {
  constexpr int H = WN / 2;
  return ((c % WN) >= H ? I : 0) + i0 + (c / WN) * H + (c % H);
}

template <class T>
__device__ __forceinline__ void swiglu_tile(const GemmArgs& a, const f32x16 (&acc)[T::TN][T::TM],
                                            uint8_t* smem, const TileWork& t, int wm, int wn,
                                            int jv) {
  // a lane holds columns 8g + 4 * (lane / 32) + q (q < 4) of each 32-column
  // block: with 64 columns per wave the up block is the second one (same
  // group g); with 32 (half tiles) groups 2 and 3 hold the up columns of
  // groups 0 and 1
  static_assert((T::TN == 2 && T::WN == 64) || (T::TN == 1 && T::WN == 32), "gate/up layout");
  constexpr int GROUPS = T::TN == 2 ? 4 : 2;  // 8-column groups of gate columns per lane
  constexpr int OC = T::BN / 2;              // output columns per tile
  constexpr int PITCH = OC * 2 + 16;         // bytes per staged row (skewed)
  const int tid = threadIdx.x, lane = tid & 63;
  const int frow = lane & 31, fhalf = lane >> 5;
#pragma unroll
  for (int j = 0; j < T::TM; ++j)
    if (j < jv) {
#pragma unroll
      for (int g = 0; g < GROUPS; ++g) {
        float h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gv = acc[0][j][4 * g + q];
          float uv;
          if constexpr (T::TN == 2)
            uv = acc[1][j][4 * g + q];
          else
            uv = acc[0][j][4 * (g + 2) + q];
          h[q] = gv / (1.0f + __expf(-gv)) * uv;
        }
        const int m = wm * T::WM + j * 32 + frow;
        const int o = wn * (T::WN / 2) + 8 * g + 4 * fhalf;
        u32x2 v;
        v[0] = pack_bf16x2(h[0], h[1]);
        v[1] = pack_bf16x2(h[2], h[3]);
        *reinterpret_cast<u32x2*>(smem + m * PITCH + o * 2) = v;
      }
    }
  __syncthreads();
  constexpr int TPR = OC * 2 / 16;           // threads per row
  constexpr int RPP = T::THREADS / TPR;      // rows per pass
  const int cr = tid / TPR, cc = tid % TPR;
  const size_t I = (size_t)(a.N / 2);
  for (int r0 = 0; r0 < t.rows; r0 += RPP) {
    const int r = r0 + cr;
    if (r < t.rows) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * PITCH + cc * 16);
      store16_nt(a.c_local + ((size_t)(t.m_abs + r) * I + t.n_abs / 2) * 2 + cc * 16, v);
    }
  }
  __syncthreads();   // the staged tile is read; the next tile may overwrite LDS
}

template <class T, int JV, class P>
__device__ __forceinline__ void run_tile_swiglu(const GemmArgs& a, uint8_t* smem, uint32_t lds0,
                                                const P& cp, int KT, int wm, int wn,
                                                int lane, const TileWork& t,
                                                PendingTiles& pending) {
  f32x16 acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  k_loop<T, JV>(acc, smem, lds0, cp, KT, wm, wn, lane, a, pending);
  swiglu_tile<T>(a, acc, smem, t, wm, wn, JV);
}

template <class T, int J, class P>
__device__ __forceinline__ void run_tile_swiglu_jv(int jv, const GemmArgs& a, uint8_t* smem,
                                                   uint32_t lds0, const P& cp, int KT,
                                                   int wm, int wn, int lane, const TileWork& t,
                                                   PendingTiles& pending) {
  if constexpr (J > 0) {
    if (jv != J) {
      run_tile_swiglu_jv<T, J - 1>(jv, a, smem, lds0, cp, KT, wm, wn, lane, t, pending);
      return;
    }
  }
  run_tile_swiglu<T, J>(a, smem, lds0, cp, KT, wm, wn, lane, t, pending);
}

// Half `h` (GEMM columns [h * BN/2, (h + 1) * BN/2), output columns
// [h * BN/4, (h + 1) * BN/4) of the item's) of a split last-round item.
template <class T>
__device__ __forceinline__ void run_half_swiglu(const GemmArgs& a, uint8_t* smem, uint32_t lds0,
                                                const int* s_base, const int* s_gbeg, int item,
                                                int h, int wave, int wm, int wn, int lane,
                                                PendingTiles& pending) {
  using H = HalfTile<T>;
  using P = SplitPlan<H>;
  const int K = a.K, N = a.N, I = a.N / 2;
  TileWork t = tile_of<T::BM, T::BN>(a, s_base, s_gbeg, item);
  if (t.empty) return;
  t.n_abs += h * H::BN;
  P hp;
  hp.wave = wave;
  hp.xa = a.x;
  hp.wb = a.w + (size_t)t.e * N * K * 2;
  const int sub = lane / H::CPR;
  auto chunk_of = [&](int r) {
    return (uint32_t)(((lane % H::CPR) ^ ((r >> H::SWZ_SHIFT) & (H::CPR - 1))) * 16);
  };
#pragma unroll
  for (int j = 0; j < P::A_PER_WAVE; ++j) {
    const int r = (wave * P::A_PER_WAVE + j) * H::ROWS_PER_COPY + sub;
    hp.voff_a[j] = (uint32_t)min(t.m_abs + r, t.g1 - 1) * (uint32_t)(K * 2) + chunk_of(r);
  }
#pragma unroll
  for (int j = 0; j < P::B_PER_WAVE; ++j) {
    const int r = (wave * P::B_PER_WAVE + j) * H::ROWS_PER_COPY + sub;
    hp.voff_b[j] =
        (uint32_t)swiglu_w_row<H::WN>(r, t.n_abs / 2, I) * (uint32_t)(K * 2) + chunk_of(r);
  }
  const int jv = min(H::TM, max(0, (t.rows - wm * H::WM + 31) / 32));
  run_tile_swiglu_jv<H, H::TM>(jv, a, smem, lds0, hp, K / H::BK, wm, wn, lane, t, pending);
}

template <class T>
__global__ __launch_bounds__(T::THREADS) void gemm_swiglu_bf16_kernel(GemmArgs a) {
  constexpr int BM = T::BM, BN = T::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
  __shared__ int s_base[kMaxLocalExperts + 1];
  __shared__ int s_gbeg[kMaxLocalExperts + 1];
  __shared__ int s_bad;
  __shared__ uint32_t s_done[kDoneWords];
  __shared__ int s_pend[kPendingMax];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int K = a.K, N = a.N, I = a.N / 2;
  const int El = a.s.n_experts;

  init_done(s_done);
  if (!build_work_table<BM, T::THREADS>(a, N / BN, s_base, s_gbeg, &s_bad)) return;
  const int total = s_base[El];

  const int G = gridDim.x;                  // a multiple of 8
  const int per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;

  PendingTiles pending;                     // stays empty: no tile is counted
  pending.done = s_done;
  pending.e = s_pend;
  pending.base = s_base;
  CopyPlan<T> cp;
  cp.q0 = wave * T::IPW;
  const bool copies_a = cp.q0 < BM / T::ROWS_PER_COPY;
  const int r0 = (copies_a ? cp.q0 : cp.q0 - BM / T::ROWS_PER_COPY) * T::ROWS_PER_COPY +
                 lane / T::CPR;
  const uint32_t lds0 = lds_addr(smem);

  // a last round that would keep at most half of the grid busy runs as half
  // tiles, as in the down-projection
  int split = total;
  const int rem = total % G;
  if (rem > 0 && 2 * rem <= G) split = total - rem;

  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= split) {
      const int v = item - split;           // split is a multiple of G: v < G
      if (v < 2 * (total - split))
        run_half_swiglu<T>(a, smem, lds0, s_base, s_gbeg, split + v / 2, v & 1, wave, wm, wn,
                           lane, pending);
      break;
    }
    const TileWork t = tile_of<BM, BN>(a, s_base, s_gbeg, item);
    if (t.empty) continue;
    // as in the down-projection; B rows go through the gate/up permutation
    cp.base = copies_a ? a.x : a.w + (size_t)t.e * N * K * 2;
#pragma unroll
    for (int j = 0; j < T::IPW; ++j) {
      const int r = r0 + j * T::ROWS_PER_COPY;
      const uint32_t chunk = ((lane % T::CPR) ^ ((r >> T::SWZ_SHIFT) & (T::CPR - 1))) * 16;
      const int grow =
          copies_a ? min(t.m_abs + r, t.g1 - 1) : swiglu_w_row<T::WN>(r, t.n_abs / 2, I);
      cp.voff[j] = (uint32_t)grow * (uint32_t)(K * 2) + chunk;
    }
    const int KT = K / T::BK;
    const int jv = min(T::TM, max(0, (t.rows - wm * T::WM + 31) / 32));
    run_tile_swiglu_jv<T, T::TM>(jv, a, smem, lds0, cp, KT, wm, wn, lane, t, pending);
  }
}

template <class T, bool WS>
hipError_t launch_bf16(const GemmArgs& a, int grid, hipStream_t st) {
  if (a.epilogue_only)
    hipLaunchKernelGGL((gemm_scatter_bf16_kernel<T, true, false, false, WS>), dim3(grid), dim3(T::THREADS), 0,
                       st, a);
  else if (a.trace)
    hipLaunchKernelGGL((gemm_scatter_bf16_kernel<T, false, true, false, WS>), dim3(grid), dim3(T::THREADS), 0,
                       st, a);
  else if (a.fused) {
    const int g = fused_grid<gemm_scatter_bf16_kernel<T, false, false, true, WS>>(T::THREADS, a.num_cus);
    if (!g) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((gemm_scatter_bf16_kernel<T, false, false, true, WS>), dim3(g), dim3(T::THREADS), 0, st, a);
  }
  else
    hipLaunchKernelGGL((gemm_scatter_bf16_kernel<T, false, false, false, WS>), dim3(grid), dim3(T::THREADS),
                       0, st, a);
  return hipGetLastError();
}

template <class T, bool WS>
hipError_t launch_bf16_decode(const GemmArgs& a, int grid, hipStream_t st) {
  if (a.epilogue_only)
    hipLaunchKernelGGL((gemm_scatter_bf16_decode_kernel<T, true, false, false, WS>), dim3(grid),
                       dim3(T::THREADS), 0, st, a);
  else if (a.trace)
    hipLaunchKernelGGL((gemm_scatter_bf16_decode_kernel<T, false, true, false, WS>), dim3(grid),
                       dim3(T::THREADS), 0, st, a);
  else if (a.fused) {
    const int g = fused_grid<gemm_scatter_bf16_decode_kernel<T, false, false, true, WS>>(T::THREADS, a.num_cus);
    if (!g) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((gemm_scatter_bf16_decode_kernel<T, false, false, true, WS>), dim3(g), dim3(T::THREADS), 0, st, a);
  }
  else
    hipLaunchKernelGGL((gemm_scatter_bf16_decode_kernel<T, false, false, false, WS>), dim3(grid),
                       dim3(T::THREADS), 0, st, a);
  return hipGetLastError();
}

using Tile256 = Bf16Tile<256, 256, 2, 4, 64, 2>;
using Tile128 = Bf16Tile<128, 128, 2, 2, 64, 2>;

}  // namespace

hipError_t launch_swiglu_bf16(const GemmArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(gemm_swiglu_bf16_kernel<Tile256>, dim3(grid), dim3(Tile256::THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, int grid, hipStream_t st) {
  switch (tile) {
    case kTile256x256:
      return a.w_slice_major ? launch_bf16<TallTile, true>(a, grid, st)
                             : launch_bf16<TallTile, false>(a, grid, st);
    case kTile128x128:
      return a.w_slice_major ? launch_bf16<Tile128, true>(a, grid, st)
                             : launch_bf16<Tile128, false>(a, grid, st);
    case kTileDecode64x128:
      return a.w_slice_major ? launch_bf16_decode<DecodeTile, true>(a, grid, st)
                             : launch_bf16_decode<DecodeTile, false>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ep
