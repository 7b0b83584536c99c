// Blockwise-scaled fp8 grouped GEMM with the receive-buffer sink epilogue, for
// gfx950.  X and W_e hold OCP e4m3fn codes; X carries one fp32 scale per
// (row, 128-wide K block) and W_e one per (128 N x 128 K block), the 1-D
// activation / 2-D weight scaling of the blockwise fp8 kernel family named in
// "P3PeerSendConfig" (description).  Output rows are bf16, accumulated in
// fp32:
//   y[m][n] = sum_b x_scale[m][b] * w_scale[e][n/128][b] * sum_{k in b} X[m][k] W_e[k][n].
//
// Tiles: 256 x 256 with 8 waves as 2 x 4 (128 x 64 per wave) when N is a
// multiple of 256, else 256 x 128 with 8 waves as 4 x 2 (64 x 64 per wave),
// 32 x 32 MFMA blocks.  A K slice is exactly one 128-wide scale block (128
// bytes per row, the bf16 kernel's LDS layout and swizzle).  The wide tile
// moves 64 KB per slice for 16.8 MFLOP where the narrow one moves 48 KB for
// 8.4, so it needs half the global -> LDS bandwidth per flop; two of its
// stages fill the LDS, so it keeps one slice in flight, the narrow tile two.
// Per slice and 32 x 32 block the two v_mfma_scale_f32_32x32x64_f8f6f4 (unit
// E8M0 scales) build a partial sum P that is promoted as
// acc += P * (x_scale * w_scale): with W_e as the first MFMA operand each
// lane's 16 results share one row and one 128-column block, so the promotion
// factor is one float per lane.  The scales travel with the slice: dword
// direct copies put the tile's 256 x_scale values and its w_scale values
// into the same LDS stage.  Work schedule, row destinations, epilogue and
// completion are those of the bf16 kernel (gemm_common.h).
#include "gemm_common.h"

namespace ep {

namespace {

// Row-tile band of the item order (tile_of): the skewed fp8 routing puts
// thousands of rows on one expert, whose 28 column slabs would otherwise each
// re-read all of its X rows; bands of 4 row tiles took that workload's GEMM
// from 514 to 497 us in one process.
constexpr int kFp8Band = 4;

using namespace gemm;

template <int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct Fp8Tile {
  static constexpr int BM = 256, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES = 8, THREADS = 512;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 32, TN = WN / 32;
  static constexpr int BK = 128, RB = 128, CPR = 8, SWZ_SHIFT = 1;
  static constexpr int STAGES = STAGES_;
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int NB = BN / 128;                 // 128-column scale blocks per tile
  static constexpr int SX_OFF = A_BYTES + B_BYTES;   // 256 fp32 row scales
  static constexpr int SW_OFF = SX_OFF + BM * 4;      // 64 / NB copies of each w_scale
  static constexpr int STAGE = SW_OFF + 64 * 4;
  static constexpr int ROWS_PER_COPY = 1024 / RB;
  static constexpr int COPIES_A = BM / ROWS_PER_COPY;        // copies of X rows
  static constexpr int COPIES = (BM + BN) / ROWS_PER_COPY;   // 16-byte copies per slice
  static constexpr int IPW = COPIES / WAVES;                 // per wave
  static constexpr int SCALE_WAVES = BM / 64 + 1;            // waves issuing one dword copy
  static constexpr int LDS_MAIN = STAGES * STAGE;
  static constexpr int LDS_C = BM * (BN * 2 + 16);
  static constexpr int LDS = LDS_MAIN > LDS_C ? LDS_MAIN : LDS_C;
  static_assert(WAVES_M * WAVES_N == WAVES, "waves");
  static_assert(IPW * WAVES == COPIES, "copies must split evenly over waves");
  static_assert(SCALE_WAVES <= WAVES, "scale copies");
  static_assert(STAGE % 256 == 0, "stage alignment");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns share one scale block");
  static_assert(STAGES == 2 || STAGES == 3, "pipeline depth");
};

using Fp8Wide = Fp8Tile<256, 2, 4, 2>;     // 256 x 256, one slice in flight
using Fp8Narrow = Fp8Tile<128, 4, 2, 3>;   // 256 x 128, two slices in flight

typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

__device__ __forceinline__ i32x8 join(i32x4 lo, i32x4 hi) {
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// MFMAs and scale promotion over one K slice (one scale block) in stage `st`;
// only the first JV MFMA row blocks of this wave are computed (the others lie
// past m_end).  Per 32 x 32 block the two 64-k MFMAs chain into one partial
// sum, promoted once.  The narrow tile reads all its fragments up front; the
// wide tile (twice the blocks per wave, 128 accumulator registers) keeps the
// W_e fragments of both halves and reads the X fragments one row block at a
// time.
// GLU: the SwiGLU up-projection, whose wave columns are TN = 2 blocks (gate,
// then up) of two different 128-row weight scale blocks: the tile's w_scale
// copies hold the gate block's value in lanes 0..31 and the up block's in
// lanes 32..63, and the promotion factor is x_scale * w_scale of the block.
template <class T, int JV, bool GLU = false>
__device__ __forceinline__ void mma_slice_fp8(f32x16 (&acc)[T::TN][T::TM], const uint8_t* st,
                                              int wm, int wn, int lane) {
  const int frow = lane & 31;
  const int lrow = frow * T::RB;
  const uint8_t* fx_base = st + (wm * T::WM) * T::RB + lrow;
  const uint8_t* fw_base = st + T::A_BYTES + (wn * T::WN) * T::RB + lrow;
  const int swz = (frow >> T::SWZ_SHIFT) & (T::CPR - 1);
  const float* sx = reinterpret_cast<const float*>(st + T::SX_OFF);
  float s[T::TM];
  float sg[T::TN];                   // GLU: w_scale of column block i
  if constexpr (GLU) {
    static_assert(T::TN == 2, "gate block, then up block");
#pragma unroll
    for (int i = 0; i < T::TN; ++i) sg[i] = reinterpret_cast<const float*>(st + T::SW_OFF)[i * 32];
#pragma unroll
    for (int j = 0; j < T::TM; ++j) s[j] = j < JV ? sx[wm * T::WM + j * 32 + frow] : 0.f;
  } else {
    const float sw =
        reinterpret_cast<const float*>(st + T::SW_OFF)[(wn * T::WN / 128) * (64 / T::NB)];
#pragma unroll
    for (int j = 0; j < T::TM; ++j) s[j] = j < JV ? sx[wm * T::WM + j * 32 + frow] * sw : 0.f;
  }
  // fragment of 64-k half ks: 32 bytes = logical chunks 4ks + 2(lane/32) + {0,1}
  auto frag = [&](const uint8_t* row, int ks) {
    const int c0 = ((4 * ks + 2 * (lane >> 5)) ^ swz) << 4;
    const int c1 = ((4 * ks + 2 * (lane >> 5) + 1) ^ swz) << 4;
    return join(*reinterpret_cast<const i32x4*>(row + c0),
                *reinterpret_cast<const i32x4*>(row + c1));
  };
  const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if constexpr (T::TM * T::TN <= 4) {
    i32x8 fw[2][T::TN], fx[2][T::TM];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < T::TN; ++i) fw[ks][i] = frag(fw_base + i * 32 * T::RB, ks);
#pragma unroll
      for (int j = 0; j < T::TM; ++j)
        if (j < JV) fx[ks][j] = frag(fx_base + j * 32 * T::RB, ks);
    }
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
#pragma unroll
      for (int i = 0; i < T::TN; ++i)
        if (j < JV) {
          // format 0 = e4m3 for both operands; E8M0 scale 127 = 1.0
          f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[0][i], fx[0][j], zero, 0,
                                                                     0, 0, 127, 0, 127);
          p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[1][i], fx[1][j], p, 0, 0, 0, 127,
                                                              0, 127);
          const float f = GLU ? s[j] * sg[i] : s[j];
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = __builtin_fmaf(p[q], f, acc[i][j][q]);
        }
  } else {
    // both 64-k halves of the W_e fragments stay live; X fragments one row
    // block at a time; each block's two MFMAs chain into one partial sum
    i32x8 fw[2][T::TN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < T::TN; ++i) fw[ks][i] = frag(fw_base + i * 32 * T::RB, ks);
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
      if (j < JV) {
        const i32x8 fx0 = frag(fx_base + j * 32 * T::RB, 0);
        const i32x8 fx1 = frag(fx_base + j * 32 * T::RB, 1);
#pragma unroll
        for (int i = 0; i < T::TN; ++i) {
          f32x16 p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[0][i], fx0, zero, 0, 0, 0,
                                                                     127, 0, 127);
          p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[1][i], fx1, p, 0, 0, 0, 127, 0,
                                                              127);
          const float f = GLU ? s[j] * sg[i] : s[j];
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = __builtin_fmaf(p[q], f, acc[i][j][q]);
        }
      }
  }
}

// Per-wave copy plan of one tile.  Copy q = wave*IPW + j moves rows
// [8q', 8q'+8) of X (q' = q < COPIES_A) or of W_e (q' = q - COPIES_A) into
// the q-th KB of the stage; the two operand bases are wave-uniform (SGPRs) and
// each copy keeps only the lane's 32-bit offset.  Waves 0..3 also copy the
// x_scale values of their 64 tile rows and wave 4 the tile's w_scale values,
// 64 / NB lanes per 128-column block (one dword per lane).
template <class T>
struct Fp8Copies {
  const uint8_t* xa;                 // X
  const uint8_t* wb;                 // W_e
  uint32_t voff[T::IPW];
  int q0;
  const uint8_t* sbase;              // x_scale or this tile's w_scale rows (slice 0)
  uint32_t soff;                     // lane's byte offset from sbase
  uint32_t sdst;                     // LDS offset of the scale copy inside a stage
  bool has_scale;
};

// Issues this wave's copies of K slice kt into the stage at LDS address `st`.
template <class T>
__device__ __forceinline__ void copy_slice_fp8(uint32_t st, const Fp8Copies<T>& c, int kt) {
  const size_t kb = (size_t)kt * T::BK;
#pragma unroll
  for (int j = 0; j < T::IPW; ++j) {
    const int q = c.q0 + j;
    g2lds16s((q < T::COPIES_A ? c.xa : c.wb) + kb, c.voff[j], st + q * 1024);
  }
  if (c.has_scale) g2lds4s(c.sbase + (size_t)kt * 4, c.soff, st + c.sdst);
}

// Waits until only the copies of the slice issued last (`one_in_flight`) may
// still be in flight: IPW copies, plus the scale copy of the waves that have one.
template <class T>
__device__ __forceinline__ void wait_fp8(const Fp8Copies<T>& c, bool one_in_flight) {
  if (!one_in_flight) wait_vm<0>();
  else if (c.has_scale) wait_vm<T::IPW + 1>();
  else wait_vm<T::IPW>();
}

// The K loop, S = STAGES stages and S - 1 slices in flight.  Each step
// copies slice k + S - 1 into the stage freed by the previous step,
// multiplies slice k, waits for slice k + 1 and synchronises the workgroup.
// The previous tile's pending completion is done right after the prologue's
// barrier.
template <class T, int JV, bool GLU = false>
__device__ __forceinline__ void k_loop_fp8(f32x16 (&acc)[T::TN][T::TM], uint8_t* smem,
                                           uint32_t lds0, const Fp8Copies<T>& c, int KT, int wm,
                                           int wn, int lane, const GemmArgs& a,
                                           PendingTiles& pending) {
  constexpr int S = T::STAGES;
  copy_slice_fp8<T>(lds0, c, 0);
  if (S == 3 && KT > 1) copy_slice_fp8<T>(lds0 + T::STAGE, c, 1);
  wait_fp8<T>(c, S == 3 && KT > 1);
  // every wave's stores of the earlier tiles are now complete: count them
  prologue_barrier(a, pending);
  for (int kt = 0; kt < KT; kt += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int k = kt + u;
      if (k >= KT) break;
      const bool ahead = k + S - 1 < KT;
      if (ahead) copy_slice_fp8<T>(lds0 + ((u + S - 1) % S) * T::STAGE, c, k + S - 1);
      if constexpr (JV > 0) mma_slice_fp8<T, JV, GLU>(acc, smem + u * T::STAGE, wm, wn, lane);
      wait_fp8<T>(c, S == 3 && ahead);
      raw_barrier();
    }
  }
}

// One tile: zeroed accumulators, the K loop, the sink epilogue.
template <class T, int JV>
__device__ __forceinline__ void run_tile_fp8(const GemmArgs& a, uint8_t* smem, uint32_t lds0,
                                             const Fp8Copies<T>& c, int KT, int wm, int wn, int lane,
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
  k_loop_fp8<T, JV>(acc, smem, lds0, c, KT, wm, wn, lane, a, pending);
  send_tile<T::BM, T::BN, T::WM, T::WN, T::TM, T::TN, T::THREADS>(a, acc, smem, s_rowdst, s_recv,
                                                                   t, wm, wn, JV, ri, pending);
}

// Runs the tile with JV = jv (this wave's MFMA row blocks before m_end) as a
// compile-time constant, as in the bf16 kernel.
template <class T, int J>
__device__ __forceinline__ void run_tile_fp8_jv(int jv, const GemmArgs& a, uint8_t* smem,
                                                uint32_t lds0, const Fp8Copies<T>& c, int KT, int wm,
                                                int wn, int lane, const TileWork& t,
                                                const RowInfo& ri, uint64_t* s_rowdst,
                                                uint8_t* const* s_recv, PendingTiles& pending) {
  if constexpr (J > 0) {
    if (jv != J) {
      run_tile_fp8_jv<T, J - 1>(jv, a, smem, lds0, c, KT, wm, wn, lane, t, ri, s_rowdst, s_recv,
                                pending);
      return;
    }
  }
  run_tile_fp8<T, J>(a, smem, lds0, c, KT, wm, wn, lane, t, ri, s_rowdst, s_recv, pending);
}

template <class T, bool EPI, bool TRACE, bool FUSED>
__global__ __launch_bounds__(T::THREADS) void gemm_scatter_fp8_kernel(GemmArgs a) {
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
  const int KB = K / 128;                   // scale blocks along K
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
  Fp8Copies<T> c;
  c.q0 = wave * T::IPW;
  c.xa = a.x;
  c.has_scale = wave < T::SCALE_WAVES;
  c.sdst = wave < BM / 64 ? T::SX_OFF + wave * 256 : T::SW_OFF;
  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= total) break;
    const TileWork t = tile_of<BM, BN, kFp8Band>(a, s_base, s_gbeg, item);
    if (t.empty) {
      signal_empty_expert(a, t.e, pending);
      continue;
    }
    // lane L fills physical chunk L%8 of row 8q' + L/8, which holds logical
    // chunk (L%8) ^ swizzle(row); rows past m_end re-read the group's last row
    c.wb = a.w + (size_t)t.e * N * K;
#pragma unroll
    for (int j = 0; j < T::IPW; ++j) {
      const int q = c.q0 + j;
      const bool is_a = q < T::COPIES_A;
      const int r = (is_a ? q : q - T::COPIES_A) * T::ROWS_PER_COPY + lane / T::CPR;
      const uint32_t off = ((lane % T::CPR) ^ ((r >> T::SWZ_SHIFT) & (T::CPR - 1))) * 16;
      const int grow = is_a ? min(t.m_abs + r, t.g1 - 1) : t.n_abs + r;
      c.voff[j] = (uint32_t)grow * (uint32_t)K + off;
    }
    if (wave < BM / 64) {
      const int m = min(t.m_abs + wave * 64 + lane, t.g1 - 1);
      c.sbase = reinterpret_cast<const uint8_t*>(a.x_scale);
      c.soff = (uint32_t)m * (uint32_t)KB * 4;
    } else {
      // lanes [64b/NB, 64(b+1)/NB) copy the w_scale of the tile's block b
      c.sbase = reinterpret_cast<const uint8_t*>(
          a.w_scale + ((size_t)t.e * (N / 128) + t.n_abs / 128) * KB);
      c.soff = (uint32_t)(lane / (64 / T::NB)) * (uint32_t)KB * 4;
    }

    const RowInfo ri = tid < BM ? load_row_info(a, t.e, t.g1, t.m_abs + tid) : RowInfo{-1, 0, 0};
    const int jv = min(T::TM, max(0, (t.rows - wm * T::WM + 31) / 32));
    if constexpr (TRACE) trace_start(a, item);
    run_tile_fp8_jv<T, T::TM>(jv, a, smem, lds0, c, KB, wm, wn, lane, t, ri, s_rowdst, s_recv,
                              pending);
    if constexpr (TRACE) trace_end(a, item, t, BN);
  }
  flush_pending(a, pending);
  if constexpr (FUSED) fused_consume(a, &s_bad);
}


// ---------------------------------------------------------------------------
// Up-projection with SwiGLU on block-scaled fp8 operands, the first GEMM of the
// fp8 expert FFN, whose output is the fp8 X of the kernel above:
//   g = sum_b x_scale[m][b] * w_scale[e][i/128][b] * sum_{k in b} X1[m][k] Wg_e[i][k]
//   u = the same with the up rows I + i,   h = silu(g) * u   (binary32)
// and H re-quantised per (row, 128 columns), the 1-D activation scaling of the
// same blockwise family: scale = amax / 448 (1 if amax = 0), code = the
// e4m3fn value of h / scale rounded to nearest even.  W1_e = [Wg_e; Wu_e] is
// stored [2I][hidden] with w_scale [2I/128][hidden/128].  The wide tile's 256
// GEMM columns are the 128 gate rows i0..i0+127 and their up rows, permuted as
// in the bf16 up-projection (each wave's 64 columns: 32 gate rows, then the 32
// matching up rows), so a lane holds gate and up of the same outputs and a
// tile's 128 outputs of a row are exactly one scale block: the row's amax is
// reduced over the tile's four column waves through LDS, then the tile writes
// 128 code bytes and one scale per row.  No sink, no completion signalling.

// W1 row of GEMM column c of a tile whose outputs start at i0 (64 columns per wave).
__device__ __forceinline__ int glu_w_row(int c, int i0, int I) {
  return ((c % 64) >= 32 ? I : 0) + i0 + (c / 64) * 32 + (c % 32);
}

// binary32 -> e4m3fn code (sign, 4 exponent bits of bias 7, 3 mantissa bits),
// rounded to nearest even; magnitudes that would round past 448 give 448.
__device__ __forceinline__ uint32_t e4m3fn_code(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t ab = b & 0x7fffffffu;
  uint32_t code;
  if (ab < 0x3c800000u) {
    // below 2^-6: the subnormal codes k * 2^-9 (k = 8 is the smallest normal)
    code = (uint32_t)__builtin_rintf(__uint_as_float(ab) * 512.0f);
  } else {
    // keep 3 mantissa bits, ties to even; a carry moves into the exponent
    const uint32_t r = ab + 0x7ffffu + ((ab >> 20) & 1u);
    code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);   // exponent - 127 + 7
    code = code > 0x7eu ? 0x7eu : code;
  }
  return sign | code;
}

template <class T>
__device__ __forceinline__ void glu_fp8_tile(const GemmArgs& a, const f32x16 (&acc)[T::TN][T::TM],
                                             uint8_t* smem, const TileWork& t, int wm, int wn) {
  static_assert(T::TN == 2 && T::WN == 64 && T::BN == 256 && T::WAVES_N == 4, "gate/up layout");
  constexpr int OC = T::BN / 2;              // outputs per tile row: one scale block
  constexpr int PITCH = OC + 16;             // bytes per staged code row (skewed)
  constexpr int AMAX_OFF = T::BM * PITCH;    // float [BM][WAVES_N] partial maxima
  static_assert(AMAX_OFF + T::BM * T::WAVES_N * 4 <= T::LDS, "epilogue LDS");
  const int tid = threadIdx.x, lane = tid & 63;
  const int frow = lane & 31, fhalf = lane >> 5;
  float* s_amax = reinterpret_cast<float*>(smem + AMAX_OFF);
  // a lane holds columns 8g + 4 * (lane / 32) + q (q < 4) of the wave's 32
  // outputs, gate in block 0 and up in block 1; h is formed twice (for the
  // row maxima, then for the codes) rather than kept in registers
  auto hval = [&](int j, int q) {
    const float g = acc[0][j][q], u = acc[1][j][q];
    return g / (1.0f + __expf(-g)) * u;
  };
#pragma unroll
  for (int j = 0; j < T::TM; ++j) {
    float mx = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = __builtin_fmaxf(mx, __builtin_fabsf(hval(j, q)));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    if (fhalf == 0) s_amax[(wm * T::WM + j * 32 + frow) * T::WAVES_N + wn] = mx;
  }
  __syncthreads();
  const size_t I = (size_t)(a.N / 2);
  const int i0 = t.n_abs / 2;
#pragma unroll
  for (int j = 0; j < T::TM; ++j) {
    const int r = wm * T::WM + j * 32 + frow;
    const float* am = s_amax + r * T::WAVES_N;
    const float amax = __builtin_fmaxf(__builtin_fmaxf(am[0], am[1]), __builtin_fmaxf(am[2], am[3]));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) w |= e4m3fn_code(hval(j, 4 * g + q) / scale) << (8 * q);
      *reinterpret_cast<uint32_t*>(smem + r * PITCH + wn * 32 + 8 * g + 4 * fhalf) = w;
    }
    if (wn == 0 && fhalf == 0 && r < t.rows)
      a.c_scale[(size_t)(t.m_abs + r) * (I / 128) + i0 / 128] = scale;
  }
  __syncthreads();
  constexpr int TPR = OC / 16;               // threads per row
  constexpr int RPP = T::THREADS / TPR;      // rows per pass
  const int cr = tid / TPR, cc = tid % TPR;
  for (int r0 = 0; r0 < t.rows; r0 += RPP) {
    const int r = r0 + cr;
    if (r < t.rows) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * PITCH + cc * 16);
      store16_nt(a.c_local + (size_t)(t.m_abs + r) * I + i0 + cc * 16, v);
    }
  }
  __syncthreads();   // the staged tile is read; the next tile may overwrite LDS
}

template <class T, int JV>
__device__ __forceinline__ void run_tile_glu(const GemmArgs& a, uint8_t* smem, uint32_t lds0,
                                             const Fp8Copies<T>& c, int KT, int wm, int wn,
                                             int lane, const TileWork& t, PendingTiles& pending) {
  f32x16 acc[T::TN][T::TM];
#pragma unroll
  for (int i = 0; i < T::TN; ++i)
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  k_loop_fp8<T, JV, true>(acc, smem, lds0, c, KT, wm, wn, lane, a, pending);
  glu_fp8_tile<T>(a, acc, smem, t, wm, wn);
}

template <class T, int J>
__device__ __forceinline__ void run_tile_glu_jv(int jv, const GemmArgs& a, uint8_t* smem,
                                                uint32_t lds0, const Fp8Copies<T>& c, int KT,
                                                int wm, int wn, int lane, const TileWork& t,
                                                PendingTiles& pending) {
  if constexpr (J > 0) {
    if (jv != J) {
      run_tile_glu_jv<T, J - 1>(jv, a, smem, lds0, c, KT, wm, wn, lane, t, pending);
      return;
    }
  }
  run_tile_glu<T, J>(a, smem, lds0, c, KT, wm, wn, lane, t, pending);
}

template <class T>
__global__ __launch_bounds__(T::THREADS) void gemm_swiglu_fp8_kernel(GemmArgs a) {
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
  const int KB = K / 128;                   // scale blocks along K
  const int El = a.s.n_experts;

  init_done(s_done);
  if (!build_work_table<BM, T::THREADS>(a, N / BN, s_base, s_gbeg, &s_bad)) return;
  const int total = s_base[El];

  const int G = gridDim.x;                  // a multiple of 8
  const int per_xcd = G >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const uint32_t lds0 = lds_addr(smem);

  PendingTiles pending;                     // stays empty: no tile is counted
  pending.done = s_done;
  pending.e = s_pend;
  pending.base = s_base;
  Fp8Copies<T> c;
  c.q0 = wave * T::IPW;
  c.xa = a.x;
  c.has_scale = wave < T::SCALE_WAVES;
  c.sdst = wave < BM / 64 ? T::SX_OFF + wave * 256 : T::SW_OFF;
  for (int round = 0;; ++round) {
    const int item = round * G + xcd * per_xcd + slot;
    if (item >= total) break;
    const TileWork t = tile_of<BM, BN, kFp8Band>(a, s_base, s_gbeg, item);
    if (t.empty) continue;
    const int i0 = t.n_abs / 2;
    // as in the down-projection; W1 rows go through the gate/up permutation
    c.wb = a.w + (size_t)t.e * N * K;
#pragma unroll
    for (int j = 0; j < T::IPW; ++j) {
      const int q = c.q0 + j;
      const bool is_a = q < T::COPIES_A;
      const int r = (is_a ? q : q - T::COPIES_A) * T::ROWS_PER_COPY + lane / T::CPR;
      const uint32_t off = ((lane % T::CPR) ^ ((r >> T::SWZ_SHIFT) & (T::CPR - 1))) * 16;
      const int grow = is_a ? min(t.m_abs + r, t.g1 - 1) : glu_w_row(r, i0, I);
      c.voff[j] = (uint32_t)grow * (uint32_t)K + off;
    }
    if (wave < BM / 64) {
      const int m = min(t.m_abs + wave * 64 + lane, t.g1 - 1);
      c.sbase = reinterpret_cast<const uint8_t*>(a.x_scale);
      c.soff = (uint32_t)m * (uint32_t)KB * 4;
    } else {
      // lanes 0..31 copy the gate rows' scale block, lanes 32..63 the up rows'
      c.sbase = reinterpret_cast<const uint8_t*>(a.w_scale + (size_t)t.e * (N / 128) * KB);
      const int blk = (lane < 32 ? 0 : I / 128) + i0 / 128;
      c.soff = (uint32_t)blk * (uint32_t)KB * 4;
    }
    const int jv = min(T::TM, max(0, (t.rows - wm * T::WM + 31) / 32));
    run_tile_glu_jv<T, T::TM>(jv, a, smem, lds0, c, KB, wm, wn, lane, t, pending);
  }
}


template <class T>
hipError_t launch_fp8(const GemmArgs& a, int grid, hipStream_t st) {
  if (a.epilogue_only)
    hipLaunchKernelGGL((gemm_scatter_fp8_kernel<T, true, false, false>), dim3(grid), dim3(T::THREADS), 0,
                       st, a);
  else if (a.trace)
    hipLaunchKernelGGL((gemm_scatter_fp8_kernel<T, false, true, false>), dim3(grid), dim3(T::THREADS), 0,
                       st, a);
  else if (a.fused) {
    const int g = fused_grid<gemm_scatter_fp8_kernel<T, false, false, true>>(T::THREADS, a.num_cus);
    if (!g) return hipErrorLaunchFailure;
    hipLaunchKernelGGL((gemm_scatter_fp8_kernel<T, false, false, true>), dim3(g), dim3(T::THREADS), 0, st, a);
  }
  else
    hipLaunchKernelGGL((gemm_scatter_fp8_kernel<T, false, false, false>), dim3(grid), dim3(T::THREADS), 0,
                       st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu_fp8(const GemmArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(gemm_swiglu_fp8_kernel<Fp8Wide>, dim3(grid), dim3(Fp8Wide::THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmArgs& a, int tile, int grid, hipStream_t st) {
  switch (tile) {
    case kTile256x256: return launch_fp8<Fp8Wide>(a, grid, st);
    case kTile256x128: return launch_fp8<Fp8Narrow>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ep
