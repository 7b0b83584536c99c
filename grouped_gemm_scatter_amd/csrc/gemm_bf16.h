// bf16 tile geometry, LDS layout, fragment MFMAs and direct-copy plans shared
// by the grouped-GEMM kernels that take whole K slices of 64 through LDS
// (the sink kernels with and without dedicated send waves, the SwiGLU
// up-projection).
#pragma once

#include "gemm_common.h"

namespace ep {

namespace {

using namespace gemm;

// LDS layout of one K slice of an operand: RB = 2*BK bytes per row, rows
// back to back; 16-byte chunk kc of row r is stored at chunk
// kc ^ ((r / (256 / RB)) % (RB / 16)).  A ds_read_b128 serves 16 lanes
// (256 bytes, all 64 banks) per cycle; 16 consecutive rows read at one kc
// then land in 16 distinct 16-byte bank groups, so fragment reads are
// conflict-free.  Whole 128-byte row pieces (BK = 64) also make every L2
// request a full line, which the load path needs for bandwidth.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int STAGES_>
struct Bf16Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BK = BK_, STAGES = STAGES_;
  static constexpr int RB = BK * 2;                 // bytes of one row in one slice
  static constexpr int CPR = RB / 16;               // 16-byte chunks per row
  static constexpr int SWZ_SHIFT = RB == 64 ? 2 : 1;  // log2(256 / RB)
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // one direct copy moves 64 lanes x 16 B = 1 KB = ROWS_PER_COPY rows
  static constexpr int ROWS_PER_COPY = 1024 / RB;
  static constexpr int COPIES = (BM + BN) / ROWS_PER_COPY;
  static constexpr int IPW = COPIES / WAVES;       // copies per wave per slice
  static constexpr int C_PITCH = BN * 2 + 16;      // bytes per staged output row
  static constexpr int LDS_MAIN = STAGES * STAGE;
  static constexpr int LDS_C = BM * C_PITCH;
  static constexpr int LDS = LDS_MAIN > LDS_C ? LDS_MAIN : LDS_C;
  // MFMA row blocks of wave row 0 (the same for every wave row here), and the
  // row tiling: whole tiles of BM rows (BAL = 0, see row_tiles)
  static constexpr int TM0 = TM, BAL = 0;
  static_assert(RB == 64 || RB == 128, "slice row width");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(STAGES >= 2 && STAGES <= 8, "pipeline depth");
};

// The 256-column tile of up to nine 32-row blocks (288 rows), fed by the
// balanced row tiling (BAL = 9, see row_tiles): an expert's ceil(M_e / 32)
// row blocks are spread evenly over the fewest tiles of at most nine blocks,
// so no tile of an expert is left with a handful of rows (with plain 256-row
// tiles an expert of 1030 rows has a fifth tile of 6 rows, which still copies
// every W_e slice of its column slab).  Wave row 0 owns tile rows [0, 128)
// (four blocks), wave row 1 rows [128, 288) (up to five); a tile of eight
// blocks, the common case, gives every wave four.  Each LDS stage holds 288
// rows of X and 256 of W_e; the staged output tile (288 rows) fits the LDS
// beside the workgroup's other arrays.
struct TallTile {
  static constexpr int BM = 288, BN = 256;
  static constexpr int WAVES_M = 2, WAVES_N = 4;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BK = 64, STAGES = 2;
  static constexpr int RB = BK * 2;
  static constexpr int CPR = RB / 16;
  static constexpr int SWZ_SHIFT = 1;
  static constexpr int WM = 128;                   // first row of wave row 1
  static constexpr int WN = BN / WAVES_N;
  static constexpr int TM = 5, TN = WN / 32;       // blocks of wave row 1; columns
  static constexpr int TM0 = 4;                    // blocks of wave row 0
  static constexpr int BAL = BM / 32;              // at most nine blocks per tile
  static constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int ROWS_PER_COPY = 1024 / RB;
  static constexpr int C_PITCH = BN * 2 + 16;
  static constexpr int LDS_MAIN = STAGES * STAGE;
  static constexpr int LDS_C = BM * C_PITCH;
  static constexpr int LDS = LDS_MAIN > LDS_C ? LDS_MAIN : LDS_C;
  static_assert(WM + TM * 32 == BM && TM0 * 32 == WM, "wave rows cover the tile");
};

// MFMAs over one K slice held in LDS stage `st`.
template <class T, int JV>
__device__ __forceinline__ void mma_slice(f32x16 (&acc)[T::TN][T::TM], const uint8_t* st,
                                          int wm, int wn, int lane) {
  // lane reads row (lane & 31) of each 32-row block at kchunk 2s + lane/32
  const int lrow = (lane & 31) * T::RB;
  const uint8_t* fx_base = st + (wm * T::WM) * T::RB + lrow;
  const uint8_t* fw_base = st + T::A_BYTES + (wn * T::WN) * T::RB + lrow;
  const int swz = ((lane & 31) >> T::SWZ_SHIFT) & (T::CPR - 1);
  bf16x8 fw[2][T::TN], fx[2][T::TM];
  auto load_frags = [&](int s, int buf) {
    const int chunk = ((2 * s + (lane >> 5)) ^ swz) << 4;
#pragma unroll
    for (int i = 0; i < T::TN; ++i)
      fw[buf][i] = *reinterpret_cast<const bf16x8*>(fw_base + i * 32 * T::RB + chunk);
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
      if (j < JV)
        fx[buf][j] = *reinterpret_cast<const bf16x8*>(fx_base + j * 32 * T::RB + chunk);
  };
  load_frags(0, 0);
#pragma unroll
  for (int s = 0; s < T::BK / 16; ++s) {
    if (s + 1 < T::BK / 16) load_frags(s + 1, (s + 1) & 1);
#pragma unroll
    for (int j = 0; j < T::TM; ++j)
#pragma unroll
      for (int i = 0; i < T::TN; ++i)
        if (j < JV)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s & 1][i], fx[s & 1][j],
                                                              acc[i][j], 0, 0, 0);
  }
}

// W_e in one of its two layouts, a compile-time choice (WS) of every copy
// plan: row-major [N][K], where K slice kt of row n (64 elements, 128 bytes)
// lies at n*2K + kt*128 bytes from the expert's base, or slice-major
// [K/64][N][64] (WS), where it lies at kt*128N + n*128, so that one K slice of
// a block of rows is one contiguous run.  Slice-major plans start their W base
// at the tile's first row, keep the row part in the lane offsets and step the
// base by 128N bytes per slice.

// This wave's direct copies of one tile.  Copy q = wave*IPW + j moves rows
// [q*RPC, (q+1)*RPC) (RPC = rows per copy) of X (A, q < BM/RPC) or of W_e
// (B) into the q-th KB of the stage; all copies of one wave move rows of the
// same operand, so the operand base is wave-uniform and each copy keeps only
// the lane's 32-bit offset from it.
template <class T, bool WS = false>
struct CopyPlan {
  static_assert(T::IPW * T::WAVES == T::COPIES, "copies must split evenly over waves");
  static_assert((T::BM / T::ROWS_PER_COPY) % T::IPW == 0, "one operand per wave");
  static_assert(T::RB == 128, "64-element K slices");
  const uint8_t* base;        // X or W_e
  uint32_t voff[T::IPW];
  int q0;
  uint32_t kstride;           // WS: bytes from one K slice of the operand to the next
};

// Issues this wave's direct copies of K slice kt into the stage at LDS
// address `st`.
// A wave-uniform pointer, moved to scalar registers: the copies take their
// base there, and the compiler does not always prove a base uniform when
// several tile shapes share one loop.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

template <class T, bool WS>
__device__ __forceinline__ void copy_slice(uint32_t st, const CopyPlan<T, WS>& c, int kt) {
  const uint8_t* base = uniform_ptr(c.base + (size_t)kt * (WS ? c.kstride : T::RB));
#pragma unroll
  for (int j = 0; j < T::IPW; ++j) g2lds16s(base, c.voff[j], st + (c.q0 + j) * 1024);
}

}  // namespace

}  // namespace ep
