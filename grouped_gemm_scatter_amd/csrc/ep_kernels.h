// Kernel argument blocks and launchers of the EP-combine step (internal to
// the library; the public surface is include/ep_combine.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"

namespace ep {

struct CombineArgs {
  const int32_t* topk_ids;   // [R][T][top_k]
  const float* topk_w;       // [R][T][top_k]
  uint8_t* out;              // [R][T][N] bf16
  const uint64_t* flags;     // R rank flags (tail of the count words)
  uint8_t* recv[kMaxRanks];
  int32_t* err;
  uint64_t epoch;
  const uint64_t* epoch_ptr;  // device epoch word (read instead of epoch), or null
  int64_t spin_limit;
  int32_t n_ranks;
  int32_t tokens;            // tokens per rank in this call
  int32_t top_k;
  int32_t N;
  int32_t msg_bytes;
  int32_t expert_lo;         // first local global expert id
  int32_t n_experts;         // E_l
  int32_t system_scope;
  int32_t per_expert;        // acquire each tagged count word instead of the rank flag
  const uint64_t* words;     // the E_l*R count words
};

struct GemmArgs {
  const uint8_t* x;          // [M][K] bf16 or e4m3fn
  const uint8_t* w;          // [E_l][N][K]
  const float* x_scale;      // [M][K/128] (fp8)
  const float* w_scale;      // [E_l][N/128][K/128] (fp8)
  const int32_t* offsets;    // [E_l*R + 1]
  const int32_t* src_info;   // [M][2]
  uint8_t* c_local;          // [M][N] bf16, sink disabled only
  float* c_scale;            // fp8 up-projection: [M][N/256] output row-block scales
  int32_t m_total;
  int32_t K;
  int32_t N;
  int32_t sink_on;           // p3_control >= 0
  int32_t epilogue_only;     // skip the K loop; accumulators = (m*131 + n*7) mod 256
  int32_t w_slice_major;     // W as [E_l][K/64][N][64] (bf16 down-projection) instead of [E_l][N][K]
  SinkState s;
  uint64_t* trace;           // tile records, 4 u64 each (null: off)
  int64_t trace_records;
  // consumer side of a fused launch (ep_grouped_gemm_scatter_combine): once its
  // tiles are done and published, every workgroup runs combine runs
  // blockIdx.x, blockIdx.x + gridDim.x, ... of comb_runs_per_rank runs per rank
  int32_t fused;
  int32_t comb_tokens_per_run;
  int32_t comb_runs_per_rank;
  int32_t comb_chunks;       // 16-byte chunks per lane per pass: 4, 8 or 14
  int32_t num_cus;           // host only: fused grids are sized from it
  CombineArgs comb;
};

// Grid of a fused launch: every workgroup resident at once (the kernel's own
// occupancy times the CU count, a multiple of 8).  0 if that cannot be known.
// The occupancy is a property of the kernel and the architecture, queried once
// per kernel.
template <auto KERNEL>
inline int fused_grid(int threads, int num_cus) {
  static const int per_cu = [threads] {
    int n = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERNEL, threads, 0) == hipSuccess ? n
                                                                                              : 0;
  }();
  const int g = per_cu * num_cus / 8 * 8;
  return g >= 8 ? g : 0;
}



// Tile configurations of the grouped GEMM.
enum GemmTile : int {
  kTile256x256 = 0,
  kTile128x128 = 1,
  kTile256x128 = 2,
  kTileDecode64x128 = 3,
  // 128 x 128, three stages, with dedicated send waves (ep_combine_params
  // send_waves = 4) or the sink inside the MFMA waves (EP_FLAG_SEND_TILE)
  kTileSend128x128 = 4,
  kTileSendNone128x128 = 5,
};

inline int gemm_tile_rows(int tile) {
  return (tile == kTile128x128 || tile >= kTileSend128x128) ? 128
         : tile == kTileDecode64x128                          ? 64
                                                              : 256;
}
inline int gemm_tile_cols(int tile) {
  return tile == kTile256x256 ? 256 : 128;
}
// workgroups resident per CU (LDS-bound)
inline int gemm_blocks_per_cu(int tile) { return tile == kTile128x128 ? 2 : 1; }

hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, int grid, hipStream_t st);
// The bf16 GEMM with `send_waves` (4, or 0: the sink inside the MFMA waves)
// dedicated send waves above its 8 MFMA waves (128 x 128 tiles).
hipError_t launch_gemm_send(const GemmArgs& a, int send_waves, int grid, hipStream_t st);
// Up-projection + SwiGLU (256 x 256 GEMM tiles, 256 x 128 outputs); a.N = 2I, a.K = hidden.
hipError_t launch_swiglu_bf16(const GemmArgs& a, int grid, hipStream_t st);
hipError_t launch_gemm_fp8(const GemmArgs& a, int tile, int grid, hipStream_t st);
// Up-projection + SwiGLU on fp8 operands (256 x 256 GEMM tiles, 256 x 128 e4m3fn
// outputs and one scale per output row and tile); a.N = 2I, a.K = hidden.
hipError_t launch_swiglu_fp8(const GemmArgs& a, int grid, hipStream_t st);
hipError_t launch_signal(const SinkState& s, const int32_t* expert, const int32_t* dst_rank,
                         const uint64_t* signal, int n, hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, int num_cus, hipStream_t st);
// word = word + 1, skipping values whose low 32 bits are zero (one thread).
hipError_t launch_advance_epoch(uint64_t* word, hipStream_t st);

struct GroupArgs {
  const int32_t* topk_ids;   // [R][T][top_k] global expert ids
  int32_t* offsets;          // [E_l*R + 1]
  int32_t* src_info;         // [M][2] (t, k), M <= R*T*top_k
  int32_t n_ranks;
  int32_t n_experts;         // E_l
  int32_t expert_lo;         // my_rank * E_l
  int32_t tokens;            // T
  int32_t top_k;
};

struct DispatchArgs {
  const uint8_t* tokens_x;   // [R][tokens][row_bytes]: each source rank's token rows
  const int32_t* offsets;    // [E_l*R + 1]
  const int32_t* src_info;   // [M][2] (t, k)
  uint8_t* x_out;            // [M][row_bytes]
  int32_t* err;
  int32_t m_total;
  int32_t row_bytes;         // multiple of 16
  int32_t tokens;
  int32_t n_ranks;
  int32_t n_experts;         // E_l
};

// Dispatch side: x_out[m] = the token row of grouped row m's pick.
hipError_t launch_dispatch(const DispatchArgs& a, int num_cus, hipStream_t st);

// W [experts][N][K] bf16 -> [experts][K/64][N][64] (K a multiple of 64).
hipError_t launch_pack_slice_major(const uint8_t* w, uint8_t* out, int64_t experts, int N, int K,
                                   int num_cus, hipStream_t st);

// Local grouping of the routing (count, scan, place; three launches on st).
hipError_t launch_grouping(const GroupArgs& a, hipStream_t st);

}  // namespace ep
