// Device code shared by the bf16 and fp8 grouped-GEMM kernels: direct
// global->LDS copies, raw barriers, the persistent work table over ragged
// expert groups, row destinations, the sink epilogue and tile completion.
#pragma once

#include "combine_common.h"
#include "ep_kernels.h"

namespace ep {
namespace gemm {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(uint8_t* lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_u8*)lds);
}

// Copies 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane L of the wave writes bytes [16L, 16L+16)
// after `lds`, a wave-uniform LDS address passed in M0 (saved and restored).
// Issued through inline assembly so that the compiler's wait-count insertion
// does not conservatively drain these copies before unrelated LDS reads; the
// K loops wait for them explicitly (vmcnt) before each workgroup barrier.
// Vector memory operations of one wave complete in issue order, so waiting
// for a later count also covers every earlier copy.
__device__ __forceinline__ void g2lds16(const void* g, uint8_t* lds) {
  const uint32_t m = lds_addr(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m)
      : "memory");
}

// Same copy addressed as a wave-uniform base (an SGPR pair) plus the lane's
// 32-bit byte offset: one VGPR per copy instead of a 64-bit address, and the
// per-slice advance stays in scalar registers.  `m` is the LDS byte address
// (wave-uniform) that lane 0 writes.
__device__ __forceinline__ void g2lds16s(const void* sbase, uint32_t voff, uint32_t m) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m)
      : "memory");
}

// Dword copy in the same SGPR-base + 32-bit-offset form: lane L writes bytes
// [4L, 4L+4) after LDS address `m`.
__device__ __forceinline__ void g2lds4s(const void* sbase, uint32_t voff, uint32_t m) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m)
      : "memory");
}

// Same with 4 bytes per lane (global_load_lds_dword): lane L writes bytes
// [4L, 4L+4) after `lds`.
__device__ __forceinline__ void g2lds4(const void* g, uint8_t* lds) {
  const uint32_t m = lds_addr(lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m)
      : "memory");
}

// Workgroup barrier without the implied memory fence of __syncthreads(): the
// fence would wait for every copy still in flight into other stages.  The
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Waits until at most `pending` * PER_SLICE of this wave's copies are in
// flight (pending in [0, MAXP]; larger values wait as for MAXP).
template <int PER_SLICE, int MAXP = 3>
__device__ __forceinline__ void wait_slices(int pending) {
  static_assert(MAXP >= 1 && MAXP <= 6 && MAXP * PER_SLICE < 64, "vmcnt range");
  const int p = pending < MAXP ? pending : MAXP;
  if constexpr (MAXP >= 6) { if (p == 6) return wait_vm<6 * PER_SLICE>(); }
  if constexpr (MAXP >= 5) { if (p == 5) return wait_vm<5 * PER_SLICE>(); }
  if constexpr (MAXP >= 4) { if (p == 4) return wait_vm<4 * PER_SLICE>(); }
  if constexpr (MAXP >= 3) { if (p == 3) return wait_vm<3 * PER_SLICE>(); }
  if constexpr (MAXP >= 2) { if (p == 2) return wait_vm<2 * PER_SLICE>(); }
  if (p == 1) return wait_vm<PER_SLICE>();
  wait_vm<0>();
}

// Expert that owns work item `item`: largest e with base[e] <= item.
__device__ __forceinline__ int find_expert(const int* base, int n_experts, int item) {
  int lo = 0, hi = n_experts;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (base[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

// Per-workgroup setup: validates the offsets, builds the prefix of work items
// per expert (ceil(M_e / BM) * n_tiles tiles, or one signal-only item for an
// empty expert) and caches the group starts (s_gbeg[e] = offsets[e*R]) in
// LDS.  Returns false (and latches EP_ERR_BAD_GROUP once) when the offsets
// are inconsistent.
// Row tiles of an expert with `me` rows: whole tiles of BM rows, or with
// BAL > 0 the fewest tiles of at most BAL 32-row blocks each, over which the
// expert's ceil(me / 32) blocks are then spread evenly (so no tile of an
// expert is left nearly empty).
template <int BM, int BAL>
__device__ __forceinline__ int row_tiles(int me) {
  if constexpr (BAL > 0) return (((me + 31) >> 5) + BAL - 1) / BAL;
  return (me + BM - 1) / BM;
}

template <int BM, int THREADS, int BAL = 0>
__device__ __forceinline__ bool build_work_table(const GemmArgs& a, int nt, int* s_base, int* s_gbeg,
                                 int* s_bad) {
  const int tid = threadIdx.x;
  const int R = a.s.n_ranks, El = a.s.n_experts;
  if (tid == 0) *s_bad = 0;
  __syncthreads();
  for (int i = tid; i <= El * R; i += THREADS) {
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
  for (int e = tid; e <= El; e += THREADS) s_gbeg[e] = a.offsets[e * R];
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < El; ++e) {
      s_base[e] = acc;
      int me = s_gbeg[e + 1] - s_gbeg[e];
      acc += me ? row_tiles<BM, BAL>(me) * nt : 1;
    }
    s_base[El] = acc;
  }
  __syncthreads();
  return true;
}

// One tile of the persistent schedule.
struct TileWork {
  int e;        // local expert
  int g1;       // m_end: exclusive end of the expert's row group
  int m_abs;    // first row of the tile
  int n_abs;    // first column of the tile
  int rows;     // valid rows in the tile
  bool empty;   // signal-only item of an expert with no rows
};

// Item -> tile: item order is expert-major, then column tile, then row tile,
// so consecutive items share W_e slabs and X rows.  With GM > 0, an expert
// with more than GM row tiles is walked in bands of GM row tiles (band-major,
// then column tile, then row tile within the band): the workgroups of one XCD
// then share a few X row tiles and a few W_e slabs at a time instead of one
// slab and many row tiles.  Experts with at most GM row tiles keep the plain
// order.
// With BAL > 0 (see row_tiles) row tile mb of mt covers blocks
// [mb*B/mt, (mb+1)*B/mt) of the expert's B = ceil(me / 32) row blocks.
template <int BM, int BN, int GM = 0, int BAL = 0>
__device__ __forceinline__ TileWork tile_of(const GemmArgs& a, const int* s_base,
                                            const int* s_gbeg, int item) {
  TileWork t;
  const int El = a.s.n_experts;
  t.e = find_expert(s_base, El, item);
  const int g0 = s_gbeg[t.e];
  t.g1 = s_gbeg[t.e + 1];
  const int me = t.g1 - g0;
  t.empty = me == 0;
  const int mt = t.empty ? 1 : row_tiles<BM, BAL>(me);
  const int local = item - s_base[t.e];
  int mb = local % mt, nb = local / mt;
  if constexpr (GM > 0) {
    const int per = GM * (a.N / BN);           // items of one full band
    const int full = mt / GM;                  // full bands
    const int band = local / per;
    const int rows = band < full ? GM : mt - full * GM;
    const int o = local - band * per;
    mb = band * GM + o % rows;
    nb = o / rows;
  }
  t.n_abs = nb * BN;
  if constexpr (BAL > 0) {
    const int nbk = (me + 31) >> 5;
    const int b0 = mb * nbk / mt, b1 = (mb + 1) * nbk / mt;
    t.m_abs = g0 + 32 * b0;
    t.rows = t.empty ? 0 : min(32 * b1, me) - 32 * b0;
  } else {
    t.m_abs = g0 + mb * BM;
    t.rows = t.empty ? 0 : min(BM, t.g1 - t.m_abs);
  }
  return t;
}

// Source coordinates of one row of a tile, loaded before the tile's K loop so
// that their latency hides under it: owner rank rk (from the offsets of the
// row's group), token index t and pick index k (src_info).  rk < 0: row past
// m_end (not sent).
struct RowInfo {
  int rk;
  int t;
  int k;
};

__device__ __forceinline__ RowInfo load_row_info(const GemmArgs& a, int e, int g1, int m) {
  RowInfo ri{-1, 0, 0};
  if (m >= g1) return ri;
  ri.rk = 0;
  if (!a.sink_on) return ri;
  const int R = a.s.n_ranks;
  const int32_t* grp = a.offsets + e * R;
  int bound[kMaxRanks];   // all loads issued together, one wait
#pragma unroll
  for (int r = 1; r < kMaxRanks; ++r) bound[r] = r < R ? grp[r] : 0x7fffffff;
#pragma unroll
  for (int r = 1; r < kMaxRanks; ++r)
    if (bound[r] <= m) ri.rk = r;
  ri.t = a.src_info[2 * (size_t)m];
  ri.k = a.src_info[2 * (size_t)m + 1];
  return ri;
}

// Destination of row m (0 = not sent): the owner rank's receive buffer at the
// "P3PeerSendConfig" slot of (src_idx, src_topk) after the bounds check, or
// the local C row when the sink is disabled.
__device__ __forceinline__ uint64_t row_destination(const GemmArgs& a, uint8_t* const* s_recv,
                                                    const RowInfo& ri, int m) {
  if (ri.rk < 0) return 0;
  if (!a.sink_on) return (uint64_t)(a.c_local + (size_t)m * a.N * 2);
  if (ri.t < 0 || ri.t >= a.s.max_tokens || ri.k < 0 || ri.k >= a.s.top_k) {
    latch_error(a.s.err, kErrSlotOob);
    return 0;
  }
  return (uint64_t)(s_recv[ri.rk] + slot_offset(ri.t, ri.k, a.s.top_k, a.s.msg_bytes));
}

// Tiles whose rows are sent but whose completion is still to be counted.
// Completion is deferred to the next tile's prologue, which drains this
// workgroup's stores (vector memory operations of a wave complete in issue
// order, so the prologue's wait for its first copies also covers the earlier
// row stores), and up to kPendingMax tiles are counted together: one release
// fence, i.e. one write-back of the XCD's L2, covers the stores of all of
// them (a write-back per tile, let alone per wave, serialises on the L2).
// Experts whose last tile this workgroup counted are marked in `done` (an LDS
// bit set that only thread 0 touches); their counts and rank elections are
// published together when the workgroup's persistent loop ends.
constexpr int kPendingMax = 8;
constexpr int kDoneWords = kMaxLocalExperts / 32;

struct PendingTiles {
  int* e;                     // LDS, kPendingMax experts of the pending tiles (thread 0's)
  int n = 0;                  // pending tiles, the same in every thread
  uint32_t* done;             // LDS, kDoneWords words, zeroed at kernel start
  const int* base;            // LDS work table: expert e owns base[e+1] - base[e] items
};

// Tiles that expert e's items produce: one per item.
__device__ __forceinline__ int tiles_of(const PendingTiles& p, int e) {
  return p.base[e + 1] - p.base[e];
}

// Counts the pending tiles; called by every thread once all waves' row
// stores of those tiles are acknowledged by the L2 (each wave waited on its
// vmcnt, then a barrier).  Thread 0 issues the release fence and a relaxed
// fetch-add per tile on its expert's tile counter (fence + RMW = a release
// RMW), all RMWs before any result is examined.  An RMW that finds its
// expert's last tile marks the expert done.
__device__ __forceinline__ void complete_pending(const GemmArgs& a, PendingTiles& p) {
  if (p.n == 0) return;
  if (a.sink_on && threadIdx.x == 0) {
    fence_release(a.s.system_scope);
    int old[kPendingMax];
#pragma unroll
    for (int i = 0; i < kPendingMax; ++i)
      if (i < p.n)
        old[i] = a.s.system_scope
                     ? __hip_atomic_fetch_add(a.s.tile_counter + p.e[i], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM)
                     : __hip_atomic_fetch_add(a.s.tile_counter + p.e[i], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < kPendingMax; ++i)
      if (i < p.n && old[i] == tiles_of(p, p.e[i]) - 1)
        p.done[p.e[i] >> 5] |= 1u << (p.e[i] & 31);
  }
  p.n = 0;
}

// The barrier of a tile's K-loop prologue, after every wave has waited for
// its copies (and so for its earlier row stores).  When a batch of pending
// tiles is to be counted after it, the barrier is bracketed by workgroup-scope
// release and acquire fences: the raw barrier orders execution only, and the
// fences make every wave's row stores happen-before thread 0's agent-scope
// release fence in complete_pending.  (p.n is the same in every thread.)
__device__ __forceinline__ void prologue_barrier(const GemmArgs& a, PendingTiles& p) {
  if (p.n >= kPendingMax) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    raw_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    complete_pending(a, p);
  } else {
    raw_barrier();
  }
}

// offsets[e*R + r] for r = 0..kMaxRanks (indices clamped to the array), all
// loads issued together: expert e's run of rank rk holds
// bound[rk + 1] - bound[rk] rows for rk < R.
__device__ __forceinline__ void load_run_bounds(const GemmArgs& a, int e,
                                                int (&bound)[kMaxRanks + 1]) {
  const int R = a.s.n_ranks, last = a.s.n_experts * R;
#pragma unroll
  for (int r = 0; r <= kMaxRanks; ++r) bound[r] = a.offsets[min(e * R + r, last)];
}

// End of the persistent loop: drain and count what is left, then publish the
// experts this workgroup finished.  Thread 0: one acquire fence (it
// synchronises with every tile's release through the tile counters'
// modification order), re-arm of their tile counters and their count words,
// one release fence, then a relaxed fetch-add on each rank counter per
// expert.  A fetch-add that finds the other E_l - 1 experts of its rank done
// makes this thread the rank's last producer: after one more acquire fence,
// the re-arm of those rank counters and one more release fence it stores the
// rank flags.  The acquire-release election of "ep_signal_completion"
// (description), with at most four fences per workgroup.  In per-expert
// completion mode the count words are instead release-stored one by one,
// tagged with the step, and there is no election.
__device__ __forceinline__ void flush_pending(const GemmArgs& a, PendingTiles& p) {
  if (p.n > 0) {
    wait_vm<0>();
    __syncthreads();
    complete_pending(a, p);
  }
  if (!a.sink_on || threadIdx.x != 0) return;
  bool any = false;
  for (int w = 0; w < kDoneWords; ++w) any |= p.done[w] != 0;
  if (!any) return;
  const SinkState& s = a.s;
  const int R = s.n_ranks;
  fence_acquire(s.system_scope);
  if (s.per_expert) {
    // per-expert completion: each count word is its own release store
    for (int w = 0; w < kDoneWords; ++w)
      for (uint32_t m = p.done[w]; m; m &= m - 1) {
        const int e = w * 32 + __builtin_ctz(m);
        int bound[kMaxRanks + 1];
        load_run_bounds(a, e, bound);
        __hip_atomic_store(s.tile_counter + e, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int rk = 0; rk < kMaxRanks; ++rk)
          if (rk < R) publish_count_release(s, e, rk, (uint64_t)(bound[rk + 1] - bound[rk]));
      }
    return;
  }
  for (int w = 0; w < kDoneWords; ++w)
    for (uint32_t m = p.done[w]; m; m &= m - 1) {
      const int e = w * 32 + __builtin_ctz(m);
      // the expert's run bounds, all loads issued before any is used
      int bound[kMaxRanks + 1];
      load_run_bounds(a, e, bound);
      __hip_atomic_store(s.tile_counter + e, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint64_t* word = s.words + count_index(e, 0, R);
      if (s.system_scope) {
#pragma unroll
        for (int rk = 0; rk < kMaxRanks; ++rk)
          if (rk < R)
            __hip_atomic_store(word + rk, (uint64_t)(bound[rk + 1] - bound[rk]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      } else {
#pragma unroll
        for (int rk = 0; rk < kMaxRanks; ++rk)
          if (rk < R)
            __hip_atomic_store(word + rk, (uint64_t)(bound[rk + 1] - bound[rk]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  fence_release(s.system_scope);
  uint32_t won = 0;               // ranks whose last producer this is
  for (int w = 0; w < kDoneWords; ++w)
    for (uint32_t m = p.done[w]; m; m &= m - 1) {
      int old[kMaxRanks];
#pragma unroll
      for (int rk = 0; rk < kMaxRanks; ++rk)
        if (rk < R)
          old[rk] = s.system_scope ? __hip_atomic_fetch_add(s.rank_counter + rk, 1,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_SYSTEM)
                                   : __hip_atomic_fetch_add(s.rank_counter + rk, 1,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int rk = 0; rk < kMaxRanks; ++rk)
        if (rk < R && old[rk] == s.n_experts - 1) won |= 1u << rk;
    }
  if (!won) return;
  fence_acquire(s.system_scope);
  uint64_t* flags = s.words + (size_t)s.n_experts * R;
  for (int rk = 0; rk < R; ++rk)
    if (won & (1u << rk))
      __hip_atomic_store(s.rank_counter + rk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  fence_release(s.system_scope);
  const uint64_t epoch = step_epoch(s);
  for (int rk = 0; rk < R; ++rk)
    if (won & (1u << rk)) {
      if (s.system_scope)
        __hip_atomic_store(flags + rk, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      else
        __hip_atomic_store(flags + rk, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Consumer side of a fused launch (ep_grouped_gemm_scatter_combine): once the
// workgroup's tiles are done and its finished experts published, it runs its
// share of the combine runs, each after acquiring its rank's completion.
// Producers never wait for consumers, and every workgroup of the launch is
// resident at once (the grid never exceeds the workgroups the GPU holds), so
// the consumers' bounded waits are met as the other workgroups finish.
__device__ __forceinline__ void fused_consume(const GemmArgs& a, int* s_ok) {
  switch (a.comb_chunks) {
    case 4:
      combine_runs_ch<4>(a.comb, blockIdx.x, gridDim.x, a.comb_tokens_per_run,
                         a.comb_runs_per_rank, s_ok);
      break;
    case 8:
      combine_runs_ch<8>(a.comb, blockIdx.x, gridDim.x, a.comb_tokens_per_run,
                         a.comb_runs_per_rank, s_ok);
      break;
    default:
      combine_runs_ch<14>(a.comb, blockIdx.x, gridDim.x, a.comb_tokens_per_run,
                          a.comb_runs_per_rank, s_ok);
  }
}

// Signal-only work item of an expert with no rows: its tiles are all done
// (there are none), so it is published with the workgroup's finished experts
// (its counts are 0).
__device__ __forceinline__ void signal_empty_expert(const GemmArgs& a, int e, PendingTiles& p) {
  if (a.sink_on && threadIdx.x == 0) p.done[e >> 5] |= 1u << (e & 31);
}

// Zeroes the finished-expert set (thread 0; the work table's barriers order
// it before any use).
__device__ __forceinline__ void init_done(uint32_t* done) {
  if (threadIdx.x == 0)
    for (int w = 0; w < kDoneWords; ++w) done[w] = 0;
}

// The sink epilogue ("EpiloguePeerSink", send_tile): the finished fp32
// accumulators (32x32 MFMA blocks, lane holding 4 consecutive columns of one
// row per group) become a bf16 tile staged in LDS; each valid row is then
// sent with coalesced 16-byte nontemporal stores to its destination (row
// coordinates `ri` were loaded before the K loop).  The tile joins `pending`:
// it is counted at a later tile's prologue (or by flush_pending).  `jv`: valid
// MFMA row blocks of this wave.
template <int BM, int BN, int WM, int WN, int TM, int TN, int THREADS>
__device__ __forceinline__ void send_tile(const GemmArgs& a, const f32x16 (&acc)[TN][TM],
                                          uint8_t* smem, uint64_t* s_rowdst,
                                          uint8_t* const* s_recv, const TileWork& t, int wm,
                                          int wn, int jv, const RowInfo& ri,
                                          PendingTiles& pending) {
  constexpr int C_PITCH = BN * 2 + 16;   // bytes per staged row (16-byte skew against conflicts)
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < BM) s_rowdst[tid] = row_destination(a, s_recv, ri, t.m_abs + tid);
  const int frow = lane & 31, fhalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
      if (j < jv) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = wn * WN + i * 32 + 8 * g + 4 * fhalf;
          const int m = wm * WM + j * 32 + frow;
          u32x2 v;
          v[0] = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          v[1] = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<u32x2*>(smem + m * C_PITCH + n * 2) = v;
        }
      }
  __syncthreads();
  constexpr int TPR = BN * 2 / 16;          // threads per row
  constexpr int RPP = THREADS / TPR;        // rows per pass
  const int cr = tid / TPR, cc = tid % TPR;
  for (int r0 = 0; r0 < t.rows; r0 += RPP) {
    const int r = r0 + cr;
    if (r < t.rows) {
      const uint64_t dst = s_rowdst[r];
      if (dst) {
        u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * C_PITCH + cc * 16);
        store16_nt(reinterpret_cast<uint8_t*>(dst) + (size_t)t.n_abs * 2 + cc * 16, v);
      }
    }
  }
  // only thread 0 counts tiles: the list lives in LDS, not in per-lane
  // scratch memory, whose accesses would wait on this tile's row stores
  if (tid == 0) pending.e[pending.n] = t.e;
  ++pending.n;
  __syncthreads();   // the staged tile is read; the next tile may overwrite LDS
}

// Tile trace (EP_FLAG_TRACE).  Thread 0 writes a tile's record at `slot` in
// two parts, so no clock value stays live across the K loop: the start clock
// (word 2) when the tile begins, the coordinates (words 0-1) and the end clock
// (word 3) once its row stores are issued.  Slots past the buffer are dropped.
typedef __attribute__((address_space(1))) uint64_t global_u64;

__device__ __forceinline__ void trace_start(const GemmArgs& a, int slot) {
  if (!a.trace || threadIdx.x != 0 || slot >= a.trace_records) return;
  *(global_u64*)(a.trace + (size_t)slot * 4 + 2) = (uint64_t)wall_clock64();
}

__device__ __forceinline__ void trace_end(const GemmArgs& a, int slot, const TileWork& t,
                                          int cols) {
  if (!a.trace || threadIdx.x != 0 || slot >= a.trace_records) return;
  const uint64_t t_end = (uint64_t)wall_clock64();
  const uint64_t w0 = (uint64_t)(uint32_t)t.m_abs << 32 | (uint32_t)t.n_abs;
  const uint64_t w1 = (uint64_t)(t.e & 0xffff) | (uint64_t)(t.rows & 0xffff) << 16 |
                      (uint64_t)(cols & 0xffff) << 32 | (uint64_t)(blockIdx.x & 0xffff) << 48;
  uint64_t* rec = a.trace + (size_t)slot * 4;
  store16_nt(rec, u32x4{(uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1, (uint32_t)(w1 >> 32)});
  *(global_u64*)(rec + 3) = t_end;
}

// Measurement mode (EP_FLAG_EPILOGUE_ONLY): a tile without its K loop.  The
// accumulator of element (m, n) (m row of X, n output column) becomes the
// exact small integer (m*131 + n*7) mod 256, in the layout send_tile reads
// (lane holds columns n0 + 4*(lane/32) + 8g + q, q < 4, of row m0 + lane % 32
// in group g); then the ordinary sink epilogue.  Pending tiles are counted
// once eight have accumulated, after every wave has drained its stores.
template <int BM, int BN, int WM, int WN, int TM, int TN, int THREADS>
__device__ __forceinline__ void epilogue_only_tile(const GemmArgs& a, uint8_t* smem,
                                                   uint64_t* s_rowdst, uint8_t* const* s_recv,
                                                   const TileWork& t, int wm, int wn, int jv,
                                                   const RowInfo& ri, PendingTiles& pending) {
  if (pending.n >= kPendingMax) {
    wait_vm<0>();
    prologue_barrier(a, pending);
  }
  const int lane = threadIdx.x & 63;
  f32x16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = t.m_abs + wm * WM + j * 32 + (lane & 31);
          const int n = t.n_abs + wn * WN + i * 32 + 8 * g + 4 * (lane >> 5) + q;
          acc[i][j][4 * g + q] = (float)((m * 131 + n * 7) & 255);
        }
  send_tile<BM, BN, WM, WN, TM, TN, THREADS>(a, acc, smem, s_rowdst, s_recv, t, wm, wn, jv, ri,
                                             pending);
}

// The persistent loop of the measurement mode: items first, first + stride,
// ...; each tile's row coordinates are loaded one tile ahead, so their latency
// hides under the previous tile's epilogue as it hides under the K loop in a
// normal launch.
template <int BM, int BN, int WM, int WN, int TM, int TN, int THREADS, int TM0 = TM, int BAL = 0>
__device__ __forceinline__ void epilogue_only_loop(const GemmArgs& a, uint8_t* smem,
                                                   uint64_t* s_rowdst, uint8_t* const* s_recv,
                                                   const int* s_base, const int* s_gbeg,
                                                   PendingTiles& pending, int first, int stride,
                                                   int total, int wm, int wn) {
  const int tid = threadIdx.x;
  TileWork t{};
  RowInfo ri{-1, 0, 0};
  if (first < total) {
    t = tile_of<BM, BN, 0, BAL>(a, s_base, s_gbeg, first);
    if (!t.empty && tid < BM) ri = load_row_info(a, t.e, t.g1, t.m_abs + tid);
  }
  for (int item = first; item < total; item += stride) {
    TileWork tn{};
    RowInfo rin{-1, 0, 0};
    if (item + stride < total) {
      tn = tile_of<BM, BN, 0, BAL>(a, s_base, s_gbeg, item + stride);
      if (!tn.empty && tid < BM) rin = load_row_info(a, tn.e, tn.g1, tn.m_abs + tid);
    }
    if (t.empty) {
      signal_empty_expert(a, t.e, pending);
    } else {
      const int jv = min(wm == 0 ? TM0 : TM, max(0, (t.rows - wm * WM + 31) / 32));
      epilogue_only_tile<BM, BN, WM, WN, TM, TN, THREADS>(a, smem, s_rowdst, s_recv, t, wm, wn,
                                                          jv, ri, pending);
    }
    t = tn;
    ri = rin;
  }
}

}  // namespace gemm
}  // namespace ep
