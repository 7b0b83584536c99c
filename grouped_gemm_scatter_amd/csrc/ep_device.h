// Device-side helpers shared by the gfx950 kernels of the EP-combine step:
// vector types, the receive-slot formula, error latching and the rank-level
// completion protocol.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kMaxRanks = 8;
constexpr int kMaxLocalExperts = 256;

constexpr int kErrSlotOob = 0x1;
constexpr int kErrFlagTimeout = 0x2;
constexpr int kErrBadGroup = 0x4;

// Runtime state of the in-epilogue row send: the receive buffers of the R
// ranks, the count/flag words, the election counters and the error word
// ("P3PeerSendConfig", fields recv_buf_ptrs, n_ranks, top_k, msg_bytes,
// max_tokens_per_rank, atomic_counter).
struct SinkState {
  uint8_t* recv[kMaxRanks];
  uint64_t* words;          // E_l*R count words, then R rank flags
  int32_t* rank_counter;    // [R] election counters
  int32_t* tile_counter;    // [E_l] finished tiles of each expert in this step
  int32_t* err;
  uint64_t epoch;
  const uint64_t* epoch_ptr;  // device epoch word (read instead of epoch), or null
  int32_t n_ranks;
  int32_t n_experts;        // E_l, the election bound
  int32_t top_k;
  int32_t msg_bytes;
  int32_t max_tokens;
  int32_t system_scope;
  int32_t per_expert;       // per-expert completion: tagged count words, no elections
};

// The step's epoch: the device word when the handle keeps it there (it does
// not change during a launch: the stream orders its advance before it).
__device__ __forceinline__ uint64_t step_epoch(const SinkState& s) {
  return s.epoch_ptr ? *s.epoch_ptr : s.epoch;
}

// Byte offset of pick src_topk of token src_idx in its owner's receive buffer
// ("P3PeerSendConfig", description: recv_buf_layout).
__device__ __forceinline__ uint64_t slot_offset(int src_idx, int src_topk, int top_k,
                                                int msg_bytes) {
  return ((uint64_t)src_idx * (uint64_t)top_k + (uint64_t)src_topk) * (uint64_t)msg_bytes;
}

// Linear index of the count word of (local expert e, rank rk)
// ("P3PeerSendConfig", description: recv_count_layout).
__device__ __forceinline__ int count_index(int e, int rk, int n_ranks) { return e * n_ranks + rk; }

__device__ __forceinline__ void latch_error(int32_t* err, int bits) {
  __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One completion signal for (local expert e, destination rank rk), made by a
// single thread ("ep_signal_completion", description, with ep_ord_r and
// has_rank_flag): the count word is a plain progress store; the fetch-add on
// rk's election counter releases it (and everything this producer made
// visible before) and acquires all earlier producers' releases; the producer
// that finds E_l - 1 there happens-after every other producer of rk, re-arms
// the counter and release-stores the rank flag.  Returns true when elected.
__device__ __forceinline__ bool signal_rank(const SinkState& s, int e, int rk, uint64_t value) {
  uint64_t* word = s.words + count_index(e, rk, s.n_ranks);
  uint64_t* flag = s.words + (size_t)s.n_experts * s.n_ranks + rk;
  int32_t* ctr = s.rank_counter + rk;
  int old;
  if (s.system_scope) {
    __hip_atomic_store(word, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_SYSTEM);
  } else {
    __hip_atomic_store(word, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (old != s.n_experts - 1) return false;
  __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (s.system_scope)
    __hip_atomic_store(flag, step_epoch(s), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  else
    __hip_atomic_store(flag, step_epoch(s), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Agent- or system-scope fences.
__device__ __forceinline__ void fence_release(int system_scope) {
  if (system_scope)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
  else
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire(int system_scope) {
  if (system_scope)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  else
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Per-expert completion: count word (e, rk) = the step's tag (low 32 bits of
// the epoch) in the high half and the row count in the low half, published
// by a release store of its own.
__device__ __forceinline__ uint64_t tagged_count(uint64_t epoch, uint64_t rows) {
  return (epoch << 32) | (rows & 0xffffffffull);
}
__device__ __forceinline__ void publish_count_release(const SinkState& s, int e, int rk,
                                                      uint64_t rows) {
  uint64_t* word = s.words + count_index(e, rk, s.n_ranks);
  const uint64_t v = tagged_count(step_epoch(s), rows);
  if (s.system_scope)
    __hip_atomic_store(word, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  else
    __hip_atomic_store(word, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Pause between polls of a bounded wait: 128 clocks for the first polls,
// doubling every 16 polls up to 16 x 128 clocks, so that many waiting
// workgroups do not keep the polled line busy while producers still work.
__device__ __forceinline__ void poll_pause(int64_t i) {
  const int reps = i < 16 ? 1 : i < 32 ? 2 : i < 48 ? 4 : i < 64 ? 8 : 16;
  for (int r = 0; r < reps; ++r) __builtin_amdgcn_s_sleep(2);
}

// Bounded acquire wait for a per-expert count word carrying this step's tag.
__device__ __forceinline__ bool acquire_count(const uint64_t* word, uint64_t epoch, int64_t limit,
                                              int system_scope) {
  for (int64_t i = 0; i < limit; ++i) {
    const uint64_t v = system_scope
                           ? __hip_atomic_load(word, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM)
                           : __hip_atomic_load(word, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if ((v >> 32) == (epoch & 0xffffffffull)) return true;
    poll_pause(i);
  }
  return false;
}

// Bounded acquire wait for a rank flag.  Returns false after `limit` polls.
__device__ __forceinline__ bool acquire_flag(const uint64_t* flag, uint64_t epoch, int64_t limit,
                                             int system_scope) {
  for (int64_t i = 0; i < limit; ++i) {
    uint64_t v = system_scope
                     ? __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM)
                     : __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if (v == epoch) return true;
    poll_pause(i);
  }
  return false;
}

// 16-byte accesses to global memory.  The pointers are cast to the global
// address space: a generic pointer (one read back from LDS, say) would make
// them flat instructions, which also count on the LDS counter, so every wait
// for an LDS read would wait for the flat stores issued before it as well.
typedef __attribute__((address_space(1))) u32x4 global_u32x4;

// Nontemporal 16-byte global store (streamed: no reuse by this kernel).
__device__ __forceinline__ void store16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, (global_u32x4*)p);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *(const global_u32x4*)p;
}

__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load((const global_u32x4*)p);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  uint16_t ua = __builtin_bit_cast(uint16_t, a), ub = __builtin_bit_cast(uint16_t, b);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

}  // namespace ep
