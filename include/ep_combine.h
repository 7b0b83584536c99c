/*
 * ep_combine.h -- C ABI of the MI355X (gfx950) MoE expert-parallel combine.
 *
 * One EP-combine step on one GPU's share of an expert-parallel MoE layer:
 *
 *   1. ep_grouped_gemm_scatter: a grouped GEMM runs every local expert's
 *      down-projection over that expert's contiguous row group and, instead
 *      of storing a local C, sends each finished bf16 output row straight to
 *      the receive buffer of the rank that owns the row ("EpiloguePeerSink",
 *      Mojo trait page: description, member Enabled, method send_tile).
 *      The row for pick src_topk of token src_idx lands at byte
 *      (src_idx*top_k + src_topk)*msg_bytes + byte_off of its owner's buffer
 *      ("P3PeerSendConfig", Mojo struct page: description).  When the last
 *      tile of expert e is stored, the kernel publishes, for every rank rk,
 *      the row count of (e, rk) in count word e*n_ranks + rk and takes part in
 *      an acquire-release election on rk's counter; the producer elected last
 *      release-stores rk's rank-completion flag ("ep_signal_completion",
 *      Mojo function page: description, parameters ep_ord_r, has_rank_flag,
 *      n_experts_per_device).
 *   2. ep_combine_reduce: the consumer acquires each source rank's flag once
 *      and forms the top-k routing-weighted sum of the slots of that rank's
 *      tokens.
 *
 * The R ranks are R logical receive buffers in this GPU's memory.  Every
 * pointer argument named "device" is GPU memory owned by the caller; the
 * library never allocates or frees device memory.  All step calls are
 * asynchronous and ordered on the given stream (a hipStream_t passed as
 * void*, NULL meaning the null stream); a handle must be used by one stream
 * at a time.  Host-detectable errors are returned synchronously as negative
 * codes; faults found by the kernels are latched into the caller's error word
 * as positive bits and read back by ep_combine_query_error.
 */
#ifndef EP_COMBINE_H
#define EP_COMBINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define EP_API __attribute__((visibility("default")))
#else
#define EP_API
#endif

#define EP_MAX_RANKS 8            /* capacity of recv_buf_ptrs ("P3PeerSendConfig", fields) */
#define EP_MAX_LOCAL_EXPERTS 256

/* return codes (negative: synchronous, host-detected) */
#define EP_OK 0
#define EP_ERR_INVALID_ARG (-1)   /* null pointer, bad size, misalignment, bad epoch */
#define EP_ERR_UNSUPPORTED (-2)   /* shape, dtype or flag combination the library does not handle */
#define EP_ERR_HIP (-3)           /* a HIP runtime call or kernel launch failed */

/* device error bits latched into ep_combine_buffers.error_word */
#define EP_ERR_SLOT_OOB 0x1       /* a row's slot fell outside its receive buffer; not written */
#define EP_ERR_FLAG_TIMEOUT 0x2   /* the combine gave up waiting for a rank flag */
#define EP_ERR_BAD_GROUP 0x4      /* offsets not monotone / not ending at m_total */

/* element types of X and W */
#define EP_DTYPE_BF16 0           /* bf16 X [M][K], bf16 W [E_l][N][K] */
#define EP_DTYPE_FP8_E4M3_B128 1  /* e4m3fn X, W + fp32 scales, 1x128 (X) and 128x128 (W) blocks */

/* flags */
#define EP_FLAG_SYSTEM_SCOPE 0x1  /* publish / acquire flags at system scope instead of agent scope */
/* Per-expert completion ("ep_signal_completion", description, the form without
   ep_ord_r, where a consumer must look at every expert's own signal): every
   count word is published by its own release store, tagged with the step as
   (epoch & 0xffffffff) << 32 | rows, and the consumer acquires each of the E_l
   count words of a rank instead of one rank flag.  No rank elections; the
   rank counters and flag words are left untouched.  E_l*R release stores per
   step instead of R.  In this mode an epoch whose low 32 bits are zero is
   rejected (EP_ERR_INVALID_ARG): zeroed count words would read as carrying
   it; epochs need only differ modulo 2^32 from one step to the next. */
#define EP_FLAG_PER_EXPERT_RELEASE 0x2
/* Measurement mode of ep_grouped_gemm_scatter: the K loop is skipped and the
   accumulator of output element (m, n) (m = row of X, n = output column) is
   set to the exact small integer (m*131 + n*7) mod 256 before the epilogue, so
   the launch times the sink epilogue alone (row lookups, scatter stores, counts
   and completion) at the real shape.  Every other effect of the call (slot
   placement, count words, elections, flags, error bits) is that of a normal
   step. */
#define EP_FLAG_EPILOGUE_ONLY 0x4
/* Tile trace ("P3PeerSendConfig" fields trace_ptr / trace_on and
   send_stamp_ptr / send_stamp_on, whose contents the pages leave open): every
   non-empty GEMM tile of ep_grouped_gemm_scatter writes one record of four
   u64 words at buffers.trace + 4*slot:
     w0 = m0 << 32 | n0        first row (in X's grouped order) and column
     w1 = e | rows << 16 | cols << 32 | workgroup << 48
                               local expert, tile rows before m_end, tile
                               columns, the workgroup that ran it
     w2 = t_start              device wall clock when the workgroup began the
                               tile (before its first K-slice copy)
     w3 = t_end                wall clock once its row stores were issued
   Clock ticks are those of the device's constant-rate wall clock
   (hipDeviceAttributeWallClockRate, kHz).  Slots are distinct within one
   launch (a tile's work item, tiles of a split last round after the others);
   records whose slot is >= buffers.trace_records are not written, nor is any
   slot without a tile, so the caller zeroes the buffer before a traced launch
   (w2 == 0 marks an unused slot).  Off by default; the measurement mode
   (EP_FLAG_EPILOGUE_ONLY) and the other calls write no records. */
#define EP_FLAG_TRACE 0x8
/* Weight layout of the down-projection (bf16 handles only; EP_ERR_UNSUPPORTED
   with fp8): ep_grouped_gemm_scatter and its variants read W as
   [E_l][K/64][N][64], the layout ep_pack_weights writes, in which the
   64-element K slice of a block of output columns is one contiguous run.
   The arithmetic and every result are those of the row-major layout; what
   changes is the HBM access pattern, which the decode-shaped GEMM (a stream
   of W with few rows per expert) reads faster, and the prefill-shaped one
   slightly slower.  The up-projection's W1 stays row-major. */
#define EP_FLAG_W_SLICE_MAJOR 0x10
/* Device-resident epoch, for callers that capture a step in a HIP graph (its
   replays cannot take a new epoch argument): every call of the handle then
   takes epoch = 0 (EP_ERR_INVALID_ARG otherwise) and its kernels read the
   step's epoch from buffers.epoch_word, which ep_advance_epoch moves one step
   forward on the stream.  A step is then ep_advance_epoch, then the producer
   and consumer calls; the flags and tagged count words carry the word's value
   exactly as they carry a host epoch. */
#define EP_FLAG_DEVICE_EPOCH 0x20
/* The bf16 GEMM on the tile of the send-wave kernel (128 x 128 outputs, three
   K-slice stages, 8 MFMA waves) with params.send_waves = 0: the same kernel
   with the sink inside the MFMA waves, the reference point for the send waves
   ("EpiloguePeerSink", SendWarps = 0).  EP_ERR_UNSUPPORTED with fp8,
   EP_FLAG_EPILOGUE_ONLY or EP_FLAG_TRACE; ep_grouped_gemm_scatter_combine
   returns EP_ERR_UNSUPPORTED for such a handle. */
#define EP_FLAG_SEND_TILE 0x40

typedef struct ep_combine_params {
  int32_t n_ranks;               /* R: ranks with a receive buffer, 1..8 */
  int32_t p2p_world_size;        /* ranks reachable by direct stores; must equal n_ranks */
  int32_t my_rank;               /* this GPU's rank; local experts are global ids
                                    [my_rank*E_l, (my_rank+1)*E_l) */
  int32_t top_k;                 /* picks per token */
  int32_t msg_bytes;             /* bytes per slot; >= 2*hidden_n, multiple of 16 */
  int32_t max_tokens_per_rank;   /* T: slots per rank = T*top_k */
  int32_t n_experts_per_device;  /* E_l: local experts, also the election bound */
  int32_t hidden_k;              /* K: reduction width, multiple of 64 (128 for fp8) */
  int32_t hidden_n;              /* N: output width, multiple of 128 */
  int32_t dtype;                 /* EP_DTYPE_* */
  uint32_t flags;                /* EP_FLAG_* */
  /* Dedicated send waves ("EpiloguePeerSink", comptime member SendWarps, and
     its methods service, drain and shutdown): 0, or 4 for bf16 handles.  With
     4, the grouped GEMM runs 8 MFMA waves and 4 send waves per workgroup on
     128 x 128 tiles, one workgroup per CU: the MFMA waves stage each finished
     tile in LDS and go on with the next tile while the send waves send the
     staged rows to their slots (service), count the tile once their stores
     are acknowledged (drain: what the previous tile left pending) and,
     after the last tile, publish the finished experts (shutdown).  Results,
     slots, counts, flags and error behaviour are those of the default kernels.
     Same restrictions as EP_FLAG_SEND_TILE; other values EP_ERR_INVALID_ARG. */
  int32_t send_waves;
  int64_t flag_spin_limit;       /* combine's bounded wait, in polls per flag; 0 = default (2^22) */
} ep_combine_params;

typedef struct ep_combine_buffers {
  /* device: R receive buffers of max_tokens_per_rank*top_k*msg_bytes bytes
     each, 16-byte aligned; entries >= n_ranks are ignored */
  void* recv_buf[EP_MAX_RANKS];
  /* device: E_l*R + R u64 words: count word e*R + rk for each (local expert e,
     rank rk), then the R rank-completion flags (word E_l*R + rk).  A count
     word holds the row count; with EP_FLAG_PER_EXPERT_RELEASE it also carries
     the step's tag in its high 32 bits */
  uint64_t* recv_count;
  int32_t* rank_counter;         /* device: R election counters, zero before first use */
  int32_t* tile_counter;         /* device: E_l per-expert tile counters, zero before first use */
  int32_t* error_word;           /* device: one int32, zero before first use */
  /* device, used only with EP_FLAG_TRACE: trace_records records of four u64
     words (16-byte aligned); NULL / 0 otherwise */
  uint64_t* trace;
  int64_t trace_records;
  /* device, used only with EP_FLAG_DEVICE_EPOCH: one u64 holding the current
     step's epoch (8-byte aligned, zero before the first ep_advance_epoch);
     NULL otherwise */
  uint64_t* epoch_word;
} ep_combine_buffers;

typedef struct ep_combine_handle* ep_combine_t;

/* Sets up the send state of one GPU's share ("P3PeerSendConfig", Mojo struct
   page: fields recv_buf_ptrs (at most 8 peer buffers), n_ranks, p2p_world_size,
   top_k, msg_bytes, max_tokens_per_rank, my_rank and atomic_counter, and the
   disabled() default, whose pointers are dereferenced only when p3_control >= 0,
   the per-call gate of ep_grouped_gemm_scatter here; "ep_signal_completion",
   Mojo function page: the count buffer with its rank-flag tail and parameter
   n_experts_per_device, the election bound).  Validates the geometry,
   records the caller's device buffers and picks kernel configurations for
   the current device.  No device work and no device memory: the buffers are
   the caller's and must outlive the handle.  Returns EP_OK and *out, or a
   negative code (EP_ERR_INVALID_ARG for a bad size, null or misaligned
   buffer; EP_ERR_UNSUPPORTED for p2p_world_size != n_ranks or a shape the
   kernels do not tile; EP_ERR_HIP when the device cannot be queried). */
EP_API int ep_combine_init(const ep_combine_params* params, const ep_combine_buffers* bufs,
                    ep_combine_t* out);

EP_API void ep_combine_destroy(ep_combine_t h);

/* Grouped GEMM + in-epilogue row scatter + fused completion signalling
   ("EpiloguePeerSink" send_tile; "P3PeerSendConfig" description;
   "ep_signal_completion" description).

   x        device, [m_total][K] bf16 (or e4m3fn bytes): the dispatched rows,
            grouped by local expert e, and inside a group by source rank rk.
   w        device, [E_l][N][K] bf16 (or e4m3fn): W_e is the logical K x N matrix,
            stored K-contiguous; with EP_FLAG_W_SLICE_MAJOR (bf16), the same
            values laid out [E_l][K/64][N][64] by ep_pack_weights.
   x_scale  device, [m_total][K/128] fp32, fp8 only (else may be NULL).
   w_scale  device, [E_l][N/128][K/128] fp32, fp8 only (else may be NULL).
   offsets  device, E_l*R + 1 int32: rows [offsets[e*R+rk], offsets[e*R+rk+1])
            come from rank rk for expert e; group e ends at m_end = offsets[(e+1)*R];
            offsets[0] = 0 and offsets[E_l*R] = m_total.
   src_info device, [m_total][2] int32: (src_idx, src_topk) = the row's token
            index on its owner rank and its pick position.
   m_total  number of rows (host value; must equal offsets[E_l*R]).
   p3_control  runtime gate: >= 0 sends rows to the receive buffers and signals;
            < 0 disables the sink: the GEMM stores bf16 [m_total][N] to c_local
            and no receive buffer, count word or flag is touched.
   c_local  device, used only when p3_control < 0 (else ignored, may be NULL).
   epoch    the value this step's rank flags are set to; nonzero, and different
            from the previous step's (callers count 1, 2, 3, ...); with
            EP_FLAG_PER_EXPERT_RELEASE its low 32 bits must be nonzero.
   stream   hipStream_t as void*.
   Slots outside a receive buffer latch EP_ERR_SLOT_OOB and are skipped;
   inconsistent offsets latch EP_ERR_BAD_GROUP and the launch does nothing. */
EP_API int ep_grouped_gemm_scatter(ep_combine_t h, const void* x, const void* w,
                            const float* x_scale, const float* w_scale,
                            const int32_t* offsets, const int32_t* src_info,
                            int32_t m_total, int32_t p3_control, void* c_local,
                            uint64_t epoch, void* stream);

/* Allocation-free form of ep_grouped_gemm_scatter, for callers that cannot
   allocate device memory or run a call that might (code under HIP graph
   capture, tight serving loops): same arguments, results and errors, but the
   election counters and per-expert tile counters the call works with are the
   library's own, a device array of EP_MAX_RANKS + EP_MAX_LOCAL_EXPERTS int32
   words (1056 bytes) that every GPU holds once, from the first ep_combine_init
   on it until the process ends; buffers.rank_counter and buffers.tile_counter
   are not touched.  The call allocates nothing: it zeroes the counters with a
   small kernel on `stream`, then launches the GEMM as ep_grouped_gemm_scatter.
   Every call on one GPU shares that array, so calls that overlap in time on one
   GPU (on different streams, or from several handles) race and must not be
   issued; and since a step's elections run on these counters, a step made with
   this call must not also signal through ep_signal_completion.
   Returns EP_ERR_HIP when no handle was ever initialised on the current device
   (the array's address is looked up there), EP_ERR_UNSUPPORTED for a geometry
   beyond the array (not reachable through ep_combine_init's own limits). */
EP_API int ep_grouped_gemm_scatter_noalloc(ep_combine_t h, const void* x, const void* w,
                                           const float* x_scale, const float* w_scale,
                                           const int32_t* offsets, const int32_t* src_info,
                                           int32_t m_total, int32_t p3_control, void* c_local,
                                           uint64_t epoch, void* stream);

/* The GEMM tile ep_grouped_gemm_scatter uses for a call with m_total rows on
   this handle (no device work): returns the tile kind (>= 0: 0 = 256 x 256 for
   fp8, and for bf16 256 columns by up to 288 rows, an expert's rows spread
   evenly over the fewest tiles of at most nine 32-row blocks, 1 = 128 x 128, 2 = 256 x 128, 3 = 64 x 128, the small-row-group tile used
   when m_total <= 48 * E_l with bf16 and N a multiple of 256, 4 = 128 x 128
   with dedicated send waves, 5 = the same tile with the sink inside the MFMA
   waves) and writes its rows and columns; a negative code for a null handle or pointer or a
   negative m_total. */
EP_API int ep_gemm_tile(ep_combine_t h, int32_t m_total, int32_t* tile_rows, int32_t* tile_cols);

/* Local grouping of the routing: the layout ep_grouped_gemm_scatter takes as
   offsets and src_info.  A pick (rk, t, k) is local when its global expert g
   lies in [my_rank*E_l, (my_rank+1)*E_l); it becomes a row of group
   e = g - my_rank*E_l ("EpiloguePeerSink", send_tile argument expert_id).
   Rows are ordered by (e, rk, t, k):
     offsets[e*R + rk]  first row of expert e's run of rank rk (the count
                        layout e*n_ranks + rk of "P3PeerSendConfig",
                        description), offsets[0] = 0, offsets[E_l*R] = M
     src_info[m]        (t, k) of row m ("P3PeerSendConfig", src_info_ptr)
   topk_ids         device [R][tokens_per_rank][top_k] int32 global expert ids;
                    ids outside the local slice (a negative id included) are
                    not rows.
   tokens_per_rank  0..max_tokens_per_rank.
   offsets          device, E_l*R + 1 int32, written.
   src_info         device, room for R*tokens_per_rank*top_k rows of 2 int32
                    (every pick local); rows [0, M) are written, nothing else.
   Deterministic: the result depends on topk_ids only.  Three stream-ordered
   launches; M is read from offsets[E_l*R]. */
EP_API int ep_group_local_picks(ep_combine_t h, const int32_t* topk_ids, int32_t tokens_per_rank,
                                int32_t* offsets, int32_t* src_info, void* stream);

/* Dispatch side of the expert FFN on this GPU's share: every grouped row m
   receives the hidden row of its pick's token, the input of the up-projection
   (the expert FFN's first GEMM; the sink epilogue of "P3PeerSendConfig",
   description, sits in the second).  In a multi-GPU layer each token's owner
   sends that row to the GPU owning the expert; here the R source ranks are R
   logical token arrays in this GPU's memory and the rows are gathered on the
   receiving side.
     x_out[m][:] = tokens_x[rk][t][:]   for m < m_total, where rk is the rank
                                        run of offsets holding m and
                                        t = src_info[m][0]
   tokens_x        device [R][tokens_per_rank][row_bytes] (16-byte aligned)
   row_bytes       bytes per row, a multiple of 16 (2*hidden for bf16 rows)
   offsets, src_info, m_total  the grouped layout (ep_group_local_picks)
   x_out           device [m_total][row_bytes], written for every row.
   A token index outside [0, tokens_per_rank) latches EP_ERR_BAD_GROUP and
   that row is not written.  One launch; nothing else is touched. */
EP_API int ep_dispatch_rows(ep_combine_t h, const void* tokens_x, int32_t tokens_per_rank,
                            int32_t row_bytes, const int32_t* offsets, const int32_t* src_info,
                            int32_t m_total, void* x_out, void* stream);

/* Moves the device-resident epoch of an EP_FLAG_DEVICE_EPOCH handle one step
   forward (epoch_word + 1, skipping values whose low 32 bits are zero, which
   per-expert completion could not tell from unwritten count words).  One
   single-thread launch on `stream`, nothing else is touched; EP_ERR_UNSUPPORTED
   for a handle without the flag.  Calls on one handle must not overlap. */
EP_API int ep_advance_epoch(ep_combine_t h, void* stream);

/* Weight re-layout for EP_FLAG_W_SLICE_MAJOR: writes
     w_out[e][s][n][j] = w[e][n][64*s + j]   (e < E_l, s < K/64, n < N, j < 64)
   for the handle's E_l, N = hidden_n and K = hidden_k.  A one-time transform
   of static weights (layout only: the values of the page "EpiloguePeerSink"'s
   W_e are unchanged), needed before a handle created with
   EP_FLAG_W_SLICE_MAJOR multiplies by them; any bf16 handle of the same shape
   may run it.
   w, w_out  device, E_l*N*K bf16 each, 16-byte aligned, not overlapping
             (EP_ERR_INVALID_ARG otherwise).
   bf16 handles only (EP_ERR_UNSUPPORTED for fp8).  One launch on `stream`;
   nothing but w_out is written. */
EP_API int ep_pack_weights(ep_combine_t h, const void* w, void* w_out, void* stream);

/* Up-projection with SwiGLU: the expert FFN's first grouped GEMM, whose
   output is the x of ep_grouped_gemm_scatter (the sink epilogue on the page
   "P3PeerSendConfig" belongs to the FFN's second GEMM; this is the first one
   feeding it).  With hidden = hidden_n and I = hidden_k of the handle:
     h_out[m][i] = bf16( silu(g) * u ),  silu(g) = g / (1 + e^-g),
     g = sum_k x1[m][k] * w1[e][i][k],  u = sum_k x1[m][k] * w1[e][I + i][k]
   accumulated in fp32, for every row m of expert e's group.
   x1       device, [m_total][hidden] bf16, grouped by local expert like x.
   w1       device, [E_l][2I][hidden] bf16: gate rows 0..I-1, then up rows.
   offsets  device, E_l*R + 1 int32, as for ep_grouped_gemm_scatter.
   h_out    device, [m_total][I] bf16, written for every row; nothing else is.
   bf16 handles only (EP_ERR_UNSUPPORTED for fp8), I a multiple of 128.
   Inconsistent offsets latch EP_ERR_BAD_GROUP and the launch does nothing.
   No receive buffer, count word or flag is touched. */
EP_API int ep_grouped_gemm_swiglu(ep_combine_t h, const void* x1, const void* w1,
                                  const int32_t* offsets, int32_t m_total, void* h_out,
                                  void* stream);

/* Up-projection with SwiGLU on block-scaled fp8 operands, the first GEMM of the
   fp8 expert FFN, whose output is the fp8 x (with x_scale) of
   ep_grouped_gemm_scatter on the same handle (the blockwise fp8 family with
   1-D activation and 2-D weight scales, "P3PeerSendConfig", description).
   With hidden = hidden_n and I = hidden_k of the handle, for every row m of
   expert e's group:
     g = sum_b x1_scale[m][b] * w1_scale[e][i/128][b] * sum_{k in block b} x1[m][k] w1[e][i][k]
     u = the same with the up rows I + i,   h = silu(g) * u   (fp32)
   then per (row, block of 128 outputs): scale = amax |h| / 448 (1 if all are
   zero), h_out = e4m3fn(h / scale) rounded to nearest even, h_scale = scale.
   x1       device, [m_total][hidden] e4m3fn codes, grouped like x.
   x1_scale device, [m_total][hidden/128] fp32.
   w1       device, [E_l][2I][hidden] e4m3fn codes: gate rows 0..I-1, then up rows.
   w1_scale device, [E_l][2I/128][hidden/128] fp32.
   offsets  device, E_l*R + 1 int32, as for ep_grouped_gemm_scatter.
   h_out    device, [m_total][I] e4m3fn codes; h_scale device, [m_total][I/128]
            fp32; both written for every row, nothing else is.
   fp8 handles only (EP_ERR_UNSUPPORTED for bf16).  Inconsistent offsets latch
   EP_ERR_BAD_GROUP and the launch does nothing.  No receive buffer, count word
   or flag is touched. */
EP_API int ep_grouped_gemm_swiglu_fp8(ep_combine_t h, const void* x1, const float* x1_scale,
                                      const void* w1, const float* w1_scale,
                                      const int32_t* offsets, int32_t m_total, void* h_out,
                                      float* h_scale, void* stream);

/* Standalone batched form of the completion signal ("ep_signal_completion",
   description and args signal_offset, signal, rank_completion_counter,
   rank_flag_offset, with ep_ord_r and has_rank_flag set): for i < n, stores
   signal[i] into count word expert[i]*R + dst_rank[i], then fetch-adds
   dst_rank[i]'s election counter with acquire-release ordering; the producer
   that brings it to E_l re-arms it and release-stores flag word E_l*R + dst_rank
   = epoch.  With EP_FLAG_PER_EXPERT_RELEASE each signal is instead one
   release store of the tagged count word, with no election.  expert, dst_rank,
   signal: device arrays of n entries; signal[i] < 2^32 in that mode.  Each
   (expert, dst_rank) pair must be signalled exactly once per step, by this
   call or by the fused GEMM epilogue, never both. */
EP_API int ep_signal_completion(ep_combine_t h, const int32_t* expert, const int32_t* dst_rank,
                         const uint64_t* signal, int32_t n, uint64_t epoch, void* stream);

/* Consumer combine ("P3PeerSendConfig", Mojo struct page: description, the
   combine kernel that reads each slot (src_idx, src_topk) of the receive
   buffers; "ep_signal_completion", Mojo function page: description, a
   consumer that acquires a source rank's completion once rather than each
   expert's).  For every source rank rk the kernel acquires flag word
   E_l*R + rk once (with EP_FLAG_PER_EXPERT_RELEASE: each count word e*R + rk,
   e < E_l, until its tag is this step's) (bounded wait: EP_ERR_FLAG_TIMEOUT,
   outputs of that rank left untouched), then for each token t <
   tokens_per_rank writes
     out[rk][t][:] = bf16( sum over k ascending with topk_ids[rk][t][k] local
                           of topk_w[rk][t][k] * slot(rk, t, k)[:] )
   accumulated in fp32; a token with no local pick gets +0.
   topk_ids device [R][tokens_per_rank][top_k] int32 global expert ids;
   topk_w   device [R][tokens_per_rank][top_k] fp32;
   out      device [R][tokens_per_rank][N] bf16.
   tokens_per_rank <= max_tokens_per_rank. */
EP_API int ep_combine_reduce(ep_combine_t h, const int32_t* topk_ids, const float* topk_w,
                      int32_t tokens_per_rank, void* out, uint64_t epoch, void* stream);

/* One EP-combine step in a single launch: ep_grouped_gemm_scatter (sink on)
   followed by ep_combine_reduce, with the consumer inside the same grid
   ("ep_signal_completion", description: a consumer fused into the kernel that
   acquires once per source rank; "P3PeerSendConfig", description: the combine
   kernel reading the receive slots).  Every workgroup first runs its share of
   the GEMM tiles with the sink epilogue and publishes the experts it finished
   (counts, rank elections, flags), then runs combine runs, each of one
   source rank's tokens, after acquiring that rank's completion with the
   bounded wait (EP_ERR_FLAG_TIMEOUT: that run's outputs left untouched).
   Producers never wait for consumers; consumers wait for producers of other
   workgroups of the same launch, so the launch takes one workgroup per GPU
   slot (every workgroup resident at once) and needs the GPU to itself: a
   kernel running beside it can hold slots a producer needs, and the waits then
   end in EP_ERR_FLAG_TIMEOUT rather than a result.
   Arguments are those of the two calls; the results (receive buffers, count
   words, flags, counters, out) equal theirs bit for bit.  Not with
   EP_FLAG_EPILOGUE_ONLY or EP_FLAG_TRACE (EP_ERR_UNSUPPORTED);
   tokens_per_rank >= 1. */
EP_API int ep_grouped_gemm_scatter_combine(ep_combine_t h, const void* x, const void* w,
                                           const float* x_scale, const float* w_scale,
                                           const int32_t* offsets, const int32_t* src_info,
                                           int32_t m_total, const int32_t* topk_ids,
                                           const float* topk_w, int32_t tokens_per_rank,
                                           void* out, uint64_t epoch, void* stream);

/* Synchronizes the stream, returns the latched device error bits (>= 0) and
   clears them, or a negative code if the read failed. */
EP_API int ep_combine_query_error(ep_combine_t h, void* stream);

/* Static description of a code: never NULL. */
EP_API const char* ep_combine_strerror(int code);

/* Library version, as major*10000 + minor*100 + patch. */
EP_API int ep_combine_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_COMBINE_H */
