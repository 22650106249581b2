/*
 * cp_attn.h -- causal ring attention, one context-parallel rank's share, on
 * AMD MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * Sources (web pages, cited by title and section):
 *   [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练"
 *         (mieleap.com/news/151524), sections 1-6.
 *   [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention"
 *         (devpress.csdn.net), sections 1-5.
 *
 * The operation.  A rank holds a local block of queries and, over the steps of
 * a ring, receives the K/V blocks of the other ranks ([RAF] section 3: the
 * RingAttention loop; at step j rank r uses the block of rank (r - j) mod N).
 * For every local query at absolute position i it computes causal softmax
 * attention over every key at position j <= i ([RAF] section 1; [RAF] section
 * 3, note 2: the mask comes from the blocks' absolute offsets):
 *
 *     LSE_i = ln sum_{j<=i} exp(tau <q_i,k_j>),   out_i = sum_{j<=i} exp(tau <q_i,k_j> - LSE_i) v_j
 *
 * Each ring step yields a partial (O, LSE) over its key block; partials are
 * combined by log-sum-exp rescaling (the exact rule behind the page's
 * simplified "add the chunk outputs" in [RAF] section 3, step 5).
 * Sharding uses the 2N zigzag split of [RAF] section 5, item 1.
 *
 * Conventions for every entry point:
 *   - Tensors are dense, contiguous, row-major [B, H, S, D] (D fastest),
 *     device pointers, 16-byte aligned.  Q/K/V/out are bf16 (raw 16-bit
 *     storage, passed as void*); O and LSE accumulators are fp32.
 *   - A "local" buffer of S tokens is n_chunks chunks of chunk_len tokens,
 *     concatenated in order; cp_chunks_t.start[i] is the absolute position of
 *     the first token of chunk i in the full sequence.
 *   - LSE is the natural-log sum of exp(tau * q.k); -INFINITY marks a row
 *     that has no visible key (its O is 0).
 *   - Ownership: the caller owns every device buffer, including workspace.
 *     The library never allocates device memory.  Host arrays and structs are
 *     read only during the call.
 *   - Asynchrony: calls only enqueue work on the given stream(s); inputs must
 *     stay valid until that work has run.  Kernel faults surface at the
 *     caller's next synchronisation.
 *   - Errors: arguments are checked before anything is enqueued.  A non-OK
 *     status leaves every output untouched and sets a thread-local message
 *     readable with cp_last_error().  No C++ exception crosses the ABI.
 *   - Thread safety: the library keeps a per-device pool of HIP events for the
 *     ring driver; calls are not re-entrant from several host threads on the
 *     same device.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_MAX_CHUNKS 8
#define CP_MAX_STEPS 64

/* Chunk table of a local buffer: n_chunks (1..CP_MAX_CHUNKS) chunks of
 * chunk_len tokens each (chunk_len > 0 and a multiple of 64); start[i] >= 0
 * is the absolute position of chunk i.  Chunks must not overlap. */
typedef struct {
    int32_t n_chunks;
    int32_t chunk_len;
    int64_t start[CP_MAX_CHUNKS];
} cp_chunks_t;

typedef enum {
    CP_OK = 0,
    CP_ERR_INVALID = 1,      /* bad argument (message in cp_last_error) */
    CP_ERR_UNSUPPORTED = 2,  /* valid but not built (e.g. head dim) */
    CP_ERR_WORKSPACE = 3,    /* workspace too small */
    CP_ERR_HIP = 4           /* a HIP runtime call or launch failed */
} cp_status_t;

enum { CP_STEP_WRITE = 0, CP_STEP_MERGE = 1 };

/* Text describing the last non-OK status returned on this host thread. */
const char* cp_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int cp_version(void);

/*
 * Zigzag shard and ring schedule ([RAF] section 5 item 1; [RAF] section 3).
 * The full sequence is cut into 2*cp_size chunks of chunk_len tokens; rank r
 * holds chunks r and 2*cp_size-1-r (ascending).  At ring step `step` the rank
 * works on the K/V block of rank (rank - step) mod cp_size.
 * Writes the query table of `rank` to *q_chunks and the K/V table of that
 * step's source rank to *kv_chunks (either pointer may be NULL).
 * Errors: CP_ERR_INVALID if cp_size < 1, rank or step outside [0, cp_size),
 * chunk_len <= 0, or the sequence (2 * cp_size * chunk_len tokens) longer
 * than 2^31 - 1 positions.
 */
cp_status_t cp_zigzag_chunks(int cp_size, int rank, int chunk_len, int step,
                             cp_chunks_t* q_chunks, cp_chunks_t* kv_chunks);

/*
 * One ring step: partial causal attention of the local queries against one
 * K/V block, merged into running fp32 accumulators (the per-step fused
 * attention call of [MLM] section 5 and [RAF] section 3, step 4, with the
 * log-sum-exp merge in place of the page's plain sum).
 *
 *   q   bf16 [B,H,Sq,D],  Sq  = q_chunks->n_chunks  * q_chunks->chunk_len
 *   k,v bf16 [B,H,Skv,D], Skv = kv_chunks->n_chunks * kv_chunks->chunk_len
 *   o   fp32 [B,H,Sq,D] running output (normalised), lse fp32 [B,H,Sq]
 *   out_bf16_or_null  bf16 [B,H,Sq,D]: if non-NULL, also write bf16(o) (RNE)
 *   mode CP_STEP_WRITE: (o,lse) := partial of this block (rows with no
 *        visible key get o = 0, lse = -inf);
 *        CP_STEP_MERGE: (o,lse) := merge((o,lse), partial); rows with no
 *        visible key keep their values.
 *   softmax_scale > 0 and finite (1/sqrt(D) for the standard definition).
 * Supported: D in {64, 128}; B, H >= 1.  q, k, v must not alias o/lse/out.
 */
cp_status_t cp_attn_step_fwd(const void* q, const void* k, const void* v,
                             float* o, float* lse, void* out_bf16_or_null,
                             int B, int H, int D,
                             const cp_chunks_t* q_chunks, const cp_chunks_t* kv_chunks,
                             float softmax_scale, int mode, hipStream_t stream);

/*
 * One ring step in fp8 ([MLM] section 4: FP8 together with context
 * parallelism): the same partial attention, fused merge and modes as
 * cp_attn_step_fwd, with Q, K and V as e4m3 codes (OCP encoding, one byte per
 * value) and per-tensor dequantisation factors (the values are code * scale).
 *   q   e4m3 [B,H,Sq,D]; k  e4m3 [B,H,Skv,D]; vt  e4m3 [B,H,D,Skv] (V transposed)
 *   o, lse, out_bf16_or_null, mode: as cp_attn_step_fwd (o row-major fp32)
 * The scores use softmax_scale * q_scale * k_scale; the probabilities are
 * rounded to e4m3 for the PV product (fp32 accumulation) and the output is
 * multiplied by v_scale.
 * Supported: D = 128, q chunk_len a multiple of 128; other shapes return
 * CP_ERR_UNSUPPORTED.  Scales must be finite and > 0.  Errors otherwise as
 * cp_attn_step_fwd.
 */
cp_status_t cp_attn_step_fwd_fp8(const void* q, const void* k, const void* vt,
                                 float* o, float* lse, void* out_bf16_or_null,
                                 int B, int H, int D,
                                 const cp_chunks_t* q_chunks, const cp_chunks_t* kv_chunks,
                                 float softmax_scale, float q_scale, float k_scale, float v_scale,
                                 int mode, hipStream_t stream);

/*
 * Standalone log-sum-exp merge of two partial results, in place on the
 * accumulator ([RAF] section 3, step 5 of the RingAttention loop: combining
 * the outputs of the chunks, which the page adds as a stated simplification;
 * this is the exact combination for softmax attention):
 * L = ln(e^La + e^Lb), O = e^(La-L) Oa + e^(Lb-L) Ob; an
 * operand with LSE = -inf contributes nothing; both empty gives (0, -inf).
 *   o_acc, o_part fp32 [B,H,Sq,D]; lse_acc, lse_part fp32 [B,H,Sq]
 *   out_bf16_or_null: if non-NULL, also write bf16 of the merged O.
 * Supported: D a multiple of 4 (any size), Sq >= 0 (Sq = 0 does nothing and
 * accepts NULL pointers).
 */
cp_status_t cp_attn_merge(float* o_acc, float* lse_acc,
                          const float* o_part, const float* lse_part,
                          int B, int H, int Sq, int D, void* out_bf16_or_null,
                          hipStream_t stream);

/*
 * Backward of one ring step ([MLM] section 2: the backward pass mirrors the
 * forward, the K/V gradients travelling back along the ring; [MLM] section
 * 5: forward and backward of one autograd function).  For a loss with
 * gradient dO with respect to the output, with P_ij = exp(tau <q_i,k_j> -
 * LSE_i) over the visible keys (position j <= i, absolute positions from the
 * chunk tables) and 0 elsewhere, the K/V block of one step contributes
 *
 *     dV_j = sum_i P_ij dO_i,       dP_ij = <dO_i, v_j>,
 *     dS_ij = P_ij (dP_ij - Delta_i),
 *     dQ_i += tau sum_j dS_ij k_j,  dK_j = tau sum_i dS_ij q_i,
 *
 * where LSE and Delta_i = <dO_i, out_i> come from the complete forward (all
 * steps).  A rank adds the dQ parts of its N steps; each block's dK and dV
 * are summed over the ranks whose queries see it.
 */
enum { CP_BWD_DQ_ACCUMULATE = 1, CP_BWD_DKV_ACCUMULATE = 2 };

/*
 * Delta_i = sum_d dO[i][d] out[i][d] in fp32, for every row of the local
 * queries (the forward's bf16 output and the upstream gradient).
 *   out, d_out bf16 [B,H,Sq,D]; delta fp32 [B,H,Sq]
 * Supported: D in {64, 128}; Sq >= 0 (Sq = 0 does nothing and accepts NULL
 * pointers).  delta must not overlap the inputs.
 */
cp_status_t cp_attn_bwd_delta(const void* out, const void* d_out, float* delta,
                              int B, int H, int Sq, int D, hipStream_t stream);

/*
 * Gradient contributions of one K/V block to the local queries and to the
 * block itself.
 *   q, d_out  bf16 [B,H,Sq,D] with table *q_chunks
 *   k, v      bf16 [B,H,Skv,D] with table *kv_chunks
 *   lse       fp32 [B,H,Sq], natural log, of the complete forward (-INFINITY:
 *             the row has no visible key and contributes nothing)
 *   delta     fp32 [B,H,Sq] from cp_attn_bwd_delta
 *   dq        fp32 [B,H,Sq,D];  dk, dv  fp32 [B,H,Skv,D]
 *   mode      bit CP_BWD_DQ_ACCUMULATE: dq += this block's part (else
 *             dq := it); bit CP_BWD_DKV_ACCUMULATE: dk, dv += (else :=).
 *             Every row of the outputs is written (with 0 where no visible
 *             pair contributes).
 * Two kernels on `stream`: one owns the dq rows, the other the dk/dv rows;
 * no atomics, so results are deterministic.
 * Supported: D in {64, 128}; B, H >= 1.  dq, dk, dv must not overlap each
 * other or any input.  Errors as cp_attn_step_fwd; mode outside [0, 3] is
 * CP_ERR_INVALID.
 */
cp_status_t cp_attn_step_bwd(const void* q, const void* k, const void* v, const void* d_out,
                             const float* lse, const float* delta,
                             float* dq, float* dk, float* dv,
                             int B, int H, int D,
                             const cp_chunks_t* q_chunks, const cp_chunks_t* kv_chunks,
                             float softmax_scale, int mode, hipStream_t stream);

/* Workspace bytes cp_ring_attn_fwd needs: two staging slots, each for the K
 * and V blocks [B,H,Skv,D] bf16 of up to four ring steps (sixteen blocks);
 * the fp32 running output [B,H,Sq,D]; and, for launches whose grid is small
 * enough that each row block's keys are split over two workgroups, the two
 * halves' fp32 partial outputs and LSE for R = min(65536, B*H*Sq) rows plus
 * 512 counters; each part rounded up to 256 bytes.  Returns 0 for
 * non-positive sizes. */
size_t cp_ring_attn_workspace_bytes(int B, int H, int Skv, int D, int Sq);

/*
 * A rank's whole share of causal ring attention, replayed on one GPU.
 *   q         bf16 [B,H,Sq,D] with table *q_chunks
 *   k_steps[j], v_steps[j]  host array of n_steps device pointers, ring order:
 *             the K/V block the rank uses at step j, bf16 [B,H,Skv,D], with
 *             table kv_chunks_steps[j] (all the same chunk_len and count).
 *             Step 0 is read in place (the rank's own block); for j >= 1 the
 *             block is first copied into one of two staging slots in the
 *             workspace on copy_stream, standing in for the peer-to-peer
 *             receive ([MLM] section 5: double buffering on a separate
 *             stream; [RAF] section 3: receive from the previous rank).
 *             After step 0, the steps are computed in the fewest groups of
 *             at most four steps and CP_MAX_CHUNKS chunks per kernel launch,
 *             smaller groups first: a slot holds the blocks of one group,
 *             and the online softmax runs on across the group's blocks,
 *             which equals merging the steps' partial results by their
 *             log-sum-exp.
 *   out       bf16 [B,H,Sq,D], lse fp32 [B,H,Sq]  (final results)
 *   workspace at least cp_ring_attn_workspace_bytes(B,H,Skv,D,Sq) bytes,
 *             256-byte aligned.
 *   copy_stream  a stream other than `stream`, on which the staging copies
 *             overlap the compute; or `stream` itself, which runs every
 *             copy in order before the launch that reads it (no overlap,
 *             for measurement).  NULL only when `stream` is NULL too.
 * The copies for launch g+1 overlap the compute of launch g; the copy into a
 * slot waits until the launch that last read that slot has finished.  On entry
 * copy_stream waits for prior work on `stream`; before returning, `stream`
 * waits for every copy, so later work on `stream` is ordered after the call.
 * Every query row must see at least one key over the steps (true for a
 * zigzag share, whose step 0 contains the diagonal).
 * Errors: CP_ERR_INVALID for bad tables or n_steps outside [1, CP_MAX_STEPS],
 * CP_ERR_WORKSPACE if workspace_bytes is too small.
 */
cp_status_t cp_ring_attn_fwd(const void* q, const cp_chunks_t* q_chunks,
                             const void* const* k_steps, const void* const* v_steps,
                             const cp_chunks_t* kv_chunks_steps, int n_steps,
                             void* out, float* lse,
                             int B, int H, int D, float softmax_scale,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream, hipStream_t copy_stream);

/*
 * The launch plan of cp_ring_attn_fwd (and cp_ring_attn_fwd_fp8) for these
 * tables, without running anything: the loop over ring steps of [MLM]
 * section 5 as this library groups it.  Writes the number of kernel launches
 * to *n_launches and, for the first max_launches launches l, the first ring
 * step it covers (first_step[l]), its number of steps (step_count[l]) and,
 * for each query chunk c, chunk_flags[l * CP_MAX_CHUNKS + c]: 0 if the launch
 * does not compute chunk c, else CP_PLAN_ACTIVE with CP_PLAN_MERGE (merge
 * into the running fp32 O read from the workspace), CP_PLAN_WRITE_O (write
 * the running O back) and CP_PLAN_FINALIZE (write out and lse).  Any output
 * array may be NULL.  Errors: as cp_ring_attn_fwd for the tables and n_steps.
 */
enum { CP_PLAN_MERGE = 1, CP_PLAN_FINALIZE = 2, CP_PLAN_WRITE_O = 4, CP_PLAN_ACTIVE = 8 };
cp_status_t cp_ring_attn_fwd_plan(const cp_chunks_t* q_chunks, const cp_chunks_t* kv_chunks_steps,
                                  int n_steps, int max_launches, int* n_launches,
                                  int* first_step, int* step_count, int* chunk_flags);

/*
 * cp_ring_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  The staging slots and the fp32 running
 * output live in a static array of the library on each device
 * (cp_ring_attn_fwd_noalloc_max_bytes() bytes, 64 MiB, held from the library's
 * load until the process ends); nothing is allocated.  The launch grouping
 * is cp_ring_attn_fwd's (up to four ring steps per launch) when its slots fit
 * the array, else fewer steps per launch; the results then differ from
 * cp_ring_attn_fwd's only by rounding order.
 * Arguments, errors and stream semantics: as cp_ring_attn_fwd.  A share whose
 * slots for one ring step per launch plus running output exceed the array is
 * refused with CP_ERR_WORKSPACE before anything is enqueued.
 * Every call on one device uses that device's single array: calls that
 * overlap in time on one device (other streams, other host threads) race and
 * must be serialised by the caller.  No part of the array needs clearing
 * between calls (every byte read is written earlier in the same call).
 */
size_t cp_ring_attn_fwd_noalloc_max_bytes(void);
cp_status_t cp_ring_attn_fwd_noalloc(const void* q, const cp_chunks_t* q_chunks,
                                     const void* const* k_steps, const void* const* v_steps,
                                     const cp_chunks_t* kv_chunks_steps, int n_steps,
                                     void* out, float* lse,
                                     int B, int H, int D, float softmax_scale,
                                     hipStream_t stream, hipStream_t copy_stream);

/* Workspace bytes cp_ring_attn_fwd_fp8 needs: two staging slots of e4m3 K and
 * V^T blocks (one byte per value) for up to four ring steps, plus the fp32
 * running output [B,H,Sq,D], each rounded up to 256 bytes.  Returns 0 for
 * non-positive sizes. */
size_t cp_ring_attn_fwd_fp8_workspace_bytes(int B, int H, int Skv, int D, int Sq);

/*
 * A rank's whole share in fp8, replayed on one GPU: the ring of
 * cp_ring_attn_fwd (same launch groups, staging slots, streams and events)
 * with the steps of cp_attn_step_fwd_fp8.
 *   q          e4m3 [B,H,Sq,D] with table *q_chunks
 *   k_steps[j] e4m3 [B,H,Skv,D]; vt_steps[j] e4m3 [B,H,D,Skv] (V transposed)
 *   out        bf16 [B,H,Sq,D]; lse fp32 [B,H,Sq]
 *   scales     as cp_attn_step_fwd_fp8
 * The staging copies move one byte per value, half of the bf16 ring's.
 * Supported: D = 128, q chunk_len a multiple of 128.  Errors as
 * cp_ring_attn_fwd; CP_ERR_UNSUPPORTED for other shapes.
 */
cp_status_t cp_ring_attn_fwd_fp8(const void* q, const cp_chunks_t* q_chunks,
                                 const void* const* k_steps, const void* const* vt_steps,
                                 const cp_chunks_t* kv_chunks_steps, int n_steps,
                                 void* out, float* lse,
                                 int B, int H, int D, float softmax_scale,
                                 float q_scale, float k_scale, float v_scale,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, hipStream_t copy_stream);

/* Workspace bytes cp_ring_attn_bwd needs: Delta fp32 [B,H,Sq], then two
 * staging slots, each for one step's K and V blocks (bf16 [B,H,Skv,D]) and
 * the dK and dV partial sums that travel with it (fp32 [B,H,Skv,D]), each
 * rounded up to 256 bytes.  Returns 0 for non-positive sizes. */
size_t cp_ring_attn_bwd_workspace_bytes(int B, int H, int Skv, int D, int Sq);

/*
 * Backward of a rank's whole share, replayed on one GPU ([MLM] section 2:
 * the backward pass mirrors the forward; the K/V blocks go around the ring
 * again and each block's gradients travel with it, collecting every rank's
 * contribution).
 *   q, d_out, out  bf16 [B,H,Sq,D] with table *q_chunks; out and lse are the
 *             complete forward results (cp_ring_attn_fwd)
 *   lse       fp32 [B,H,Sq]
 *   k_steps[j], v_steps[j]  as for cp_ring_attn_fwd (ring order, step 0 the
 *             rank's own block)
 *   dk_steps[j], dv_steps[j]  host array of n_steps device pointers, fp32
 *             [B,H,Skv,D]: the partial sums of dK and dV of step j's block.
 *             They are read and added to where dkv_accumulate[j] != 0, else
 *             overwritten with this rank's contribution.
 *   dkv_accumulate  host array [n_steps], or NULL for the ring's own pattern:
 *             step 0 (the block's first visit) writes, later steps add.
 *   dq        fp32 [B,H,Sq,D]: written, the sum of every step's part.
 * Delta = rowsum(d_out * out) goes to the workspace first.  Step 0 reads its
 * K/V in place and writes dk_steps[0], dv_steps[0] directly.  For j >= 1, on
 * copy_stream, the block and (when adding) its partial sums are copied into
 * staging slot (j-1) % 2 (the receive), the kernels on `stream` update the
 * slot's partial sums, and they are copied back to dk_steps[j], dv_steps[j]
 * (the send).  Step j+2's receive into the same slot follows that send on
 * copy_stream.  Stream semantics and copy_stream == stream as for
 * cp_ring_attn_fwd: on return `stream` is ordered after every copy.
 * Supported: D in {64, 128}.  dq, every dK/dV buffer and the workspace must
 * not overlap one another or any input.  Errors as cp_ring_attn_fwd.
 */
cp_status_t cp_ring_attn_bwd(const void* q, const cp_chunks_t* q_chunks,
                             const void* d_out, const void* out, const float* lse,
                             const void* const* k_steps, const void* const* v_steps,
                             const cp_chunks_t* kv_chunks_steps, int n_steps,
                             float* const* dk_steps, float* const* dv_steps,
                             const int* dkv_accumulate, float* dq,
                             int B, int H, int D, float softmax_scale,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream, hipStream_t copy_stream);

/*
 * Kernel timing for measurement.  While enabled, every attention-step kernel
 * launched by cp_attn_step_fwd / cp_ring_attn_fwd / cp_attn_step_fwd_fp8, and each of the two
 * kernels of cp_attn_step_bwd and of every step of cp_ring_attn_bwd (dq
 * first, then dk/dv), is bracketed by two HIP
 * events on its stream.  cp_profile_read waits for those events, writes up to
 * max_entries elapsed times (milliseconds, launch order) to kernel_ms and
 * their count to *n_entries, and clears the record.  At most 4096 launches
 * are kept; later ones are not timed.  Enabling or disabling clears the record.
 */
cp_status_t cp_profile_enable(int enable);
cp_status_t cp_profile_read(float* kernel_ms, int max_entries, int* n_entries);

/* As cp_profile_read, and also writes the name of each timed kernel (the
 * variant the launch chose, e.g. "step_kernel_256<128>"; "" for a launch
 * with an empty grid) to kernel_names[i] when kernel_names is non-NULL.  The
 * strings are static and owned by the library.  Either array may be NULL. */
cp_status_t cp_profile_read_named(float* kernel_ms, const char** kernel_names,
                                  int max_entries, int* n_entries);

/*
 * Stream-ordering test hook.  While set, the ring drivers (cp_ring_attn_fwd,
 * cp_ring_attn_fwd_fp8, cp_ring_attn_bwd) precede every kernel launch that
 * reads a staging slot with a bounded device-side spin of compute_us
 * microseconds on the compute stream, and every staging copy (receive or
 * send) with one of copy_us on the copy stream.  A launch then reads its slot
 * late while later copies run ahead, or a copy lands late, so a missing wait
 * in the double-buffered staging of [MLM] section 5 would change the result;
 * with correct ordering results are bit-identical.  0 disables a side.
 * Errors: CP_ERR_INVALID outside [0, 100000].  Process-wide setting.
 */
cp_status_t cp_test_set_delays(int compute_us, int copy_us);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
