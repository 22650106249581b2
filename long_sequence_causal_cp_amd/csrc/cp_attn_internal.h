// Internal interface between the host library (validation, ring driver) and
// the gfx950 kernels.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

constexpr int kMaxChunks = 8;
constexpr int kTileKeys = 64;  // keys per K/V tile staged through LDS

// Per-query-chunk work flags for one step launch.
enum : int {
  kFlagMerge = 1,     // read the running (O, LSE) and merge; else overwrite
  kFlagFinalize = 2,  // write bf16 output
  kFlagWriteO = 4,    // write the fp32 running O
  kFlagLaneO = 8,     // the running O is kept in the step kernel's lane order (see the kernel)
};

// Everything one launch of the step kernel needs; passed by value.
struct StepArgs {
  const uint16_t* q;  // bf16 [BH, Sq, D]
  // K/V chunk c: its first row for (b, h) = 0; (b, h) adds bh * Skv * D.  The
  // chunks of one launch may come from different [BH, Skv, D] blocks (one
  // launch can cover two ring steps), so each has its own base.
  const uint16_t* kc[kMaxChunks];
  const uint16_t* vc[kMaxChunks];
  float* o_run;       // fp32 [BH, Sq, D] (may be null when no chunk has kFlagWriteO/kFlagMerge)
  float* lse_run;     // fp32 [BH, Sq]
  uint16_t* out;      // bf16 [BH, Sq, D] (may be null when no chunk finalizes)
  int BH, D;
  int Sq, Skv;                // rows per (b, h) of the query block and of every K/V block
  int q_chunk_len, kv_chunk_len;
  int n_kv_chunks;            // chunks of this launch, visited in index order
  int n_order;                // active query chunks in this launch
  int order[kMaxChunks];      // their indices, heaviest first
  int flags[kMaxChunks];      // per query chunk index
  int q_start[kMaxChunks];    // absolute positions
  int kv_start[kMaxChunks];
  int rb_per_chunk;           // row blocks per query chunk
  int heads_per_xcd;          // > 0: keep each (b,h) on one XCD
  int heads_per_group;        // divides heads_per_xcd; set by the launch
  float scale_log2;           // tau * log2(e)
  // Key split (launch_step may split each row block's key tiles over two
  // workgroups when the grid is small and these are set): the two halves'
  // normalised partials, fp32 [2][part_rows][D] in the lane order of the
  // running O, their LSE [2][part_rows], and one counter per row block, zero
  // before the launch (the merging workgroup resets it).
  float* part_o;
  float* part_lse;
  unsigned* part_cnt;
  int part_rows;              // capacity in rows; 0: no key split
  // Non-null: the kSplitMaxBlocks counters still hold the caller's garbage.
  // An unsplit launch clears them from its first workgroup (stream order
  // makes that visible to later launches); a split launch clears them with
  // a small kernel before it starts.
  unsigned* cnt_to_clear;
};

// Rows of the key-split partial buffers a ring workspace holds: a launch
// splits only when its grid of 128-row workgroups has fewer than
// kSplitMaxBlocks workgroups, so it never needs more rows than this.
constexpr int kSplitMaxBlocks = 512;
constexpr int kSplitRows = kSplitMaxBlocks * 128;

// Everything one backward launch of one K/V block needs (both backward
// kernels); passed by value.
struct BwdArgs {
  const uint16_t* q;     // bf16 [BH, Sq, D]
  const uint16_t* dout;  // bf16 [BH, Sq, D], upstream gradient of the output
  const uint16_t* k;     // bf16 [BH, Skv, D], one K/V block (its chunks concatenated)
  const uint16_t* v;
  const float* lse;      // fp32 [BH, Sq], natural log, of the complete forward
  const float* delta;    // fp32 [BH, Sq], rowsum(dO * O) of the complete forward
  float* dq;             // fp32 [BH, Sq, D]
  float* dk;             // fp32 [BH, Skv, D], this block's rows
  float* dv;
  int BH, D;
  int Sq, Skv;
  int q_chunk_len, kv_chunk_len;
  int n_q_chunks, n_kv_chunks;
  int q_start[kMaxChunks];
  int kv_start[kMaxChunks];
  int accumulate;        // bit 0: dq += contribution (else =); bit 1: dk, dv += (else =)
  int heads_per_xcd;     // > 0: keep each (b,h) on one XCD
  int heads_per_group;   // divides heads_per_xcd; set by the launch
  float scale;           // tau
  float scale_log2;      // tau * log2(e)
};

// Backward of one K/V block: the query-stationary dq kernel and the
// key-stationary dk/dv kernel (rows and keys per workgroup for a chunk length).
int bwd_dq_rows(int q_chunk_len);
int bwd_dkdv_keys(int kv_chunk_len);
// *name (if name is non-null) receives the launched kernel's name, or null
// when the grid is empty; the same holds for launch_step.
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream, const char** name = nullptr);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream, const char** name = nullptr);
// delta[r] = sum_d dout[r][d] * out[r][d] over `rows` rows of D bf16 values.
hipError_t launch_bwd_delta(const uint16_t* out, const uint16_t* dout, float* delta, int64_t rows, int D,
                            hipStream_t stream);

// Row-block height (queries per workgroup) the step kernel uses for a chunk length.
int step_block_rows(int q_chunk_len);

// Launch the step kernel; `grid` = n_order * rb_per_chunk * BH workgroups.
hipError_t launch_step(const StepArgs& a, int D, hipStream_t stream, const char** name = nullptr);

// Copy one ring step's K and V blocks (`bytes` each, a multiple of 16) into a
// staging slot on `stream` (the copy stream of the ring driver).
hipError_t launch_stage_copy(const void* k_src, void* k_dst, const void* v_src, void* v_dst, size_t bytes,
                             hipStream_t stream);

// Zero n 32-bit words (the key-split counters) with a fill kernel.
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream);

// A single-wave spin of `us` microseconds of the device's constant-rate
// clock on `stream` (stream-ordering tests only); it always ends.
hipError_t launch_delay(int us, hipStream_t stream);

// Standalone merge kernel.
hipError_t launch_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                        uint16_t* out, int64_t rows, int D, hipStream_t stream);

}  // namespace cpattn
