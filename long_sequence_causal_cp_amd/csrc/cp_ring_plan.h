// Host-only planning of the one-GPU ring replay: argument checks of chunk
// tables, visible-pair counts, the zigzag tables, and the ordered list of
// stream operations (staging copies, kernel launches, event records and
// waits) that the forward and backward ring drivers issue.  No HIP call is
// made here: the drivers in cp_attn_api.cpp execute a plan, and a CPU test
// builds this file with address and undefined-behaviour sanitizers and checks
// every plan's happens-before order for races on the staging slots.
//
// Sources (web pages, cited by title and section):
//   [MLM] "Megatron-LM源码解析：Context Parallel如何革新长序列训练", section 5
//         (double-buffered loop: while step i computes on one buffer, the
//         transfer for the next step fills the other on its own stream).
//   [RAF] "如何用Context并行加速大模型训练？手把手教你配置RingAttention+FlashAttention",
//         section 3 (step j uses the block of rank (r - j) mod N) and section
//         5, item 1 (2N zigzag chunks).
#pragma once

#include <string>
#include <vector>

#include "../../include/cp_attn.h"

namespace cpplan {

// Per-query-chunk work flags of one launch (the step kernels' flag values).
enum : int {
  kMerge = 1,     // merge into the running (O, LSE); else overwrite
  kFinalize = 2,  // write the bf16 output (the row's last launch)
  kWriteO = 4,    // write the fp32 running O
};

// Checks of one chunk table: 1..CP_MAX_CHUNKS chunks of a positive multiple
// of 64 tokens, starts in [0, 2^31 - chunk_len], no two chunks overlapping.
// Returns CP_OK, or CP_ERR_INVALID with the reason in *err.
cp_status_t check_chunks(const cp_chunks_t* t, const char* name, std::string* err);

// Visible (query, key) pairs (key position <= query position) between a
// query chunk at qs of lq tokens and a key chunk at ks of lk tokens.
long long chunk_pairs(long long qs, long long lq, long long ks, long long lk);
// Visible pairs of query chunk c of *q against every chunk of *kv.
long long pairs_for_chunk(const cp_chunks_t* q, int c, const cp_chunks_t* kv);

// Zigzag table of rank r: chunks r and 2N-1-r of chunk_len tokens ([RAF]
// section 5, item 1).  Arguments must be valid (checked by the caller).
void zigzag_table(int cp_size, int r, int chunk_len, cp_chunks_t* t);

// One operation of a ring replay, in host issue order.
enum class OpKind {
  Record,   // record `event` on `stream`
  Wait,     // `stream` waits for `event`
  Stage,    // forward: copy the K/V blocks of launch `index` into its slot
  Launch,   // forward: the step kernel of launch `index`
  Delta,    // backward: Delta of the local rows
  Receive,  // backward: copy step `index`'s K/V block (and, when it adds, its
            // travelling dK/dV partial sums) into slot (index - 1) % 2
  Kernels,  // backward: the dq and dk/dv kernels of step `index`
  Send,     // backward: copy the slot's updated dK/dV partial sums back out
};
enum Stream : int { kCompute = 0, kCopy = 1 };

struct Op {
  OpKind kind;
  int stream;
  int event;  // Record, Wait
  int index;  // Stage, Launch: launch; Receive, Kernels, Send: ring step
};

// One kernel launch of the forward ring: steps [first_step, first_step +
// count), its staging slot (-1: the rank's own block, read in place), the
// query chunks it computes with their flags, and each chunk's visible pairs.
struct FwdLaunch {
  int first_step = 0, count = 0;
  int slot = -1;
  int n_active = 0;
  int active[CP_MAX_CHUNKS] = {};
  int flags[CP_MAX_CHUNKS] = {};
  long long work[CP_MAX_CHUNKS] = {};
};

struct FwdPlan {
  std::vector<FwdLaunch> launches;
  std::vector<Op> ops;
  int n_events = 0;
  int steps_per_launch = 0;  // most steps a launch covers = blocks a slot holds
};

// The forward ring of cp_ring_attn_fwd.  Step 0 is one launch on the rank's
// own block; steps 1 .. n_steps-1 follow in the fewest groups of at most
// max_steps_per_launch steps (and CP_MAX_CHUNKS key chunks), split as evenly
// as possible, smaller groups first.  Launch l >= 1 reads slot (l-1) % 2,
// staged on the copy stream while launch l-1 computes; the staging of launch
// l waits for launch l-2 to release the same slot.  Events: 0 = entry (on
// the compute stream; the copy stream waits for it), 1 = done (on the copy
// stream; the compute stream waits for it before returning), then per
// launch one "staged" and one "released" event.  Tables must be valid.
void plan_ring_fwd(const cp_chunks_t* q, const cp_chunks_t* kv_steps, int n_steps, int max_steps_per_launch,
                   FwdPlan* plan);

struct BwdPlan {
  std::vector<Op> ops;
  int n_events = 0;
};

// The backward ring of cp_ring_attn_bwd.  Step 0 works on the rank's own
// block in place; for j >= 1 the block (with its travelling dK/dV partial
// sums when the step adds to them) is received into slot (j-1) % 2, the
// kernels update the slot's sums and they are sent back; step j+2's receive
// into the same slot follows that send on the copy stream.  Events: 0 =
// entry, 1 = done, then per step "received" and "computed".
void plan_ring_bwd(int n_steps, BwdPlan* plan);

}  // namespace cpplan
