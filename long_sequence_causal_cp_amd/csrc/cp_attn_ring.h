// Internal entry of the forward ring driver, shared by cp_ring_attn_fwd
// (caller's workspace) and cp_ring_attn_fwd_noalloc (the library's
// static scratch array).  Not part of the public C ABI.
#pragma once

#include <stddef.h>

#include "../../include/cp_attn.h"

namespace cpattn {

// Most ring steps one step-kernel launch covers; a staging slot holds this
// many K/V blocks.
constexpr int kMaxStepsPerLaunch = 4;

// Workspace bytes of the forward ring when a launch covers at most
// steps_per_launch ring steps: two staging slots of steps_per_launch K and V
// blocks, plus the fp32 running output, each rounded up to 256 bytes.
size_t ring_fwd_workspace_bytes(int B, int H, int Skv, int D, int Sq, int steps_per_launch);

// cp_ring_attn_fwd with the launch grouping limited to steps_per_launch
// (1 .. kMaxStepsPerLaunch) ring steps per launch; argument checks, errors and
// stream semantics as cp_ring_attn_fwd.
cp_status_t ring_fwd(const void* q, const cp_chunks_t* q_chunks, const void* const* k_steps,
                     const void* const* v_steps, const cp_chunks_t* kv_chunks_steps, int n_steps, void* out, float* lse,
                     int B, int H, int D, float softmax_scale, void* workspace, size_t workspace_bytes,
                     int steps_per_launch, hipStream_t stream, hipStream_t copy_stream);

// Set the thread-local message of cp_last_error and return st.
cp_status_t fail_status(cp_status_t st, const char* msg);

}  // namespace cpattn
