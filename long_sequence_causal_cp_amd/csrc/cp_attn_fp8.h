// Internal interface of the fp8 attention-step kernel (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cp_attn_internal.h"

namespace cpattn {

// One launch of the fp8 step kernel; passed by value.  Q, K and V hold fp8
// e4m3 codes (OCP encoding); V is transposed, [BH, D, Skv], so that the
// operand of the PV product is read along its rows.
struct Fp8StepArgs {
  const uint8_t* q;                // [BH, Sq, D]
  const uint8_t* kc[kMaxChunks];   // K chunk c: its first row for (b, h) = 0; (b, h) adds bh * Skv * D
  const uint8_t* vtc[kMaxChunks];  // V^T chunk c: its first column in row 0 for (b, h) = 0; (b, h) adds
                                   // bh * D * Skv, rows are Skv apart
  float* o;                        // fp32 [BH, Sq, D], row-major
  float* lse;                      // fp32 [BH, Sq]
  uint16_t* out;                   // bf16 [BH, Sq, D] or null
  int BH;
  int Sq, Skv;
  int q_chunk_len, kv_chunk_len;
  int n_kv_chunks;
  int n_order;
  int order[kMaxChunks];
  int flags[kMaxChunks];           // kFlagMerge, kFlagWriteO, kFlagFinalize
  int q_start[kMaxChunks];
  int kv_start[kMaxChunks];
  int rb_per_chunk;                // set by launch_step_fp8 from its row-block choice
  int heads_per_xcd;
  int heads_per_group;             // set by launch_step_fp8
  float scale_log2;                // tau * q_scale * k_scale * log2(e)
  float v_scale;                   // the dequantisation factor of V
};

// Rows per workgroup of the fp8 step kernel (D = 128): 256, or 128 where a grid
// of 256-row workgroups would leave compute units idle or the query chunk
// length is not a multiple of 256.  Query chunk lengths must be multiples of
// kFp8RowQuantum.
constexpr int kFp8BlockRows = 256;
constexpr int kFp8RowQuantum = 128;

// *name (if name is non-null) receives the launched kernel's name, or null
// when the grid is empty.
hipError_t launch_step_fp8(const Fp8StepArgs& a, hipStream_t stream, const char** name = nullptr);

}  // namespace cpattn
