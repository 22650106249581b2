// Which block and (b, h) each workgroup of an attention launch owns: the
// XCD-aware job order shared by the step, fp8 and backward kernels, and the
// host's choice of its head-group size.  Host and device code; the host
// planning checks (tests/sanitize) build it on the CPU.
#pragma once

#include <hip/hip_runtime.h>

namespace cpattn {

// Workgroups are dealt to the 8 XCDs round-robin (workgroup i runs on XCD
// i mod 8).  With heads_per_xcd > 0 (B*H a multiple of 8) each (b, h) stays
// on one XCD, so that its tiles are shared through that XCD's L2, and an
// XCD's heads are taken in groups of heads_per_group (a divisor of
// heads_per_xcd) whose blocks run together; inside a group blocks go in
// index order, the group's heads interleaved.  Otherwise (b, h) is the
// fastest-varying index.  Maps job in [0, blocks_per_head * BH) one to one
// onto (blk, bh) in [0, blocks_per_head) x [0, BH).
__host__ __device__ inline void xcd_job(int job, int BH, int heads_per_xcd, int heads_per_group,
                                        int blocks_per_head, int& blk, int& bh) {
  if (heads_per_xcd > 0) {
    const int x = job & 7, kk = job >> 3;
    const int per_group = heads_per_group * blocks_per_head;
    const int grp = kk / per_group, in_grp = kk - grp * per_group;
    blk = in_grp / heads_per_group;
    bh = x * heads_per_xcd + grp * heads_per_group + in_grp % heads_per_group;
  } else {
    blk = job / BH;
    bh = job % BH;
  }
}

// The two workgroups of a key-split launch that share a row block: workgroup
// w of the doubled grid is half `ks` of job `job`.  With the XCD-aware order
// both halves keep the job's number modulo 8 (one XCD); the grid of jobs is
// then a multiple of 8.
__host__ __device__ inline void split_job(int w, int heads_per_xcd, int& job, int& ks) {
  if (heads_per_xcd > 0) {
    ks = (w >> 3) & 1;
    job = (w & 7) | ((w >> 4) << 3);
  } else {
    ks = w & 1;
    job = w >> 1;
  }
}

// Heads per group of the XCD-aware job order: the most heads (a divisor of
// heads_per_xcd) whose blocks_per_head workgroups each fit in `slots`, the
// workgroups one XCD runs at once; at least 1.
inline int heads_per_group(int heads_per_xcd, long long blocks_per_head, long long slots) {
  int hpg = 1;
  for (int d = 1; d <= heads_per_xcd; ++d)
    if (heads_per_xcd % d == 0 && d * blocks_per_head <= slots) hpg = d;
  return hpg;
}

}  // namespace cpattn
