"""Causal ring attention for one context-parallel rank, native on MI355X (gfx950).

The compute path is the HIP library ``libcp_attn.so`` (C ABI declared in
``include/cp_attn.h``); ``binding`` marshals torch tensors into it.
"""
from .binding import (CpChunks, CpError, CP_BWD_DKV_ACCUMULATE, CP_BWD_DQ_ACCUMULATE, CP_PLAN_ACTIVE,
                      CP_PLAN_FINALIZE, CP_PLAN_MERGE, CP_PLAN_WRITE_O, CP_STEP_MERGE,
                      CP_STEP_WRITE, cp_attn_bwd_delta, cp_attn_merge, cp_attn_step_bwd, cp_attn_step_fwd, cp_attn_step_fwd_fp8,
                      cp_last_error, cp_profile_enable, cp_profile_read, cp_profile_read_named, cp_ring_attn_bwd,
                      cp_ring_attn_bwd_workspace_bytes, cp_ring_attn_fwd, cp_ring_attn_fwd_fp8, cp_ring_attn_fwd_noalloc,
                      cp_ring_attn_fwd_plan,
                      cp_ring_attn_fwd_fp8_workspace_bytes, cp_ring_attn_workspace_bytes, cp_test_set_delays, cp_version,
                      cp_zigzag_chunks, load_library)

__all__ = [
    "CpChunks", "CpError", "CP_BWD_DKV_ACCUMULATE", "CP_BWD_DQ_ACCUMULATE", "CP_PLAN_ACTIVE", "CP_PLAN_FINALIZE",
    "CP_PLAN_MERGE", "CP_PLAN_WRITE_O", "CP_STEP_MERGE", "CP_STEP_WRITE",
    "cp_attn_bwd_delta", "cp_attn_merge", "cp_attn_step_bwd", "cp_attn_step_fwd", "cp_attn_step_fwd_fp8", "cp_last_error",
    "cp_profile_enable", "cp_profile_read", "cp_profile_read_named", "cp_ring_attn_bwd", "cp_ring_attn_bwd_workspace_bytes", "cp_ring_attn_fwd", "cp_ring_attn_fwd_fp8", "cp_ring_attn_fwd_noalloc", "cp_ring_attn_fwd_plan", "cp_ring_attn_fwd_fp8_workspace_bytes", "cp_ring_attn_workspace_bytes", "cp_test_set_delays", "cp_version",
    "cp_zigzag_chunks", "load_library",
]
