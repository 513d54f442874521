"""MI355X (gfx950) split-KV decode attention.

The compute lives in libmxfa.so (hand-written HIP kernels behind the C ABI in
include/mxfa.h); ``mxfa`` is its ctypes binding.
"""
from .mxfa import (EXPORTS, MXFA_BF16, MXFA_ERR_HIP, MXFA_ERR_INVALID_ARG, MXFA_ERR_UNSUPPORTED,
                   MXFA_ERR_WORKSPACE, MXFA_FP16, MXFA_OK, NOALLOC_SCRATCH_BYTES, MxfaError, Plan,
                   PreparedCall, fwd_kvcache, fwd_kvcache_append, fwd_kvcache_dkdv,
                   fwd_kvcache_paged, fwd_varlen, last_plan, lib, plan, read_probe,
                   set_timing_events, status_string, version, workspace_size,
                   workspace_size_dkdv, workspace_size_paged)

__all__ = ["EXPORTS", "MXFA_BF16", "MXFA_ERR_HIP", "MXFA_ERR_INVALID_ARG", "MXFA_ERR_UNSUPPORTED",
           "MXFA_ERR_WORKSPACE", "MXFA_FP16", "MXFA_OK", "NOALLOC_SCRATCH_BYTES", "MxfaError",
           "Plan", "PreparedCall", "fwd_kvcache", "fwd_kvcache_append", "fwd_kvcache_dkdv",
           "fwd_kvcache_paged", "fwd_varlen", "last_plan", "lib", "plan", "read_probe",
           "set_timing_events", "status_string", "version", "workspace_size",
           "workspace_size_dkdv", "workspace_size_paged"]
