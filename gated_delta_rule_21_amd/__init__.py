"""Gated delta-rule linear attention for AMD Instinct MI355X (gfx950).

Public calls (thin wrappers over the C ABI in include/gdr.h):
    chunk_fwd(q, k, v, beta, log_a=None, S0=None, form="page")        -> (o, S_T)
    chunk_fwd_varlen(q, k, v, beta, log_a, cu_seqlens, S0=None)        -> (o, S_T), sequences packed along T
    recurrent_step(q, k, v, beta, log_a, S, form="page")               -> (o, S_new)
    precond_scan(k, beta, eta, r=None, d0=None)                        -> (kw, d_T), the write keys
                                                                          of the preconditioned rule
    chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T=None, cu_seqlens=None) -> dict of dq, dk, dv, dbeta,
                                                                          dlog_a, dS0 (the gradients)
    chunk_attn(q, k, v, beta, log_a=None, S0=None, cu_seqlens=None)    -> (o, S_T) as a torch autograd
                                                                          function (backward: chunk_bwd)
    chunk_workspace_size(B, T, H, d_k, d_v, dtype, gate)               -> bytes of scratch
    chunk_varlen_workspace_size(T, n_seq, H, d_k, d_v, dtype, gate)    -> bytes of scratch
    chunk_bwd_workspace_size(B, T, H, d_k, d_v, dtype, gate)           -> bytes of scratch
"""

from ._lib import (EXPORTED, GdrError, LIB_PATH, chunk_attn, chunk_bwd, chunk_bwd_workspace_size, chunk_fwd,
                   chunk_fwd_varlen, chunk_varlen_workspace_size, chunk_workspace_size, load, precond_scan,
                   recurrent_step)

__all__ = ["EXPORTED", "GdrError", "LIB_PATH", "chunk_attn", "chunk_bwd", "chunk_bwd_workspace_size", "chunk_fwd",
           "chunk_fwd_varlen", "chunk_varlen_workspace_size", "chunk_workspace_size", "load", "precond_scan",
           "recurrent_step"]
