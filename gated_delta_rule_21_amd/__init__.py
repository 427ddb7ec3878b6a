"""Gated delta-rule linear attention for AMD Instinct MI355X (gfx950).

Public calls (thin wrappers over the C ABI in include/gdr.h):
    chunk_fwd(q, k, v, beta, log_a=None, S0=None, form="page")        -> (o, S_T)
    chunk_fwd_varlen(q, k, v, beta, log_a, cu_seqlens, S0=None)        -> (o, S_T), sequences packed along T
    chunk_fwd_noalloc(q, k, v, beta, log_a=None, S0=None)             -> (o, S_T), scratch in a static
                                                                          device array (no workspace)
    recurrent_step(q, k, v, beta, log_a, S, form="page")               -> (o, S_new)
    precond_scan(k, beta, eta, r=None, d0=None)                        -> (kw, d_T), the write keys
                                                                          of the preconditioned rule
    precond_scan_bwd(k, beta, eta, r, d0, dkw, dd_T)                  -> dict of dk, dbeta, dr, dd0 (the
                                                                          scan's gradients)
    chunk_fwd_save(q, k, v, beta, log_a, S0, cu_seqlens=None, kw=None)  -> (o, S_T, ws), the training forward:
                                                                          ws keeps the transform and the
                                                                          chunk-start states for the backward
    chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T=None, cu_seqlens=None) -> dict of dq, dk, dv, dbeta,
                                                                          dlog_a, dS0 (the gradients; kw=
                                                                          adds dkw; saved=ws takes what
                                                                          chunk_fwd_save kept)
    chunk_attn(q, k, v, beta, log_a=None, S0=None, cu_seqlens=None)    -> (o, S_T) as a torch autograd
                                                                          function (backward: chunk_bwd)
    precond_attn(k, beta, eta, r=None, d0=None)                        -> (kw, d_T) as a torch autograd
                                                                          function (backward: precond_scan_bwd)
    chunk_workspace_size(B, T, H, d_k, d_v, dtype, gate)               -> bytes of scratch
    chunk_varlen_workspace_size(T, n_seq, H, d_k, d_v, dtype, gate)    -> bytes of scratch
    chunk_bwd_workspace_size(B, T, H, d_k, d_v, dtype, gate)           -> bytes of scratch
"""

from ._lib import (EXPORTED, GdrError, LIB_PATH, chunk_attn, chunk_bwd, chunk_bwd_workspace_size, chunk_fwd,
                   chunk_fwd_noalloc, chunk_fwd_save, chunk_fwd_varlen, chunk_varlen_workspace_size, chunk_workspace_size, load, precond_attn,
                   precond_scan, precond_scan_bwd, precond_scan_bwd_workspace_size, recurrent_step)

__all__ = ["EXPORTED", "GdrError", "LIB_PATH", "chunk_attn", "chunk_bwd", "chunk_bwd_workspace_size", "chunk_fwd",
           "chunk_fwd_noalloc", "chunk_fwd_save", "chunk_fwd_varlen", "chunk_varlen_workspace_size", "chunk_workspace_size", "load",
           "precond_attn", "precond_scan", "precond_scan_bwd", "precond_scan_bwd_workspace_size", "recurrent_step"]
