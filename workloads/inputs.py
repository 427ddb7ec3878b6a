"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and rounds them to the I/O dtype.  It
holds none of the recurrence's arithmetic, so both the CPU oracle and the GPU
path can take their inputs from here without sharing any computation.

Recipe (per workload, per (batch b, head h) slice, so a sampled slice can be
regenerated on its own):

  * stream  = numpy PCG64 seeded with SeedSequence([seed, b, h]).
  * one draw of a [T, 2*d_k + d_v + 1 + g] standard-normal array in row-major
    order, where g = 0 (no gate), 1 (scalar gate) or d_k (per-channel gate);
    row t holds [q_t | k_t | v_t | beta logit | gate logit(s)].  Because rows
    are drawn in order, the inputs for a shorter T are a prefix of those for a
    longer T.
  * q_t, k_t are divided by their own L2 norm (unit keys and queries);
    beta = sigmoid(logit); log_a = -softplus(logit).
  * S0 (when requested) comes from a second stream SeedSequence([seed, b, h, 1])
    as N(0, s0_std^2) in a [d_k, d_v] array; otherwise it is zero.
  * every tensor is rounded float64 -> float32 (round to nearest even) and, for
    bf16 I/O, float32 -> bf16 (round to nearest even).  S0 stays float32.

Preconditioner-scan inputs reuse k and beta of the (b, h) slice above (the
scan runs over the same keys as the forward) and draw, per (b, h), the
retention r_t = sigmoid(z + 3) (z standard normal, stream SeedSequence([seed, b,
h, 2]); median 0.95, all in (0, 1)) and a starting preconditioner
d0 ~ U(0.5, 1.5) (stream SeedSequence([seed, b, h, 3]), float32).  The step
size is PRECOND_ETA.  The pages give no value for either; these keep d of order
one over long sequences.

Backward workloads add, per (b, h), the gradients of a loss L = <dO, o> +
<dS_T, S_T>: dO ~ N(0, 1) as a [T, d_v] array (stream SeedSequence([seed, b, h,
4]), rounded like the inputs) and dS_T ~ N(0, 1) as [d_k, d_v] float32 (stream
SeedSequence([seed, b, h, 5])), the scale of the outputs and states they stand for.

Decode workloads draw, per (sequence n, head h), S0 from SeedSequence([seed, n,
h, 1]) and the token stream from SeedSequence([seed, n, h]) as a [steps,
2*d_k + d_v + 2] array (row s = step s: q, k, v, beta logit, gate logit).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "CONFIGS", "DECODE_CONFIG", "round_to_io", "bf16_round",
    "slice_inputs", "chunk_inputs", "decode_slice", "decode_inputs", "PRECOND_ETA",
    "precond_slice", "precond_inputs", "precond_factors", "grad_slice", "grad_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape, dtype and distribution of one chunk-forward workload."""
    name: str
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    chunk: int = 64
    io: str = "bf16"          # "f32" or "bf16": dtype of q, k, v, beta, log_a and o
    gate: str = "none"        # "none", "scalar" or "channel"
    s0_std: float = 0.0       # 0 => S0 = 0
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """Shape and distribution of the recurrent decode-step workload."""
    name: str
    N: int                     # independent sequences
    H: int
    d_k: int
    d_v: int
    steps: int
    io: str = "bf16"
    gate: str = "scalar"
    s0_std: float = 0.02
    seed: int = 5

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# The five workloads the path is measured and checked on.
CONFIGS: Dict[int, Workload] = {
    1: Workload("deltanet_b1h1t256d64_f32", B=1, T=256, H=1, d_k=64, d_v=64, io="f32",
                gate="none", s0_std=0.0, seed=1),
    2: Workload("deltanet_b4h16t4096d128_bf16", B=4, T=4096, H=16, d_k=128, d_v=128, io="bf16",
                gate="none", s0_std=0.0, seed=2),
    3: Workload("gated_deltanet_scalar_b8h16t8192d128_bf16", B=8, T=8192, H=16, d_k=128, d_v=128,
                io="bf16", gate="scalar", s0_std=0.0, seed=3),
    4: Workload("kda_channel_b2h32t32768d128_bf16", B=2, T=32768, H=32, d_k=128, d_v=128,
                io="bf16", gate="channel", s0_std=0.02, seed=4),
}
DECODE_CONFIG = DecodeWorkload("decode_gated_n256h32d128_bf16_state_f32", N=256, H=32, d_k=128,
                               d_v=128, steps=1000, io="bf16", gate="scalar", s0_std=0.02, seed=5)


def bf16_round(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    holding bf16-representable values.  NaN/Inf are not expected here."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def round_to_io(x: np.ndarray, io: str) -> np.ndarray:
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if io == "f32":
        return x32
    if io == "bf16":
        return bf16_round(x32)
    raise ValueError(f"unknown io dtype {io!r}")


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _neg_softplus(x: np.ndarray) -> np.ndarray:
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def _gate_width(gate: str, d_k: int) -> int:
    return {"none": 0, "scalar": 1, "channel": d_k}[gate]


def slice_inputs(wl: Workload, b: int, h: int, T: Optional[int] = None) -> dict:
    """Inputs of one (b, h) slice: q, k [T, d_k]; v [T, d_v]; beta [T];
    log_a None / [T] / [T, d_k]; S0 [d_k, d_v] float32.  All float32 arrays
    holding values exactly representable in the I/O dtype."""
    T = wl.T if T is None else T
    dk, dv = wl.d_k, wl.d_v
    g = _gate_width(wl.gate, dk)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h])))
    z = rng.standard_normal((T, 2 * dk + dv + 1 + g))
    q = _unit_rows(z[:, :dk])
    k = _unit_rows(z[:, dk:2 * dk])
    v = z[:, 2 * dk:2 * dk + dv]
    beta = _sigmoid(z[:, 2 * dk + dv])
    if wl.gate == "none":
        log_a = None
    elif wl.gate == "scalar":
        log_a = round_to_io(_neg_softplus(z[:, 2 * dk + dv + 1]), wl.io)
    else:
        log_a = round_to_io(_neg_softplus(z[:, 2 * dk + dv + 1:]), wl.io)
    if wl.s0_std > 0.0:
        rs = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h, 1])))
        S0 = (wl.s0_std * rs.standard_normal((dk, dv))).astype(np.float32)
    else:
        S0 = np.zeros((dk, dv), np.float32)
    return dict(q=round_to_io(q, wl.io), k=round_to_io(k, wl.io), v=round_to_io(v, wl.io),
                beta=round_to_io(beta, wl.io), log_a=log_a, S0=S0)


def chunk_inputs(wl: Workload, T: Optional[int] = None) -> dict:
    """Full-workload inputs in the token-major layout: q, k [B, T, H, d_k];
    v [B, T, H, d_v]; beta [B, T, H]; log_a None / [B, T, H] / [B, T, H, d_k];
    S0 [B, H, d_k, d_v] (float32; zeros when s0_std == 0)."""
    T = wl.T if T is None else T
    B, H, dk, dv = wl.B, wl.H, wl.d_k, wl.d_v
    q = np.empty((B, T, H, dk), np.float32)
    k = np.empty((B, T, H, dk), np.float32)
    v = np.empty((B, T, H, dv), np.float32)
    beta = np.empty((B, T, H), np.float32)
    log_a = None
    if wl.gate == "scalar":
        log_a = np.empty((B, T, H), np.float32)
    elif wl.gate == "channel":
        log_a = np.empty((B, T, H, dk), np.float32)
    S0 = np.zeros((B, H, dk, dv), np.float32)
    for b in range(B):
        for h in range(H):
            s = slice_inputs(wl, b, h, T)
            q[b, :, h] = s["q"]
            k[b, :, h] = s["k"]
            v[b, :, h] = s["v"]
            beta[b, :, h] = s["beta"]
            if log_a is not None:
                log_a[b, :, h] = s["log_a"]
            S0[b, h] = s["S0"]
    return dict(q=q, k=k, v=v, beta=beta, log_a=log_a, S0=S0)


def decode_slice(wl: DecodeWorkload, n: int, h: int, steps: Optional[int] = None) -> dict:
    """Token stream and initial state of one (sequence, head): q, k [steps, d_k];
    v [steps, d_v]; beta [steps]; log_a None / [steps] / [steps, d_k]; S0 [d_k, d_v]."""
    steps = wl.steps if steps is None else steps
    dk, dv = wl.d_k, wl.d_v
    g = _gate_width(wl.gate, dk)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, n, h])))
    z = rng.standard_normal((steps, 2 * dk + dv + 1 + g))
    rs = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, n, h, 1])))
    S0 = (wl.s0_std * rs.standard_normal((dk, dv))).astype(np.float32)
    log_a = None
    if wl.gate == "scalar":
        log_a = round_to_io(_neg_softplus(z[:, 2 * dk + dv + 1]), wl.io)
    elif wl.gate == "channel":
        log_a = round_to_io(_neg_softplus(z[:, 2 * dk + dv + 1:]), wl.io)
    return dict(q=round_to_io(_unit_rows(z[:, :dk]), wl.io),
                k=round_to_io(_unit_rows(z[:, dk:2 * dk]), wl.io),
                v=round_to_io(z[:, 2 * dk:2 * dk + dv], wl.io),
                beta=round_to_io(_sigmoid(z[:, 2 * dk + dv]), wl.io),
                log_a=log_a, S0=S0)


def decode_inputs(wl: DecodeWorkload, steps: Optional[int] = None) -> dict:
    """All slices: q, k [steps, N, H, d_k]; v [steps, N, H, d_v]; beta [steps, N, H];
    log_a None / [steps, N, H] / [steps, N, H, d_k]; S0 [N, H, d_k, d_v] float32."""
    steps = wl.steps if steps is None else steps
    N, H, dk, dv = wl.N, wl.H, wl.d_k, wl.d_v
    q = np.empty((steps, N, H, dk), np.float32)
    k = np.empty((steps, N, H, dk), np.float32)
    v = np.empty((steps, N, H, dv), np.float32)
    beta = np.empty((steps, N, H), np.float32)
    log_a = None
    if wl.gate == "scalar":
        log_a = np.empty((steps, N, H), np.float32)
    elif wl.gate == "channel":
        log_a = np.empty((steps, N, H, dk), np.float32)
    S0 = np.empty((N, H, dk, dv), np.float32)
    for n in range(N):
        for h in range(H):
            s = decode_slice(wl, n, h, steps)
            q[:, n, h] = s["q"]
            k[:, n, h] = s["k"]
            v[:, n, h] = s["v"]
            beta[:, n, h] = s["beta"]
            if log_a is not None:
                log_a[:, n, h] = s["log_a"]
            S0[n, h] = s["S0"]
    return dict(q=q, k=k, v=v, beta=beta, log_a=log_a, S0=S0)


PRECOND_ETA = 1.0


def _precond_factor_slice(wl: Workload, b: int, h: int, T: int):
    rr = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h, 2])))
    r = round_to_io(_sigmoid(rr.standard_normal(T) + 3.0), wl.io)
    rd = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h, 3])))
    d0 = rd.uniform(0.5, 1.5, wl.d_k).astype(np.float32)
    return r, d0


def precond_slice(wl: Workload, b: int, h: int, T: Optional[int] = None) -> dict:
    """Preconditioner-scan inputs of one (b, h) slice: k [T, d_k]; beta [T];
    r [T] (retention); d0 [d_k] float32."""
    T = wl.T if T is None else T
    s = slice_inputs(wl, b, h, T)
    r, d0 = _precond_factor_slice(wl, b, h, T)
    return dict(k=s["k"], beta=s["beta"], r=r, d0=d0)


def precond_factors(wl: Workload, T: Optional[int] = None) -> dict:
    """The scan's own inputs for all slices (the keys and beta being those of
    chunk_inputs): r [B, T, H]; d0 [B, H, d_k] float32."""
    T = wl.T if T is None else T
    r = np.empty((wl.B, T, wl.H), np.float32)
    d0 = np.empty((wl.B, wl.H, wl.d_k), np.float32)
    for b in range(wl.B):
        for h in range(wl.H):
            r[b, :, h], d0[b, h] = _precond_factor_slice(wl, b, h, T)
    return dict(r=r, d0=d0)


def precond_inputs(wl: Workload, T: Optional[int] = None) -> dict:
    """All slices: k [B, T, H, d_k]; beta, r [B, T, H]; d0 [B, H, d_k] float32."""
    T = wl.T if T is None else T
    B, H, dk = wl.B, wl.H, wl.d_k
    k = np.empty((B, T, H, dk), np.float32)
    beta = np.empty((B, T, H), np.float32)
    r = np.empty((B, T, H), np.float32)
    d0 = np.empty((B, H, dk), np.float32)
    for b in range(B):
        for h in range(H):
            s = precond_slice(wl, b, h, T)
            k[b, :, h] = s["k"]
            beta[b, :, h] = s["beta"]
            r[b, :, h] = s["r"]
            d0[b, h] = s["d0"]
    return dict(k=k, beta=beta, r=r, d0=d0)


def grad_slice(wl: Workload, b: int, h: int, T: Optional[int] = None) -> dict:
    """Output gradients of one (b, h) slice: dO [T, d_v] (I/O dtype values);
    dS_T [d_k, d_v] float32."""
    T = wl.T if T is None else T
    ro = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h, 4])))
    dO = round_to_io(ro.standard_normal((T, wl.d_v)), wl.io)
    rs = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h, 5])))
    dS_T = rs.standard_normal((wl.d_k, wl.d_v)).astype(np.float32)
    return dict(dO=dO, dS_T=dS_T)


def grad_inputs(wl: Workload, T: Optional[int] = None) -> dict:
    """All slices: dO [B, T, H, d_v]; dS_T [B, H, d_k, d_v] float32."""
    T = wl.T if T is None else T
    dO = np.empty((wl.B, T, wl.H, wl.d_v), np.float32)
    dS_T = np.empty((wl.B, wl.H, wl.d_k, wl.d_v), np.float32)
    for b in range(wl.B):
        for h in range(wl.H):
            g = grad_slice(wl, b, h, T)
            dO[b, :, h], dS_T[b, h] = g["dO"], g["dS_T"]
    return dict(dO=dO, dS_T=dS_T)
