"""The C-ABI library loads, exports every symbol the header declares, and rejects
bad arguments before anything is launched (CPU only: every call below fails
validation, so no kernel is ever enqueued and no pointer is dereferenced)."""

import ctypes
import os
import re

import pytest

import gated_delta_rule_21_amd as gdr
from gated_delta_rule_21_amd._lib import GdrDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP = range(6)
FAKE = 0x10000          # a 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdr.LIB_PATH):
        from gated_delta_rule_21_amd.build import build
        build()
    return gdr.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gdr_\w+)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    assert set(declared_functions()) == set(gdr.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in gdr.h but not exported"


def test_status_strings(lib):
    for s in range(6):
        assert lib.gdr_status_string(s).startswith(b"GDR_")
    assert b"WORKSPACE" in lib.gdr_status_string(WORKSPACE)
    assert lib.gdr_version() >= 100


def _desc(**kw):
    d = dict(B=1, T=8, H=2, d_k=128, d_v=128, chunk=64, io=1, gate=1, form=0)
    d.update(kw)
    return GdrDesc(**d)


def _ptrs(n=9, start=FAKE, stride=1 << 24):
    return [start + i * stride for i in range(n)]


def _ws_size(lib, d):
    n = ctypes.c_size_t(12345)
    st = lib.gdr_chunk_fwd_workspace_size(None if d is None else ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def _chunk(lib, d, ptrs, ws_bytes=None):
    q, k, v, beta, log_a, S0, o, S_T = ptrs[:8]
    ws = ptrs[8] if len(ptrs) > 8 else None
    if ws_bytes is None:
        ws_bytes = _ws_size(lib, d)[1] if d is not None else 0
    return lib.gdr_chunk_fwd(None if d is None else ctypes.byref(d), q, k, v, beta, log_a, S0, o, S_T,
                             ws, ws_bytes, None)


def test_workspace_size(lib):
    rec = lambda esz: 2 * 10 * 256 * esz + 6 * 64 * 4    # ten 16x16 blocks of T and of P, six factor rows
    assert _ws_size(lib, _desc(B=2, T=130, H=3)) == (OK, 2 * 3 * 3 * rec(2))        # bf16, 3 chunks
    assert _ws_size(lib, _desc(io=0, d_k=64, T=64)) == (OK, 2 * 1 * rec(4))         # fp32, 1 chunk
    # bf16 with a per-channel gate: the three decayed [64][d_k] operands follow each record
    assert _ws_size(lib, _desc(gate=2, T=65)) == (OK, 2 * 2 * (rec(2) + 3 * 64 * 128 * 2))
    assert _ws_size(lib, _desc(gate=2, d_k=64, T=64)) == (OK, 2 * (rec(2) + 3 * 64 * 64 * 2))
    assert _ws_size(lib, _desc(gate=2, io=0, d_k=64, T=64)) == (OK, 2 * rec(4))     # fp32: no operands
    assert _ws_size(lib, _desc(T=0)) == (OK, 0)
    assert _ws_size(lib, None) == (INVALID, 0)
    assert _ws_size(lib, _desc(d_k=96)) == (UNSUPPORTED, 0)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc()), None) == INVALID


def test_workspace_checks(lib):
    p = _ptrs()
    p[8] = None
    assert _chunk(lib, _desc(), p) == WORKSPACE                # missing workspace
    assert b"workspace" in lib.gdr_last_error()
    need = _ws_size(lib, _desc())[1]
    assert _chunk(lib, _desc(), _ptrs(), ws_bytes=need - 1) == WORKSPACE
    assert b"needed" in lib.gdr_last_error()
    p = _ptrs()
    p[8] += 8
    assert _chunk(lib, _desc(), p) == ALIGN                    # workspace 16-byte alignment
    p = _ptrs()
    p[8] = p[6] + 64                                           # workspace inside o
    assert _chunk(lib, _desc(), p) == INVALID
    assert b"overlaps" in lib.gdr_last_error()


def test_per_sequence_offset_limit(lib):
    """The kernels address one (sequence, head) slice with 32-bit byte offsets: the
    longest sequence at H16 d128 bf16 is T = 524,287 (T*H*d*2 = 2^31 - 4096); one
    token more is refused before anything is enqueued, by the size query and the call."""
    assert _ws_size(lib, _desc(B=1, T=524287, H=16))[0] == OK
    assert _ws_size(lib, _desc(B=1, T=524288, H=16))[0] == UNSUPPORTED
    assert b"2^31 - 1 per sequence" in lib.gdr_last_error()
    assert _chunk(lib, _desc(B=1, T=524288, H=16), _ptrs(), ws_bytes=1 << 40) == UNSUPPORTED
    assert _ws_size(lib, _desc(B=1, T=524287, H=16, io=0, d_k=64, d_v=64))[0] == OK     # fp32 d64: as many bytes
    assert _ws_size(lib, _desc(B=1, T=524288, H=16, io=0, d_k=64, d_v=64))[0] == UNSUPPORTED
    assert _ws_size(lib, _desc(B=1, T=1048575, H=8))[0] == OK                            # half the heads: twice T
    assert _ws_size(lib, _desc(B=1, T=1048576, H=8))[0] == UNSUPPORTED


def test_null_desc(lib):
    assert _chunk(lib, None, _ptrs()) == INVALID
    assert b"desc" in lib.gdr_last_error()


@pytest.mark.parametrize("field,value,code", [
    ("d_k", 96, UNSUPPORTED), ("d_v", 256, UNSUPPORTED), ("chunk", 32, UNSUPPORTED),
    ("io", 7, INVALID), ("gate", 3, INVALID), ("form", 2, INVALID),
    ("B", 0, INVALID), ("H", -1, INVALID), ("T", -5, INVALID),
])
def test_bad_descriptor_fields(lib, field, value, code):
    assert _chunk(lib, _desc(**{field: value}), _ptrs()) == code


def test_fp32_io_with_dk128_per_channel_gate_is_unsupported(lib):
    # fp32 I/O at d_k = 128 is offered without a gate or with a scalar gate only
    assert _chunk(lib, _desc(io=0, gate=2), _ptrs()) == UNSUPPORTED
    n = ctypes.c_size_t(7)
    for gate, code in ((0, OK), (1, OK), (2, UNSUPPORTED)):
        assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(_desc(io=0, gate=gate)), ctypes.byref(n)) == code, gate


@pytest.mark.parametrize("which", range(5))
def test_null_required_pointer(lib, which):
    p = _ptrs()
    p[[0, 1, 2, 3, 6][which]] = None
    assert _chunk(lib, _desc(), p) == INVALID


def test_gate_pointer_consistency(lib):
    p = _ptrs()
    p[4] = None
    assert _chunk(lib, _desc(gate=1), p) == INVALID          # gate requested, no log_a
    assert _chunk(lib, _desc(gate=0), _ptrs()) == INVALID    # log_a given without a gate


def test_misaligned_pointers(lib):
    for idx in (0, 1, 2, 6, 5, 7):
        p = _ptrs()
        p[idx] += 8
        assert _chunk(lib, _desc(), p) == ALIGN, idx
    p = _ptrs()
    p[3] += 1                                                  # beta (bf16) must be 2-byte aligned
    assert _chunk(lib, _desc(), p) == ALIGN


def test_output_overlapping_input_is_rejected(lib):
    p = _ptrs()
    p[6] = p[0] + 64                                           # o inside q
    assert _chunk(lib, _desc(), p) == INVALID
    assert b"overlaps" in lib.gdr_last_error()
    p = _ptrs()
    p[7] = p[5] + 256                                          # S_T partially over S0
    assert _chunk(lib, _desc(), p) == INVALID


def _step(lib, d, ptrs):
    q, k, v, beta, log_a, S, S_new, o = ptrs[:8]
    return lib.gdr_recurrent_step(ctypes.byref(d), q, k, v, beta, log_a, S, S_new, o, None)


def test_decode_checks(lib):
    assert _step(lib, _desc(T=4), _ptrs()) == INVALID           # one token per step
    p = _ptrs()
    p[6] = p[5] + 1024                                          # S_new partially over S
    assert _step(lib, _desc(T=1), p) == INVALID
    p = _ptrs()
    p[5] = None
    assert _step(lib, _desc(T=1), p) == INVALID
    assert _step(lib, _desc(T=1, d_k=32), _ptrs()) == UNSUPPORTED


# ---- packed variable-length sequences -------------------------------------------------------
def _ws_varlen(lib, d, n_seq):
    n = ctypes.c_size_t(12345)
    st = lib.gdr_chunk_fwd_varlen_workspace_size(None if d is None else ctypes.byref(d), n_seq, ctypes.byref(n))
    return st, n.value


def _chunk_varlen(lib, d, cu, n_seq, ptrs, ws_bytes=None):
    q, k, v, beta, log_a, S0, o, S_T = ptrs[:8]
    ws = ptrs[8] if len(ptrs) > 8 else None
    if ws_bytes is None:
        ws_bytes = _ws_varlen(lib, d, n_seq)[1] if d is not None else 0
    return lib.gdr_chunk_fwd_varlen(None if d is None else ctypes.byref(d), cu, n_seq, q, k, v, beta, log_a, S0, o,
                                    S_T, ws, ws_bytes, None)


def test_varlen_workspace_size(lib):
    rec = 2 * 10 * 256 * 2 + 6 * 64 * 4
    # record slots per head: ceil(T / 64) + n_seq (sequence i starts at slot floor(cu[i] / 64) + i),
    # then the longest-first order of the sequences (n_seq int32, padded to 16 bytes)
    assert _ws_varlen(lib, _desc(T=130, H=3), 4) == (OK, 3 * (3 + 4) * rec + 16)
    assert _ws_varlen(lib, _desc(T=130, H=3), 5) == (OK, 3 * (3 + 5) * rec + 32)
    assert _ws_varlen(lib, _desc(T=130, H=3, gate=2), 2) == (OK, 3 * (3 + 2) * (rec + 3 * 64 * 128 * 2) + 16)
    assert _ws_varlen(lib, _desc(T=130, H=3), 0) == (INVALID, 0)
    assert _ws_varlen(lib, _desc(B=2), 2) == (INVALID, 0)                  # packed tensors take B = 1
    rec32 = 2 * 10 * 256 * 4 + 6 * 64 * 4                                  # fp32 records
    assert _ws_varlen(lib, _desc(io=0, d_k=64), 2) == (OK, 2 * (1 + 2) * rec32 + 16)
    assert _ws_varlen(lib, _desc(io=0, d_k=128, gate=2), 2) == (UNSUPPORTED, 0)   # fp32 per-channel: d_k = 64
    assert _ws_varlen(lib, None, 2) == (INVALID, 0)


def test_varlen_argument_checks(lib):
    cu = FAKE + 0x7F000000                     # never dereferenced
    assert _chunk_varlen(lib, _desc(B=2), cu, 2, _ptrs()) == INVALID
    assert _chunk_varlen(lib, _desc(), None, 2, _ptrs()) == INVALID
    assert b"cu_seqlens" in lib.gdr_last_error()
    assert _chunk_varlen(lib, _desc(), cu, 0, _ptrs()) == INVALID
    assert _chunk_varlen(lib, _desc(io=0, d_k=128, gate=2), cu, 2, _ptrs()) == UNSUPPORTED
    assert _chunk_varlen(lib, _desc(), cu + 2, 2, _ptrs()) == ALIGN
    p = _ptrs()
    assert _chunk_varlen(lib, _desc(), p[6] + 16, 2, p) == INVALID        # offsets inside o
    assert b"overlaps" in lib.gdr_last_error()
    need = _ws_varlen(lib, _desc(), 2)[1]
    assert _chunk_varlen(lib, _desc(), cu, 2, _ptrs(), ws_bytes=need - 1) == WORKSPACE


# ---- write key (the preconditioned delta rule) -------------------------------------------
def _chunk_wkey(lib, d, kw, ptrs, ws_bytes=None):
    q, k, v, beta, log_a, S0, o, S_T = ptrs[:8]
    ws = ptrs[8] if len(ptrs) > 8 else None
    if ws_bytes is None:
        ws_bytes = _ws_size(lib, d)[1] if d is not None else 0
    return lib.gdr_chunk_fwd_wkey(None if d is None else ctypes.byref(d), q, k, kw, v, beta, log_a, S0, o, S_T, ws,
                                  ws_bytes, None)


def test_write_key_chunk_checks(lib):
    kw = FAKE + 0x7F000000                     # never dereferenced
    p = _ptrs()
    p[4] = None
    assert _chunk_wkey(lib, _desc(gate=1), kw, p) == INVALID                # a gate needs log_a
    assert b"log_a" in lib.gdr_last_error()
    assert _chunk_wkey(lib, _desc(gate=2, d_k=64), kw, _ptrs()) == UNSUPPORTED   # per-channel: d_k = 128
    assert _chunk_wkey(lib, _desc(gate=0), kw, _ptrs()) == INVALID          # log_a given without a gate
    assert _chunk_wkey(lib, _desc(gate=0), None, _ptrs()) == INVALID
    assert b"kw" in lib.gdr_last_error()
    assert _chunk_wkey(lib, _desc(gate=1, io=0, d_k=64), kw, _ptrs()) == UNSUPPORTED   # bf16 only
    assert _chunk_wkey(lib, _desc(gate=1), kw + 8, _ptrs()) == ALIGN
    p = _ptrs()
    assert _chunk_wkey(lib, _desc(gate=1), p[6] + 64, p) == INVALID          # kw inside o
    assert b"overlaps" in lib.gdr_last_error()


def test_write_key_step_checks(lib):
    kw = FAKE + 0x7F000000
    p = _ptrs()
    d = _desc(T=1, gate=0)
    call = lambda d, kw, la=None: lib.gdr_recurrent_step_wkey(ctypes.byref(d), p[0], p[1], kw, p[2], p[3], la, p[5],
                                                              p[7], p[6], None)
    assert call(_desc(T=1, gate=1), kw) == INVALID                         # a gate needs log_a
    assert call(d, kw, p[4]) == INVALID                                    # log_a given without a gate
    assert call(d, None) == INVALID
    assert call(d, kw + 4) == ALIGN
    assert call(d, p[7] + 64) == INVALID                                   # kw inside S_new
    assert b"overlaps" in lib.gdr_last_error()


def _scan(lib, d, k, beta, r, eta, d0, kw, d_T):
    return lib.gdr_precond_scan(None if d is None else ctypes.byref(d), k, beta, r, eta, d0, kw, d_T, None)


def test_precond_scan_checks(lib):
    k, beta, r, d0, kw, dT = _ptrs(6)
    d = _desc(gate=0)
    assert _scan(lib, None, k, beta, r, 1.0, d0, kw, dT) == INVALID
    for field, value, code in (("io", 7, INVALID), ("B", 0, INVALID), ("H", 0, INVALID), ("T", -1, INVALID),
                               ("d_k", 96, UNSUPPORTED)):
        assert _scan(lib, _desc(gate=0, **{field: value}), k, beta, r, 1.0, d0, kw, dT) == code, field
    for eta in (float("nan"), float("inf"), -float("inf")):
        assert _scan(lib, d, k, beta, r, eta, d0, kw, dT) == INVALID
    assert _scan(lib, d, None, beta, r, 1.0, d0, kw, dT) == INVALID
    assert _scan(lib, d, k, None, r, 1.0, d0, kw, dT) == INVALID
    assert _scan(lib, d, k, beta, r, 1.0, d0, None, dT) == INVALID
    assert _scan(lib, d, k + 8, beta, r, 1.0, d0, kw, dT) == ALIGN
    assert _scan(lib, d, k, beta, r, 1.0, d0, kw + 8, dT) == ALIGN
    assert _scan(lib, d, k, beta + 1, r, 1.0, d0, kw, dT) == ALIGN
    assert _scan(lib, d, k, beta, r + 1, 1.0, d0, kw, dT) == ALIGN
    assert _scan(lib, d, k, beta, r, 1.0, d0 + 2, kw, dT) == ALIGN
    assert _scan(lib, _desc(gate=0, io=0, d_k=64), k, beta + 2, r, 1.0, d0, kw, dT) == ALIGN   # fp32: 4 bytes
    assert _scan(lib, d, k, beta, r, 1.0, d0, k + 64, dT) == INVALID            # kw inside k
    assert b"kw overlaps k" in lib.gdr_last_error()
    assert _scan(lib, d, k, beta, r, 1.0, d0, kw, kw + 256) == INVALID          # d_T inside kw
    assert _scan(lib, d, k, beta, r, 1.0, d0, kw, d0 + 16) == INVALID           # d_T partly over d0
    assert _scan(lib, d, k, beta, r, 1.0, dT, k + 64, dT) == INVALID            # d_T == d0 is allowed ...
    assert b"kw overlaps k" in lib.gdr_last_error()                             # ... the error is kw's


def _bwd(lib, d, p, ws_bytes=1 << 40):
    """gdr_chunk_bwd with p = (q, k, v, beta, log_a, S0, dO, dS_T, dq, dk, dv, dbeta, dlog_a, dS0, ws)."""
    return lib.gdr_chunk_bwd(None if d is None else ctypes.byref(d), *p[:14], p[14], ws_bytes, None)


def test_backward_workspace_size(lib):
    n = ctypes.c_size_t(7)
    d = _desc(B=2, T=130, H=3)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value == 2 * 3 * 3 * (11776 + 4 * 128 * 128)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(_desc(T=0)), ctypes.byref(n)) == OK and n.value == 0
    for fields, code in (({"io": 0}, UNSUPPORTED), ({"gate": 2, "d_k": 64}, UNSUPPORTED), ({"d_k": 96}, UNSUPPORTED),
                         ({"B": 0}, INVALID), ({"form": 2}, INVALID)):
        n.value = 7
        assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(_desc(**fields)), ctypes.byref(n)) == code, fields
        assert n.value == 0
    # both forms, with and without a gate
    for gate in (0, 1, 2):
        assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(_desc(gate=gate, form=1)), ctypes.byref(n)) == OK
    # per-channel gate (d_k = 128): the records also hold the three decayed [64][d_k] operands
    d = _desc(B=2, T=130, H=3, gate=2)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value == 2 * 3 * 3 * (11776 + 3 * 64 * 128 * 2 + 4 * 128 * 128)


def test_backward_argument_checks(lib):
    p = _ptrs(15)
    d = _desc()
    assert _bwd(lib, None, p) == INVALID
    for i, name in enumerate(("q", "k", "v", "beta", "log_a", None, "dO", None, "dq", "dk", "dv", "dbeta", "dlog_a",
                              None, "workspace")):
        if name is None:          # S0, dS_T and dS0 may be NULL
            continue
        bad = list(p)
        bad[i] = None
        assert _bwd(lib, d, bad) == (WORKSPACE if name == "workspace" else INVALID), name
        assert name.encode() in lib.gdr_last_error()
    assert _bwd(lib, d, p, ws_bytes=16) == WORKSPACE                       # workspace too small
    assert _bwd(lib, _desc(gate=0), p) == INVALID                          # log_a given without a gate
    bad = list(p)
    bad[4] = None
    assert _bwd(lib, _desc(gate=0), bad) == INVALID                        # dlog_a given without a gate
    for i in (0, 6, 8, 13):                                                # 16-byte operands
        bad = list(p)
        bad[i] += 8
        assert _bwd(lib, d, bad) == ALIGN, i
    bad = list(p)
    bad[11] += 1
    assert _bwd(lib, d, bad) == ALIGN                                      # dbeta: 2 bytes
    bad = list(p)
    bad[9] = bad[1] + 64                                                   # dk inside k
    assert _bwd(lib, d, bad) == INVALID
    assert b"dk overlaps k" in lib.gdr_last_error()
    bad = list(p)
    bad[14] = bad[8] + 256                                                 # workspace over dq
    assert _bwd(lib, d, bad) == INVALID
    bad = list(p)
    bad[13] = bad[7]                                                       # dS0 == dS_T is allowed ...
    bad[9] = bad[1] + 64
    assert _bwd(lib, d, bad) == INVALID
    assert b"dk overlaps k" in lib.gdr_last_error()                        # ... the error is dk's


def _bwd_wkey(lib, d, p, ws_bytes=1 << 40):
    """gdr_chunk_bwd_wkey with p = (q, k, kw, v, beta, log_a, S0, dO, dS_T, dq, dk, dkw, dv, dbeta, dlog_a,
    dS0, ws)."""
    return lib.gdr_chunk_bwd_wkey(None if d is None else ctypes.byref(d), *p[:16], p[16], ws_bytes, None)


def test_backward_write_key_checks(lib):
    p = _ptrs(17)
    d = _desc()
    assert _bwd_wkey(lib, None, p) == INVALID
    for i, name in ((2, "kw"), (11, "dkw"), (0, "q"), (9, "dq")):
        bad = list(p)
        bad[i] = None
        assert _bwd_wkey(lib, d, bad) == INVALID, name
        assert name.encode() in lib.gdr_last_error()
    assert _bwd_wkey(lib, _desc(gate=2), p) == UNSUPPORTED                 # no per-channel gate with a write key
    assert _bwd_wkey(lib, _desc(io=0), p) == UNSUPPORTED                   # bf16 only
    assert _bwd_wkey(lib, d, p, ws_bytes=16) == WORKSPACE
    for i in (2, 11):                                                      # kw, dkw: 16-byte operands
        bad = list(p)
        bad[i] += 8
        assert _bwd_wkey(lib, d, bad) == ALIGN, i
    bad = list(p)
    bad[11] = bad[2] + 64                                                  # dkw inside kw
    assert _bwd_wkey(lib, d, bad) == INVALID
    assert b"dkw overlaps kw" in lib.gdr_last_error()
    bad = list(p)
    bad[11] = bad[10]                                                      # dkw == dk
    assert _bwd_wkey(lib, d, bad) == INVALID


def test_backward_varlen_checks(lib):
    n = ctypes.c_size_t(7)
    d = _desc(B=1, T=300, H=2)
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(d), 5, ctypes.byref(n)) == OK
    slots = 2 * (-(-300 // 64) + 5)
    assert n.value == slots * (11776 + 4 * 128 * 128)
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(d), 0, ctypes.byref(n)) == INVALID
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(_desc(B=2, T=300)), 3, ctypes.byref(n)) == INVALID
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(_desc(B=1, io=0)), 3, ctypes.byref(n)) == UNSUPPORTED
    p = _ptrs(16)
    call = lambda d, cu, ns, q=p: lib.gdr_chunk_bwd_varlen(ctypes.byref(d), cu, ns, *q[:14], q[14], 1 << 40, None)
    assert call(d, None, 5) == INVALID                                     # no offsets table
    assert b"cu_seqlens" in lib.gdr_last_error()
    assert call(d, p[15], 0) == INVALID                                    # n_seq < 1
    assert call(_desc(B=2, T=300), p[15], 5) == INVALID                    # B must be 1
    assert call(d, p[15] + 2, 5) == ALIGN                                  # int32 table
    bad = list(p)
    bad[9] = bad[15]                                                       # dk over the offsets table
    assert call(d, p[15], 5, bad) == INVALID


def test_binding_rejects_strided_offsets(lib):
    """The kernels read cu_seqlens as a dense int32 array: a strided view is refused by
    both packed-sequence wrappers before anything reaches the library."""
    import torch
    T, H, d = 40, 2, 64
    x = torch.zeros((1, T, H, d), dtype=torch.bfloat16)
    beta = torch.zeros((1, T, H), dtype=torch.bfloat16)
    cu = torch.tensor([0, 99, 10, 99, 40], dtype=torch.int32)[::2]
    assert not cu.is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        gdr.chunk_bwd(x, x, x, beta, None, None, x, cu_seqlens=cu)
    with pytest.raises(ValueError, match="contiguous"):
        gdr.chunk_fwd_varlen(x, x, x, beta, None, cu)
    with pytest.raises(ValueError, match="GPU tensor"):          # a dense table passes this check
        gdr.chunk_bwd(x, x, x, beta, None, None, x, cu_seqlens=cu.contiguous())


def _scan_bwd(lib, d, p, eta=1.0, ws_bytes=1 << 40):
    """gdr_precond_scan_bwd with p = (k, beta, r, d0, dkw, dd_T, dk, dbeta, dr, dd0, ws)."""
    return lib.gdr_precond_scan_bwd(None if d is None else ctypes.byref(d), p[0], p[1], p[2], ctypes.c_float(eta),
                                    *p[3:10], p[10], ws_bytes, None)


def test_precond_scan_backward_checks(lib):
    n = ctypes.c_size_t(7)
    d = _desc(B=2, T=100, H=3, d_k=64)
    assert lib.gdr_precond_scan_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value == 2 * 3 * 100 * (64 + 2) * 4
    assert lib.gdr_precond_scan_bwd_workspace_size(ctypes.byref(_desc(d_k=96)), ctypes.byref(n)) == UNSUPPORTED
    assert n.value == 0
    p = _ptrs(11)
    d = _desc()
    assert _scan_bwd(lib, None, p) == INVALID
    for i, name in ((0, "k"), (1, "beta"), (6, "dk"), (7, "dbeta")):
        bad = list(p)
        bad[i] = None
        assert _scan_bwd(lib, d, bad) == INVALID, name
        assert name.encode() in lib.gdr_last_error()
    bad = list(p)
    bad[10] = None
    assert _scan_bwd(lib, d, bad) == WORKSPACE
    assert _scan_bwd(lib, d, p, ws_bytes=16) == WORKSPACE
    bad = list(p)
    bad[2] = None                                                          # dr given without r
    assert _scan_bwd(lib, d, bad) == INVALID
    assert _scan_bwd(lib, d, p, eta=float("nan")) == INVALID
    assert _scan_bwd(lib, _desc(d_k=96), p) == UNSUPPORTED
    for i in (0, 4, 6):                                                    # k, dkw, dk: 16-byte operands
        bad = list(p)
        bad[i] += 8
        assert _scan_bwd(lib, d, bad) == ALIGN, i
    bad = list(p)
    bad[6] = bad[0] + 64                                                   # dk inside k
    assert _scan_bwd(lib, d, bad) == INVALID
    assert b"dk overlaps k" in lib.gdr_last_error()
    bad = list(p)
    bad[9] = bad[5] + 4                                                    # dd0 inside dd_T, not equal
    assert _scan_bwd(lib, d, bad) == INVALID


def test_packed_write_key_checks(lib):
    d = _desc(B=1, T=300, H=2)
    p = _ptrs(12)
    fwd = lambda d, cu, ns, q: lib.gdr_chunk_fwd_varlen_wkey(ctypes.byref(d), cu, ns, *q[:9], q[9], 1 << 40, None)
    assert fwd(d, None, 3, p) == INVALID                                   # no offset table
    bad = list(p)
    bad[2] = None
    assert fwd(d, FAKE, 3, bad) == INVALID                                 # no write key
    assert b"kw" in lib.gdr_last_error()
    assert fwd(_desc(B=1, T=300, H=2, io=0), FAKE, 3, p) == UNSUPPORTED    # write key: bf16 only
    q = _ptrs(18)
    bwd = lambda d, cu, ns, q: lib.gdr_chunk_bwd_varlen_wkey(ctypes.byref(d), cu, ns, *q[:16], q[16], 1 << 40, None)
    assert bwd(d, None, 3, q) == INVALID
    for i, name in ((2, "kw"), (11, "dkw")):
        bad = list(q)
        bad[i] = None
        assert bwd(d, FAKE, 3, bad) == INVALID, name
    assert bwd(_desc(B=1, T=300, H=2, gate=2), FAKE, 3, q) == UNSUPPORTED  # no per-channel gate with a write key


def _fwd_save(lib, d, cu, n_seq, p, ws_bytes=1 << 40):
    """gdr_chunk_fwd_save with p = (q, k, kw, v, beta, log_a, S0, o, S_T, ws)."""
    return lib.gdr_chunk_fwd_save(None if d is None else ctypes.byref(d), cu, n_seq, *p[:9], p[9], ws_bytes, None)


def test_training_forward_checks(lib):
    """The training forward takes the backward's configurations and the backward's
    workspace size (its records plus the chunk-start states)."""
    p = _ptrs(11)
    p[2] = None                                                            # no write key
    d = _desc(B=2, T=130, H=3)
    assert _fwd_save(lib, None, None, 0, p) == INVALID
    n_fwd, n_bwd = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.gdr_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n_fwd)) == OK
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n_bwd)) == OK
    assert n_bwd.value > n_fwd.value
    assert _fwd_save(lib, d, None, 0, p, ws_bytes=n_fwd.value) == WORKSPACE    # the forward's size is not enough
    assert _fwd_save(lib, d, None, 0, p, ws_bytes=n_bwd.value - 1) == WORKSPACE
    bad = list(p)
    bad[9] = None
    assert _fwd_save(lib, d, None, 0, bad) == WORKSPACE                    # no workspace
    assert _fwd_save(lib, _desc(io=0, d_k=64, d_v=64), None, 0, p) == UNSUPPORTED   # bf16 only
    assert _fwd_save(lib, _desc(gate=2, d_k=64), None, 0, p) == UNSUPPORTED        # per-channel: d_k = 128
    kw = list(p)
    kw[2] = p[10]
    assert _fwd_save(lib, _desc(gate=2), None, 0, kw) == UNSUPPORTED       # per-channel gate with a write key
    assert _fwd_save(lib, d, None, 3, p) == INVALID                        # n_seq without an offset table
    assert b"cu_seqlens" in lib.gdr_last_error()
    for i, name in ((0, "q"), (1, "k"), (3, "v"), (4, "beta"), (7, "o")):
        bad = list(p)
        bad[i] = None
        assert _fwd_save(lib, d, None, 0, bad) == INVALID, name
    bad = list(p)
    bad[7] = bad[9] + 256                                                  # o inside the workspace
    assert _fwd_save(lib, d, None, 0, bad) == INVALID
    # packed sequences
    dp = _desc(B=1, T=300, H=2)
    assert _fwd_save(lib, _desc(B=2, T=300, H=2), FAKE, 3, p) == INVALID  # B must be 1
    assert _fwd_save(lib, dp, FAKE, 0, p) == INVALID                       # n_seq < 1
    assert _fwd_save(lib, dp, FAKE + 2, 3, p) == ALIGN                     # int32 table
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(dp), 3, ctypes.byref(n)) == OK
    assert _fwd_save(lib, dp, FAKE, 3, p, ws_bytes=n.value - 16) == WORKSPACE


def _bwd_saved(lib, d, cu, n_seq, p, ws_bytes=1 << 40):
    """gdr_chunk_bwd_saved with p = (q, k, kw, v, beta, log_a, S0, dO, dS_T, dq, dk, dkw, dv, dbeta, dlog_a,
    dS0, ws)."""
    return lib.gdr_chunk_bwd_saved(None if d is None else ctypes.byref(d), cu, n_seq, *p[:16], p[16], ws_bytes, None)


def test_saved_backward_checks(lib):
    p = _ptrs(18)
    p[2] = p[11] = None                                                    # no write key
    d = _desc(B=2, T=130, H=3)
    assert _bwd_saved(lib, None, None, 0, p) == INVALID
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert _bwd_saved(lib, d, None, 0, p, ws_bytes=n.value - 1) == WORKSPACE
    bad = list(p)
    bad[16] = None
    assert _bwd_saved(lib, d, None, 0, bad) == WORKSPACE
    assert _bwd_saved(lib, _desc(io=0), None, 0, p) == UNSUPPORTED
    assert _bwd_saved(lib, d, None, 2, p) == INVALID                       # n_seq without an offset table
    half = list(p)
    half[2] = p[17]                                                        # kw without dkw
    assert _bwd_saved(lib, d, None, 0, half) == INVALID
    assert b"kw and dkw" in lib.gdr_last_error()
    both = list(half)
    both[11] = p[17] + (1 << 22)
    assert _bwd_saved(lib, _desc(gate=2), None, 0, both) == UNSUPPORTED    # per-channel gate with a write key
    for i, name in ((0, "q"), (7, "dO"), (9, "dq"), (13, "dbeta")):
        bad = list(p)
        bad[i] = None
        assert _bwd_saved(lib, d, None, 0, bad) == INVALID, name
    bad = list(p)
    bad[10] = bad[1] + 64                                                  # dk inside k
    assert _bwd_saved(lib, d, None, 0, bad) == INVALID
    assert _bwd_saved(lib, _desc(B=2, T=300, H=2), FAKE, 3, p) == INVALID  # packed: B must be 1
