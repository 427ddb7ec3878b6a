"""Stage-level GPU checks of the chunk forward's state-independent transform.

The transform writes one record per (sequence, head, chunk) into the caller's
workspace; the state pass only reads those records, q, k, v and the state.  Each
test runs gdr_chunk_fwd with a caller-owned workspace, copies the workspace back
and compares every record with the fp64 chunk form (tests/chunk_form.py, itself
checked against the token-by-token oracle by pin P-h) on the same bf16- or
fp32-exact inputs:

- T = (I + A)^-1 with A = strict_lower(diag(beta) (K e^{g_read})(K~ e^{-g})^T),
  the UT/WY transform of "Moonshot AI's New Attention Architecture: Key
  Innovations Explained", §3 Hardware-Friendly Algorithm (K~ = the write key of
  "OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
  Attention", §2.1, K~ = K without one), compared as T - I;
- P = lower_incl((Q e^{g})(K~ e^{-g})^T), the masked intra-chunk scores of the
  same section, where the transform forms them (fp32 I/O and the per-channel gate);
- the gate rows without a gate or with a scalar gate (beta, e^{g_read}, e^{g},
  e^{g_C - g}, e^{g_C}, g; g the inclusive running sum of log a inside the
  chunk, g_C its last valid value); for the per-channel gate the mark of chunks
  whose decay within a 16-token block leaves the split factors' range, and in
  bf16 also beta, e^{g_C} per channel and the three decayed operands
  K e^{g_read}, Q e^{g}, K~ e^{g_C - g}.

Only the rows and columns of real tokens are compared (the ragged last chunk
of T = 200 has 8).  The record layout is the library's internal one: blocks of
16 x 16 elements in the order (0,0) (1,0) (1,1) (2,0) ... (3,3); a T block
holds (T_RJ)^T, a P block P_RJ; six fp32 rows of 64 after the twenty blocks; for
the per-channel gate, three 64 x d_k bf16 operands after those.
Tolerances: 2e-2 relative L2 for bf16 records and products, 1e-4 for fp32, 2e-5
for the fp32 gate rows.
"""

import numpy as np
import pytest

from tests.chunk_form import chunk_forward
from tests.gpu_util import dev, need_gpu, say, torch
from tests.report import report
from oracle import rel_l2
from workloads import Workload, chunk_inputs

pytestmark = pytest.mark.gpu

CH = 64
BLOCKS = [(R, J) for R in range(4) for J in range(R + 1)]


def _rec_layout(io, gate, dk):
    esz = 2 if io == "bf16" else 4
    t_off, p_off, f_off = 0, 10 * 256 * esz, 20 * 256 * esz
    nbytes = f_off + 6 * CH * 4
    x_off = nbytes
    if io == "bf16" and gate == "channel":
        nbytes += 3 * CH * dk * 2
    return esz, t_off, p_off, f_off, x_off, nbytes


def _elems(buf, io):
    if io == "f32":
        return np.frombuffer(buf.tobytes(), np.float32).astype(np.float64)
    u = np.frombuffer(buf.tobytes(), np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _blocks(rec, off, io, esz, transposed):
    """The 64 x 64 matrix held by the ten blocks at byte offset `off`."""
    M = np.zeros((CH, CH))
    for u, (R, J) in enumerate(BLOCKS):
        blk = _elems(rec[off + u * 256 * esz: off + (u + 1) * 256 * esz], io).reshape(16, 16)
        M[16 * R:16 * R + 16, 16 * J:16 * J + 16] = blk.T if transposed else blk
    return M


def _check(name, got, ref, tol, minus_identity=False):
    if minus_identity:
        got, ref = got - np.eye(len(got)), ref - np.eye(len(ref))
    e = rel_l2(got, ref) if np.any(ref) else float(np.max(np.abs(got)))
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert e <= tol, f"{name}: rel_l2 {e:.3e} > {tol:.1e}"
    return e


def _run(inp, io, gate, form="page", kw=None, expect_marked=()):
    need_gpu()
    import gated_delta_rule_21_amd as gdr
    B, T, H, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    nch = -(-T // CH)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    ws = torch.zeros(gdr.chunk_workspace_size(B, T, H, dk, dv, dt, gate), dtype=torch.uint8, device="cuda")
    gdr.chunk_fwd(dev(inp["q"], io), dev(inp["k"], io), dev(inp["v"], io), dev(inp["beta"], io),
                  dev(inp["log_a"], io), torch.from_numpy(inp["S0"]).cuda(), form=form, workspace=ws,
                  kw=None if kw is None else dev(kw, io))
    torch.cuda.synchronize()
    wsh = ws.cpu().numpy()
    esz, t_off, p_off, f_off, x_off, rb = _rec_layout(io, gate, dk)
    tol = 2e-2 if io == "bf16" else 1e-4
    worst = {}
    for b in range(B):
        for h in range(H):
            sl = lambda x: None if x is None else x[b:b + 1, :, h:h + 1]
            kws = sl(kw)
            _, _, inter = chunk_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]),
                                        sl(inp["log_a"]), inp["S0"][b:b + 1, h:h + 1], CH, form=form, keep=True,
                                        kw=kws)
            for n, it in enumerate(inter):
                c = it["T"].shape[0]
                rec = wsh[((b * H + h) * nch + n) * rb:((b * H + h) * nch + n + 1) * rb]
                f = np.frombuffer(rec[f_off:f_off + 6 * CH * 4].tobytes(), np.float32).astype(np.float64)
                f = f.reshape(6, CH)
                rows = slice(n * CH, n * CH + c)
                be = inp["beta"][b, rows, h].astype(np.float64)
                errs = {"T": _check(f"T b{b} h{h} n{n}", _blocks(rec, t_off, io, esz, True)[:c, :c], it["T"], tol,
                                    minus_identity=True)}
                if io == "f32" or gate == "channel":
                    errs["P"] = _check(f"P b{b} h{h} n{n}", _blocks(rec, p_off, io, esz, False)[:c, :c], it["P"], tol)
                if gate in ("none", "scalar"):
                    errs["beta"] = _check("beta", f[0, :c], be, 2e-5)
                    g = it["g"][:, 0]
                    la = np.zeros(c) if inp["log_a"] is None else inp["log_a"][b, rows, h].astype(np.float64)
                    g_read = g if form == "page" else g - la
                    for i, ref in enumerate([np.exp(g_read), np.exp(g), np.exp(g[-1] - g), np.exp(g[-1]) + 0 * g]):
                        errs[f"f{i + 1}"] = _check(f"factor row {i + 1} b{b} h{h} n{n}", f[i + 1, :c], ref, 2e-5)
                    errs["g"] = _check(f"g b{b} h{h} n{n}", f[5, :c], g, 2e-5)
                if gate == "channel":
                    mark = f[5, 0]
                    assert mark == (1.0 if (b, h, n) in expect_marked else 0.0), \
                        f"mark of chunk b{b} h{h} n{n}: {mark}"
                if gate == "channel" and io == "bf16":
                    g = it["g"]
                    la = inp["log_a"][b, rows, h].astype(np.float64)
                    g_read = g if form == "page" else g - la
                    K = inp["k"][b, rows, h].astype(np.float64)
                    Q = inp["q"][b, rows, h].astype(np.float64)
                    KW = K if kw is None else kw[b, rows, h].astype(np.float64)
                    errs["beta"] = _check("beta", f[0, :c], be, 2e-5)
                    errs["eC"] = _check(f"e^gC b{b} h{h} n{n}", f[1:3].reshape(-1)[:dk], np.exp(g[-1]), 2e-5)
                    X = _elems(rec[x_off:x_off + 3 * CH * dk * 2], "bf16").reshape(3, CH, dk)
                    for i, ref in enumerate([K * np.exp(g_read), Q * np.exp(g), KW * np.exp(g[-1] - g)]):
                        errs[f"x{i}"] = _check(f"operand {i} b{b} h{h} n{n}", X[i, :c], ref, 1e-2)
                for key, e in errs.items():
                    worst[key] = max(worst.get(key, 0.0), e)
    line = ", ".join(f"{k} {v:.2e}" for k, v in sorted(worst.items()))
    say("  worst per record field: " + line)
    report(f"transform records io={io} d_k={dk} gate={gate} form={form}{' write key' if kw is not None else ''}"
           f" ({B * H * nch} records): {line}")


def _wl(B, T, H, dk, dv, io, gate, seed):
    return Workload("stages", B=B, T=T, H=H, d_k=dk, d_v=dv, io=io, gate=gate, s0_std=0.02, seed=seed)


@pytest.mark.parametrize("io,dk", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_transform_records(io, dk, gate):
    if gate == "channel" and io == "bf16" and dk != 128:
        pytest.skip("the per-channel bf16 forward takes d_k = 128")
    if gate == "channel" and io == "f32" and dk != 64:
        pytest.skip("the per-channel fp32 forward takes d_k = 64")
    say(f"case transform records io={io} d_k={dk} gate={gate}")
    _run(chunk_inputs(_wl(2, 200, 3, dk, 128, io, gate, seed=101 + dk + len(gate))), io, gate)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_transform_records_literal(io, gate):
    dk = 128 if io == "bf16" else 64
    say(f"case transform records, literal form, io={io} gate={gate}")
    _run(chunk_inputs(_wl(1, 150, 2, dk, 64, io, gate, seed=131)), io, gate, form="literal")


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_transform_records_write_key(gate):
    inp = chunk_inputs(_wl(1, 200, 2, 128, 128, "bf16", gate, seed=151))
    rng = np.random.default_rng(152)
    kw = (inp["k"] * rng.uniform(0.2, 2.0, inp["k"].shape)).astype(np.float32)
    kw = (torch.from_numpy(kw).to(torch.bfloat16).float().numpy()) if torch is not None else kw
    say(f"case transform records, write key, gate={gate}")
    _run(inp, "bf16", gate, kw=kw)


@pytest.mark.parametrize("io,form", [("bf16", "page"), ("bf16", "literal"), ("f32", "page")])
def test_transform_records_marked_chunks(io, form):
    """Channels that decay by e^-6 per token for 20 tokens: their chunks are marked
    and formed by the generic transform; the others keep the split factors."""
    dk = 128 if io == "bf16" else 64
    inp = chunk_inputs(_wl(2, 200, 2, dk, 64, io, "channel", seed=171))
    inp["log_a"][0, 20:40, 1, :16] = -6.0       # chunk 0 of (b 0, h 1)
    inp["log_a"][1, 150:172, 0, 40:] = -6.0     # chunk 2 of (b 1, h 0)
    say(f"case transform records, marked chunks, io={io} form={form}")
    _run(inp, io, "channel", form=form, expect_marked={(0, 1, 0), (1, 0, 2)})
