"""A fixed set of library calls on seeded inputs, for the serialized-launch check
(tests/test_gpu_serialized.py): run in the test process and again in a child
process whose HIP runtime serializes every kernel launch (AMD_SERIALIZE_KERNEL).

    python tests/serial_run.py OUT.npz     # writes every result to OUT.npz

No oracle here: the two runs are compared with each other, bit for bit."""

from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run_all() -> dict:
    import torch
    import gated_delta_rule_21_amd as gdr
    from workloads import Workload, chunk_inputs, decode_inputs, grad_inputs, precond_inputs, DECODE_CONFIG

    out = {}

    def keep(prefix, **ts):
        for n, t in ts.items():
            if t is not None:
                out[f"{prefix}.{n}"] = t.detach().float().cpu().numpy()

    def dev(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()

    for gate, seed in (("scalar", 501), ("channel", 502), ("none", 503)):
        wl = Workload(f"serial_{gate}", B=2, T=1000, H=4, d_k=128, d_v=128, io="bf16", gate=gate, s0_std=0.1,
                      seed=seed)
        x = chunk_inputs(wl)
        x.update(grad_inputs(wl))
        q, k, v, beta, log_a = (dev(x[n]) for n in ("q", "k", "v", "beta", "log_a"))
        S0 = torch.from_numpy(x["S0"]).cuda()
        dO, dS_T = dev(x["dO"]), torch.from_numpy(x["dS_T"]).cuda()
        o, S_T = gdr.chunk_fwd(q, k, v, beta, log_a, S0)
        keep(f"fwd_{gate}", o=o, S_T=S_T)
        g = gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T)
        keep(f"bwd_{gate}", **g)
        o2, S2, ws = gdr.chunk_fwd_save(q, k, v, beta, log_a, S0)
        g2 = gdr.chunk_bwd(q, k, v, beta, log_a, S0, dO, dS_T, saved=ws)
        keep(f"saved_{gate}", o=o2, S_T=S2, **g2)

    wl = Workload("serial_scan", B=2, T=1000, H=4, d_k=128, d_v=128, io="bf16", gate="scalar", s0_std=0.0, seed=504)
    x = precond_inputs(wl)
    kw, d_T = gdr.precond_scan(dev(x["k"]), dev(x["beta"]), 0.5, dev(x["r"]), torch.from_numpy(x["d0"]).cuda())
    keep("scan", kw=kw, d_T=d_T)

    dwl = DECODE_CONFIG.replace(N=16, H=4, steps=20)
    d = decode_inputs(dwl)
    S = torch.from_numpy(d["S0"]).cuda()
    for s in range(20):
        o, S = gdr.recurrent_step(dev(d["q"][s]), dev(d["k"][s]), dev(d["v"][s]), dev(d["beta"][s]),
                                  dev(d["log_a"][s]), S)
        keep(f"decode{s}", o=o)
    keep("decode", S=S)
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    print(f"serial_run: AMD_SERIALIZE_KERNEL={os.environ.get('AMD_SERIALIZE_KERNEL')}", flush=True)
    np.savez(sys.argv[1], **run_all())
    print("serial_run: done", flush=True)
