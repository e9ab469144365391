"""Runs one scenario of a workgroup-cap test in a process of its own: the
library reads its tuning caps (MUON_CAST_WG_CAP, MUON_F32_SCALE_WG_CAP) once
per process, so a test that lowers one starts this module with the variable
set, and compares what it saves with its own results.

    python -m tests.cap_child <scenario> <inputs.npz> <outputs.npz>

Scenarios: "cast" (X0, NS5 and the fused Muon step of the batched entry
points) and "f32scale" (the float32 iteration, steps 5 and 0)."""

import sys

import numpy as np


def run(scenario, d):
    """The scenario's outputs (a flat list of arrays) for the arrays of the
    .npz ``d``; also called in-process by the tests for the reference run."""
    import torch

    from newton_schulz_09_amd import muon
    n = int(d["n"])
    Gs = [torch.from_numpy(np.ascontiguousarray(d[f"G{k}"])).cuda() for k in range(n)]
    outs = []
    if scenario == "cast":
        bufs = [torch.from_numpy(np.ascontiguousarray(d[f"B{k}"])).cuda() for k in range(n)]
        outs += muon.ns5_batched(Gs, steps=0)
        outs += muon.ns5_batched(Gs)
        outs += muon.ns5_batched(Gs, bufs=bufs)
        outs += bufs
    elif scenario == "f32scale":
        outs += muon.newton_schulz_f32(Gs)
        outs += muon.newton_schulz_f32(Gs, steps=0)
    else:
        raise ValueError(scenario)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def main():
    scenario, src, dst = sys.argv[1:4]
    with np.load(src) as d:
        res = run(scenario, d)
    np.savez(dst, *res)
    print(f"cap_child {scenario}: {len(res)} arrays", flush=True)


if __name__ == "__main__":
    main()
